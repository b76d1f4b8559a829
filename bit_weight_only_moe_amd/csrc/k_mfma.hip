// MFMA grouped GEMM (prefill) -- filled in below.
