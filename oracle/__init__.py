"""CPU oracle for the 4-bit weight-only mixture-of-experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only the test suite, the graft
smoke check and the benchmark's ``cpu_baseline`` leg use it.  The HIP
library and this package share no code, tables or constants.

Everything is computed in float64 with numpy, as a plain and slow reading
of what the layer computes:

* the layer shape (256 routed experts, 6 chosen per token, one always-on
  shared expert) follows the architecture table in "Recursive Flint: 40B
  Local Coding Model, Benchmarks" (section "What is Recursive Flint?") and
  the table in "Recursive Flint: 125 tok/s on an M4 Pro, measured where it
  matters least" (section "What actually shipped");
* weight-only 4-bit serving (W4A16), the fused top-k router and the
  expert-indexed GEMVs follow "[Model] Add Flint (RecursiveSI/flint)",
  section "What happened";
* the two 4-bit formats (NVFP4, group-64 affine INT4) follow the same
  "What actually shipped" table and "Run the Flint coding model on a CPU
  VPS", section "Which Flint tag to pull on a CPU VPS".

Where the pages are silent (router score function, expert activation,
byte layouts, rounding points) the module docstrings state the reading
taken.  Parity status: every function here is pinned by the CPU tests in
``tests/test_oracle_*.py``; none is "parity unpinned".
"""

from .formats import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    fp16_bits_to_f64,
    e2m1_value,
    e4m3fn_value,
    unpack_nibbles,
    dequant_matrix,
    dequant_matrix_f32,
    rne_bf16,
)
from .moe import (  # noqa: F401
    router_logits,
    topk_select,
    topk_weights,
    route,
    expert_ffn,
    permute,
    grouped_ffn,
    combine,
    moe_layer,
    rms_norm,
    chain_layer,
    dense_gemv,
)
