// Dense 4-bit GEMV for gfx950: out[t, n] = W[n] . x_t for one packed
// matrix, the shape of the 4-bit output head of "Recursive Flint: 40B Local
// Coding Model, Benchmarks" (section "How Recursive built Flint"; its rows
// are the 150,144-token vocabulary of "What is Recursive Flint?") and of a
// dense layer's projections.
//
// Persistent blocks: each stages its nt <= NT tokens in LDS once, then takes
// row groups rb = blockIdx.x, blockIdx.x + gridDim.x, ...; a group is RB = 4 *
// 64 / LPR rows, LPR lanes per row, every lane PPL pieces of 32 weights.  The
// next group's weight pieces are loaded before the current group's dot
// products, so each wave keeps two groups of loads in flight.  fp32 results,
// the NVFP4 tensor scale applied last, as in the expert GEMVs.
#include "gemv.cuh"
#include "launch.h"

namespace moe {

constexpr int kDenseNT = 8;       // tokens staged per launch (8 rows of up to 3840 in 64 KB of LDS)
constexpr int kDenseLpr = 16;     // lanes per row
constexpr int kDenseMaxPcl = 8;   // pieces per lane held in registers
// From this many tokens NVFP4 runs on the matrix cores.  Head (150,144 x 2048), same box:
// vector units 38 / 50 / 82 / 160 us at 2 / 4 / 8 / 16 tokens, matrix cores 67 us at all four
// (587 blocks of 256 columns, two per CU: a second partial wave of blocks).
constexpr int kDenseMfmaMinT = 8;

struct DenseArgs {
  MatDev m;
  int e, rows, nt;
  const uint16_t* x;  // [nt, cols]
  float* out;         // [nt, rows]
};

// Pieces of row n for this lane: p = lir + q * LPR, q < ppl.
template <int FMT, int PCL>
MOE_DEV void dense_load(const DenseArgs& g, int n, int lir, int lpr, int ppl, int q0, RawPiece (&r)[PCL]) {
  const int nc = min(n, g.rows - 1);  // a lane group past the last row loads the last row (unused)
  const uint8_t* rc = row_codes<FMT>(g.m, g.e, nc);
  const uint8_t* rs = row_scales<FMT>(g.m, g.e, nc);
  const uint8_t* rz = row_zeros<FMT>(g.m, g.e, nc);
#pragma unroll
  for (int q = 0; q < PCL; ++q)
    if (q0 + q < ppl) r[q] = load_piece<FMT>(rc, rs, rz, lir + (q0 + q) * lpr);
}

template <int FMT, int NT, int PCL, int LPR>
MOE_DEV void dense_dot_store(const DenseArgs& g, int n, int lir, int lpr, int ppl, int q0, bool last_chunk,
                             const RawPiece (&r)[PCL], const uint16_t* xs, const float* xsum, int K,
                             float (&acc)[NT]) {
#pragma unroll
  for (int q = 0; q < PCL; ++q)
    if (q0 + q < ppl) piece_dot<FMT, NT>(r[q], lir + (q0 + q) * lpr, xs, K, xsum, K / 32, g.nt, acc);
  if (!last_chunk) return;
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (t < g.nt) acc[t] = LPR ? group_sum_last<LPR>(acc[t]) : group_sum_last_dyn(acc[t], lpr);
  if (n < g.rows && lir == lpr - 1) {
    const float ts = tensor_scale<FMT>(g.m, g.e);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (t < g.nt) g.out[(size_t)t * g.rows + n] = acc[t] * ts;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
}

// KP > 0: K = 32 KP columns and PPL = KP / kDenseLpr pieces per lane, compile
// time, two row groups in flight.  KP == 0: the runtime shape, lanes per row
// lpr (a power of two dividing K / 32), pieces in chunks of kDenseMaxPcl.
template <int FMT, int NT, int KP>
__global__ void __launch_bounds__(256) k_dense_gemv(DenseArgs g, int lpr_rt) {
  extern __shared__ __align__(16) uint8_t smem[];
  constexpr bool FIX = KP > 0;
  constexpr int LPR = FIX ? kDenseLpr : 0;
  constexpr int PPL = FIX ? KP / kDenseLpr : kDenseMaxPcl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = FIX ? 32 * KP : g.m.cols;
  const int lpr = FIX ? LPR : lpr_rt;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = FIX ? PPL : (K / 32) / lpr;
  const int rpb = 4 * rpw;
  const int nrb = (g.rows + rpb - 1) / rpb;
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)NT * K * sizeof(uint16_t));
  int rb = blockIdx.x;
  const int row_in = wave * rpw + rsub;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.f;
  if (FIX) {
    RawPiece ra[PPL], rbuf[PPL];
    if (rb < nrb) dense_load<FMT, PPL>(g, rb * rpb + row_in, lir, lpr, ppl, 0, ra);
    stage_rows<FMT>(xs, xsum, g.x, [](int t) { return t; }, g.nt, K);
    __syncthreads();
    for (; rb < nrb; rb += 2 * gridDim.x) {
      const int rb2 = rb + gridDim.x;
      if (rb2 < nrb) dense_load<FMT, PPL>(g, rb2 * rpb + row_in, lir, lpr, ppl, 0, rbuf);
      dense_dot_store<FMT, NT, PPL, LPR>(g, rb * rpb + row_in, lir, lpr, ppl, 0, true, ra, xs, xsum, K, acc);
      if (rb2 >= nrb) break;
      if (rb2 + gridDim.x < nrb) dense_load<FMT, PPL>(g, (rb2 + gridDim.x) * rpb + row_in, lir, lpr, ppl, 0, ra);
      dense_dot_store<FMT, NT, PPL, LPR>(g, rb2 * rpb + row_in, lir, lpr, ppl, 0, true, rbuf, xs, xsum, K, acc);
    }
  } else {
    stage_rows<FMT>(xs, xsum, g.x, [](int t) { return t; }, g.nt, K);
    __syncthreads();
    RawPiece r[kDenseMaxPcl];
    for (; rb < nrb; rb += gridDim.x) {
      const int n = rb * rpb + row_in;
      for (int q0 = 0; q0 < ppl; q0 += kDenseMaxPcl) {
        dense_load<FMT, kDenseMaxPcl>(g, n, lir, lpr, ppl, q0, r);
        dense_dot_store<FMT, NT, kDenseMaxPcl, 0>(g, n, lir, lpr, ppl, q0, q0 + kDenseMaxPcl >= ppl, r, xs, xsum, K,
                                                  acc);
      }
    }
  }
}

static MatDev dense_mat(const moe_w4_matrix& m) {
  MatDev d;
  d.codes = m.codes;
  d.scales = (const uint8_t*)m.scales;
  d.zeros = m.fmt == kFmtInt4Sb ? (const uint8_t*)m.biases : m.zeros;
  d.ts = m.tensor_scale;
  d.rows = m.rows;
  d.cols = m.cols;
  return d;
}

template <int FMT, int NT>
static void dense_launch(const DenseArgs& g, int blocks, size_t lds, hipStream_t s) {
  if (g.m.cols == 2048) {
    hipLaunchKernelGGL((k_dense_gemv<FMT, NT, 64>), dim3(blocks), dim3(256), lds, s, g, kDenseLpr);
  } else {
    int lpr = kDenseLpr;
    while (lpr > 1 && (g.m.cols / 32) % lpr) lpr >>= 1;
    hipLaunchKernelGGL((k_dense_gemv<FMT, NT, 0>), dim3(blocks), dim3(256), lds, s, g, lpr);
  }
}

template <int FMT>
static void dense_launch_nt(const DenseArgs& g, int blocks, size_t lds, hipStream_t s) {
  if (g.nt == 1) dense_launch<FMT, 1>(g, blocks, lds, s);
  else if (g.nt == 2) dense_launch<FMT, 2>(g, blocks, lds, s);
  else if (g.nt <= 4) dense_launch<FMT, 4>(g, blocks, lds, s);
  else dense_launch<FMT, 8>(g, blocks, lds, s);
}

int dense_max_tokens() { return kDenseNT; }

hipError_t launch_dense_gemv(const moe_w4_matrix* m, int expert, const uint16_t* x, int T, float* out,
                             hipStream_t s) {
  if (m->fmt == kFmtBf16) return hipErrorInvalidValue;  // 4-bit formats only
  // several NVFP4 tokens: the matrix cores (the vector units would issue T dot products per
  // weight; the matrix once per 64 tokens instead of once per 8)
  if (T >= kDenseMfmaMinT && m->fmt == kFmtNvfp4 && m->cols % 256 == 0 && m->cols <= 2048)
    return launch_dense_mfma(m, expert, x, T, out, s);
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
  }
  DenseArgs g;
  g.m = dense_mat(*m);
  g.e = expert;
  g.rows = m->rows;
  const int K = m->cols;
  int lpr = kDenseLpr;
  while (lpr > 1 && (K / 32) % lpr) lpr >>= 1;
  const int rpb = 4 * (64 / lpr);
  const int nrb = (g.rows + rpb - 1) / rpb;
  const int blocks = std::max(1, std::min(nrb, 4 * cus));
  // tokens in batches of up to kDenseNT; each batch streams the matrix once
  for (int t0 = 0; t0 < T; t0 += kDenseNT) {
    g.nt = std::min(kDenseNT, T - t0);
    g.x = x + (size_t)t0 * K;
    g.out = out + (size_t)t0 * g.rows;
    const int ntc = g.nt == 1 ? 1 : g.nt == 2 ? 2 : g.nt <= 4 ? 4 : 8;
    const size_t lds = (size_t)ntc * K * 2 + (size_t)ntc * (K / 32) * 4;
    if (m->fmt == kFmtNvfp4) dense_launch_nt<kFmtNvfp4>(g, blocks, lds, s);
    else if (m->fmt == kFmtInt4Sb) dense_launch_nt<kFmtInt4Sb>(g, blocks, lds, s);
    else dense_launch_nt<kFmtInt4>(g, blocks, lds, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace moe
