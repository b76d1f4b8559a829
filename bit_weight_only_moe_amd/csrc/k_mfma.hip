// Grouped SwiGLU experts on the bf16 matrix cores (gfx950 MFMA), for
// prefill and large batches: the "grouped-GEMM path" that "[Model] Add Flint
// (RecursiveSI/flint)" (section "What happened") uses when a batch gives
// each expert many tokens.
//
// Per expert e with rows [offsets[e], offsets[e+1]) (tokens gathered through
// sorted_pairs):
//   gate/up kernel: G = X_e Wg_e^T, U = X_e Wu_e^T over K = H, then
//                   h = bf16(silu(G) * U);
//   down kernel:    O = h_e Wd_e^T over K = I, fp32.
// A device-side table lists (expert, first row) for every row tile.
// Main path (k_mfma_bl for NVFP4, k_mfma_bd for INT4): 64-row tiles; each
// lane dequantises its own weight column in registers.  With Zipf-skewed
// routing most experts get a few dozen rows, so small tiles waste little
// matrix work on padding.  Other shapes: 128-row tiles with the weights
// dequantised into LDS, and an expert's final remainder of at most 64 rows
// in a 64-row tile (4 waves side by side instead of 2 x 2).
//
// Weights are dequantised once per 64-wide K step, as bf16:
//   NVFP4: e4m3 * e2m1 has at most 6 significant bits, so the bf16 operand is
//          exact; the fp32 tensor scale multiplies the accumulator at the end;
//   INT4:  the operand is the exact integer (q - z); each 64-wide K step is one
//          quantisation group, accumulated separately and scaled by its fp16
//          scale in fp32 (s * (q - z) itself would not be exact in bf16).
// MFMA: v_mfma_f32_32x32x16_bf16.  Operands: lane l supplies row (A) or column
// (B) l % 32 and 8 consecutive k values; the accumulator register i of lane l
// holds row (i / 4) * 8 + (l / 32) * 4 + i % 4, column l % 32.  Each wave
// owns a 64 x 64 output tile (2 x 2 accumulators).
// LDS tiles are [rows][64 k] bf16 with the 16-byte chunk index XOR-ed by
// row & 7: a 128-byte row spans all 32 banks, so the 8 lanes that one LDS
// cycle serves for a 16-byte access (8 consecutive rows at one chunk, or 4
// rows at chunks c and c + 4) land on distinct banks.
#include "common.cuh"
#include "launch.h"
#include "mfma.cuh"
#include "route.cuh"

namespace moe {

constexpr int kBM = 128;  // rows per full tile; remainders of <= 64 rows may use 64-row tiles
constexpr int kBK = 64;   // reduction step = one INT4 group

struct MfmaArgs {
  int H, I, k, rows;
  const uint16_t* x;            // gate/up: tokens [T, H]
  const int32_t* sorted_pairs;  // NULL: sorted row r is token r
  const int32_t* offsets;       // [E + 1]; NULL: one expert over rows [0, rows)
  const int32_t* tiles;         // [0] = count, then (expert, first row) pairs
  int tile_rows;                // rows per tile of that table: 128 or 64
  const uint8_t *gc, *gs, *gz;  // gate codes / scales / zeros
  const uint8_t *uc, *us, *uz;  // up
  const uint8_t *dc, *ds, *dz;  // down
  const float *gts, *uts, *dts; // NVFP4 tensor scales
  uint16_t* h;                  // [rows, I]
  float* out;                   // [rows, H]
  int ldo;                      // dense form: row stride of out
};

MOE_DEV bool tile_of(const MfmaArgs& g, int mt, int& e, int& r0, int& r1) {
  if (mt >= g.tiles[0]) return false;
  e = g.tiles[1 + 2 * mt];
  r0 = g.tiles[2 + 2 * mt];
  const int end = g.offsets ? g.offsets[e + 1] : g.rows;
  r1 = min(end, r0 + g.tile_rows);
  return true;
}

// Tile tables, one block (one thread per expert, E <= 1024): each expert's
// rows in tiles of bm rows (`big`); with `split` (bm = 128), a final remainder
// of 1..64 rows becomes one 64-row tile (`small`) instead.  Each table: [0] =
// count, then (expert, first row) pairs.
__global__ void __launch_bounds__(1024) k_tile_table(const int32_t* __restrict__ offsets, int E, int rows, int bm,
                                                     int split, int32_t* __restrict__ big, int32_t* __restrict__ small) {
  __shared__ int scan_lds[17];
  const int e = threadIdx.x;
  int r0 = 0, r1 = 0;
  if (e < E) {
    r0 = offsets ? offsets[e] : 0;
    r1 = offsets ? offsets[e + 1] : rows;
  }
  const int c = r1 - r0, rem = c % bm;
  const bool to_small = split && rem > 0 && rem <= 64;
  const int nb = c / bm + ((rem > 0 && !to_small) ? 1 : 0);
  const int ns = to_small ? 1 : 0;
  int tb, ts;
  const int fb = block_exclusive_scan(nb, scan_lds, tb);
  const int fs = block_exclusive_scan(ns, scan_lds, ts);
  for (int t = 0; t < nb; ++t) {
    big[1 + 2 * (fb + t)] = e;
    big[2 + 2 * (fb + t)] = r0 + t * bm;
  }
  if (ns) {
    small[1 + 2 * fs] = e;
    small[2 + 2 * fs] = r0 + (c / bm) * bm;
  }
  if (e == 0) {
    big[0] = tb;
    small[0] = ts;
  }
}

// One K step's global data for this thread is loaded two steps ahead of its
// use, into two sets of plain registers in turn (a struct or array here is
// copied through private memory by the compiler), so the memory latency is
// covered by the matrix work of the steps in between.  A set: activation
// chunks a0..a3 (2 x 2 waves: 4 per thread; 4 x 1: a0, a1), weight codes b0
// (4 x 1: and b1, the row's next 32 weights), NVFP4 block scales sc, INT4
// zero point z and this wave's two per-column group scales s0, s1.
#define MOE_STAGE_VARS(p) \
  uint4 p##a0, p##a1, p##a2, p##a3, p##b0, p##b1; \
  uint32_t p##sc = 0; \
  int p##z = 0; \
  float p##s0 = 1.f, p##s1 = 1.f
#define MOE_STAGE_ARGS(p) p##a0, p##a1, p##a2, p##a3, p##b0, p##b1, p##sc, p##z, p##s0, p##s1

// Map the block index to (row tile, column slice) so that every column slice
// of a row tile runs on the same XCD (blocks go to XCDs round-robin), and the
// tile's activation rows stay in that XCD's L2.
// Contiguous tile ranges per XCD: XCD x takes tiles [x * per, (x + 1) * per)
// in order, each with all its column slices back to back.  Neighbouring row
// tiles of one expert then run on the same XCD at about the same time and
// read that expert's weights from its L2 after the first.  A block whose tile
// is past the table's end returns (tile_of).
MOE_DEV void block_tile_chunked(int nslices, int ntiles, int& tile, int& slice) {
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  const int per = (ntiles + 7) >> 3;
  const int t = j / nslices;
  tile = t < per ? xcd * per + t : 0x7fffffff;
  slice = j % nslices;
}

MOE_DEV void block_tile(int nslices, int& tile, int& slice) {
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  tile = (j / nslices) * 8 + xcd;
  slice = j % nslices;
}

// Write one K step's activation chunks and dequantised weights into the
// (single) LDS tiles, between two barriers.  WM = 2: thread = (row tid >> 1,
// chunks (tid & 1) * 4 .. + 4) for A and (row (tid >> 1) & 63 of matrix
// tid >> 7, half tid & 1) for B.  WM = 1: (row tid >> 2, chunks (tid & 3) * 2
// .. + 2) for A and (row tid & 127 of matrix tid >> 7, both halves) for B.
template <int FMT, int WM>
MOE_DEV void mfma_step(uint4 a0, uint4 a1, uint4 a2, uint4 a3, uint4 b0, uint4 b1, uint32_t sc, int z, uint4* As,
                       uint4* Bs, int a_row, int a_c0, int b_lrow, int b_half) {
  __syncthreads();
  As[swz(a_row, a_c0)] = a0;
  As[swz(a_row, a_c0 + 1)] = a1;
  if (WM == 2) {
    As[swz(a_row, a_c0 + 2)] = a2;
    As[swz(a_row, a_c0 + 3)] = a3;
  }
  uint4 o[4];
  dequant32<FMT>(b0, sc, z, o);
#pragma unroll
  for (int c = 0; c < 4; ++c) Bs[swz(b_lrow, b_half * 4 + c)] = o[c];
  if (WM == 1) {
    dequant32<FMT>(b1, sc >> 16, z, o);
#pragma unroll
    for (int c = 0; c < 4; ++c) Bs[swz(b_lrow, 4 + c)] = o[c];
  }
  __syncthreads();
}

// Load K step kt's data for this thread (see MOE_STAGE_VARS).
template <int FMT, int WM>
MOE_DEV void mfma_load(int kt, const uint16_t* arow, int a_c0, const uint8_t* bcodes, const uint8_t* bscales,
                       const uint8_t* bzeros_row, const uint16_t* sc0, const uint16_t* sc1, uint4& a0, uint4& a1,
                       uint4& a2, uint4& a3, uint4& b0, uint4& b1, uint32_t& sc, int& z, float& s0, float& s1) {
  const uint4* xa = (const uint4*)(arow + kt * kBK) + a_c0;
  const uint4* wb = (const uint4*)(bcodes + kt * (kBK / 2));
  a0 = xa[0];
  b0 = wb[0];
  a1 = xa[1];
  if (WM == 2) {
    a2 = xa[2];
    a3 = xa[3];
  } else {
    b1 = wb[1];
  }
  if (FMT == kFmtNvfp4) {
    sc = WM == 2 ? *(const uint16_t*)(bscales + kt * 4) : *(const uint32_t*)(bscales + kt * 4);
  } else {
    z = bzeros_row[kt];
    s0 = f16_to_f32(sc0[kt]);
    s1 = f16_to_f32(sc1[kt]);
  }
}

// ------------------------------------------------------------------ gate/up
// Block: 4 waves as WM (rows) x WN = 4 / WM (features); each wave owns a
// 64-row x 32-feature tile of both G and U.  The block covers 64 * WM rows and
// 32 * WN features of gate and of up.
template <int FMT, int WM>
__global__ void __launch_bounds__(256, 2) k_mfma_gateup(MfmaArgs g) {
  constexpr int WN = 4 / WM, BMr = 64 * WM, NF = 32 * WN;
  __shared__ uint4 As[BMr * 8];     // [BMr][64] bf16, swizzled
  __shared__ uint4 Bs[2 * NF * 8];  // rows 0..NF-1 gate, NF..2NF-1 up
  int tile, slice;
  block_tile(g.I / NF, tile, slice);
  int e, r0, r1;
  if (!tile_of(g, tile, e, r0, r1)) return;
  const int H = g.H, I = g.I;
  const int n0 = slice * NF;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int a_row = WM == 2 ? tid >> 1 : tid >> 2, a_c0 = WM == 2 ? (tid & 1) * 4 : (tid & 3) * 2;
  // rows past the tile's end load a valid row; their outputs are never stored
  const int arow = min(r0 + a_row, r1 - 1);
  const int tok = g.sorted_pairs ? g.sorted_pairs[arow] / g.k : arow;
  const uint16_t* xrow = g.x + (size_t)tok * H;
  const int b_mat = tid >> 7, b_row = WM == 2 ? (tid >> 1) & 63 : tid & 127, b_half = WM == 2 ? tid & 1 : 0;
  const int b_lrow = b_mat * NF + b_row;
  const size_t wrow = (size_t)e * I + n0 + b_row;
  const uint8_t* bcodes = (b_mat ? g.uc : g.gc) + wrow * (H / 2) + b_half * 16;
  const uint8_t* bscales = (b_mat ? g.us : g.gs) + wrow * (H / 16) + b_half * 2;
  const uint8_t* bzeros = b_mat ? g.uz : g.gz;
  // this wave's gate / up feature column (INT4 group scales)
  const int ncol = n0 + wn * 32 + (lane & 31);
  const uint16_t* gsc = (const uint16_t*)g.gs + ((size_t)e * I + ncol) * (H / 64);
  const uint16_t* usc = (const uint16_t*)g.us + ((size_t)e * I + ncol) * (H / 64);

  f32x16_t acc[2][2];  // [gate / up][row sub-tile]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[a][m] = f32x16_t{};

  const int nk = H / kBK;
  const uint8_t* bzrow = bzeros ? bzeros + wrow * (H / 64) : nullptr;
  // NVFP4 accumulates straight into acc; INT4 accumulates one group in part
  // and adds it to acc times the group's scale.
  auto mma = [&](f32x16_t (&c)[2][2]) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      const bf16x8_t a0 = lds_frag(As, wm * 64 + (lane & 31), chunk);
      const bf16x8_t a1 = lds_frag(As, wm * 64 + 32 + (lane & 31), chunk);
      const bf16x8_t bg = lds_frag(Bs, wn * 32 + (lane & 31), chunk);
      const bf16x8_t bu = lds_frag(Bs, NF + wn * 32 + (lane & 31), chunk);
      c[0][0] = mfma(a0, bg, c[0][0]);
      c[0][1] = mfma(a1, bg, c[0][1]);
      c[1][0] = mfma(a0, bu, c[1][0]);
      c[1][1] = mfma(a1, bu, c[1][1]);
    }
  };
  auto compute = [&](float sg, float su) {
    if (FMT == kFmtNvfp4) {
      mma(acc);
    } else {
      f32x16_t part[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int m = 0; m < 2; ++m) part[a][m] = f32x16_t{};
      mma(part);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[0][m][i] = fmaf(sg, part[0][m][i], acc[0][m][i]);
          acc[1][m][i] = fmaf(su, part[1][m][i], acc[1][m][i]);
        }
      }
    }
  };
  MOE_STAGE_VARS(p_);
  MOE_STAGE_VARS(q_);
  mfma_load<FMT, WM>(0, xrow, a_c0, bcodes, bscales, bzrow, gsc, usc, MOE_STAGE_ARGS(p_));
  if (nk > 1) mfma_load<FMT, WM>(1, xrow, a_c0, bcodes, bscales, bzrow, gsc, usc, MOE_STAGE_ARGS(q_));
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    mfma_step<FMT, WM>(p_a0, p_a1, p_a2, p_a3, p_b0, p_b1, p_sc, p_z, As, Bs, a_row, a_c0, b_lrow, b_half);
    float gs0 = p_s0, gs1 = p_s1;
    if (kt + 2 < nk) mfma_load<FMT, WM>(kt + 2, xrow, a_c0, bcodes, bscales, bzrow, gsc, usc, MOE_STAGE_ARGS(p_));
    compute(gs0, gs1);
    mfma_step<FMT, WM>(q_a0, q_a1, q_a2, q_a3, q_b0, q_b1, q_sc, q_z, As, Bs, a_row, a_c0, b_lrow, b_half);
    gs0 = q_s0;
    gs1 = q_s1;
    if (kt + 3 < nk) mfma_load<FMT, WM>(kt + 3, xrow, a_c0, bcodes, bscales, bzrow, gsc, usc, MOE_STAGE_ARGS(q_));
    compute(gs0, gs1);
  }
  if (kt < nk) {  // odd number of K steps
    mfma_step<FMT, WM>(p_a0, p_a1, p_a2, p_a3, p_b0, p_b1, p_sc, p_z, As, Bs, a_row, a_c0, b_lrow, b_half);
    compute(p_s0, p_s1);
  }
  // epilogue: h = bf16(silu(ts_g * G) * (ts_u * U))
  const float tsg = FMT == kFmtNvfp4 ? g.gts[e] : 1.f, tsu = FMT == kFmtNvfp4 ? g.uts[e] : 1.f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = wm * 64 + m * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      if (r0 + row < r1) {
        const float gv = acc[0][m][i] * tsg, uv = acc[1][m][i] * tsu;
        g.h[(size_t)(r0 + row) * I + ncol] = (uint16_t)f32_to_bf16_rne(silu_f32(gv) * uv);
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Block: 4 waves as WM x WN = 4 / WM, each a 64-row x 64-column tile; the
// block covers 64 * WM rows and 64 * WN output columns.
template <int FMT, int WM>
__global__ void __launch_bounds__(256, (WM == 1 && FMT == kFmtNvfp4) ? 3 : 2) k_mfma_down(MfmaArgs g) {
  constexpr int WN = 4 / WM, BMr = 64 * WM, NC = 64 * WN;
  __shared__ uint4 As[BMr * 8];
  __shared__ uint4 Bs[NC * 8];
  int tile, slice;
  block_tile(g.H / NC, tile, slice);
  int e, r0, r1;
  if (!tile_of(g, tile, e, r0, r1)) return;
  const int H = g.H, I = g.I;
  const int n0 = slice * NC;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int a_row = WM == 2 ? tid >> 1 : tid >> 2, a_c0 = WM == 2 ? (tid & 1) * 4 : (tid & 3) * 2;
  const uint16_t* hrow = g.h + (size_t)min(r0 + a_row, r1 - 1) * I;
  const int b_row = WM == 2 ? tid >> 1 : tid, b_half = WM == 2 ? tid & 1 : 0;
  const size_t wrow = (size_t)e * H + n0 + b_row;
  const uint8_t* bcodes = g.dc + wrow * (I / 2) + b_half * 16;
  const uint8_t* bscales = g.ds + wrow * (I / 16) + b_half * 2;
  const int ncol0 = n0 + wn * 64 + (lane & 31);
  const uint16_t* dsc0 = (const uint16_t*)g.ds + ((size_t)e * H + ncol0) * (I / 64);
  const uint16_t* dsc1 = (const uint16_t*)g.ds + ((size_t)e * H + ncol0 + 32) * (I / 64);

  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x16_t{};
  const int nk = I / kBK;
  const uint8_t* bzrow = g.dz ? g.dz + wrow * (I / 64) : nullptr;
  auto mma = [&](f32x16_t (&c)[2][2]) {
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      const bf16x8_t a0 = lds_frag(As, wm * 64 + (lane & 31), chunk);
      const bf16x8_t a1 = lds_frag(As, wm * 64 + 32 + (lane & 31), chunk);
      const bf16x8_t b0 = lds_frag(Bs, wn * 64 + (lane & 31), chunk);
      const bf16x8_t b1 = lds_frag(Bs, wn * 64 + 32 + (lane & 31), chunk);
      c[0][0] = mfma(a0, b0, c[0][0]);
      c[0][1] = mfma(a0, b1, c[0][1]);
      c[1][0] = mfma(a1, b0, c[1][0]);
      c[1][1] = mfma(a1, b1, c[1][1]);
    }
  };
  auto compute = [&](float s0, float s1) {
    if (FMT == kFmtNvfp4) {
      mma(acc);
    } else {
      f32x16_t part[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) part[m][n] = f32x16_t{};
      mma(part);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[m][0][i] = fmaf(s0, part[m][0][i], acc[m][0][i]);
          acc[m][1][i] = fmaf(s1, part[m][1][i], acc[m][1][i]);
        }
      }
    }
  };
  MOE_STAGE_VARS(p_);
  MOE_STAGE_VARS(q_);
  mfma_load<FMT, WM>(0, hrow, a_c0, bcodes, bscales, bzrow, dsc0, dsc1, MOE_STAGE_ARGS(p_));
  if (nk > 1) mfma_load<FMT, WM>(1, hrow, a_c0, bcodes, bscales, bzrow, dsc0, dsc1, MOE_STAGE_ARGS(q_));
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    mfma_step<FMT, WM>(p_a0, p_a1, p_a2, p_a3, p_b0, p_b1, p_sc, p_z, As, Bs, a_row, a_c0, b_row, b_half);
    float ds0 = p_s0, ds1 = p_s1;
    if (kt + 2 < nk) mfma_load<FMT, WM>(kt + 2, hrow, a_c0, bcodes, bscales, bzrow, dsc0, dsc1, MOE_STAGE_ARGS(p_));
    compute(ds0, ds1);
    mfma_step<FMT, WM>(q_a0, q_a1, q_a2, q_a3, q_b0, q_b1, q_sc, q_z, As, Bs, a_row, a_c0, b_row, b_half);
    ds0 = q_s0;
    ds1 = q_s1;
    if (kt + 3 < nk) mfma_load<FMT, WM>(kt + 3, hrow, a_c0, bcodes, bscales, bzrow, dsc0, dsc1, MOE_STAGE_ARGS(q_));
    compute(ds0, ds1);
  }
  if (kt < nk) {  // odd number of K steps
    mfma_step<FMT, WM>(p_a0, p_a1, p_a2, p_a3, p_b0, p_b1, p_sc, p_z, As, Bs, a_row, a_c0, b_row, b_half);
    compute(p_s0, p_s1);
  }
  const float ts = FMT == kFmtNvfp4 ? g.dts[e] : 1.f;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = wm * 64 + m * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (r0 + row < r1) g.out[(size_t)(r0 + row) * H + ncol0 + n * 32] = acc[m][n][i] * ts;
      }
    }
  }
}

// ------------------------------------------------------------------ 64-row tiles, streamed weights
// Block: 4 waves side by side over the columns, each covering all 32 * RF
// rows of the tile; only HBM-sized state is per block, so two blocks share a
// CU.  Each lane dequantises the packed codes of its own B column (l % 32)
// in registers and hands them to the matrix core as the B operand; the
// activations, which the 4 waves share, go through LDS (two buffers, one
// barrier per K step).
// K order inside a 64-wide step (one INT4 group, four NVFP4 blocks): matrix
// slice ks takes k = ks*8 .. +8 from lane half 0 and k = 32 + ks*8 .. +8 from
// lane half 1, so a lane's 32 weights of a step are one contiguous 16-byte
// run of codes; the activation fragments are read from LDS in the same order.
// Both halves of a slice lie in the same INT4 group.
// INT4 (k_mfma_bd): each lane loads its column's codes straight from HBM into
// registers, a ring of 4 single steps (its group partial sums leave no
// registers for more).
// NVFP4 (k_mfma_bl): the codes of 4 K steps (one 128-byte line per weight
// row) are loaded cooperatively, 8 lanes per row, into a double-buffered LDS
// tile, from which each lane reads its column's 16 bytes per step; the block
// scales of those 4 steps are one 16-byte load per lane.
// GU: column pair cf = 0 / 1 is gate / up feature f = n0 + wave*32 + l%32
//     (the block covers 128 features); h = bf16(silu(G) * U).
// !GU: columns n0 + wave*64 + cf*32 + l%32 (the block covers 256 outputs).
constexpr int kBdMaxSteps = 32;  // K <= 2048

// NVFP4 needs K to be a whole number of 4-step groups.
static inline bool bd_k_ok(int fmt, int K) {
  return K <= kBK * kBdMaxSteps && (fmt != kFmtNvfp4 || K % (4 * kBK) == 0);
}

template <int FMT, int RF, bool GU>
__global__ void __launch_bounds__(256, 2) k_mfma_bd(MfmaArgs g) {
  static_assert(FMT == kFmtInt4, "INT4 only (NVFP4: k_mfma_bl)");
  constexpr int BM = 32 * RF, D = 4, NB = GU ? 128 : 256;
  constexpr int AV = BM / 32;       // activation uint4 per thread per K step
  __shared__ uint4 As[2][BM * 8];   // [BM][64] bf16, swizzled, two buffers
  const int K = GU ? g.H : g.I, N = GU ? g.I : g.H;
  int tile, slice;
  block_tile_chunked(N / NB, g.tiles[0], tile, slice);
  int e, r0, r1;
  if (!tile_of(g, tile, e, r0, r1)) return;
  const int n0 = slice * NB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Activations: load v of a thread is row v * 32 + tid / 8, 16-byte chunk
  // tid % 8, so 8 lanes read one row's 128 bytes of a K step.  Rows past the
  // tile's end load a valid row; their outputs are never stored.
  const int a_chunk = tid & 7;
  const u32x4_t* asrc[AV];
#pragma unroll
  for (int v = 0; v < AV; ++v) {
    const int arow = min(r0 + v * 32 + (tid >> 3), r1 - 1);
    if (GU) {
      const int tok = g.sorted_pairs ? g.sorted_pairs[arow] / g.k : arow;
      asrc[v] = (const u32x4_t*)(g.x + (size_t)tok * K) + a_chunk;
    } else {
      asrc[v] = (const u32x4_t*)(g.h + (size_t)arow * K) + a_chunk;
    }
  }
  // this lane's two B columns
  const uint8_t* bcp[2];
  const uint8_t* bsp[2];
  const uint8_t* bzp[2];
#pragma unroll
  for (int cf = 0; cf < 2; ++cf) {
    const size_t row = GU ? (size_t)e * N + n0 + wave * 32 + l32 : (size_t)e * N + n0 + wave * 64 + cf * 32 + l32;
    const uint8_t* codes = GU ? (cf ? g.uc : g.gc) : g.dc;
    const uint8_t* scales = GU ? (cf ? g.us : g.gs) : g.ds;
    const uint8_t* zeros = GU ? (cf ? g.uz : g.gz) : g.dz;
    bcp[cf] = codes + row * (K / 2) + hf * 16;
    bsp[cf] = scales + row * (K / 64) * 2;
    bzp[cf] = zeros + row * (K / 64);
  }
  // Plain vectors, not uint4: a struct copy from global memory becomes a
  // block copy through private memory.  Activations: ring of D steps.
  u32x4_t ar[AV][D];
  // weights: ring of D steps
  u32x4_t bq[D][2];
  int bz[D][2];
  float bgs[D][2];
  auto load_a = [&](int kt, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < AV; ++v) ar[v][j] = asrc[v][kt * 8];
  };
  auto load_b = [&](int kt, int j) __attribute__((always_inline)) {  // one step
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
      bq[j][cf] = *(const u32x4_t*)(bcp[cf] + kt * 32);
      bz[j][cf] = bzp[cf][kt];
      bgs[j][cf] = f16_to_f32(((const uint16_t*)bsp[cf])[kt]);
    }
  };
  auto write_a = [&](int j, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < AV; ++v) ((u32x4_t*)As[buf])[swz(v * 32 + (tid >> 3), a_chunk)] = ar[v][j];
  };

  f32x16_t acc[2][RF];
#pragma unroll
  for (int cf = 0; cf < 2; ++cf)
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) acc[cf][rf] = f32x16_t{};

  const int nk = K / kBK;
  // loads past the last K step repeat it (in bounds, never used)
  load_a(0, 0);
  load_b(0, 0);
  load_a(min(1, nk - 1), 1);
  load_b(min(1, nk - 1), 1);
  load_a(min(2, nk - 1), 2);
  load_b(min(2, nk - 1), 2);
  load_a(min(3, nk - 1), 3);
  load_b(min(3, nk - 1), 3);
  write_a(0, 0);
  __syncthreads();
  auto step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int kt = decltype(kc)::value, j = kt % D;
    write_a((j + 1) % D, (kt + 1) & 1);  // after the last step: unused
    uint4 o[2][4];
    dequant32<FMT>(to_uint4(bq[j][0]), 0, bz[j][0], o[0]);
    dequant32<FMT>(to_uint4(bq[j][1]), 0, bz[j][1], o[1]);
    const float s0 = bgs[j][0], s1 = bgs[j][1];
    load_a(min(kt + D, nk - 1), j);
    load_b(min(kt + D, nk - 1), j);
    const uint4* at = As[kt & 1];
    f32x16_t part[2][RF];
#pragma unroll
    for (int cf = 0; cf < 2; ++cf)
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) part[cf][rf] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t a[RF];
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) a[rf] = lds_frag(at, rf * 32 + l32, hf * 4 + ks);
#pragma unroll
      for (int cf = 0; cf < 2; ++cf) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, o[cf][ks]);
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) part[cf][rf] = mfma(a[rf], b, part[cf][rf]);
      }
    }
    // each K step is one quantisation group: scale its partial sums in fp32
#pragma unroll
    for (int rf = 0; rf < RF; ++rf)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[0][rf][i] = fmaf(s0, part[0][rf][i], acc[0][rf][i]);
        acc[1][rf][i] = fmaf(s1, part[1][rf][i], acc[1][rf][i]);
      }
    __syncthreads();
  };
  // Straight-line code (no loop back edge): the compiler then waits for each
  // step's own loads only, not for every load in flight.
  unrolled_steps<0, kBdMaxSteps>(nk, step);
  if (GU) {
    const int f = n0 + wave * 32 + l32;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = rf * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
        if (r0 + row < r1)
          g.h[(size_t)(r0 + row) * N + f] = (uint16_t)f32_to_bf16_rne(silu_f32(acc[0][rf][i]) * acc[1][rf][i]);
      }
    }
  } else {
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
      const int col = n0 + wave * 64 + cf * 32 + l32;
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = rf * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
          if (r0 + row < r1) g.out[(size_t)(r0 + row) * N + col] = acc[cf][rf][i];
        }
      }
    }
  }
}

// NVFP4: the 256 weight rows of a block (gate + up features, or down
// columns) are loaded 4 K steps (128 bytes of a row) at a time by 8
// consecutive lanes, so one load instruction covers 8 whole cache lines
// rather than 16-byte pieces of 32 (measured: 2-4% faster than per-lane
// streaming into registers).  LDS: activations 2 x 8 KB, codes 2 x 32 KB.
// DENSE (down form only): one matrix and one tile of g.rows <= 64 rows (no
// tile table); block b takes output columns [256 b, 256 b + 256) of N, the
// last slice partial (weight rows clamped to N - 1, their outputs not
// stored); outputs at row stride g.ldo.
template <int FMT, bool GU, bool DENSE = false>
__global__ void __launch_bounds__(256, 2) k_mfma_bl(MfmaArgs g) {
  static_assert(FMT == kFmtNvfp4, "NVFP4 only");
  static_assert(!(DENSE && GU), "the dense form is a plain product");
  constexpr int RF = 2, BM = 64, D = 4, NB = GU ? 128 : 256, AV = 2;
  __shared__ uint4 As[2][BM * 8];
  __shared__ uint4 Bs[2][256 * 8];  // [256 weight rows][128 bytes], chunk c at c ^ (row & 7)
  const int K = GU ? g.H : g.I, N = GU ? g.I : g.H;
  int tile, slice;
  int e, r0, r1;
  if (DENSE) {
    slice = blockIdx.x;
    e = 0;
    r0 = 0;
    r1 = g.rows;
  } else {
    block_tile_chunked(N / NB, g.tiles[0], tile, slice);
    if (!tile_of(g, tile, e, r0, r1)) return;
  }
  const int n0 = slice * NB;
  // weight row n of this block, clamped into the matrix (dense: the last slice is partial)
  auto wrow = [&](int n) __attribute__((always_inline)) { return DENSE ? min(n, N - 1) : n; };
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  const int a_chunk = tid & 7;
  const u32x4_t* asrc[AV];
#pragma unroll
  for (int v = 0; v < AV; ++v) {
    const int arow = min(r0 + v * 32 + (tid >> 3), r1 - 1);
    if (GU) {
      const int tok = g.sorted_pairs ? g.sorted_pairs[arow] / g.k : arow;
      asrc[v] = (const u32x4_t*)(g.x + (size_t)tok * K) + a_chunk;
    } else {
      asrc[v] = (const u32x4_t*)(g.h + (size_t)arow * K) + a_chunk;
    }
  }
  // block weight row br: GU: gate feature br (br < 128) or up feature br - 128;
  // down: output column br
  auto brow_codes = [&](int br) __attribute__((always_inline)) {
    if (GU) return (br < 128 ? g.gc : g.uc) + ((size_t)e * N + n0 + (br & 127)) * (K / 2);
    return g.dc + ((size_t)e * N + wrow(n0 + br)) * (K / 2);
  };
  // this thread's 8 group loads: rows i*32 + tid/8, 16-byte chunk tid % 8
  const uint8_t* gsrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) gsrc[i] = brow_codes(i * 32 + (tid >> 3)) + a_chunk * 16;
  // this lane's two B columns (rows of Bs) and their block scales
  int lrow[2];
  const uint8_t* bsp[2];
#pragma unroll
  for (int cf = 0; cf < 2; ++cf) {
    lrow[cf] = GU ? cf * 128 + wave * 32 + l32 : wave * 64 + cf * 32 + l32;
    const size_t row = GU ? (size_t)e * N + n0 + wave * 32 + l32 : (size_t)e * N + wrow(n0 + lrow[cf]);
    bsp[cf] = (GU ? (cf ? g.us : g.gs) : g.ds) + row * (K / 16);
  }
  u32x4_t ar[AV][D];
  u32x4_t gr[8];        // next group's codes, in flight
  u32x4_t gsv[2][2];    // block scales of the current and next group
  auto load_a = [&](int kt, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < AV; ++v) ar[v][j] = asrc[v][kt * 8];
  };
  auto write_a = [&](int j, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < AV; ++v) ((u32x4_t*)As[buf])[swz(v * 32 + (tid >> 3), a_chunk)] = ar[v][j];
  };
  auto load_group = [&](int grp_step0, int sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) gr[i] = *(const u32x4_t*)(gsrc[i] + grp_step0 * 32);
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) gsv[sb][cf] = *(const u32x4_t*)(bsp[cf] + grp_step0 * 4);
  };
  auto write_group = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int br = i * 32 + (tid >> 3);
      ((u32x4_t*)Bs[buf])[br * 8 + (a_chunk ^ (br & 7))] = gr[i];
    }
  };
  f32x16_t acc[2][RF];
#pragma unroll
  for (int cf = 0; cf < 2; ++cf)
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) acc[cf][rf] = f32x16_t{};
  const int nk = K / kBK;
  load_group(0, 0);
  load_a(0, 0);
  load_a(min(1, nk - 1), 1);
  load_a(min(2, nk - 1), 2);
  load_a(min(3, nk - 1), 3);
  write_group(0);
  write_a(0, 0);
  __syncthreads();
  auto step = [&](auto kc) __attribute__((always_inline)) {
    constexpr int kt = decltype(kc)::value, j = kt % D, grp = (kt / 4) & 1;
    write_a((j + 1) % D, (kt + 1) & 1);  // after the last step: unused
    uint4 o[2][4];
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
      const int br = lrow[cf], c = 2 * j + hf;
      const uint4 codes = Bs[grp][br * 8 + (c ^ (br & 7))];
      const uint32_t sc = gsv[grp][cf][j] >> (16 * hf);
      dequant32<FMT>(codes, sc, 0, o[cf]);
    }
    load_a(min(kt + D, nk - 1), j);
    const bool more = kt + 4 < nk;
    if (j == 0 && more) load_group(kt + 4, grp ^ 1);
    const uint4* at = As[kt & 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t a[RF];
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) a[rf] = lds_frag(at, rf * 32 + l32, hf * 4 + ks);
#pragma unroll
      for (int cf = 0; cf < 2; ++cf) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, o[cf][ks]);
#pragma unroll
        for (int rf = 0; rf < RF; ++rf) acc[cf][rf] = mfma(a[rf], b, acc[cf][rf]);
      }
    }
    if (j == 3 && more) write_group(grp ^ 1);  // the other buffer's last reader was step kt - 3
    __syncthreads();
  };
  unrolled_steps<0, kBdMaxSteps>(nk, step);
  if (GU) {
    const float tsg = g.gts[e], tsu = g.uts[e];
    const int f = n0 + wave * 32 + l32;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = rf * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
        if (r0 + row < r1) {
          const float gv = acc[0][rf][i] * tsg, uv = acc[1][rf][i] * tsu;
          g.h[(size_t)(r0 + row) * N + f] = (uint16_t)f32_to_bf16_rne(silu_f32(gv) * uv);
        }
      }
    }
  } else {
    const float ts = g.dts[e];
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
      const int col = n0 + lrow[cf];
#pragma unroll
      for (int rf = 0; rf < RF; ++rf) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = rf * 32 + (i >> 2) * 8 + hf * 4 + (i & 3);
          if (r0 + row < r1 && (!DENSE || col < N))
            g.out[(size_t)(r0 + row) * (DENSE ? g.ldo : N) + col] = acc[cf][rf][i] * ts;
        }
      }
    }
  }
}

// Dense product out[t, n] = tensor_scale * sum_k x[t, k] W[n, k] for one NVFP4
// matrix (expert `expert` of the stack) on the matrix cores: tokens in tiles
// of up to 64 rows, one block per 256 output columns.  Needs K % 256 == 0 and
// K <= 2048.
hipError_t launch_dense_mfma(const moe_w4_matrix* m, int expert, const uint16_t* x, int T, float* out,
                             hipStream_t s) {
  if (m->fmt != kFmtNvfp4 || !bd_k_ok(m->fmt, m->cols)) return hipErrorInvalidValue;
  const size_t rc = (size_t)m->rows * m->cols;
  MfmaArgs g{};
  g.H = m->rows;  // N: output columns
  g.I = m->cols;  // K
  g.k = 1;
  g.dc = m->codes + (size_t)expert * (rc / 2);
  g.ds = (const uint8_t*)m->scales + (size_t)expert * (rc / 16);
  g.dts = m->tensor_scale + expert;
  g.ldo = m->rows;
  const int nblk = (m->rows + 255) / 256;
  for (int t0 = 0; t0 < T; t0 += 64) {
    g.rows = std::min(64, T - t0);
    g.h = const_cast<uint16_t*>(x) + (size_t)t0 * m->cols;
    g.out = out + (size_t)t0 * m->rows;
    MOE_LAUNCH((k_mfma_bl<kFmtNvfp4, false, true>), dim3(nblk), dim3(256), 0, s, g);
  }
  return hipSuccess;
}

// ------------------------------------------------------------------ router (large batches)
// logits[t, e] = sum_h x[t, h] * w[e, h] on the matrix cores.  Each fp32
// router weight is split exactly into three bf16 parts, w = hi + mid + lo,
// by truncation: hi keeps the top 8 significant bits of w, mid the top 8 of
// the exact residual w - hi (at most 16 bits), lo the rest (at most 8 bits,
// so exact in bf16).  Every product x * part is exact in fp32 and the three
// MFMAs accumulate them in fp32, as the VALU router's fused multiply-adds do
// (in another order).  Block: 64 tokens x 64 experts, 4 waves as 2 x 2 of
// 32 x 32; 64-wide K steps staged through LDS, global data loaded two steps
// ahead.
// Named, interleaved fields: adjacent copies from adjacent global addresses
// are merged into one block copy that the compiler keeps in private memory.
struct RouterStage {
  uint4 a0;     // bf16 0..7 of one token row's 16
  float4 w0;    // fp32 0..3 of one router row's 16
  uint4 a1;     // bf16 8..15
  float4 w1, w2, w3;
};

MOE_DEV void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t hb = __float_as_uint(w) & 0xFFFF0000u;
  const float t1 = w - __uint_as_float(hb);
  const uint32_t mb = __float_as_uint(t1) & 0xFFFF0000u;
  const float t2 = t1 - __uint_as_float(mb);
  hi = hb >> 16;
  mid = mb >> 16;
  lo = __float_as_uint(t2) >> 16;
}

// Split two fp32 values into packed bf16 pairs of their hi / mid / lo parts.
MOE_DEV void split3_pair(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  uint32_t ha, ma, la, hb, mb, lb;
  split3(a, ha, ma, la);
  split3(b, hb, mb, lb);
  hi = ha | (hb << 16);
  mid = ma | (mb << 16);
  lo = la | (lb << 16);
}

// Split 8 fp32 weights into three uint4 of 8 bf16 each.
MOE_DEV void split3_x8(float4 p, float4 q, uint4& hi, uint4& mid, uint4& lo) {
  split3_pair(p.x, p.y, hi.x, mid.x, lo.x);
  split3_pair(p.z, p.w, hi.y, mid.y, lo.y);
  split3_pair(q.x, q.y, hi.z, mid.z, lo.z);
  split3_pair(q.z, q.w, hi.w, mid.w, lo.w);
}

MOE_DEV void router_load(const uint16_t* xrow, const float* wrow, int kt, RouterStage& st) {
  const uint4* xa = (const uint4*)(xrow + kt * 64);
  const float4* wa = (const float4*)(wrow + kt * 64);
  st.a0 = xa[0];
  st.w0 = wa[0];
  st.a1 = xa[1];
  st.w1 = wa[1];
  st.w2 = wa[2];
  st.w3 = wa[3];
}

// Write one K step's token chunk and split router chunks into the tiles.
MOE_DEV void router_stage(const RouterStage& st, int lrow, int lq, uint4* As, uint4 (*Bs)[64 * 8]) {
  __syncthreads();
  As[swz(lrow, lq * 2)] = st.a0;
  As[swz(lrow, lq * 2 + 1)] = st.a1;
  uint4 h, m, l;
  split3_x8(st.w0, st.w1, h, m, l);  // two chunks of 8 weights
  Bs[0][swz(lrow, lq * 2)] = h;
  Bs[1][swz(lrow, lq * 2)] = m;
  Bs[2][swz(lrow, lq * 2)] = l;
  split3_x8(st.w2, st.w3, h, m, l);
  Bs[0][swz(lrow, lq * 2 + 1)] = h;
  Bs[1][swz(lrow, lq * 2 + 1)] = m;
  Bs[2][swz(lrow, lq * 2 + 1)] = l;
  __syncthreads();
}

// All 16 fragments of the step are read before the 12 MFMAs: one LDS wait
// per step instead of one per MFMA (a lone wave per SIMD hides none of it).
MOE_DEV void router_compute(const uint4* As, const uint4 (*Bs)[64 * 8], int wm, int wn, int lane, f32x16_t& acc) {
  bf16x8_t a[4], b[4][3];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int chunk = ks * 2 + (lane >> 5);
    a[ks] = lds_frag(As, wm * 32 + (lane & 31), chunk);
    const int brow = wn * 32 + (lane & 31);
#pragma unroll
    for (int p = 0; p < 3; ++p) b[ks][p] = lds_frag(Bs[p], brow, chunk);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    acc = mfma(a[ks], b[ks][2], acc);
    acc = mfma(a[ks], b[ks][1], acc);
    acc = mfma(a[ks], b[ks][0], acc);
  }
}

__global__ void __launch_bounds__(256) k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     int T, int H, int E, float* __restrict__ logits) {
  __shared__ uint4 As[64 * 8];      // [64 tokens][64 k] bf16, swizzled
  __shared__ uint4 Bs[3][64 * 8];   // hi / mid / lo parts of [64 experts][64 k]
  const int nte = (E + 63) / 64;
  // consecutive logical tiles on one XCD (block b runs on XCD b % 8): the
  // expert tiles of one token tile share its activations in that XCD's L2
  const int nb = gridDim.x;
  const int lb = nb % 8 == 0 ? (int)(blockIdx.x % 8) * (nb / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int t0 = (lb / nte) * 64, e0 = (lb % nte) * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // loaders: token row tid >> 2, 16 bf16 at (tid & 3) * 16; router row tid >> 2, 16 fp32 at (tid & 3) * 16
  const int lrow = tid >> 2, lq = tid & 3;
  const uint16_t* xrow = x + (size_t)min(t0 + lrow, T - 1) * H + lq * 16;
  const float* wrow = wr + (size_t)min(e0 + lrow, E - 1) * H + lq * 16;
  f32x16_t acc = f32x16_t{};
  const int nk = H / 64;
  // Prefetches are unconditional (step index clamped; the surplus loads at
  // the end are re-reads): under a branch the compiler waits for every load
  // in flight, the one just issued included, before each staging.
  RouterStage s0, s1;
  router_load(xrow, wrow, 0, s0);
  router_load(xrow, wrow, min(1, nk - 1), s1);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    router_stage(s0, lrow, lq, As, Bs);
    router_load(xrow, wrow, min(kt + 2, nk - 1), s0);
    router_compute(As, Bs, wm, wn, lane, acc);
    router_stage(s1, lrow, lq, As, Bs);
    router_load(xrow, wrow, min(kt + 3, nk - 1), s1);
    router_compute(As, Bs, wm, wn, lane, acc);
  }
  if (kt < nk) {
    router_stage(s0, lrow, lq, As, Bs);
    router_compute(As, Bs, wm, wn, lane, acc);
  }
  const int col = e0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = t0 + wm * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    if (row < T && col < E) logits[(size_t)row * E + col] = acc[i];
  }
}

hipError_t launch_router_mfma(const uint16_t* x, const float* wr, int T, int H, int E, float* logits, hipStream_t s) {
  const unsigned blocks = (unsigned)(((T + 63) / 64) * ((E + 63) / 64));
  hipLaunchKernelGGL(k_router_mfma, dim3(blocks), dim3(256), 0, s, x, wr, T, H, E, logits);
  return hipGetLastError();
}

static size_t big_tiles_max(int E, int total_rows) { return (size_t)total_rows / 64 + E + 1; }
static size_t tables_bytes(int E, int total_rows) {
  const size_t t = (1 + 2 * big_tiles_max(E, total_rows) + 1 + 2 * ((size_t)E + 1)) * sizeof(int32_t);
  return (t + 255) & ~(size_t)255;
}

size_t mfma_ws_bytes(int E, int H, int I, int total_rows) {
  (void)H;
  return tables_bytes(E, total_rows) + (((size_t)total_rows * I * 2 + 255) & ~(size_t)255);
}

bool mfma_shape_ok(int H, int I) { return H % 128 == 0 && I % 64 == 0; }

// 64-row remainder tiles need 128-feature gate/up slices and 256-column down slices.
static bool small_tiles_ok(int H, int I) { return I % 128 == 0 && H % 256 == 0; }

hipError_t launch_grouped_mfma(const moe_ffn_weights* w, int E, const int32_t* offsets, const int32_t* sorted_pairs,
                               int k, const uint16_t* x, int H, int I, int total_rows, float* out, void* ws,
                               hipStream_t s) {
  if (w->gate.fmt != kFmtNvfp4 && w->gate.fmt != kFmtInt4) return hipErrorInvalidValue;  // NVFP4, INT4 only
  const size_t max_big = big_tiles_max(E, total_rows);
  int32_t* big = (int32_t*)ws;
  int32_t* small = big + 1 + 2 * max_big;
  uint16_t* h = (uint16_t*)((char*)ws + tables_bytes(E, total_rows));
  const bool split = small_tiles_ok(H, I);
  MfmaArgs g;
  g.H = H;
  g.I = I;
  g.k = k;
  g.rows = total_rows;
  g.x = x;
  g.sorted_pairs = sorted_pairs;
  g.offsets = offsets;
  g.gc = w->gate.codes;
  g.gs = (const uint8_t*)w->gate.scales;
  g.gz = w->gate.zeros;
  g.uc = w->up.codes;
  g.us = (const uint8_t*)w->up.scales;
  g.uz = w->up.zeros;
  g.dc = w->down.codes;
  g.ds = (const uint8_t*)w->down.scales;
  g.dz = w->down.zeros;
  g.gts = w->gate.tensor_scale;
  g.uts = w->up.tensor_scale;
  g.dts = w->down.tensor_scale;
  g.h = h;
  g.out = out;
  // 64-row tiles everywhere (k_mfma_bl / k_mfma_bd).
  if (split && bd_k_ok(w->gate.fmt, H) && bd_k_ok(w->gate.fmt, I)) {
    MOE_LAUNCH(k_tile_table, dim3(1), dim3(1024), 0, s, offsets, E, total_rows, 64, 0, big, small);
    const unsigned b8 = (unsigned)((max_big + 7) / 8 * 8);
    MfmaArgs ga = g;
    ga.tiles = big;
    ga.tile_rows = 64;
    if (w->gate.fmt == kFmtNvfp4) {
      MOE_LAUNCH((k_mfma_bl<kFmtNvfp4, true>), dim3(b8 * (I / 128)), dim3(256), 0, s, ga);
      MOE_LAUNCH((k_mfma_bl<kFmtNvfp4, false>), dim3(b8 * (H / 256)), dim3(256), 0, s, ga);
    } else {
      MOE_LAUNCH((k_mfma_bd<kFmtInt4, 2, true>), dim3(b8 * (I / 128)), dim3(256), 0, s, ga);
      MOE_LAUNCH((k_mfma_bd<kFmtInt4, 2, false>), dim3(b8 * (H / 256)), dim3(256), 0, s, ga);
    }
    return hipGetLastError();
  }
  // Otherwise LDS-staged weights: 128-row tiles, with a final remainder of at
  // most 64 rows in a 64-row tile when the shapes allow.
  MOE_LAUNCH(k_tile_table, dim3(1), dim3(1024), 0, s, offsets, E, total_rows, kBM, split ? 1 : 0, big, small);
  // one block per (row tile, column slice); tiles rounded up to a multiple of the 8 XCDs
  const unsigned big8 = (unsigned)((max_big + 7) / 8 * 8), small8 = (unsigned)((E + 7) / 8 * 8);
  MfmaArgs gb = g, gs = g;
  gb.tiles = big;
  gb.tile_rows = kBM;
  gs.tiles = small;
  gs.tile_rows = 64;
  const dim3 gu_small(small8 * (I / 128)), dn_small(small8 * (H / 256));
  if (w->gate.fmt == kFmtNvfp4) {
    MOE_LAUNCH((k_mfma_gateup<kFmtNvfp4, 2>), dim3(big8 * (I / 64)), dim3(256), 0, s, gb);
    if (split) MOE_LAUNCH((k_mfma_gateup<kFmtNvfp4, 1>), gu_small, dim3(256), 0, s, gs);
    MOE_LAUNCH((k_mfma_down<kFmtNvfp4, 2>), dim3(big8 * (H / 128)), dim3(256), 0, s, gb);
    if (split) MOE_LAUNCH((k_mfma_down<kFmtNvfp4, 1>), dn_small, dim3(256), 0, s, gs);
  } else {
    MOE_LAUNCH((k_mfma_gateup<kFmtInt4, 2>), dim3(big8 * (I / 64)), dim3(256), 0, s, gb);
    if (split) MOE_LAUNCH((k_mfma_gateup<kFmtInt4, 1>), gu_small, dim3(256), 0, s, gs);
    MOE_LAUNCH((k_mfma_down<kFmtInt4, 2>), dim3(big8 * (H / 128)), dim3(256), 0, s, gb);
    if (split) MOE_LAUNCH((k_mfma_down<kFmtInt4, 1>), dn_small, dim3(256), 0, s, gs);
  }
  return hipGetLastError();
}

}  // namespace moe
