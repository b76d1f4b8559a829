// Grouped SwiGLU experts on the bf16 matrix cores (gfx950 MFMA), for
// prefill and large batches: the "grouped-GEMM path" that "[Model] Add Flint
// (RecursiveSI/flint)" (section "What happened") uses when a batch gives
// each expert many tokens.
//
// Per expert e with rows [offsets[e], offsets[e+1]) (tokens gathered through
// sorted_pairs):
//   gate/up kernel: G = X_e Wg_e^T, U = X_e Wu_e^T over K = H, then
//                   h = bf16(silu(G) * U) for a 128-row x 64-feature tile;
//   down kernel:    O = h_e Wd_e^T over K = I, fp32, 128 x 128 tiles.
// A device-side tile table lists (expert, first row) for every 128-row tile.
//
// Weights are dequantised once per 64-wide K step into LDS as bf16:
//   NVFP4: e4m3 * e2m1 has at most 6 significant bits, so the bf16 operand is
//          exact; the fp32 tensor scale multiplies the accumulator at the end;
//   INT4:  the operand is the exact integer (q - z); each 64-wide K step is one
//          quantisation group, accumulated separately and scaled by its fp16
//          scale in fp32 (s * (q - z) itself would not be exact in bf16).
// MFMA: v_mfma_f32_32x32x16_bf16.  Operands: lane l supplies row (A) or column
// (B) l % 32 and 8 consecutive k values; the accumulator register i of lane l
// holds row (i / 4) * 8 + (l / 32) * 4 + i % 4, column l % 32.
// LDS tiles are [128 rows][64 k] bf16 with the 16-byte chunk index XOR-ed by
// row & 7: a 128-byte row spans all 32 banks, so the 8 lanes that one LDS
// cycle serves for a 16-byte access (8 consecutive rows at one chunk, or 4
// rows at chunks c and c + 4) land on distinct banks.  Two tile buffers
// alternate between K steps, so each step needs one barrier.
#include "common.cuh"
#include "launch.h"
#include "route.cuh"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;  // rows (tokens) per tile
constexpr int kBK = 64;   // reduction step = one INT4 group

struct MfmaArgs {
  int H, I, k, rows;
  const uint16_t* x;            // gate/up: tokens [T, H]
  const int32_t* sorted_pairs;  // NULL: sorted row r is token r
  const int32_t* offsets;       // [E + 1]; NULL: one expert over rows [0, rows)
  const int32_t* tiles;         // [0] = count, then (expert, first row) pairs
  const uint8_t *gc, *gs, *gz;  // gate codes / scales / zeros
  const uint8_t *uc, *us, *uz;  // up
  const uint8_t *dc, *ds, *dz;  // down
  const float *gts, *uts, *dts; // NVFP4 tensor scales
  uint16_t* h;                  // [rows, I]
  float* out;                   // [rows, H]
};

MOE_DEV int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }  // in 16-byte units

// Dequantise 32 consecutive weights (16 bytes of codes) of one row into 4
// bf16 chunks of 8.  NVFP4: two e4m3 block scales (bytes 0, 1 of `sc`).
// INT4: zero point z; the result is the exact integer q - z.  Every value is
// exact in fp32 and in bf16, so the hardware fp32 -> bf16 conversion does
// not round.
MOE_DEV uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <int FMT>
MOE_DEV void dequant32(uint4 c, uint32_t sc, int z, uint4 (&o)[4]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
    if (FMT == kFmtNvfp4) {
      const float b = e4m3_to_f32(sc, q >> 1);
      const moe_f32x2 p0 = e2m1x2_to_f32<0>(w[q]), p1 = e2m1x2_to_f32<1>(w[q]);
      const moe_f32x2 p2 = e2m1x2_to_f32<2>(w[q]), p3 = e2m1x2_to_f32<3>(w[q]);
      v[0] = p0.x * b; v[1] = p0.y * b; v[2] = p1.x * b; v[3] = p1.y * b;
      v[4] = p2.x * b; v[5] = p2.y * b; v[6] = p3.x * b; v[7] = p3.y * b;
    } else {
      // 2^23 + q as fp32 bits, minus 2^23 + z: exact
      const float off = 8388608.0f + (float)z;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(0x4B000000u | ((w[q] >> (4 * j)) & 15u)) - off;
    }
    o[q].x = pack_bf16(v[0], v[1]);
    o[q].y = pack_bf16(v[2], v[3]);
    o[q].z = pack_bf16(v[4], v[5]);
    o[q].w = pack_bf16(v[6], v[7]);
  }
}

MOE_DEV bf16x8_t lds_frag(const uint4* tile, int row, int chunk) {
  return __builtin_bit_cast(bf16x8_t, tile[swz(row, chunk)]);
}

MOE_DEV f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

MOE_DEV bool tile_of(const MfmaArgs& g, int mt, int& e, int& r0, int& r1) {
  if (mt >= g.tiles[0]) return false;
  e = g.tiles[1 + 2 * mt];
  r0 = g.tiles[2 + 2 * mt];
  const int end = g.offsets ? g.offsets[e + 1] : g.rows;
  r1 = min(end, r0 + kBM);
  return true;
}

// Tile table: one block; expert e contributes ceil(count_e / 128) tiles.
__global__ void __launch_bounds__(1024) k_tile_table(const int32_t* __restrict__ offsets, int E, int rows,
                                                     int32_t* __restrict__ tiles) {
  __shared__ int scan_lds[17];
  const int e = threadIdx.x;
  int r0 = 0, r1 = 0;
  if (e < E) {
    r0 = offsets ? offsets[e] : 0;
    r1 = offsets ? offsets[e + 1] : rows;
  }
  const int nt = (r1 - r0 + kBM - 1) / kBM;
  int total;
  const int first = block_exclusive_scan(nt, scan_lds, total);
  for (int t = 0; t < nt; ++t) {
    tiles[1 + 2 * (first + t)] = e;
    tiles[2 + 2 * (first + t)] = r0 + t * kBM;
  }
  if (e == 0) tiles[0] = total;
}

// One K step's global data for this thread, loaded two steps ahead of its
// use (two register sets in turn) so that the memory latency is covered by
// the matrix work of the steps in between.
struct MfmaStage {
  uint4 a[4];      // 4 x 8 bf16 of one activation row
  uint4 b;         // 32 packed 4-bit weights of one weight row
  uint32_t sc;     // NVFP4: the two e4m3 block scales of those 32 weights
  int z;           // INT4: zero point of this K step's group
  float s0, s1;    // INT4: this wave's two per-column group scales (fp16 -> fp32)
};

// Map the block index to (row tile, column slice) so that every column slice
// of a row tile runs on the same XCD (blocks go to XCDs round-robin), and the
// tile's activation rows stay in that XCD's L2.
MOE_DEV void block_tile(int nslices, int& tile, int& slice) {
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3;
  tile = (j / nslices) * 8 + xcd;
  slice = j % nslices;
}

// ------------------------------------------------------------------ gate/up
// Block: 4 waves as 2 (rows) x 2 (features); each wave owns a 64-row x 32-
// feature tile of both G and U (2 x 2 accumulators of 32 x 32).
template <int FMT>
__global__ void __launch_bounds__(256) k_mfma_gateup(MfmaArgs g) {
  __shared__ uint4 As2[2][kBM * 8];  // [128][64] bf16, swizzled
  __shared__ uint4 Bs2[2][128 * 8];  // rows 0..63 gate, 64..127 up
  int tile, slice;
  block_tile(g.I / 64, tile, slice);
  int e, r0, r1;
  if (!tile_of(g, tile, e, r0, r1)) return;
  const int H = g.H, I = g.I;
  const int n0 = slice * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // loader roles: A row tid >> 1, 4 chunks from (tid & 1) * 4; B matrix tid >> 7, row (tid >> 1) & 63, half tid & 1
  const int a_row = tid >> 1, a_c0 = (tid & 1) * 4;
  const bool a_valid = r0 + a_row < r1;
  const int tok = a_valid ? (g.sorted_pairs ? g.sorted_pairs[r0 + a_row] / g.k : r0 + a_row) : 0;
  const uint16_t* xrow = g.x + (size_t)tok * H;
  const int b_mat = tid >> 7, b_row = (tid >> 1) & 63, b_half = tid & 1;
  const size_t wrow = (size_t)e * I + n0 + b_row;
  const uint8_t* bcodes = (b_mat ? g.uc : g.gc) + wrow * (H / 2) + b_half * 16;
  const uint8_t* bscales = b_mat ? g.us : g.gs;
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
  auto load = [&](int kt, MfmaStage& st) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.a[c] = a_valid ? ((const uint4*)(xrow + kt * kBK))[a_c0 + c] : make_uint4(0, 0, 0, 0);
    st.b = *(const uint4*)(bcodes + kt * (kBK / 2));
    if (FMT == kFmtNvfp4) {
      st.sc = *(const uint16_t*)(bscales + wrow * (H / 16) + kt * 4 + b_half * 2);
    } else {
      st.z = bzeros[wrow * (H / 64) + kt];
      st.s0 = f16_to_f32(gsc[kt]);
      st.s1 = f16_to_f32(usc[kt]);
    }
  };
  // Write this K step's tiles into buffer `buf`.  The buffer was last read
  // two steps ago, before every wave passed the previous step's barrier.
  auto step = [&](const MfmaStage& st, int buf) {
    uint4* As = As2[buf];
    uint4* Bs = Bs2[buf];
#pragma unroll
    for (int c = 0; c < 4; ++c) As[swz(a_row, a_c0 + c)] = st.a[c];
    {
      uint4 o[4];
      dequant32<FMT>(st.b, st.sc, st.z, o);
#pragma unroll
      for (int c = 0; c < 4; ++c) Bs[swz(b_mat * 64 + b_row, b_half * 4 + c)] = o[c];
    }
    __syncthreads();
  };
  // NVFP4 accumulates straight into acc; INT4 accumulates one group in part
  // and adds it to acc times the group's scale.
  auto mma = [&](f32x16_t (&c)[2][2], int buf) {
    const uint4* As = As2[buf];
    const uint4* Bs = Bs2[buf];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      const bf16x8_t a0 = lds_frag(As, wm * 64 + (lane & 31), chunk);
      const bf16x8_t a1 = lds_frag(As, wm * 64 + 32 + (lane & 31), chunk);
      const bf16x8_t bg = lds_frag(Bs, wn * 32 + (lane & 31), chunk);
      const bf16x8_t bu = lds_frag(Bs, 64 + wn * 32 + (lane & 31), chunk);
      c[0][0] = mfma(a0, bg, c[0][0]);
      c[0][1] = mfma(a1, bg, c[0][1]);
      c[1][0] = mfma(a0, bu, c[1][0]);
      c[1][1] = mfma(a1, bu, c[1][1]);
    }
  };
  auto compute = [&](float sg, float su, int buf) {
    if (FMT == kFmtNvfp4) {
      mma(acc, buf);
    } else {
      f32x16_t part[2][2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int m = 0; m < 2; ++m) part[a][m] = f32x16_t{};
      mma(part, buf);
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
  MfmaStage s0, s1;
  load(0, s0);
  if (nk > 1) load(1, s1);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(s0, 0);
    const float q0 = s0.s0, q1 = s0.s1;
    if (kt + 2 < nk) load(kt + 2, s0);
    compute(q0, q1, 0);
    step(s1, 1);
    const float p0 = s1.s0, p1 = s1.s1;
    if (kt + 3 < nk) load(kt + 3, s1);
    compute(p0, p1, 1);
  }
  if (kt < nk) {  // odd number of K steps
    step(s0, 0);
    compute(s0.s0, s0.s1, 0);
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
// Block: 4 waves as 2 x 2, each a 64-row x 64-column tile (2 x 2 accumulators).
template <int FMT>
__global__ void __launch_bounds__(256) k_mfma_down(MfmaArgs g) {
  __shared__ uint4 As2[2][kBM * 8];
  __shared__ uint4 Bs2[2][128 * 8];
  int tile, slice;
  block_tile(g.H / 128, tile, slice);
  int e, r0, r1;
  if (!tile_of(g, tile, e, r0, r1)) return;
  const int H = g.H, I = g.I;
  const int n0 = slice * 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int a_row = tid >> 1, a_c0 = (tid & 1) * 4;
  const bool a_valid = r0 + a_row < r1;
  const uint16_t* hrow = g.h + (size_t)(a_valid ? r0 + a_row : r0) * I;
  const int b_row = tid >> 1, b_half = tid & 1;
  const size_t wrow = (size_t)e * H + n0 + b_row;
  const uint8_t* bcodes = g.dc + wrow * (I / 2) + b_half * 16;
  const int ncol0 = n0 + wn * 64 + (lane & 31);
  const uint16_t* dsc0 = (const uint16_t*)g.ds + ((size_t)e * H + ncol0) * (I / 64);
  const uint16_t* dsc1 = (const uint16_t*)g.ds + ((size_t)e * H + ncol0 + 32) * (I / 64);

  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x16_t{};
  const int nk = I / kBK;
  auto load = [&](int kt, MfmaStage& st) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      st.a[c] = a_valid ? ((const uint4*)(hrow + kt * kBK))[a_c0 + c] : make_uint4(0, 0, 0, 0);
    st.b = *(const uint4*)(bcodes + kt * (kBK / 2));
    if (FMT == kFmtNvfp4) {
      st.sc = *(const uint16_t*)(g.ds + wrow * (I / 16) + kt * 4 + b_half * 2);
    } else {
      st.z = g.dz[wrow * (I / 64) + kt];
      st.s0 = f16_to_f32(dsc0[kt]);
      st.s1 = f16_to_f32(dsc1[kt]);
    }
  };
  auto step = [&](const MfmaStage& st, int buf) {
    uint4* As = As2[buf];
    uint4* Bs = Bs2[buf];
#pragma unroll
    for (int c = 0; c < 4; ++c) As[swz(a_row, a_c0 + c)] = st.a[c];
    {
      uint4 o[4];
      dequant32<FMT>(st.b, st.sc, st.z, o);
#pragma unroll
      for (int c = 0; c < 4; ++c) Bs[swz(b_row, b_half * 4 + c)] = o[c];
    }
    __syncthreads();
  };
  auto mma = [&](f32x16_t (&c)[2][2], int buf) {
    const uint4* As = As2[buf];
    const uint4* Bs = Bs2[buf];
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
  auto compute = [&](float s0, float s1, int buf) {
    if (FMT == kFmtNvfp4) {
      mma(acc, buf);
    } else {
      f32x16_t part[2][2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) part[m][n] = f32x16_t{};
      mma(part, buf);
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
  MfmaStage s0, s1;
  load(0, s0);
  if (nk > 1) load(1, s1);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(s0, 0);
    const float q0 = s0.s0, q1 = s0.s1;
    if (kt + 2 < nk) load(kt + 2, s0);
    compute(q0, q1, 0);
    step(s1, 1);
    const float p0 = s1.s0, p1 = s1.s1;
    if (kt + 3 < nk) load(kt + 3, s1);
    compute(p0, p1, 1);
  }
  if (kt < nk) {  // odd number of K steps
    step(s0, 0);
    compute(s0.s0, s0.s1, 0);
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

// ------------------------------------------------------------------ router (large batches)
// logits[t, e] = sum_h x[t, h] * w[e, h] on the matrix cores.  Each fp32
// router weight is split exactly into three bf16 parts, w = hi + mid + lo
// (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid, each residual exact
// in fp32 and the last one exact in bf16), so every product x * part is exact
// in fp32 and the three MFMAs accumulate them in fp32, as the VALU router's
// fused multiply-adds do (in another order).  Block: 64 tokens x 64 experts,
// 4 waves as 2 x 2 of 32 x 32; 64-wide K steps staged through LDS, global
// data loaded two steps ahead.
// Named, interleaved fields: adjacent copies from adjacent global addresses
// are merged into one block copy that the compiler keeps in private memory.
struct RouterStage {
  uint4 a0;     // bf16 0..7 of one token row's 16
  float4 w0;    // fp32 0..3 of one router row's 16
  uint4 a1;     // bf16 8..15
  float4 w1, w2, w3;
};

MOE_DEV void split3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const __bf16 h = (__bf16)w;
  const float r1 = w - (float)h;
  const __bf16 m = (__bf16)r1;
  const __bf16 l = (__bf16)(r1 - (float)m);
  hi = __builtin_bit_cast(uint16_t, h);
  mid = __builtin_bit_cast(uint16_t, m);
  lo = __builtin_bit_cast(uint16_t, l);
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

MOE_DEV void router_compute(const uint4* As, const uint4 (*Bs)[64 * 8], int wm, int wn, int lane, f32x16_t& acc) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int chunk = ks * 2 + (lane >> 5);
    const bf16x8_t a = lds_frag(As, wm * 32 + (lane & 31), chunk);
    const int brow = wn * 32 + (lane & 31);
    acc = mfma(a, lds_frag(Bs[2], brow, chunk), acc);
    acc = mfma(a, lds_frag(Bs[1], brow, chunk), acc);
    acc = mfma(a, lds_frag(Bs[0], brow, chunk), acc);
  }
}

__global__ void __launch_bounds__(256) k_router_mfma(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                     int T, int H, int E, float* __restrict__ logits) {
  __shared__ uint4 As[64 * 8];      // [64 tokens][64 k] bf16, swizzled
  __shared__ uint4 Bs[3][64 * 8];   // hi / mid / lo parts of [64 experts][64 k]
  const int nte = (E + 63) / 64;
  const int t0 = (blockIdx.x / nte) * 64, e0 = (blockIdx.x % nte) * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // loaders: token row tid >> 2, 16 bf16 at (tid & 3) * 16; router row tid >> 2, 16 fp32 at (tid & 3) * 16
  const int lrow = tid >> 2, lq = tid & 3;
  const uint16_t* xrow = x + (size_t)min(t0 + lrow, T - 1) * H + lq * 16;
  const float* wrow = wr + (size_t)min(e0 + lrow, E - 1) * H + lq * 16;
  f32x16_t acc = f32x16_t{};
  const int nk = H / 64;
  RouterStage s0, s1;
  router_load(xrow, wrow, 0, s0);
  if (nk > 1) router_load(xrow, wrow, 1, s1);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    router_stage(s0, lrow, lq, As, Bs);
    if (kt + 2 < nk) router_load(xrow, wrow, kt + 2, s0);
    router_compute(As, Bs, wm, wn, lane, acc);
    router_stage(s1, lrow, lq, As, Bs);
    if (kt + 3 < nk) router_load(xrow, wrow, kt + 3, s1);
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

size_t mfma_ws_bytes(int E, int H, int I, int total_rows) {
  const size_t max_tiles = (size_t)total_rows / kBM + E + 1;
  const size_t t = (1 + 2 * max_tiles) * sizeof(int32_t);
  (void)H;
  return ((t + 255) & ~(size_t)255) + (((size_t)total_rows * I * 2 + 255) & ~(size_t)255);
}

bool mfma_shape_ok(int H, int I) { return H % 128 == 0 && I % 64 == 0; }

hipError_t launch_grouped_mfma(const moe_ffn_weights* w, int E, const int32_t* offsets, const int32_t* sorted_pairs,
                               int k, const uint16_t* x, int H, int I, int total_rows, float* out, void* ws,
                               hipStream_t s) {
  const size_t max_tiles = (size_t)total_rows / kBM + E + 1;
  int32_t* tiles = (int32_t*)ws;
  const size_t t = (1 + 2 * max_tiles) * sizeof(int32_t);
  uint16_t* h = (uint16_t*)((char*)ws + ((t + 255) & ~(size_t)255));
  MfmaArgs g;
  g.H = H;
  g.I = I;
  g.k = k;
  g.rows = total_rows;
  g.x = x;
  g.sorted_pairs = sorted_pairs;
  g.offsets = offsets;
  g.tiles = tiles;
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
  hipLaunchKernelGGL(k_tile_table, dim3(1), dim3(1024), 0, s, offsets, E, total_rows, tiles);
  // one block per (row tile, column slice); tiles rounded up to a multiple of the 8 XCDs
  const unsigned tiles8 = (unsigned)((max_tiles + 7) / 8 * 8);
  const dim3 ga(tiles8 * (I / 64)), gd(tiles8 * (H / 128));
  if (w->gate.fmt == kFmtNvfp4) {
    hipLaunchKernelGGL(k_mfma_gateup<kFmtNvfp4>, ga, dim3(256), 0, s, g);
    hipLaunchKernelGGL(k_mfma_down<kFmtNvfp4>, gd, dim3(256), 0, s, g);
  } else {
    hipLaunchKernelGGL(k_mfma_gateup<kFmtInt4>, ga, dim3(256), 0, s, g);
    hipLaunchKernelGGL(k_mfma_down<kFmtInt4>, gd, dim3(256), 0, s, g);
  }
  return hipGetLastError();
}

}  // namespace moe
