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
// (row >> 1) & 7, so the 16 lanes of an LDS pass hit distinct banks.
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

MOE_DEV int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }  // in 16-byte units

// Dequantise 32 consecutive weights (16 bytes of codes) of one row into 4
// bf16 chunks of 8.  NVFP4: two e4m3 block scales (bytes 0, 1 of `sc`).
// INT4: zero point z; the result is the exact integer q - z.
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
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = (float)((int)((w[q] >> (4 * j)) & 15u) - z);
    }
    // exact values: the conversion to bf16 does not round
    o[q].x = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    o[q].y = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
    o[q].z = f32_to_bf16_rne(v[4]) | (f32_to_bf16_rne(v[5]) << 16);
    o[q].w = f32_to_bf16_rne(v[6]) | (f32_to_bf16_rne(v[7]) << 16);
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

// ------------------------------------------------------------------ gate/up
// Block: 4 waves as 2 (rows) x 2 (features); each wave owns a 64-row x 32-
// feature tile of both G and U (2 x 2 accumulators of 32 x 32).
template <int FMT>
__global__ void __launch_bounds__(256) k_mfma_gateup(MfmaArgs g) {
  __shared__ uint4 As[kBM * 8];  // [128][64] bf16, swizzled
  __shared__ uint4 Bs[128 * 8];  // rows 0..63 gate, 64..127 up
  int e, r0, r1;
  if (!tile_of(g, blockIdx.x, e, r0, r1)) return;
  const int H = g.H, I = g.I;
  const int n0 = blockIdx.y * 64;
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

  f32x16_t acc[2][2];  // [gate / up][row sub-tile]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int m = 0; m < 2; ++m) acc[a][m] = f32x16_t{};

  const int nk = H / kBK;
  uint4 ra[4], rb;
  uint32_t rsc = 0;
  int rz = 0;
  auto load = [&](int kt) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ra[c] = a_valid ? ((const uint4*)(xrow + kt * kBK))[a_c0 + c] : make_uint4(0, 0, 0, 0);
    rb = *(const uint4*)(bcodes + kt * (kBK / 2));
    if (FMT == kFmtNvfp4) {
      rsc = *(const uint16_t*)(bscales + wrow * (H / 16) + kt * 4 + b_half * 2);
    } else {
      rsc = 0;
      rz = bzeros[wrow * (H / 64) + kt];
    }
  };
  // per-lane INT4 group scales of this wave's gate / up feature column
  const int ncol = n0 + wn * 32 + (lane & 31);
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) As[swz(a_row, a_c0 + c)] = ra[c];
    {
      uint4 o[4];
      dequant32<FMT>(rb, rsc, rz, o);
#pragma unroll
      for (int c = 0; c < 4; ++c) Bs[swz(b_mat * 64 + b_row, b_half * 4 + c)] = o[c];
    }
    __syncthreads();
    float sg = 1.f, su = 1.f;
    if (FMT == kFmtInt4) {
      sg = f16_to_f32(((const uint16_t*)g.gs)[((size_t)e * I + ncol) * (H / 64) + kt]);
      su = f16_to_f32(((const uint16_t*)g.us)[((size_t)e * I + ncol) * (H / 64) + kt]);
    }
    if (kt + 1 < nk) load(kt + 1);
    f32x16_t part[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int m = 0; m < 2; ++m) part[a][m] = (FMT == kFmtInt4) ? f32x16_t{} : acc[a][m];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      const bf16x8_t a0 = lds_frag(As, wm * 64 + (lane & 31), chunk);
      const bf16x8_t a1 = lds_frag(As, wm * 64 + 32 + (lane & 31), chunk);
      const bf16x8_t bg = lds_frag(Bs, wn * 32 + (lane & 31), chunk);
      const bf16x8_t bu = lds_frag(Bs, 64 + wn * 32 + (lane & 31), chunk);
      part[0][0] = mfma(a0, bg, part[0][0]);
      part[0][1] = mfma(a1, bg, part[0][1]);
      part[1][0] = mfma(a0, bu, part[1][0]);
      part[1][1] = mfma(a1, bu, part[1][1]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (FMT == kFmtInt4) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[0][m][i] = fmaf(sg, part[0][m][i], acc[0][m][i]);
          acc[1][m][i] = fmaf(su, part[1][m][i], acc[1][m][i]);
        }
      } else {
        acc[0][m] = part[0][m];
        acc[1][m] = part[1][m];
      }
    }
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
  __shared__ uint4 As[kBM * 8];
  __shared__ uint4 Bs[128 * 8];
  int e, r0, r1;
  if (!tile_of(g, blockIdx.x, e, r0, r1)) return;
  const int H = g.H, I = g.I;
  const int n0 = blockIdx.y * 128;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int a_row = tid >> 1, a_c0 = (tid & 1) * 4;
  const bool a_valid = r0 + a_row < r1;
  const uint16_t* hrow = g.h + (size_t)(a_valid ? r0 + a_row : r0) * I;
  const int b_row = tid >> 1, b_half = tid & 1;
  const size_t wrow = (size_t)e * H + n0 + b_row;
  const uint8_t* bcodes = g.dc + wrow * (I / 2) + b_half * 16;

  f32x16_t acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x16_t{};
  const int nk = I / kBK;
  uint4 ra[4], rb;
  uint32_t rsc = 0;
  int rz = 0;
  auto load = [&](int kt) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ra[c] = a_valid ? ((const uint4*)(hrow + kt * kBK))[a_c0 + c] : make_uint4(0, 0, 0, 0);
    rb = *(const uint4*)(bcodes + kt * (kBK / 2));
    if (FMT == kFmtNvfp4) {
      rsc = *(const uint16_t*)(g.ds + wrow * (I / 16) + kt * 4 + b_half * 2);
    } else {
      rz = g.dz[wrow * (I / 64) + kt];
    }
  };
  const int ncol0 = n0 + wn * 64 + (lane & 31);
  load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) As[swz(a_row, a_c0 + c)] = ra[c];
    {
      uint4 o[4];
      dequant32<FMT>(rb, rsc, rz, o);
#pragma unroll
      for (int c = 0; c < 4; ++c) Bs[swz(b_row, b_half * 4 + c)] = o[c];
    }
    __syncthreads();
    float s0 = 1.f, s1 = 1.f;
    if (FMT == kFmtInt4) {
      s0 = f16_to_f32(((const uint16_t*)g.ds)[((size_t)e * H + ncol0) * (I / 64) + kt]);
      s1 = f16_to_f32(((const uint16_t*)g.ds)[((size_t)e * H + ncol0 + 32) * (I / 64) + kt]);
    }
    if (kt + 1 < nk) load(kt + 1);
    f32x16_t part[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) part[m][n] = (FMT == kFmtInt4) ? f32x16_t{} : acc[m][n];
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      const bf16x8_t a0 = lds_frag(As, wm * 64 + (lane & 31), chunk);
      const bf16x8_t a1 = lds_frag(As, wm * 64 + 32 + (lane & 31), chunk);
      const bf16x8_t b0 = lds_frag(Bs, wn * 64 + (lane & 31), chunk);
      const bf16x8_t b1 = lds_frag(Bs, wn * 64 + 32 + (lane & 31), chunk);
      part[0][0] = mfma(a0, b0, part[0][0]);
      part[0][1] = mfma(a0, b1, part[0][1]);
      part[1][0] = mfma(a1, b0, part[1][0]);
      part[1][1] = mfma(a1, b1, part[1][1]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (FMT == kFmtInt4) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc[m][0][i] = fmaf(s0, part[m][0][i], acc[m][0][i]);
          acc[m][1][i] = fmaf(s1, part[m][1][i], acc[m][1][i]);
        }
      } else {
        acc[m][0] = part[m][0];
        acc[m][1] = part[m][1];
      }
    }
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
  const dim3 ga((unsigned)max_tiles, I / 64), gd((unsigned)max_tiles, H / 128);
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
