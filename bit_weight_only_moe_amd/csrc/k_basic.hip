// Router, top-k, grouping, combine and dequantisation kernels (gfx950).
//
// The layer routes every token to the k best of E experts through a "fused
// top-k router", groups the (token, expert) pairs for "expert-indexed GEMVs"
// or a grouped GEMM ("[Model] Add Flint (RecursiveSI/flint)", section "What
// happened"), and adds the weighted expert outputs to an always-on shared
// expert ("Recursive Flint: 125 tok/s on an M4 Pro, measured where it matters
// least", table under "What actually shipped").
#include "common.cuh"
#include "launch.h"
#include "route.cuh"

namespace moe {

// ---------------------------------------------------------------- dequant
// One thread per 8 consecutive elements (one 32-bit word of codes); the
// tensor scale of the expert is read from device memory.
__global__ void __launch_bounds__(256) k_dequant_dev_ts(int fmt, int rows, int cols, const uint8_t* __restrict__ codes,
                                                        const void* __restrict__ scales,
                                                        const uint8_t* __restrict__ zeros,
                                                        const float* __restrict__ ts_ptr, float* __restrict__ out) {
  const float ts = (fmt == kFmtNvfp4) ? *ts_ptr : 1.0f;
  const int words_per_row = cols / 8;
  const long long w = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= (long long)rows * words_per_row) return;
  const int r = (int)(w / words_per_row);
  const int c0 = (int)(w % words_per_row) * 8;
  float v[8];
  if (fmt == kFmtBf16) {
    const uint4 b = *(const uint4*)(codes + ((size_t)r * cols + c0) * 2);
    const uint32_t h[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(h[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(h[i] >> 16);
    }
    float4* o = (float4*)(out + (size_t)r * cols + c0);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
    return;
  }
  const uint32_t word = *(const uint32_t*)(codes + (size_t)r * (cols / 2) + c0 / 2);
  if (fmt == kFmtNvfp4) {
    const uint8_t sb = ((const uint8_t*)scales)[(size_t)r * (cols / 16) + c0 / 16];
    const float b = e4m3_to_f32(sb, 0);
    moe_f32x2 p0 = e2m1x2_to_f32<0>(word), p1 = e2m1x2_to_f32<1>(word);
    moe_f32x2 p2 = e2m1x2_to_f32<2>(word), p3 = e2m1x2_to_f32<3>(word);
    v[0] = p0.x; v[1] = p0.y; v[2] = p1.x; v[3] = p1.y;
    v[4] = p2.x; v[5] = p2.y; v[6] = p3.x; v[7] = p3.y;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (b * v[i]) * ts;
  } else if (fmt == kFmtInt4Sb) {
    // one fused multiply-add: the single rounding of s * q + b
    const size_t g = (size_t)r * (cols / 64) + c0 / 64;
    const float s = f16_to_f32(((const uint16_t*)scales)[g]);
    const float b = f16_to_f32(((const uint16_t*)zeros)[g]);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = fmaf(s, (float)((word >> (4 * i)) & 15u), b);
  } else {
    const size_t g = (size_t)r * (cols / 64) + c0 / 64;
    const float s = f16_to_f32(((const uint16_t*)scales)[g]);
    const int z = zeros[g];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s * (float)((int)((word >> (4 * i)) & 15u) - z);
  }
  float4* o = (float4*)(out + (size_t)r * cols + c0);
  o[0] = make_float4(v[0], v[1], v[2], v[3]);
  o[1] = make_float4(v[4], v[5], v[6], v[7]);
}

hipError_t launch_dequant_expert(int fmt, int rows, int cols, const uint8_t* codes, const void* scales,
                                 const uint8_t* zeros, const float* ts_dev, float* out, hipStream_t s) {
  const long long words = (long long)rows * (cols / 8);
  const int blocks = (int)((words + 255) / 256);
  hipLaunchKernelGGL(k_dequant_dev_ts, dim3(blocks), dim3(256), 0, s, fmt, rows, cols, codes, scales, zeros, ts_dev,
                     out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- router GEMV
// logits[t, e] = sum_h x[t, h] * w_router[e, h], fp32 accumulation.
// Block: 4 waves = 4 experts; up to kRouteTok tokens staged in LDS as bf16
// (at most 64 KB).
constexpr int kRouteTok = 16;
constexpr int kRouteT4 = 4;  // tokens per block when the logits stay in LDS
constexpr int kRouterMfmaMinT = 256;

__global__ void __launch_bounds__(256) k_router_logits(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                       int T, int H, int E, int tpb, float* __restrict__ logits) {
  extern __shared__ __align__(16) uint16_t xs[];  // [tpb][H], tpb <= kRouteTok
  const int t0 = blockIdx.y * tpb;
  const int nt = min(tpb, T - t0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + wave;
  float4 wv[kRouterC];
  router_prefetch(wr + (size_t)min(e, E - 1) * H, H, lane, wv);  // past the last expert: unused
  copy_to_lds((uint4*)xs, (const uint4*)(x + (size_t)t0 * H), nt * H / 8);
  __syncthreads();
  if (e >= E) return;
  float acc[kRouteTok];
  router_dots<kRouteTok>(wr + (size_t)e * H, xs, H, nt, lane, acc, wv);
#pragma unroll
  for (int t = 0; t < kRouteTok; ++t)
    if (t < nt && lane == 63) logits[(size_t)(t0 + t) * E + e] = acc[t];
}

hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                                hipStream_t s) {
  // large batches: the matrix-core router (decode-sized batches keep the fused path's reduction order)
  if (T >= kRouterMfmaMinT) return launch_router_mfma(x, wr, T, H, E, logits, s);
  const int tpb = std::max(1, std::min(kRouteTok, 32768 / H));  // <= 64 KB of LDS
  dim3 grid((E + 3) / 4, (T + tpb - 1) / tpb);
  const size_t lds = (size_t)tpb * H * sizeof(uint16_t);
  hipLaunchKernelGGL(k_router_logits, grid, dim3(256), lds, s, x, wr, T, H, E, tpb, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------- top-k + softmax
__global__ void __launch_bounds__(256) k_topk_softmax(const float* __restrict__ logits, int T, int E, int k,
                                                      int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ __align__(16) uint64_t scratch[4 * kWaveRankScratch];
  const int wave = threadIdx.x >> 6, t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  if (E <= 256)
    wave_topk_rank(logits + (size_t)t * E, E, k, threadIdx.x & 63, scratch + wave * kWaveRankScratch,
                   ids + (size_t)t * k, w + (size_t)t * k);
  else
    wave_topk_softmax(logits + (size_t)t * E, E, k, threadIdx.x & 63, ids + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s) {
  hipLaunchKernelGGL(k_topk_softmax, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------- router + top-k, logits on chip
// moe_route without a logits buffer: one block per batch of tpb <= 4 tokens
// computes the batch's logits against every expert (wave w takes experts w,
// w + 4, ...; the same per-expert dot product as k_router_logits, so the
// logits are the same bits), keeps them in LDS and selects each token's top
// k with one wave per token.  Every block re-reads the router weights (from
// L2), which is the price of not writing the logits out.
__global__ void __launch_bounds__(256) k_route_topk_lds(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                        int T, int H, int E, int k, int tpb,
                                                        int32_t* __restrict__ ids, float* __restrict__ w) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * tpb, nt = min(tpb, T - t0);
  uint16_t* xs = (uint16_t*)smem;                             // [tpb][H]
  float* s_log = (float*)(smem + (size_t)tpb * H * 2);        // [tpb][E]
  uint64_t* rk = (uint64_t*)(smem + (((size_t)tpb * H * 2 + (size_t)tpb * E * 4 + 15) & ~(size_t)15));
  copy_to_lds((uint4*)xs, (const uint4*)(x + (size_t)t0 * H), nt * H / 8);
  __syncthreads();
  for (int e = wave; e < E; e += 4) {
    float4 wv[kRouterC];
    router_prefetch(wr + (size_t)e * H, H, lane, wv);
    float acc[kRouteT4];
    router_dots<kRouteT4>(wr + (size_t)e * H, xs, H, nt, lane, acc, wv);
#pragma unroll
    for (int t = 0; t < kRouteT4; ++t)
      if (t < nt && lane == 63) s_log[t * E + e] = acc[t];
  }
  __syncthreads();
  if (wave >= nt) return;
  const int t = t0 + wave;
  if (E <= 256)
    wave_topk_rank(s_log + wave * E, E, k, lane, rk + wave * kWaveRankScratch, ids + (size_t)t * k, w + (size_t)t * k);
  else
    wave_topk_softmax(s_log + wave * E, E, k, lane, ids + (size_t)t * k, w + (size_t)t * k);
}

// Tokens per block of k_route_topk_lds within 64 KB of LDS (0: H too large).
int route_lds_tokens(int H, int E) {
  for (int tpb = kRouteT4; tpb >= 1; --tpb) {
    const size_t lds = (((size_t)tpb * H * 2 + (size_t)tpb * E * 4 + 15) & ~(size_t)15) + 4 * kWaveRankScratch * 8;
    if (lds <= 64 * 1024) return tpb;
  }
  return 0;
}

hipError_t launch_route_topk_lds(const uint16_t* x, const float* wr, int T, int H, int E, int k, int32_t* ids,
                                 float* w, hipStream_t s) {
  const int tpb = route_lds_tokens(H, E);
  const size_t lds = (((size_t)tpb * H * 2 + (size_t)tpb * E * 4 + 15) & ~(size_t)15) + 4 * kWaveRankScratch * 8;
  hipLaunchKernelGGL(k_route_topk_lds, dim3((T + tpb - 1) / tpb), dim3(256), lds, s, x, wr, T, H, E, k, tpb, ids, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------- permute
// Stable counting sort of pairs p = t*k + j by expert id, in chunks of
// kPermChunk pairs: per-chunk histograms, one scan, per-chunk scatter.
constexpr int kPermChunk = 256;

__global__ void __launch_bounds__(256) k_perm_hist(const int32_t* __restrict__ ids, int n, int E,
                                                   int32_t* __restrict__ hist) {
  extern __shared__ int32_t h[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * kPermChunk + threadIdx.x;
  if (p < n) atomicAdd(&h[ids[p]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)blockIdx.x * E + e] = h[e];
}

// Per-expert running counts over the chunks: each histogram entry becomes
// the count of its expert in the earlier chunks, and counts[e] the total.
// Block b takes experts [64b, 64b + 64): wave g sums the g-th quarter of the
// chunks for its 64 experts with all its loads in flight at once (a batch of
// 32), the quarter totals meet in LDS, and each wave then writes its
// quarter's running counts.  Small blocks (256 threads) fit beside the
// matrix-core kernels that may share the chip.
constexpr int kScanBatch = 32;

__global__ void __launch_bounds__(256) k_perm_scan(int nchunks, int E, int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ counts) {
  __shared__ int gtot[256];  // [quarter][expert of the block]
  const int tid = threadIdx.x, el = tid & 63, g = tid >> 6;
  const int e = blockIdx.x * 64 + el;
  const bool act = e < E;
  const int cpg = (nchunks + 3) / 4;
  const int c0 = g * cpg, c1 = act ? min(nchunks, c0 + cpg) : 0;
  int v[kScanBatch] = {};
  int sum = 0;
  for (int c = c0; c < c1; c += kScanBatch) {
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) v[u] = c + u < c1 ? hist[(size_t)(c + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) sum += v[u];
  }
  gtot[tid] = sum;
  __syncthreads();
  if (!act) return;
  int run = 0, tot = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = gtot[q * 64 + el];
    run += q < g ? t : 0;
    tot += t;
  }
  if (g == 0) counts[e] = tot;
  if (c1 - c0 <= kScanBatch) {  // the one batch is still in registers
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      if (c0 + u < c1) hist[(size_t)(c0 + u) * E + e] = run;
      run += v[u];
    }
  } else {
    for (int c = c0; c < c1; c += kScanBatch) {
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) v[u] = c + u < c1 ? hist[(size_t)(c + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) {
        if (c + u < c1) hist[(size_t)(c + u) * E + e] = run;
        run += v[u];
      }
    }
  }
}

// Every block first turns the experts' counts into their offsets (one block
// scan over E <= 1024 counts; block 0 publishes them).  Then the rank of each
// pair among its chunk's earlier pairs of the same expert: inside the wave
// from a match mask (one ballot per bit of the expert id and a valid bit),
// plus the counts of that expert in the chunk's earlier waves (each wave's
// lowest lane of a value stores it).
__global__ void __launch_bounds__(256) k_perm_scatter(const int32_t* __restrict__ ids, int n, int E,
                                                      const int32_t* __restrict__ counts,
                                                      const int32_t* __restrict__ base,
                                                      int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ sorted_pairs,
                                                      int32_t* __restrict__ pair_pos) {
  __shared__ int32_t wcnt[4 * 1024];  // [wave][expert]
  __shared__ int32_t s_off[1024];
  __shared__ int scan_tmp[17];
  const int i = threadIdx.x, wave = i >> 6, lane = i & 63;
  const int p = blockIdx.x * kPermChunk + i;
  const int v = p < n ? ids[p] : 1024;  // 1024: no pair (never an expert id)
  int c4[4], loc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = i * 4 + q;
    c4[q] = counts[min(e, E - 1)];
    c4[q] = e < E ? c4[q] : 0;
    loc += c4[q];
  }
  for (int j = i; j < 4 * E; j += 256) wcnt[j] = 0;
  int total;
  int pre = block_exclusive_scan(loc, scan_tmp, total);  // its barriers also order the zeroing
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = i * 4 + q;
    if (e < E) {
      s_off[e] = pre;
      if (blockIdx.x == 0) offsets[e] = pre;
    }
    pre += c4[q];
  }
  if (blockIdx.x == 0 && i == 0) offsets[E] = total;
  unsigned long long m = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    const bool bit = (v >> b) & 1;
    const unsigned long long bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  const int rw = __popcll(m & ((1ull << lane) - 1ull));
  if (p < n && rw == 0) wcnt[wave * E + v] = __popcll(m);
  __syncthreads();
  if (p >= n) return;
  int rank = rw;
  for (int w = 0; w < wave; ++w) rank += wcnt[w * E + v];
  const int pos = s_off[v] + base[(size_t)blockIdx.x * E + v] + rank;
  sorted_pairs[pos] = p;
  pair_pos[p] = pos;
}

// x_perm[r] = x[sorted_pairs[r] / k]; one block per row, 16 bytes per thread-step.
__global__ void __launch_bounds__(256) k_gather_rows(const uint16_t* __restrict__ x,
                                                     const int32_t* __restrict__ sorted_pairs, int k, int H,
                                                     uint16_t* __restrict__ x_perm) {
  const int r = blockIdx.x;
  const int t = sorted_pairs[r] / k;
  const uint4* src = (const uint4*)(x + (size_t)t * H);
  uint4* dst = (uint4*)(x_perm + (size_t)r * H);
  for (int c = threadIdx.x; c < H / 8; c += blockDim.x) dst[c] = src[c];
}

size_t permute_ws_bytes(int T, int k, int E) {
  const long long n = (long long)T * k;
  const long long nchunks = (n + kPermChunk - 1) / kPermChunk;
  return (size_t)(nchunks * E * sizeof(int32_t));
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, const uint16_t* x, uint16_t* x_perm, int H,
                          void* ws, hipStream_t s) {
  const int n = T * k;
  const int nchunks = (n + kPermChunk - 1) / kPermChunk;
  int32_t* hist = (int32_t*)ws;
  MOE_LAUNCH(k_perm_hist, dim3(nchunks), dim3(kPermChunk), E * sizeof(int32_t), s, ids, n, E, hist);
  MOE_LAUNCH(k_perm_scan, dim3((E + 63) / 64), dim3(256), 0, s, nchunks, E, hist, counts);
  MOE_LAUNCH(k_perm_scatter, dim3(nchunks), dim3(kPermChunk), 0, s, ids, n, E, counts, hist, offsets,
                     sorted_pairs, pair_pos);
  if (x && x_perm) MOE_LAUNCH(k_gather_rows, dim3(n), dim3(256), 0, s, x, sorted_pairs, k, H, x_perm);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine
// y[t] = residual[t] + sum_j w[t,j] * out_perm[pair_pos[t*k+j]] + out_shared[t];
// accumulation order: slots 0..k-1, then shared, then residual.
__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ out_perm,
                                                 const int32_t* __restrict__ pair_pos, const float* __restrict__ w,
                                                 const float* __restrict__ out_shared,
                                                 const uint16_t* __restrict__ residual, int k, int H,
                                                 uint16_t* __restrict__ y, float* __restrict__ y_f32) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 elements
  if (c * 4 >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float4 o = ((const float4*)(out_perm + (size_t)pair_pos[(size_t)t * k + j] * H))[c];
    acc.x = fmaf(wj, o.x, acc.x);
    acc.y = fmaf(wj, o.y, acc.y);
    acc.z = fmaf(wj, o.z, acc.z);
    acc.w = fmaf(wj, o.w, acc.w);
  }
  if (out_shared) {
    const float4 o = ((const float4*)(out_shared + (size_t)t * H))[c];
    acc.x += o.x;
    acc.y += o.y;
    acc.z += o.z;
    acc.w += o.w;
  }
  if (residual) {
    const uint2 r = ((const uint2*)(residual + (size_t)t * H))[c];
    acc.x += bf16_to_f32(r.x & 0xffffu);
    acc.y += bf16_to_f32(r.x >> 16);
    acc.z += bf16_to_f32(r.y & 0xffffu);
    acc.w += bf16_to_f32(r.y >> 16);
  }
  uint2 o;
  o.x = f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16);
  o.y = f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16);
  ((uint2*)(y + (size_t)t * H))[c] = o;
  if (y_f32) ((float4*)(y_f32 + (size_t)t * H))[c] = acc;
}

hipError_t launch_combine(const float* out_perm, const int32_t* pair_pos, const float* w, const float* out_shared,
                          const uint16_t* residual, int T, int k, int H, uint16_t* y, float* y_f32, hipStream_t s) {
  dim3 grid((H / 4 + 255) / 256, T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, s, out_perm, pair_pos, w, out_shared, residual, k, H, y, y_f32);
  return hipGetLastError();
}

// ---------------------------------------------------------------- chain normalisation
// x[t] = bf16(r[t] / sqrt(mean_h(r[t]^2) + eps)), one wave per token (four
// tokens per block).  Each bf16 square is exact in fp32; the sum order, the
// rounded reciprocal root and the per-element product rounded to bf16
// (nearest, ties to even) are those of rms_norm_row_wave, which the chained
// decode step's first launch also uses.  x may alias r.
__global__ void __launch_bounds__(256) k_rms_norm(const uint16_t* r, int T, int H, float eps, uint16_t* x) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);  // one wave per token
  if (t < T) rms_norm_row_wave(r + (size_t)t * H, H, eps, threadIdx.x & 63, x + (size_t)t * H, nullptr);
}

hipError_t launch_rms_norm(const uint16_t* r, int T, int H, float eps, uint16_t* x, hipStream_t s) {
  hipLaunchKernelGGL(k_rms_norm, dim3((T + 3) / 4), dim3(256), 0, s, r, T, H, eps, x);
  return hipGetLastError();
}

// ---------------------------------------------------------------- active experts
// active[0] = number of experts with rows, active[1 + a] = their ids (increasing).
__global__ void __launch_bounds__(1024) k_active_list(const int32_t* __restrict__ offsets, int E,
                                                      int32_t* __restrict__ active) {
  __shared__ int scan_lds[17];
  const int e = threadIdx.x;
  const int flag = (e < E) && (offsets[e + 1] > offsets[e]);
  int total;
  const int pos = block_exclusive_scan(flag, scan_lds, total);
  if (flag) active[1 + pos] = e;
  if (e == 0) active[0] = total;
}

hipError_t launch_active_list(const int32_t* offsets, int E, int32_t* active, hipStream_t s) {
  hipLaunchKernelGGL(k_active_list, dim3(1), dim3(1024), 0, s, offsets, E, active);
  return hipGetLastError();
}

}  // namespace moe
