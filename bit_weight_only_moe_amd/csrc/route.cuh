// Wave-level top-k with softmax weights, and a block-wide exclusive scan,
// for the "fused top-k router" of "[Model] Add Flint (RecursiveSI/flint)",
// section "What happened".
#pragma once

#include "common.cuh"

namespace moe {

// Router logits of one expert (one wave) against nt <= RT tokens staged in
// LDS as bf16 rows of H (token t at xs + t*H, H % 4 == 0): fp32 products
// accumulated per lane in ascending column order, then one fixed-order wave
// reduction; lane 63 holds acc[t].  Both router kernels use this, so they
// produce identical bits.
constexpr int kRouterC = 8;  // float4 router loads in flight per lane

// Load a wave's first kRouterC float4 of router row `wrow` (lane l takes
// float4 l, l+64, ...): issued before the tokens are staged.
// Chunks past the row's end load its last chunk instead (unconditional
// loads: no zero-fill of a destination register between them); router_dots
// never uses them.
MOE_DEV void router_prefetch(const float* __restrict__ wrow, int H, int lane, float4 (&wv)[kRouterC]) {
  const float4* wr = (const float4*)wrow;
  const int nc = H / 4;
#pragma unroll
  for (int q = 0; q < kRouterC; ++q) wv[q] = wr[min(lane + 64 * q, nc - 1)];
}

// acc[t] = wrow . x_t for the nt <= RT tokens staged at xs (bf16, row t at
// xs + t*H), reduced over the wave.  The tokens are the inner loop and every
// token slot is computed, so the RT accumulation chains interleave instead
// of running one after another.
template <int RT>
MOE_DEV void router_dots(const float* __restrict__ wrow, const uint16_t* __restrict__ xs, int H, int nt, int lane,
                         float (&acc)[RT], float4 (&wv)[kRouterC]) {
  const float4* wr = (const float4*)wrow;
  const uint2* xv2 = (const uint2*)xs;
  const int nc = H / 4;
#pragma unroll
  for (int t = 0; t < RT; ++t) acc[t] = 0.f;
  for (int cb = 0; cb < nc; cb += 64 * kRouterC) {
    if (cb > 0) {
#pragma unroll
      for (int q = 0; q < kRouterC; ++q) wv[q] = wr[min(cb + lane + 64 * q, nc - 1)];
    }
#pragma unroll
    for (int q = 0; q < kRouterC; ++q) {
      const int c = cb + lane + 64 * q;
      if (c < nc) {
        // slots past nt read the last staged token (no branch between the
        // LDS reads); their sums are never stored
        uint2 v[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) v[t] = xv2[min(t, nt - 1) * nc + c];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          float a = acc[t];
          a = fmaf(wv[q].x, __uint_as_float(v[t].x << 16), a);
          a = fmaf(wv[q].y, __uint_as_float(v[t].x & 0xffff0000u), a);
          a = fmaf(wv[q].z, __uint_as_float(v[t].y << 16), a);
          a = fmaf(wv[q].w, __uint_as_float(v[t].y & 0xffff0000u), a);
          acc[t] = a;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < RT; ++t)
    if (t < nt) acc[t] = group_sum_last<64>(acc[t]);
}

// Copy n16 16-byte chunks from global to LDS.  A thread's first eight
// chunks are straight-line code with all loads issued before the stores, so
// loads the caller issued just before (the router weights) stay in flight
// with these (a loop header here would make the compiler wait for them
// first); the rare remainder is a plain loop.  Named registers, not an
// array, so nothing goes through private memory.
MOE_DEV void copy_to_lds(uint4* __restrict__ dst, const uint4* __restrict__ src, int n16) {
  const int nthr = blockDim.x, i0 = threadIdx.x;
  const int i1 = i0 + nthr, i2 = i0 + 2 * nthr, i3 = i0 + 3 * nthr;
  const int i4 = i0 + 4 * nthr, i5 = i0 + 5 * nthr, i6 = i0 + 6 * nthr, i7 = i0 + 7 * nthr;
  uint4 v0, v1, v2, v3, v4, v5, v6, v7;
  if (i0 < n16) v0 = src[i0];
  if (i1 < n16) v1 = src[i1];
  if (i2 < n16) v2 = src[i2];
  if (i3 < n16) v3 = src[i3];
  if (i4 < n16) v4 = src[i4];
  if (i5 < n16) v5 = src[i5];
  if (i6 < n16) v6 = src[i6];
  if (i7 < n16) v7 = src[i7];
  if (i0 < n16) dst[i0] = v0;
  if (i1 < n16) dst[i1] = v1;
  if (i2 < n16) dst[i2] = v2;
  if (i3 < n16) dst[i3] = v3;
  if (i4 < n16) dst[i4] = v4;
  if (i5 < n16) dst[i5] = v5;
  if (i6 < n16) dst[i6] = v6;
  if (i7 < n16) dst[i7] = v7;
  for (int i = i0 + 8 * nthr; i < n16; i += nthr) dst[i] = src[i];
}

// Copy n floats from global to LDS, eight loads in flight per thread.
MOE_DEV void copy_f32_to_lds(float* __restrict__ dst, const float* __restrict__ src, int n) {
  const int nthr = blockDim.x;
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * nthr) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i0 + u * nthr < n ? src[i0 + u * nthr] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u * nthr < n) dst[i0 + u * nthr] = v[u];
  }
}

// Maximum of a float over the wave, in every lane: inclusive max-scan with
// row_shr 1, 2, 3, 4, 8 and row_bcast 15, 31 (lanes without a source keep
// their own value), then lane 63 is broadcast.
template <int CTRL, int ROW_MASK, int BANK_MASK>
MOE_DEV float dpp_keep_f32(float v) {
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, ROW_MASK, BANK_MASK, false));
}
MOE_DEV float wave_max_f32(float v) {
  v = fmaxf(v, dpp_keep_f32<0x111, 0xf, 0xf>(v));
  v = fmaxf(v, dpp_keep_f32<0x112, 0xf, 0xf>(v));
  v = fmaxf(v, dpp_keep_f32<0x113, 0xf, 0xf>(v));
  v = fmaxf(v, dpp_keep_f32<0x114, 0xf, 0xe>(v));
  v = fmaxf(v, dpp_keep_f32<0x118, 0xf, 0xc>(v));
  v = fmaxf(v, dpp_keep_f32<0x142, 0xa, 0xf>(v));
  v = fmaxf(v, dpp_keep_f32<0x143, 0xc, 0xf>(v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Top-k selection over one row of E <= 64*PER values (lane l holds entries
// i*64 + l).  Each of the k rounds takes the wave maximum of the remaining
// values, then the lowest index holding it (ballots in ascending index
// order), so ties go to the lower index; -0 and +0 compare equal.  NaN never
// wins over a number; once only NaN remain, the lowest unselected index is
// taken, so the k indices are always distinct and in [0, E) whatever the
// values.  sv/se (wave-uniform) receive values and indices in rank order.
template <int PER>
MOE_DEV void wave_topk_select(const float* __restrict__ row, int E, int k, int lane, float (&sv)[8], int (&se)[8]) {
  float v[PER];
  uint32_t inr = 0, num = 0;  // bit i: entry i*64 + lane exists / holds a number (not NaN)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * 64 + lane;
    const float x = e < E ? row[e] : 0.f;
    v[i] = x;
    inr |= e < E ? (1u << i) : 0u;
    num |= (e < E && x == x) ? (1u << i) : 0u;
  }
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sv[j] = 0.f;
    se[j] = 0;
    if (j < k) {
      const uint32_t cand = num & ~taken;
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < PER; ++i) m = fmaxf(m, (cand >> i) & 1u ? v[i] : -INFINITY);
      m = wave_max_f32(m);
      int e = -1;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint64_t b = __ballot(((cand >> i) & 1u) && v[i] == m);
        if (e < 0 && b) e = i * 64 + (int)__builtin_ctzll(b);
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {  // only NaN left: lowest unselected index
        const uint64_t b = __ballot(((inr & ~taken) >> i) & 1u);
        if (e < 0 && b) e = i * 64 + (int)__builtin_ctzll(b);
      }
      sv[j] = m;
      se[j] = e;
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
    }
  }
}

MOE_DEV void wave_topk_select_any(const float* __restrict__ row, int E, int k, int lane, float (&sv)[8],
                                  int (&se)[8]) {
  if (E <= 64) wave_topk_select<1>(row, E, k, lane, sv, se);
  else if (E <= 128) wave_topk_select<2>(row, E, k, lane, sv, se);
  else if (E <= 256) wave_topk_select<4>(row, E, k, lane, sv, se);
  else if (E <= 512) wave_topk_select<8>(row, E, k, lane, sv, se);
  else wave_topk_select<16>(row, E, k, lane, sv, se);
}

// Softmax over the k selected values (in rank order, sv[0] the largest);
// lane 0 writes ids_out[0..k) and w_out[0..k).
MOE_DEV void topk_softmax_write(const float (&sv)[8], const int (&se)[8], int k, int lane, int32_t* ids_out,
                                float* w_out) {
  if (lane == 0) {
    float ex[8], sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ex[j] = 0.f;
      if (j < k) {
        ex[j] = expf(sv[j] - sv[0]);
        sum += ex[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ids_out[j] = se[j];
        w_out[j] = ex[j] / sum;
      }
    }
  }
}

// Top-k + softmax of one row of E <= 1024 logits by one wave.
MOE_DEV void wave_topk_softmax(const float* __restrict__ row, int E, int k, int lane, int32_t* ids_out,
                               float* w_out) {
  float sv[8];
  int se[8];
  wave_topk_select_any(row, E, k, lane, sv, se);
  topk_softmax_write(sv, se, k, lane, ids_out, w_out);
}

// Top-k + softmax of one row of E <= 1024 logits (in LDS) by the 4 waves of
// a block: wave w selects the top min(k, n_w) of its quarter of the row
// (contiguous index ranges, in ascending order), the candidates are stored
// in wave order, and wave 0 selects among them.  Within a quarter, tied
// candidates are in ascending index order and the quarters are ordered, so
// candidate position order is index order and the result equals the
// one-wave selection.  cand_v / cand_e: LDS scratch of 4*k entries.  Call
// from all 4 waves; contains one __syncthreads.
MOE_DEV void block_topk_softmax(const float* __restrict__ row, int E, int k, int wave, int lane,
                                float* __restrict__ cand_v, int32_t* __restrict__ cand_e, int32_t* ids_out,
                                float* w_out) {
  const int q = (E + 3) / 4;
  int base = 0, ncand = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int nw = max(0, min(q, E - w * q));
    if (w < wave) base += min(k, nw);
    ncand += min(k, nw);
  }
  const int nw = max(0, min(q, E - wave * q)), kw = min(k, nw);
  if (kw > 0) {
    float sv[8];
    int se[8];
    wave_topk_select_any(row + wave * q, nw, kw, lane, sv, se);
    if (lane < kw) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j == lane) {
          cand_v[base + j] = sv[j];
          cand_e[base + j] = wave * q + se[j];
        }
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    float sv[8];
    int se[8];
    wave_topk_select<1>(cand_v, ncand, k, lane, sv, se);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) se[j] = cand_e[se[j]];
    topk_softmax_write(sv, se, k, lane, ids_out, w_out);
  }
}

// ---- top-k by rank counting (E <= 256) -------------------------------------
// Latency-bound variant for the routing tails, where one block routes a few
// tokens while the rest of the chip waits.  Every entry gets a unique 64-bit
// key whose unsigned order is the selection order above: the order-
// preserving bits of the value (NaN mapped below every number, -0 folded
// onto +0) over the complemented index, so equal values rank by lower index.
// An entry's rank is the number of larger keys, counted with fully unrolled
// compares against keys read 16 bytes at a time (no serial maximum rounds,
// no loop branches).  Stage 1 ranks within 64-entry chunks and keeps each
// chunk's top k; stage 2 ranks those <= 32 candidates.  The selected values
// and the softmax are those of the round-based selection, bit for bit
// (a NaN-only pick has the value -inf there, and here).
constexpr int kWaveRankScratch = 104;  // u64 LDS words per wave: 64 heads, 32 candidates, 8 winners
// u64 LDS words of a block's rank scratch: one token by the block (256 keys,
// 32 candidates, 8 winners) or one token per wave (4 x kWaveRankScratch)
constexpr int kRankScratch = 4 * kWaveRankScratch;

MOE_DEV uint64_t topk_key(float v, int idx) {
  const uint32_t hi = (v == v) ? f32_order_key(v) : 0u;
  return ((uint64_t)hi << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)idx);
}
MOE_DEV float topk_key_value(uint64_t key) {
  const uint32_t hi = (uint32_t)(key >> 32);
  return hi == 0u ? -INFINITY : f32_from_order_key(hi);
}
MOE_DEV int topk_key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// Number of the N keys at K (LDS, 16-byte aligned) larger than `mine`.
template <int N>
MOE_DEV int key_rank(const uint64_t* K, uint64_t mine) {
  const uint4* K4 = (const uint4*)K;
  int r0 = 0, r1 = 0;
#pragma unroll
  for (int b = 0; b < N / 2; b += 8) {
    uint4 q0 = K4[b], q1 = K4[b + 1], q2 = K4[b + 2], q3 = K4[b + 3];
    uint4 q4 = K4[b + 4], q5 = K4[b + 5], q6 = K4[b + 6], q7 = K4[b + 7];
#define MOE_RANK_PAIR(q)                                                          \
  r0 += (((uint64_t)q.y << 32) | q.x) > mine;                                    \
  r1 += (((uint64_t)q.w << 32) | q.z) > mine;
    MOE_RANK_PAIR(q0) MOE_RANK_PAIR(q1) MOE_RANK_PAIR(q2) MOE_RANK_PAIR(q3)
    MOE_RANK_PAIR(q4) MOE_RANK_PAIR(q5) MOE_RANK_PAIR(q6) MOE_RANK_PAIR(q7)
#undef MOE_RANK_PAIR
  }
  return r0 + r1;
}

// Stage 2 + softmax for one token, by one wave: C[0..32) holds the stage-1
// candidates (unused slots 0); F: 8 LDS words.  Lanes j < k write ids_out[j]
// and w_out[j] = exp(v_j - v_0) / sum_i exp(v_i - v_0), summed in rank order.
MOE_DEV void rank_finish(const uint64_t* C, uint64_t* F, int k, int lane, int32_t* ids_out, float* w_out) {
  const uint64_t c = lane < 32 ? C[lane] : 0ull;
  const int r = key_rank<32>(C, c);
  if (c != 0ull && r < k) F[r] = c;
  wave_lds_sync();
  const uint64_t f = F[lane < k ? lane : 0];
  const float v0 = topk_key_value(F[0]);
  const float ex = expf(topk_key_value(f) - v0);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), j));
  if (lane < k) {
    ids_out[lane] = topk_key_index(f);
    w_out[lane] = ex / sum;
  }
}

// One token (E <= 256) by the 4 waves of a block; thread i owns entry i.
// S: kRankScratch LDS words.  Call from all 256 threads; two __syncthreads.
MOE_DEV void block_topk_rank(const float* __restrict__ row, int E, int k, uint64_t* S, int32_t* ids_out,
                             float* w_out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  uint64_t* K = S;
  uint64_t* C = S + 256;
  uint64_t* F = S + 288;
  const uint64_t mine = tid < E ? topk_key(row[tid], tid) : 0ull;
  K[tid] = mine;
  if (tid < 32) C[tid] = 0ull;
  __syncthreads();
  const int r = key_rank<64>(K + wave * 64, mine);
  if (tid < E && r < k) C[wave * k + r] = mine;
  __syncthreads();
  if (wave == 0) rank_finish(C, F, k, lane, ids_out, w_out);
}

// One token row of E <= 256 logits by one wave (lane l owns entries
// i*64 + l).  Each lane sorts its 4 keys; a key among the k largest has at
// most k - 1 larger keys, so its lane's largest key ranks below k among the
// 64 lanes' largest keys.  The 4 keys of each such lane (at most 4k <= 32)
// are the candidates; rank_finish ranks them.  W: kWaveRankScratch LDS words
// of this wave (16-byte aligned).
MOE_DEV void wave_topk_rank(const float* __restrict__ row, int E, int k, int lane, uint64_t* W, int32_t* ids_out,
                            float* w_out) {
  uint64_t q0, q1, q2, q3;
  {
    const int e0 = lane, e1 = 64 + lane, e2 = 128 + lane, e3 = 192 + lane;
    q0 = e0 < E ? topk_key(row[e0], e0) : 0ull;
    q1 = e1 < E ? topk_key(row[e1], e1) : 0ull;
    q2 = e2 < E ? topk_key(row[e2], e2) : 0ull;
    q3 = e3 < E ? topk_key(row[e3], e3) : 0ull;
  }
  auto cx = [](uint64_t& a, uint64_t& b) {  // a >= b afterwards
    const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
    a = hi;
    b = lo;
  };
  cx(q0, q1);
  cx(q2, q3);
  cx(q0, q2);
  cx(q1, q3);
  cx(q1, q2);
  uint64_t* heads = W;
  uint64_t* C = W + 64;
  uint64_t* F = W + 96;
  heads[lane] = q0;
  if (lane < 32) C[lane] = 0ull;
  wave_lds_sync();
  const int r = key_rank<64>(heads, q0);
  if (q0 != 0ull && r < k) {
    C[r * 4 + 0] = q0;
    C[r * 4 + 1] = q1;
    C[r * 4 + 2] = q2;
    C[r * 4 + 3] = q3;
  }
  wave_lds_sync();
  rank_finish(C, F, k, lane, ids_out, w_out);
}

// Exclusive prefix sum over a block of up to 1024 threads (all threads must
// call).  `lds` holds at least 17 ints.  Returns this thread's prefix and
// the block total in `total`.
template <int CTRL, int ROW_MASK, int BANK_MASK>
MOE_DEV int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, BANK_MASK, false);
}

// Inclusive prefix sum over the 64 lanes of a wave (row_shr 1, 2, 4, 8 within
// rows, then row_bcast 15 and 31 across rows).
MOE_DEV int wave_inclusive_scan(int v) {
  v += dpp_i32<0x111, 0xf, 0xf>(v);
  v += dpp_i32<0x112, 0xf, 0xf>(v);
  v += dpp_i32<0x114, 0xf, 0xf>(v);
  v += dpp_i32<0x118, 0xf, 0xf>(v);
  v += dpp_i32<0x142, 0xa, 0xf>(v);
  v += dpp_i32<0x143, 0xc, 0xf>(v);
  return v;
}

MOE_DEV int block_exclusive_scan(int v, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  // every thread sums the wave totals itself (at most 16): no serial pass
  int before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    const int t = lds[w];
    before += w < wave ? t : 0;
    all += t;
  }
  total = all;
  __syncthreads();  // the caller may reuse lds
  return before + inc - v;
}

}  // namespace moe
