// Wave-level top-k with softmax weights, and a block-wide exclusive scan,
// for the "fused top-k router" of "[Model] Add Flint (RecursiveSI/flint)",
// section "What happened".
#pragma once

#include "common.cuh"

namespace moe {

// Top-k of one row of E <= 64*PER logits and softmax over the selection.
// Every logit becomes a 64-bit key (order-preserving fp32 bits, then
// 1024 - index) so one unsigned maximum ranks by (larger logit, lower
// index); k rounds of a DPP wave maximum pick the winners in rank order.
// Lane 0 writes ids_out[0..k) and w_out[0..k).
template <int PER, bool COH = false>
MOE_DEV void wave_topk_softmax_t(const float* __restrict__ row, int E, int k, int lane, int32_t* ids_out,
                                 float* w_out) {
  uint64_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = i * 64 + lane;
    const float v = e < E ? (COH ? ld_dev(row + e) : row[e]) : 0.f;
    key[i] = e < E ? (((uint64_t)f32_order_key(v) << 32) | (uint32_t)(1024 - e)) : 0ull;
  }
  float sv[8];
  int se[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    sv[j] = 0.f;
    se[j] = 0;
    if (j < k) {
      uint64_t m = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) m = max_u64(m, key[i]);
      m = wave_max_u64(m);
      const int e = 1024 - (int)(uint32_t)m;
      sv[j] = f32_from_order_key((uint32_t)(m >> 32));
      se[j] = e;
      if ((e & 63) == lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (i == (e >> 6)) key[i] = 0ull;
      }
    }
  }
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

// COH: read the logits with device-coherent loads (they were written by
// other blocks of the same launch).
template <bool COH = false>
MOE_DEV void wave_topk_softmax(const float* __restrict__ row, int E, int k, int lane, int32_t* ids_out,
                               float* w_out) {
  if (E <= 64) wave_topk_softmax_t<1, COH>(row, E, k, lane, ids_out, w_out);
  else if (E <= 128) wave_topk_softmax_t<2, COH>(row, E, k, lane, ids_out, w_out);
  else if (E <= 256) wave_topk_softmax_t<4, COH>(row, E, k, lane, ids_out, w_out);
  else if (E <= 512) wave_topk_softmax_t<8, COH>(row, E, k, lane, ids_out, w_out);
  else wave_topk_softmax_t<16, COH>(row, E, k, lane, ids_out, w_out);
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
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nwaves; ++w) {
      const int t = lds[w];
      lds[w] = run;
      run += t;
    }
    lds[16] = run;
  }
  __syncthreads();
  const int res = lds[wave] + inc - v;
  total = lds[16];
  __syncthreads();
  return res;
}

}  // namespace moe
