// Wave-level top-k with softmax weights, and a block-wide exclusive scan,
// for the "fused top-k router" of "[Model] Add Flint (RecursiveSI/flint)",
// section "What happened".
#pragma once

#include "common.cuh"

namespace moe {

// One wave per token.  Each lane holds E/64 logits; k rounds of a wave-wide
// (larger value, then lower index) argmax; softmax over the selection.
MOE_DEV void wave_topk_softmax(const float* __restrict__ row, int E, int k, int lane, int32_t* ids_out,
                               float* w_out) {
  constexpr int kMaxPer = 16;  // E <= 1024
  float v[kMaxPer];
  uint32_t taken = 0;
  const int per = (E + 63) / 64;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int e = i * 64 + lane;
    v[i] = (i < per && e < E) ? row[e] : 0.f;
    if (!(i < per && e < E)) taken |= 1u << i;
  }
  float sel_v[8];
  int sel_e[8];
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int e = i * 64 + lane;
      if (!(taken & (1u << i)) && (be == 0x7fffffff || v[i] > bv)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const bool take = (oe != 0x7fffffff) && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
    sel_v[j] = bv;
    sel_e[j] = be;
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
  }
  if (lane == 0) {
    const float m = sel_v[0];
    float ex[8], sum = 0.f;
    for (int j = 0; j < k; ++j) {
      ex[j] = expf(sel_v[j] - m);
      sum += ex[j];
    }
    for (int j = 0; j < k; ++j) {
      ids_out[j] = sel_e[j];
      w_out[j] = ex[j] / sum;
    }
  }
}


// Exclusive prefix sum over a block of up to 1024 threads (all threads must
// call).  `lds` holds at least 17 ints.  Returns this thread's prefix and
// the block total in `total`.
MOE_DEV int block_exclusive_scan(int v, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = (blockDim.x + 63) >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
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
