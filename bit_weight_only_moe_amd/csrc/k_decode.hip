// Routing step of the fused decode layer: top-k, softmax weights and the
// expert grouping of a decode-sized batch (T <= 64 tokens) in one block,
// so the expert kernels can read each touched expert once ("fused top-k
// router" and "expert-indexed GEMVs" of "[Model] Add Flint
// (RecursiveSI/flint)", section "What happened").
#include "launch.h"
#include "route.cuh"

namespace moe {

constexpr int kDecodeMaxT = 64;

__global__ void __launch_bounds__(1024) k_decode_route(const float* __restrict__ logits, int T, int E, int k,
                                                       int32_t* __restrict__ ids, float* __restrict__ w,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ sorted_pairs,
                                                       int32_t* __restrict__ pair_pos, int32_t* __restrict__ active,
                                                       int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  __shared__ int32_t sid[kDecodeMaxT * 8];
  __shared__ float sw[kDecodeMaxT * 8];
  __shared__ int32_t cnt[1024];
  __shared__ int32_t off[1025];
  __shared__ int scan_lds[17];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int t = wave; t < T; t += 16) wave_topk_softmax(logits + (size_t)t * E, E, k, lane, sid + t * k, sw + t * k);
  cnt[tid] = 0;
  __syncthreads();
  const int n = T * k;
  for (int p = tid; p < n; p += 1024) atomicAdd(&cnt[sid[p]], 1);
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  int total;
  const int pref = block_exclusive_scan(c, scan_lds, total);
  if (tid < E) off[tid] = pref;
  if (tid == 0) off[E] = total;
  int nact;
  const int apos = block_exclusive_scan(c > 0 ? 1 : 0, scan_lds, nact);
  if (c > 0) active[1 + apos] = tid;
  if (tid == 0) active[0] = nact;
  __syncthreads();
  for (int p = tid; p < n; p += 1024) {
    const int e = sid[p];
    int rank = 0;
    for (int q = 0; q < p; ++q) rank += (sid[q] == e);
    const int pos = off[e] + rank;
    sorted_pairs[pos] = p;
    pair_pos[p] = pos;
    ids[p] = e;
    w[p] = sw[p];
    if (ids_out) ids_out[p] = e;
    if (w_out) w_out[p] = sw[p];
  }
  for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];
}

hipError_t launch_decode_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                               int32_t* sorted_pairs, int32_t* pair_pos, int32_t* active, int32_t* ids_out,
                               float* w_out, hipStream_t s) {
  hipLaunchKernelGGL(k_decode_route, dim3(1), dim3(1024), 0, s, logits, T, E, k, ids, w, offsets, sorted_pairs,
                     pair_pos, active, ids_out, w_out);
  return hipGetLastError();
}

}  // namespace moe
