// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moe_w4a16.h"

namespace moe {

// Dense GEMV out[T, rows] = W_expert x (tokens in batches of dense_max_tokens()).
int dense_max_tokens();
// The same product on the matrix cores (NVFP4, K % 256 == 0, K <= 2048), any T.
hipError_t launch_dense_mfma(const moe_w4_matrix* m, int expert, const uint16_t* x, int T, float* out,
                             hipStream_t s);
hipError_t launch_dense_gemv(const moe_w4_matrix* m, int expert, const uint16_t* x, int T, float* out,
                             hipStream_t s);
hipError_t launch_dequant_expert(int fmt, int rows, int cols, const uint8_t* codes, const void* scales,
                                 const uint8_t* zeros, const float* ts_dev, float* out, hipStream_t s);
// Router logits on the matrix cores (fp32 weights split exactly into three
// bf16 parts); used for large batches.
hipError_t launch_router_mfma(const uint16_t* x, const float* wr, int T, int H, int E, float* logits, hipStream_t s);
hipError_t launch_router_logits(const uint16_t* x, const float* wr, int T, int H, int E, float* logits,
                                hipStream_t s);
// Router and top-k in one kernel, the logits kept in LDS (moe_route without
// a logits buffer); route_lds_tokens() == 0 means H is too large for it.
int route_lds_tokens(int H, int E);
hipError_t launch_route_topk_lds(const uint16_t* x, const float* wr, int T, int H, int E, int k, int32_t* ids,
                                 float* w, hipStream_t s);
hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* ids, float* w, hipStream_t s);
size_t permute_ws_bytes(int T, int k, int E);
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, const uint16_t* x, uint16_t* x_perm, int H,
                          void* ws, hipStream_t s);
hipError_t launch_combine(const float* out_perm, const int32_t* pair_pos, const float* w, const float* out_shared,
                          const uint16_t* residual, int T, int k, int H, uint16_t* y, float* y_f32, hipStream_t s);
hipError_t launch_rms_norm(const uint16_t* r, int T, int H, float eps, uint16_t* x, hipStream_t s);
hipError_t launch_active_list(const int32_t* offsets, int E, int32_t* active, hipStream_t s);
hipError_t launch_grouped_gemv(const moe_ffn_weights* w, const int32_t* active, const int32_t* offsets,
                               const int32_t* sorted_pairs, int k, int max_active, const uint16_t* x, int H, int I,
                               uint16_t* h, float* out, int rows, hipStream_t s);

size_t layer_decode_lds(int T, int H, int I, int Is, int E, int k);
int layer_decode_sync_words(int H);
size_t layer_decode_rec_ints(int T, int E, int k);

// Workspace buffers of the three-launch decode layer.
// Launch a kernel and return from the enclosing function with its launch
// status if that failed (taken at once, before a later launch or status
// query can replace or clear it).
#define MOE_LAUNCH(...)                       \
  do {                                        \
    hipLaunchKernelGGL(__VA_ARGS__);          \
    const hipError_t moe_e_ = hipGetLastError(); \
    if (moe_e_ != hipSuccess) return moe_e_;  \
  } while (0)

struct LayerDecodeBufs {
  int* sync;           // ticket counters, zero before the first call, left zero
  float* logits;       // [T, E]
  int32_t* ids;        // [T*k]
  float* w;            // [T*k]
  int32_t* pair_pos;   // [T*k]
  int32_t* n_active;   // [1]
  int32_t* rec;        // [layer_decode_rec_ints]
  uint16_t* h_routed;  // [T*k, I]
  uint16_t* h_shared;  // [T, Is]
  float* o_routed;     // [T*k, H]
  float* o_shared;     // [T, H]
};
// norm_r != NULL (chained step): x is a [T, H] buffer that the first launch
// fills with rms_norm(norm_r) (eps) before the later launches read it.
hipError_t launch_layer_decode(const moe_layer_weights* L, const uint16_t* x, const uint16_t* residual, int T,
                               uint16_t* y, const LayerDecodeBufs& b, int32_t* ids_out, float* w_out, hipStream_t s,
                               const uint16_t* norm_r = nullptr, float eps = 0.f);

size_t mfma_ws_bytes(int E, int H, int I, int total_rows);
bool mfma_shape_ok(int H, int I);
hipError_t launch_grouped_mfma(const moe_ffn_weights* w, int E, const int32_t* offsets, const int32_t* sorted_pairs,
                               int k, const uint16_t* x, int H, int I, int total_rows, float* out, void* ws,
                               hipStream_t s);

}  // namespace moe
