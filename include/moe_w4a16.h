/*
 * moe_w4a16.h -- C ABI of a 4-bit weight-only (W4A16) mixture-of-experts
 * layer for AMD Instinct MI355X (gfx950).
 *
 * The layer (sources: "Recursive Flint: 40B Local Coding Model, Benchmarks",
 * architecture table under "What is Recursive Flint?"; "Recursive Flint: 125
 * tok/s on an M4 Pro, measured where it matters least", table under "What
 * actually shipped"; "[Model] Add Flint (RecursiveSI/flint)", section "What
 * happened"): a router scores each token against E routed experts and keeps
 * the top k (Flint: 256 and 6); each chosen expert, plus one always-on
 * shared expert, is a SwiGLU feed-forward network whose weights are stored
 * in 4 bits and dequantised on the fly against 16-bit activations; the
 * outputs are summed with the router weights.
 *
 * Numerics contract (all entry points):
 *   logits   fp32 accumulation of bf16 x times fp32 router weights;
 *   top-k    ranked by (larger logit, then lower expert index), ids written
 *            in rank order; weights = softmax over the k selected logits;
 *   experts  g = W_gate x, u = W_up x accumulated in fp32 from exactly
 *            dequantised weights; h = silu(g) * u rounded to bf16 (nearest,
 *            ties to even); o = W_down h accumulated in fp32;
 *   combine  y = residual + sum_j w_j o_j + o_shared in fp32, in that fixed
 *            order (no atomics: reruns are bit-identical), rounded once to
 *            bf16 (nearest, ties to even).
 *
 * Conventions:
 *   - Tensor arguments are DEVICE pointers owned by the caller, except the
 *     weight descriptor structs themselves, which live in host memory (their
 *     members point to device memory).  The library allocates and frees
 *     nothing and keeps no device state between calls.
 *   - bf16 and fp16 values are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work; they never synchronise and never read device
 *     memory on the host, so they may be captured in a HIP graph.
 *   - Every argument is validated on the host before anything is enqueued;
 *     a failing call enqueues nothing.  T == 0 is a no-op returning MOE_OK.
 *   - Device-side preconditions (documented, not checked): expert ids in
 *     [0, E); finite activations, logits and weights; offsets consistent with
 *     total_rows; buffers at least the sizes stated.
 *   - Pointers to packed weights, activations and outputs must be 16-byte
 *     aligned.
 *
 * Canonical weight layout (a matrix stack of E experts, row-major [out, in],
 * quantisation groups along `in`):
 *   codes   uint8 [E, rows, cols/2]; element 2i of a row in the LOW nibble of
 *           byte i, element 2i+1 in the HIGH nibble.
 *   NVFP4   (fmt 1) code = e2m1 (sign, 2 exponent bits bias 1, 1 mantissa
 *           bit); scales = e4m3fn uint8 [E, rows, cols/16] (one per 16
 *           consecutive elements, NaN codes invalid); tensor_scale fp32 [E];
 *           w = tensor_scale[e] * e4m3(scale) * e2m1(code).
 *   INT4    (fmt 2) group-64 affine with zero point: scales = fp16
 *           [E, rows, cols/64], zeros = uint8 [E, rows, cols/64] in 0..15;
 *           w = scale * (code - zero).
 *   Gate and up are [I, H], down is [H, I].  H and I must be multiples of 64.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, misalignment, bad size, small workspace */
  MOE_ERR_UNSUPPORTED = -2, /* E > 1024, a matrix with cols > 3840 or rows > 65536,
                               unknown format or mode */
  MOE_ERR_HIP = -3          /* a HIP launch failed; see moe_last_error() */
};

enum { MOE_FMT_NVFP4 = 1, MOE_FMT_INT4_G64 = 2 };
enum { MOE_MODE_AUTO = 0, MOE_MODE_GEMV = 1, MOE_MODE_MFMA = 2 };

/* One packed 4-bit matrix stack (host struct, device pointers). */
typedef struct moe_w4_matrix {
  int fmt;                   /* MOE_FMT_NVFP4 or MOE_FMT_INT4_G64 */
  int num_experts;           /* E of this stack */
  int rows, cols;            /* out, in (cols = reduction axis); cols <= 3840 (the GEMV
                                kernels stage 8 tokens' rows of cols in 64 KB of LDS) */
  const uint8_t* codes;      /* [E, rows, cols/2] */
  const void* scales;        /* NVFP4: uint8 e4m3 [E, rows, cols/16]; INT4: fp16 [E, rows, cols/64] */
  const uint8_t* zeros;      /* INT4: uint8 [E, rows, cols/64]; NVFP4: NULL */
  const float* tensor_scale; /* NVFP4: fp32 [E]; INT4: NULL */
} moe_w4_matrix;

/* A SwiGLU expert stack: gate [I, H], up [I, H], down [H, I]; same fmt. */
typedef struct moe_ffn_weights {
  moe_w4_matrix gate, up, down;
} moe_ffn_weights;

/* One MoE layer. */
typedef struct moe_layer_weights {
  int H, I, E, k;                 /* hidden, routed-expert inter, experts, top-k */
  const float* w_router;          /* fp32 [E, H] */
  moe_ffn_weights experts;        /* E experts of inter I */
  const moe_ffn_weights* shared;  /* one always-on expert (its own inter size, gate.rows), or NULL */
} moe_layer_weights;

/* ABI version (MOE_ABI_VERSION) and the calling thread's last error text. */
int moe_abi_version(void);
const char* moe_last_error(void);

/* Dequantise expert `expert` of matrix `m` to fp32 out[rows, cols].
 * Exact: NVFP4 gives the single fp32 rounding of tensor_scale*e4m3*e2m1,
 * INT4 gives scale*(code-zero) exactly.  (Test export of the format
 * definition above.) */
int moe_dequant_w4(const moe_w4_matrix* m, int expert, float* out, void* stream);

/* Router: logits[t, e] = sum_h x[t, h] * w_router[e, h] (fp32 accumulation)
 * for x bf16 [T, H], then top-k and softmax weights as in moe_topk_softmax.
 * logits_out fp32 [T, E] is required and receives the logits.  topk_ids
 * int32 [T, k] in rank order,
 * topk_w fp32 [T, k].  Source: the fused top-k router of "[Model] Add Flint
 * (RecursiveSI/flint)", section "What happened". */
int moe_route(const uint16_t* x, const float* w_router, int T, int H, int E, int k,
              float* logits_out, int32_t* topk_ids, float* topk_w, void* stream);

/* Top-k and softmax weights from given fp32 logits [T, E]: ids ranked by
 * (larger logit, lower index); w = exp(l - l_max) / sum over the selection.
 * 1 <= k <= min(E, 8). */
int moe_topk_softmax(const float* logits, int T, int E, int k,
                     int32_t* topk_ids, float* topk_w, void* stream);

/* Group the T*k (token, slot) pairs p = t*k + j by expert (stable counting
 * sort): counts int32 [E], offsets int32 [E+1] (exclusive prefix sum),
 * sorted_pairs int32 [T*k] (the pair at each sorted position) and pair_pos
 * int32 [T*k] (its inverse).  If x (bf16 [T, H]) and x_perm are both given,
 * x_perm bf16 [T*k, H] receives row sorted_pairs[r]/k of x at row r.
 * Workspace: moe_permute_workspace_size(T, k, E) bytes of device memory.
 * Source: the expert-indexed grouping implied by "[Model] Add Flint
 * (RecursiveSI/flint)", section "What happened". */
size_t moe_permute_workspace_size(int T, int k, int E);
int moe_permute(const int32_t* topk_ids, int T, int k, int E,
                int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                const uint16_t* x, uint16_t* x_perm, int H,
                void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU experts: for every sorted row r in [offsets[e], offsets[e+1])
 * out[r] = W_down_e (bf16(silu(W_gate_e x_t) * (W_up_e x_t))), fp32 [total_rows, H],
 * unweighted, where x_t is row sorted_pairs[r]/k of x (or row r when
 * sorted_pairs is NULL).  offsets: device int32 [E+1] with offsets[E] ==
 * total_rows.  mode: MOE_MODE_GEMV streams weights through VALU dot
 * products (few tokens per expert), MOE_MODE_MFMA runs a bf16 matrix-core
 * grouped GEMM (many tokens per expert), MOE_MODE_AUTO picks per call from
 * total_rows / E.  The shared expert is this call with E = 1, offsets
 * {0, T} and sorted_pairs NULL.  Workspace: moe_grouped_ffn_workspace_size.
 * Source: "expert-indexed GEMVs" and the "grouped-GEMM path" of "[Model]
 * Add Flint (RecursiveSI/flint)", section "What happened". */
size_t moe_grouped_ffn_workspace_size(int E, int H, int I, int total_rows, int mode);
int moe_grouped_w4a16_ffn(const moe_ffn_weights* w, int E, int H, int I,
                          const uint16_t* x, const int32_t* sorted_pairs, int k,
                          const int32_t* offsets, int total_rows, float* out,
                          int mode, void* ws, size_t ws_bytes, void* stream);

/* Combine: y[t] = residual[t] + sum_{j<k} topk_w[t, j] * out_perm[pair_pos[t*k+j]]
 * + out_shared[t], fp32, fixed order, rounded once to bf16 y [T, H]; y_f32
 * fp32 [T, H] (unrounded) may be NULL; out_shared and residual may be NULL.
 * Source: the shared-expert sum of "Recursive Flint: 125 tok/s on an M4 Pro,
 * measured where it matters least", table under "What actually shipped". */
int moe_combine(const float* out_perm, const int32_t* pair_pos, const float* topk_w,
                const float* out_shared, const uint16_t* residual,
                int T, int k, int H, uint16_t* y, float* y_f32, void* stream);

/* Whole layer for decode-sized batches (1 <= T <= 64 takes the fused path;
 * larger T is composed from the calls above): router, top-k, routed and
 * shared SwiGLU experts on 4-bit weights, combine.  Same numerics as
 * composing moe_route, moe_permute, moe_grouped_w4a16_ffn and moe_combine;
 * for 2 <= T <= 64 the result equals that composition (GEMV mode) bit for
 * bit, while a lone token splits its dot products over more lanes (same
 * contract, possibly different last bits).
 * residual bf16 [T, H] may be NULL; y bf16 [T, H]; ids_out int32 [T, k] and
 * w_out fp32 [T, k] may be NULL.  Workspace: moe_layer_decode_workspace_size
 * bytes, 256-byte aligned, ZERO-FILLED before its first use: its first
 * 64 * (17 + ceil(H / 32)) bytes hold int32 ticket counters that the decode
 * kernels use to hand work to the last block of a group; every call leaves
 * them reset to zero.  Calls sharing a
 * workspace must not run concurrently.  The shared expert must have the
 * same format and hidden size as the routed experts. */
size_t moe_layer_decode_workspace_size(const moe_layer_weights* L, int T);
int moe_layer_decode(const moe_layer_weights* L, const uint16_t* x, const uint16_t* residual,
                     int T, uint16_t* y, int32_t* ids_out, float* w_out,
                     void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
