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
 *     nothing and keeps no device state between calls, except the static
 *     scratch array of moe_layer_decode_noalloc (see there).
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
 *   INT4_SB (fmt 3) group-64 affine with scale and bias (the other reading
 *           of "group-64 affine INT4" in the table under "What actually
 *           shipped" of "Recursive Flint: 125 tok/s on an M4 Pro, measured
 *           where it matters least"; MLX stores its affine groups so):
 *           scales = fp16 [E, rows, cols/64], biases = fp16 [E, rows,
 *           cols/64]; w = scale * code + bias (codes 0..15).  The zero-point
 *           form is its special case bias = -scale * zero.  The matrix-core
 *           grouped GEMM takes NVFP4 and INT4 only: scale+bias weights run the
 *           GEMV kernels at every batch size.
 *   BF16    (fmt 4) unquantised 16-bit weights, the BF16 checkpoint that
 *           "[Model] Add Flint (RecursiveSI/flint)", section "What happened",
 *           serves beside the NVFP4 one: codes = bf16 [E, rows, cols] (2 bytes
 *           per weight), no scales.  The layer and grouped-FFN calls take it
 *           (GEMV kernels at every batch size); the dense GEMV and the
 *           matrix-core mode do not.
 *   Gate and up are [I, H], down is [H, I].  H and I must be multiples of 64.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, misalignment, bad size, small workspace */
  MOE_ERR_UNSUPPORTED = -2, /* E > 1024, a matrix with cols > 3840 or rows > 65536,
                               unknown format or mode */
  MOE_ERR_HIP = -3          /* a HIP launch failed; see moe_last_error() */
};

enum { MOE_FMT_NVFP4 = 1, MOE_FMT_INT4_G64 = 2, MOE_FMT_INT4_SB = 3, MOE_FMT_BF16 = 4 };
enum { MOE_MODE_AUTO = 0, MOE_MODE_GEMV = 1, MOE_MODE_MFMA = 2 };

/* One weight matrix stack: packed 4-bit, or BF16 (host struct, device pointers). */
typedef struct moe_w4_matrix {
  int fmt;                   /* MOE_FMT_NVFP4, MOE_FMT_INT4_G64, MOE_FMT_INT4_SB or MOE_FMT_BF16 */
  int num_experts;           /* E of this stack */
  int rows, cols;            /* out, in (cols = reduction axis); cols <= 3840 (the GEMV
                                kernels stage 8 tokens' rows of cols in 64 KB of LDS) */
  const uint8_t* codes;      /* [E, rows, cols/2]; BF16: bf16 [E, rows, cols] */
  const void* scales;        /* NVFP4: uint8 e4m3 [E, rows, cols/16]; INT4, INT4_SB: fp16 [E, rows, cols/64] */
  const uint8_t* zeros;      /* INT4: uint8 [E, rows, cols/64]; else NULL */
  const float* tensor_scale; /* NVFP4: fp32 [E]; else NULL */
  const void* biases;        /* INT4_SB: fp16 [E, rows, cols/64]; else NULL */
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

/* Dequantise expert `expert` of matrix `m` to fp32 out[rows, cols] (device,
 * caller-owned, 16-byte aligned).  Exact: NVFP4 gives the single fp32
 * rounding of tensor_scale*e4m3*e2m1, INT4 gives scale*(code-zero) exactly.
 * The formats are the NVFP4 checkpoint served weight-only as W4A16 of
 * "[Model] Add Flint (RecursiveSI/flint)", section "What happened", and the
 * group-64 affine INT4 of "Recursive Flint: 125 tok/s on an M4 Pro,
 * measured where it matters least", table under "What actually shipped".
 * Errors: MOE_ERR_INVALID_ARG for a null or misaligned pointer or an expert
 * outside [0, num_experts); MOE_ERR_UNSUPPORTED for an unknown format.
 * (A test export: it states the format definition above as code.) */
int moe_dequant_w4(const moe_w4_matrix* m, int expert, float* out, void* stream);

/* Dense 4-bit GEMV: out[t, n] = sum_c W[n, c] * x[t, c] for matrix `expert`
 * of `m` (rows n < m->rows, up to 2^24; cols as for every matrix, a multiple
 * of 64 up to 3840), x bf16 [T, cols], out fp32 [T, rows] (device,
 * caller-owned, 16-byte aligned); weights exactly dequantised, fp32
 * accumulation, the NVFP4 tensor scale applied last.  Tokens are taken in
 * batches of 8, each batch streaming the matrix once; from 8 tokens NVFP4
 * with cols a multiple of 256 up to 2048 runs on the matrix cores instead
 * (batches of 64 tokens; the same bound, another summation order).  Source: the 4-bit
 * output head of "Recursive Flint: 40B Local Coding Model, Benchmarks"
 * (section "How Recursive built Flint") over its 150,144-token vocabulary
 * ("What is Recursive Flint?"); the same call serves any dense projection.
 * Errors: MOE_ERR_INVALID_ARG for null or misaligned pointers, a bad expert
 * or T < 0; MOE_ERR_UNSUPPORTED for more than 2^24 rows or 3840 columns. */
int moe_dense_w4a16_gemv(const moe_w4_matrix* m, int expert, const uint16_t* x, int T, float* out,
                         void* stream);

/* Router: logits[t, e] = sum_h x[t, h] * w_router[e, h] (fp32 accumulation)
 * for x bf16 [T, H] and w_router fp32 [E, H] (both 16-byte aligned), then
 * top-k and softmax weights as in moe_topk_softmax: topk_ids int32 [T, k] in
 * rank order, topk_w fp32 [T, k].  logits_out fp32 [T, E] receives the
 * logits, or is NULL: the logits then stay on chip (one kernel per batch of
 * up to 4 tokens, which re-reads the router weights from cache), which
 * needs 2*H + 4*E + 3328 <= 65536 bytes of LDS for a one-token batch (else
 * MOE_ERR_UNSUPPORTED).  Both forms select the same experts from the same
 * fp32 logits below 256 tokens; from 256 tokens with logits_out the logits
 * come from the matrix cores (same contract, possibly other last bits).
 * Source: the fused top-k router of "[Model] Add Flint (RecursiveSI/flint)",
 * section "What happened"; 6 of 256 routed experts per token in the
 * architecture table of "Recursive Flint: 40B Local Coding Model,
 * Benchmarks", section "What is Recursive Flint?". */
int moe_route(const uint16_t* x, const float* w_router, int T, int H, int E, int k,
              float* logits_out, int32_t* topk_ids, float* topk_w, void* stream);

/* Top-k and softmax weights from given fp32 logits [T, E] (device): ids
 * int32 [T, k] ranked by (larger logit, lower index); topk_w fp32 [T, k] =
 * exp(l - l_max) / sum over the selection, so each row sums to 1.
 * 1 <= k <= min(E, 8), E <= 1024.  NaN logits rank below every number and
 * ties go to the lower index, so the k ids are always distinct and in
 * [0, E).  Source: the fused top-k router of "[Model] Add Flint
 * (RecursiveSI/flint)", section "What happened" (routing as the first of the
 * layer's steps); top-6 of 256 in "Recursive Flint: 40B Local Coding Model,
 * Benchmarks", section "What is Recursive Flint?". */
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

/* Normalisation between chained layers: x[t] = bf16(r[t] / sqrt(mean_h
 * r[t, h]^2 + eps)) for r, x bf16 [T, H] (device, 16-byte aligned; x may
 * equal r), H a multiple of 64, eps finite and >= 0.  Squares are summed in
 * fp32 in a fixed order; each element is multiplied by the fp32 reciprocal
 * of the fp32 root and rounded to bf16 (nearest, ties to even), within one
 * bf16 ulp of the exact quotient.  The pages chain 47 MoE layers
 * ("Recursive Flint: 40B Local Coding Model, Benchmarks", section "What is
 * Recursive Flint?") but do not describe the norms between them: this
 * gain-free RMS normalisation is the stand-in that keeps a chained decode
 * step in range while every layer's routing depends on the layer before. */
int moe_rms_norm(const uint16_t* r, int T, int H, float eps, uint16_t* x, void* stream);

/* Whole layer for decode-sized batches.  Source: the mixture-of-experts
 * layer of "Recursive Flint: 40B Local Coding Model, Benchmarks" (section
 * "What is Recursive Flint?": 256 routed experts, 6 per token, one shared
 * expert) with the always-on shared expert of "Recursive Flint: 125 tok/s on
 * an M4 Pro, measured where it matters least" (table under "What actually
 * shipped"), run as the small-batch fused router + expert-indexed GEMV
 * kernels of "[Model] Add Flint (RecursiveSI/flint)", section "What
 * happened".  (1 <= T <= 64 takes the fused path;
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
 * same format and hidden size as the routed experts.  MOE_FMT_BF16 weights
 * with T > 1 take the composed path at every T (the same results as the
 * separate calls in GEMV mode). */
size_t moe_layer_decode_workspace_size(const moe_layer_weights* L, int T);
int moe_layer_decode(const moe_layer_weights* L, const uint16_t* x, const uint16_t* residual,
                     int T, uint16_t* y, int32_t* ids_out, float* w_out,
                     void* ws, size_t ws_bytes, void* stream);

/* One decode step through n_layers chained MoE layers (the 47 MoE layers of
 * "Recursive Flint: 40B Local Coding Model, Benchmarks", section "What is
 * Recursive Flint?"), issued as one call:
 *   r_0 = r_in;  for l < n_layers:  x_l = moe_rms_norm(r_l, eps),
 *                r_{l+1} = moe_layer_decode(layers[l], x_l, residual = r_l);
 *   r_out = r_{n_layers}.
 * The norms between the layers are not on the pages: the gain-free RMS
 * normalisation stands in for them (see moe_rms_norm), so every layer's
 * routing depends on the layer before.  layers: host array of n_layers
 * layer descriptors of one shape and format (one workspace serves all).
 * r_in, r_out bf16 [T, H]; r_all bf16 [n_layers, T, H] or NULL receives
 * r_1 .. r_{n_layers}; ids_out int32 [n_layers, T, k] and w_out fp32
 * [n_layers, T, k] may be NULL (both or neither).  Workspace:
 * moe_decode_step_workspace_size(layers, n_layers, T, r_all != NULL) bytes,
 * 256-byte aligned, zero-filled before its first use (it holds a layer
 * workspace).  The result equals the same sequence of moe_rms_norm and
 * moe_layer_decode calls bit for bit. */
size_t moe_decode_step_workspace_size(const moe_layer_weights* layers, int n_layers, int T, int with_r_all);
int moe_decode_step(const moe_layer_weights* layers, int n_layers, const uint16_t* r_in, int T, float eps,
                    uint16_t* r_out, uint16_t* r_all, int32_t* ids_out, float* w_out, void* ws,
                    size_t ws_bytes, void* stream);

/* moe_layer_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same kernels, numerics and
 * arguments as moe_layer_decode; its scratch memory is a static device array
 * of moe_layer_decode_noalloc_max_bytes() bytes (8 MiB) that each GPU the
 * library runs on holds from the first use until the process ends; the call
 * allocates and frees nothing.  Only the fused path: 0 <= T <= 64, and the
 * layer's workspace at T (moe_layer_decode_workspace_size) must fit the
 * array, else MOE_ERR_UNSUPPORTED with nothing enqueued (a Flint-shaped
 * layer needs about 4.5 MiB at 64 tokens).  The array belongs to the
 * calling thread's current device, which must be the stream's device.
 * Every call on one GPU shares that GPU's array and leaves in it the state
 * the next call expects (ticket counters at zero), so calls that overlap on
 * one GPU (two streams, two threads) race and must be serialised by the
 * caller. */
size_t moe_layer_decode_noalloc_max_bytes(void);
int moe_layer_decode_noalloc(const moe_layer_weights* L, const uint16_t* x, const uint16_t* residual,
                             int T, uint16_t* y, int32_t* ids_out, float* w_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
