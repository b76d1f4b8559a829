"""The mixture-of-experts layer, step by step, in float64.

Test infrastructure only (see the package docstring).

What the layer computes, in the order the pages give it:

1. A router scores every token against all routed experts and keeps the top
   k ("[Model] Add Flint (RecursiveSI/flint)", section "What happened": a
   fused top-k router; "Recursive Flint: 40B Local Coding Model,
   Benchmarks", architecture table: 256 routed experts, 6 per token).
2. Each selected expert -- a small feed-forward sub-network ("What is
   Recursive Flint?" on the same page) -- runs on the token with its 4-bit
   weights dequantised (W4A16, "What happened").
3. The outputs are summed with the router weights, and one always-on shared
   expert is added ("Recursive Flint: 125 tok/s on an M4 Pro, measured where
   it matters least", table in "What actually shipped").

Readings taken where the pages are silent:

* router: logits = x . w_router[e] (fp32 router weights, bf16 tokens);
  select on the logits, ranked by (larger logit, then lower expert index);
  weights = softmax over the k selected logits (the same numbers as the full
  softmax renormalised over the selection); no extra routed scaling;
* expert: SwiGLU with separate gate, up and down matrices:
  h = silu(gate . x) * (up . x), silu(z) = z / (1 + exp(-z)), o = down . h;
  the down projection consumes h rounded to bfloat16 (the "A16" of W4A16),
  rounded once from the exact value; every other intermediate is exact;
* shared expert: ungated, weight 1;
* combine: y = residual + sum_j w_j o_j + o_shared, rounded once to bf16;
* grouping: pairs p = t*k + j sorted stably by expert (counting sort), with
  its inverse permutation.
"""

import numpy as np

from .formats import bf16_bits_to_f64, dequant_matrix, f64_to_bf16_bits, rne_bf16


def router_logits(x_bits, w_router):
    """logits[t, e] = sum_h x[t, h] * w_router[e, h] in float64."""
    x = bf16_bits_to_f64(x_bits)
    wr = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    return x @ wr.T


def topk_select(logits, k):
    """Top-k expert ids per row, in rank order: larger logit first, ties to the lower index."""
    lg = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-lg, axis=-1, kind="stable")
    return order[..., :k].astype(np.int64)


def topk_weights(logits, ids):
    """Softmax over the selected logits of each row."""
    lg = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(lg, np.asarray(ids), axis=-1)
    z = np.exp(sel - sel.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def route(x_bits, w_router, k, logits=None):
    """Router logits (computed unless given), top-k ids and weights."""
    if logits is None:
        logits = router_logits(x_bits, w_router)
    else:
        logits = np.asarray(logits, dtype=np.float32).astype(np.float64)
    ids = topk_select(logits, k)
    return logits, ids, topk_weights(logits, ids)


def silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(ffn, expert, x, weights=None, return_h=False):
    """SwiGLU expert on token rows x (float64 [n, H]) -> float64 [n, H].

    ``weights`` may carry the already dequantised (gate, up, down) matrices.
    """
    if weights is None:
        weights = tuple(dequant_matrix(ffn[m], expert) for m in ("gate", "up", "down"))
    wg, wu, wd = weights
    g = x @ wg.T
    u = x @ wu.T
    h = rne_bf16(silu(g) * u)
    o = h @ wd.T
    return (o, h) if return_h else o


def permute(ids, num_experts):
    """Counting sort of the pairs p = t*k + j by expert, stable in p.

    Returns counts [E], offsets [E+1] (exclusive prefix sum), sorted_pairs
    [T*k] (pair at each sorted position) and pair_pos [T*k] (its inverse).
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=num_experts)[:num_experts]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    sorted_pairs = np.argsort(flat, kind="stable")
    pair_pos = np.empty_like(sorted_pairs)
    pair_pos[sorted_pairs] = np.arange(flat.size)
    return (counts.astype(np.int64), offsets.astype(np.int64),
            sorted_pairs.astype(np.int64), pair_pos.astype(np.int64))


def grouped_ffn(ffn, x_bits, offsets, sorted_pairs=None, k=1):
    """Unweighted expert outputs, one row per sorted position.

    Row r in [offsets[e], offsets[e+1]) is expert e applied to token
    sorted_pairs[r] // k (or to token r when sorted_pairs is None).
    """
    x = bf16_bits_to_f64(x_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    rows = int(offsets[-1])
    out = np.zeros((rows, x.shape[1]), dtype=np.float64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        r = np.arange(lo, hi)
        tok = r if sorted_pairs is None else np.asarray(sorted_pairs)[r] // k
        out[lo:hi] = expert_ffn(ffn, e, x[tok])
    return out


def combine(o_pairs, w, o_shared=None, residual_bits=None):
    """y[t] = residual[t] + sum_j w[t, j] * o_pairs[t, j] + o_shared[t] (float64)."""
    o_pairs = np.asarray(o_pairs, dtype=np.float64)
    y = np.einsum("tj,tjh->th", np.asarray(w, dtype=np.float64), o_pairs)
    if o_shared is not None:
        y = y + o_shared
    if residual_bits is not None:
        y = y + bf16_bits_to_f64(residual_bits)
    return y


def moe_layer(layer, x_bits, residual_bits=None, logits=None, tokens=None):
    """The whole layer for the given tokens.

    ``layer``: dict with ``k``, ``w_router`` float32 [E, H], ``experts``
    (gate/up/down matrices over E experts) and ``shared`` (the same over one
    expert, or None).  ``logits`` (float32 [T, E]) replaces the router GEMV
    when given.  ``tokens`` restricts the work to those rows of x.

    Returns a dict: logits, ids, w, o_pairs [T, k, H], o_shared [T, H] or
    None, y (float64) and y_bf16 (y rounded once to bfloat16).
    """
    x_bits = np.asarray(x_bits)
    if tokens is not None:
        tokens = np.asarray(tokens)
        x_bits = x_bits[tokens]
        if residual_bits is not None:
            residual_bits = np.asarray(residual_bits)[tokens]
        if logits is not None:
            logits = np.asarray(logits)[tokens]
    k = int(layer["k"])
    logits, ids, w = route(x_bits, layer["w_router"], k, logits)
    x = bf16_bits_to_f64(x_bits)
    T, H = x.shape
    o_pairs = np.zeros((T, k, H), dtype=np.float64)
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        o_pairs[t_idx, j_idx] = expert_ffn(layer["experts"], int(e), x[t_idx])
    o_shared = None
    if layer.get("shared") is not None:
        o_shared = expert_ffn(layer["shared"], 0, x)
    y = combine(o_pairs, w, o_shared, residual_bits)
    return {"logits": logits, "ids": ids, "w": w, "o_pairs": o_pairs,
            "o_shared": o_shared, "y": y, "y_bf16": rne_bf16(y)}


def rms_norm(r_bits, eps):
    """The normalisation that feeds one chained layer from the residual stream.

    The pages chain 47 MoE layers ("Recursive Flint: 40B Local Coding Model,
    Benchmarks", section "What is Recursive Flint?") but describe none of the
    norms between them.  Reading taken: x = r / sqrt(mean_h(r^2) + eps), no
    learned gain, computed exactly and rounded once to bfloat16 (returned as
    bit patterns).
    """
    r = bf16_bits_to_f64(r_bits)
    ms = np.mean(r * r, axis=-1, keepdims=True)
    return f64_to_bf16_bits(rne_bf16(r / np.sqrt(ms + eps)))


def chain_layer(layer, r_bits, eps, logits=None):
    """One layer of the chained decode step: x = rms_norm(r), then the MoE
    layer with the residual r (its bf16 output is the next residual).
    Returns (x_bits, the moe_layer result dict)."""
    x_bits = rms_norm(r_bits, eps)
    return x_bits, moe_layer(layer, x_bits, residual_bits=r_bits, logits=logits)


def dense_gemv(mat, expert, x_bits, rows=None):
    """out[t, n] = sum_c W[n, c] x[t, c] for one packed 4-bit matrix (the
    4-bit output head of "Recursive Flint: 40B Local Coding Model,
    Benchmarks", section "How Recursive built Flint", is such a matrix over
    the 150,144-token vocabulary).  ``rows`` restricts it to those output rows."""
    x = bf16_bits_to_f64(x_bits)
    return x @ dequant_matrix(mat, expert, rows).T
