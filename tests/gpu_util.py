"""Helpers for the GPU parity tests: device inputs from the seeded generators,
host copies for the oracle, error metrics and near-tie detection."""

import numpy as np
import torch

import oracle
import synth

DEV = "cuda"

# Layer output tolerance: max over tokens of the normwise relative error of
# the bf16 output against the unrounded float64 result.
TOL_LAYER = 2e-3
# Unweighted expert outputs (fp32) against float64: only the bf16 rounding of
# h can differ (a flip moves h by one bf16 ulp), so the bound is tighter.
TOL_EXPERT = 1e-3


def bits_of(t):
    """bf16 tensor (any device) -> numpy uint16 bits."""
    return synth.bits16(t)


def normwise_err(y, ref):
    """max_t ||y_t - ref_t|| / ||ref_t|| (rows with ||ref_t|| == 0 use the absolute norm)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(y - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num))) if y.size else 0.0


def near_tie_tokens(x_bits, w_router, k):
    """Tokens whose fp64 margin between the k-th and (k+1)-th logit is below
    tau = 2**-20 * max_e sum_h |x_h w_eh| (fp32 accumulation cannot order them)."""
    x = oracle.bf16_bits_to_f64(x_bits)
    wr = np.asarray(w_router, dtype=np.float64)
    lg = x @ wr.T
    tau = 2.0 ** -20 * (np.abs(x) @ np.abs(wr).T).max(axis=1)
    srt = -np.sort(-lg, axis=1)
    if lg.shape[1] <= k:
        return np.zeros(lg.shape[0], dtype=bool)
    return (srt[:, k - 1] - srt[:, k]) < tau


def y_diagnostics(y_bits, ref):
    """Elementwise check: |y - ref| <= ulp_bf16(ref) + 2**-8 * rms(ref_t) (reported, not graded)."""
    y = oracle.bf16_bits_to_f64(y_bits)
    ref = np.asarray(ref)
    _, e = np.frexp(ref)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    return float(np.mean(np.abs(y - ref) > ulp + 2.0 ** -8 * rms))


def ulp_bf16(v):
    """One bf16 unit in the last place of each value (8 significant bits)."""
    _, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def decode_ws_views(ws, H, I, Is, E, k, T):
    """Host views of the fused decode workspace after a call (1 <= T <= 64).

    Mirrors the order in which the library carves the workspace (each buffer
    256-byte aligned): ticket words, logits, ids, w, counts, offsets,
    sorted_pairs, pair_pos, active list, h of the routed pairs (grouped row
    order), h of the shared expert (token order).  The caller checks the ids
    view against ids_out, so a change of layout fails loudly."""
    host = ws.cpu().numpy()
    off = 0
    n = T * k

    def take(nbytes):
        nonlocal off
        o = off
        off += (nbytes + 255) // 256 * 256
        return o

    take(4 * 16 * (17 + (H + 31) // 32))
    take(4 * T * E)
    o_ids = take(4 * n)
    o_w = take(4 * n)
    take(4 * E)
    take(4 * (E + 1))
    take(4 * n)
    o_pp = take(4 * n)
    take(4 * (E + 1))
    o_hr = take(2 * n * I)
    o_hs = take(2 * T * Is)
    return {"ids": host[o_ids:o_ids + 4 * n].view(np.int32).reshape(T, k),
            "w": host[o_w:o_w + 4 * n].view(np.float32).reshape(T, k),
            "pair_pos": host[o_pp:o_pp + 4 * n].view(np.int32).reshape(T, k),
            "h_routed": host[o_hr:o_hr + 2 * n * I].view(np.uint16).reshape(n, I),
            "h_shared": host[o_hs:o_hs + 2 * T * Is].view(np.uint16).reshape(T, Is) if Is else None}


# Slack for an fp32 dot product against its float64 value, relative to the
# sum of the absolute products (sum |w x|): about 6e-5, several times the
# typical sqrt(n) * 2**-24 of a 2048-term fp32 sum, yet far below what one
# wrong or missing 32-element piece (1.5% of the terms at H = 2048) moves.
DOT_SLACK = 2.0 ** -14
MAX_H_FLIPS = 5e-3


def check_decode_stages(layer, x, residual, y, ids, w, ws, tokens=None):
    """Tight checks of the fused decode kernels through the kernel's own h.

    gate/up + SwiGLU: every h element the kernel stored is within one bf16
    ulp (plus the fp32 slack of g and u) of the exact silu(g) * u, and at
    most MAX_H_FLIPS of them differ from its nearest bf16 value.
    down + combine: the bf16 output is within one bf16 ulp (plus the fp32
    slack of the down products and the combine) of res + sum_j w_j (Wd_j h_j)
    + Wd_sh h_sh computed in float64 from the kernel's own h and weights w.
    Returns (flip fraction, number of h elements)."""
    from oracle.moe import silu
    T = x.shape[0]
    H, I, E, k = layer["H"], layer["I"], layer["E"], layer["k"]
    sh = layer.get("shared")
    Is = sh["gate"]["rows"] if sh is not None else 0
    v = decode_ws_views(ws, H, I, Is, E, k, T)
    gids = ids.cpu().numpy()
    gw = w.cpu().numpy().astype(np.float64)
    assert np.array_equal(v["ids"], gids), "decode workspace layout differs from the test's mirror"
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    x64 = oracle.bf16_bits_to_f64(bits_of(x))
    r64 = np.zeros((T, H)) if residual is None else oracle.bf16_bits_to_f64(bits_of(residual))
    y_own = r64[tokens].copy()
    y_sl = np.abs(r64[tokens])
    host = synth.layer_to_numpy(layer, experts=set(gids[tokens].ravel().tolist()))
    flips, count = 0, 0

    def stage(ffn, e, xe, hbits, what):
        nonlocal flips, count
        wg, wu, wd = (oracle.dequant_matrix(ffn[m], e) for m in ("gate", "up", "down"))
        g, u = xe @ wg.T, xe @ wu.T
        sg, su = np.abs(xe) @ np.abs(wg).T, np.abs(xe) @ np.abs(wu).T
        sl = silu(g)
        h64 = sl * u
        slack = DOT_SLACK * (1.1 * np.abs(u) * sg + np.abs(sl) * su)
        hg = oracle.bf16_bits_to_f64(hbits)
        bad = np.abs(hg - h64) > ulp_bf16(h64) + slack
        assert not bad.any(), "%s: %d h elements more than one bf16 ulp from silu(g)*u" % (what, int(bad.sum()))
        flips += int(np.sum(hbits != oracle.f64_to_bf16_bits(oracle.rne_bf16(h64))))
        count += hbits.size
        return hg @ wd.T, np.abs(hg) @ np.abs(wd).T

    pos = {int(t): i for i, t in enumerate(tokens)}
    sel = gids[tokens]
    for e in np.unique(sel):
        ti, ji = np.nonzero(sel == e)
        tt = tokens[ti]
        rows = v["pair_pos"][tt, ji]
        o, so = stage(host["experts"], int(e), x64[tt], v["h_routed"][rows], "expert %d" % e)
        wt = gw[tt, ji][:, None]
        for i, t in enumerate(tt):
            y_own[pos[int(t)]] += wt[i] * o[i]
            y_sl[pos[int(t)]] += np.abs(wt[i]) * so[i]
    if sh is not None:
        o, so = stage(host["shared"], 0, x64[tokens], v["h_shared"][tokens], "shared expert")
        y_own += o
        y_sl += so
    yg = oracle.bf16_bits_to_f64(bits_of(y)[tokens])
    bad = np.abs(yg - y_own) > ulp_bf16(y_own) + DOT_SLACK * y_sl
    assert not bad.any(), "%d outputs more than one bf16 ulp from the float64 combine of the kernel's h" % int(
        bad.sum())
    frac = flips / max(count, 1)
    assert frac <= MAX_H_FLIPS, "h flips %.2e > %.0e" % (frac, MAX_H_FLIPS)
    return frac, count
