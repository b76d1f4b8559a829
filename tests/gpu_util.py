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
