"""Pins for the oracle's expert FFN, combine and whole layer (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.formats import f64_to_bf16_bits, dequant_matrix, rne_bf16
from tests import scalar_reference


def int4_matrix(q, z, s_bits):
    """Pack explicit INT4 codes q [E, rows, cols] with zeros/scales per 64 columns."""
    q = np.asarray(q, dtype=np.uint8)
    codes = (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)
    return {"fmt": 2, "num_experts": q.shape[0], "rows": q.shape[1], "cols": q.shape[2],
            "codes": codes, "scales": np.asarray(s_bits, dtype=np.uint16),
            "zeros": np.asarray(z, dtype=np.uint8), "tensor_scale": None}


def test_swiglu_closed_form():
    """One expert, token = unit vector e_0.

    gate row i . x = 2, up row i . x = 3 for every i, so
    h_i = silu(2) * 3 = 6 / (1 + e**-2) = 5.2847824678...; rounded to bf16
    (step 2**-5 in [4, 8)) it is 169 * 2**-5 = 5.28125.  With every down
    weight 1 and I = 64, y_n = 64 * 5.28125 = 338 exactly.  Swapping gate and
    up would give 64 * bf16(2 * silu(3)) = 366; sigmoid instead of silu
    gives 169; skipping the bf16 rounding gives 338.2260...
    """
    H = I = 64
    one = 0x3C00
    qg = np.full((1, I, H), 8)
    qg[0, :, 0] = 10
    qu = np.full((1, I, H), 8)
    qu[0, :, 0] = 11
    qd = np.full((1, H, I), 9)
    zeros = np.full((1, I, 1), 8)
    scales = np.full((1, I, 1), one)
    ffn = {"gate": int4_matrix(qg, zeros, scales), "up": int4_matrix(qu, zeros, scales),
           "down": int4_matrix(qd, np.full((1, H, 1), 8), np.full((1, H, 1), one))}
    layer = {"k": 1, "w_router": np.ones((1, H), dtype=np.float32), "experts": ffn, "shared": None}
    x = np.zeros((1, H))
    x[0, 0] = 1.0
    out = oracle.moe_layer(layer, f64_to_bf16_bits(x))
    assert out["ids"].tolist() == [[0]] and out["w"].tolist() == [[1.0]]
    assert np.all(out["y"] == 338.0)
    assert math.isclose(6.0 / (1.0 + math.exp(-2.0)), 5.284782467867294, rel_tol=1e-15)


def _tiny_layer(fmt, seed, E=8, H=128, I=64, k=3, shared=True):
    return synth.layer_to_numpy(synth.make_layer(fmt, H, I, E, k, seed, "cpu", shared=shared))


@pytest.mark.parametrize("fmt", [1, 2])
def test_one_expert_equals_dense_swiglu(fmt):
    L = _tiny_layer(fmt, 3, E=1, k=1, shared=False)
    xb = synth.bits16(synth.make_tokens(5, L["H"], 3))
    out = oracle.moe_layer(L, xb)
    wg, wu, wd = (torch.from_numpy(dequant_matrix(L["experts"][m], 0)) for m in ("gate", "up", "down"))
    x = torch.from_numpy(oracle.bf16_bits_to_f64(xb))
    h = torch.nn.functional.silu(x @ wg.T) * (x @ wu.T)
    y = torch.from_numpy(rne_bf16(h.numpy())) @ wd.T
    assert np.all(out["w"] == 1.0)
    assert np.allclose(out["y"], y.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", [1, 2])
def test_identical_experts_double_the_ffn(fmt):
    """All routed experts and the shared expert share one weight set: y = res + 2 FFN(x)."""
    L = _tiny_layer(fmt, 4, E=1, k=1, shared=False)
    E, k = 8, 3
    one = L["experts"]
    rep = {m: {key: (np.repeat(v, E, axis=0) if isinstance(v, np.ndarray) else v)
               for key, v in one[m].items()} for m in one}
    rng = np.random.default_rng(4)
    layer = {"k": k, "w_router": (rng.standard_normal((E, L["H"])) * 0.02).astype(np.float32),
             "experts": rep, "shared": one}
    xb = synth.bits16(synth.make_tokens(6, L["H"], 4))
    res = synth.bits16(synth.make_tokens(6, L["H"], 5))
    out = oracle.moe_layer(layer, xb, residual_bits=res)
    f = oracle.expert_ffn(one, 0, oracle.bf16_bits_to_f64(xb))
    assert np.allclose(out["y"], oracle.bf16_bits_to_f64(res) + 2.0 * f, rtol=1e-12, atol=1e-12)


def test_down_scale_tags_each_slot():
    """Experts differ only in the down tensor scale c_e, so o_e = c_e * o_1 and
    y = (sum_j w_j c_{id_j} + c_shared) * o_1: pairs each weight with its own
    expert and adds the shared expert once."""
    base = _tiny_layer(1, 6, E=1, k=1, shared=False)["experts"]
    E, k = 16, 4
    rep = {m: {key: (np.repeat(v, E, axis=0) if isinstance(v, np.ndarray) else v)
               for key, v in base[m].items()} for m in base}
    c = np.exp2(np.arange(E, dtype=np.float64) - 8).astype(np.float32)   # distinct powers of two
    rep["down"]["tensor_scale"] = c
    shared = {m: dict(base[m]) for m in base}
    shared["down"] = dict(base["down"], tensor_scale=np.array([0.75], dtype=np.float32))
    rng = np.random.default_rng(6)
    H = base["gate"]["cols"]
    layer = {"k": k, "w_router": (rng.standard_normal((E, H)) * 0.05).astype(np.float32),
             "experts": rep, "shared": shared}
    xb = synth.bits16(synth.make_tokens(10, H, 6))
    out = oracle.moe_layer(layer, xb)
    unit = {m: dict(base[m]) for m in base}
    unit["down"] = dict(base["down"], tensor_scale=np.array([1.0], dtype=np.float32))
    o1 = oracle.expert_ffn(unit, 0, oracle.bf16_bits_to_f64(xb))
    coef = (out["w"] * c.astype(np.float64)[out["ids"]]).sum(axis=1) + 0.75
    assert np.allclose(out["y"], coef[:, None] * o1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("fmt", [1, 2])
def test_token_independence_and_residual(fmt):
    L = _tiny_layer(fmt, 7)
    xb = synth.bits16(synth.make_tokens(7, L["H"], 7))
    res = synth.bits16(synth.make_tokens(7, L["H"], 8))
    batch = oracle.moe_layer(L, xb, residual_bits=res)
    for t in range(7):
        one = oracle.moe_layer(L, xb[t:t + 1], residual_bits=res[t:t + 1])
        assert np.array_equal(one["ids"][0], batch["ids"][t])
        assert np.allclose(one["y"][0], batch["y"][t], rtol=1e-13, atol=1e-13)
    nores = oracle.moe_layer(L, xb)
    assert np.allclose(batch["y"] - nores["y"], oracle.bf16_bits_to_f64(res), rtol=0, atol=1e-12)
    sub = oracle.moe_layer(L, xb, residual_bits=res, tokens=[5, 2])
    assert np.allclose(sub["y"], batch["y"][[5, 2]], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("fmt", [1, 2])
def test_grouped_ffn_and_combine_compose_to_the_layer(fmt):
    L = _tiny_layer(fmt, 9, E=8, k=3)
    T, k = 11, 3
    xb = synth.bits16(synth.make_tokens(T, L["H"], 9))
    out = oracle.moe_layer(L, xb)
    counts, offsets, sp, pp = oracle.permute(out["ids"], 8)
    rows = oracle.grouped_ffn(L["experts"], xb, offsets, sp, k)
    assert np.allclose(rows[pp].reshape(T, k, -1), out["o_pairs"], rtol=1e-13, atol=1e-13)
    sh = oracle.grouped_ffn(L["shared"], xb, np.array([0, T]))
    assert np.allclose(sh, out["o_shared"], rtol=1e-13, atol=1e-13)
    y = oracle.combine(rows[pp].reshape(T, k, -1), out["w"], sh)
    assert np.allclose(y, out["y"], rtol=1e-13, atol=1e-13)


def test_scalar_loop_form_agrees_on_tiny_layer():
    """Tiny shape (hidden 256, 32 experts top-6 + shared, inter 128, INT4 g64),
    two tokens, evaluated by plain Python loops against the vectorised oracle."""
    L = synth.layer_to_numpy(synth.make_layer(2, 256, 128, 32, 6, 0, "cpu"))
    xb = synth.bits16(synth.make_tokens(2, 256, 0))
    res = synth.bits16(synth.make_tokens(2, 256, 1))
    vec = oracle.moe_layer(L, xb, residual_bits=res)
    ref = scalar_reference.layer(L, xb.tolist(), res.tolist())
    for t, (ids, w, y) in enumerate(ref):
        assert vec["ids"][t].tolist() == ids
        assert np.allclose(vec["w"][t], w, rtol=1e-13, atol=0)
        assert np.allclose(vec["y"][t], y, rtol=1e-11, atol=1e-12)


def test_zero_down_weights_pass_the_residual_through():
    L = _tiny_layer(1, 10)
    for ffn in (L["experts"], L["shared"]):
        ffn["down"]["codes"] = np.zeros_like(ffn["down"]["codes"])
    xb = synth.bits16(synth.make_tokens(4, L["H"], 10))
    out = oracle.moe_layer(L, xb, residual_bits=xb)
    assert np.array_equal(out["y"], oracle.bf16_bits_to_f64(xb))
    assert np.array_equal(f64_to_bf16_bits(out["y_bf16"]), xb)


def test_dense_gemv_one_hot_columns_and_row_subsets():
    """The dense product against one-hot tokens returns the dequantised columns
    exactly, a row subset equals those rows of the full product, and the
    subset dequantisation equals the full one's rows (all three formats)."""
    rng = np.random.default_rng(11)
    for fmt in (1, 2, 3):
        m = synth.matrix_to_numpy(synth.make_matrix(fmt, 2, 40, 128, seed=fmt, device="cpu"))
        w = dequant_matrix(m, 1)
        cols = np.array([0, 5, 63, 64, 127])
        x = np.zeros((len(cols), 128))
        x[np.arange(len(cols)), cols] = 1.0
        out = oracle.dense_gemv(m, 1, f64_to_bf16_bits(x))
        assert np.array_equal(out, w[:, cols].T)
        rows = np.array([39, 0, 17, 17])
        assert np.array_equal(dequant_matrix(m, 1, rows), w[rows])
        xt = f64_to_bf16_bits(rne_bf16(rng.standard_normal((3, 128))))
        assert np.array_equal(oracle.dense_gemv(m, 1, xt, rows), oracle.dense_gemv(m, 1, xt)[:, rows])
