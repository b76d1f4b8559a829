"""Pins for the oracle's chain normalisation (CPU only).

The chained decode step feeds each layer x = bf16(r / sqrt(mean(r^2) + eps))
from the residual stream r (a reading: the pages chain the MoE layers but do
not describe the norms between them).  These checks tie oracle.rms_norm to
closed forms and exact invariants, not to a second copy of its formula."""

import numpy as np

import oracle
from oracle.formats import bf16_bits_to_f64, f64_to_bf16_bits


def bits(v):
    return f64_to_bf16_bits(np.asarray(v, dtype=np.float64))


def test_constant_row_normalises_to_one():
    # r = 2 everywhere: mean square 4, x = 2 / sqrt(4 + 1e-6) = 0.99999988 -> bf16 1.0 exactly
    r = bits(np.full((3, 64), 2.0))
    x = bf16_bits_to_f64(oracle.rms_norm(r, 1e-6))
    assert np.array_equal(x, np.ones((3, 64)))
    # negative constant: -1 exactly
    x = bf16_bits_to_f64(oracle.rms_norm(bits(np.full((1, 64), -0.75)), 1e-6))
    assert np.array_equal(x, -np.ones((1, 64)))


def test_hand_example_three_four():
    # r = (3, 4, 0, 0): mean square 25/4, sqrt 2.5, x = (1.2, 1.6, 0, 0) before rounding;
    # bf16 neighbours of 1.2 are 1.1953125 and 1.203125 (midpoint 1.19921875), of 1.6 are
    # 1.59375 and 1.6015625 (midpoint 1.59765625): x = (1.203125, 1.6015625, 0, 0)
    x = bf16_bits_to_f64(oracle.rms_norm(bits([[3.0, 4.0, 0.0, 0.0]]), 0.0))
    assert x.tolist() == [[1.203125, 1.6015625, 0.0, 0.0]]
    # with eps the row still rounds the same way (the shift is about 1e-7 relative)
    x = bf16_bits_to_f64(oracle.rms_norm(bits([[3.0, 4.0, 0.0, 0.0]]), 1e-6))
    assert x.tolist() == [[1.203125, 1.6015625, 0.0, 0.0]]


def test_power_of_two_scale_invariance():
    # without eps the normalisation ignores any power-of-two scale exactly
    rng = np.random.default_rng(3)
    r = bits(rng.standard_normal((5, 2048)))
    x0 = oracle.rms_norm(r, 0.0)
    for p in (-20, -3, 1, 7, 40):
        rs = bits(bf16_bits_to_f64(r) * 2.0 ** p)
        assert np.array_equal(oracle.rms_norm(rs, 0.0), x0)


def test_output_mean_square_and_rounding():
    # before rounding mean(x^2) = ms / (ms + eps); after one bf16 rounding per element
    # (relative error <= 2**-9) the mean square is within 2**-8 of that
    rng = np.random.default_rng(4)
    r = bits(rng.standard_normal((7, 2048)) * rng.uniform(0.01, 100.0, size=(7, 1)))
    eps = 1e-2
    rv = bf16_bits_to_f64(r)
    ms = np.mean(rv * rv, axis=1)
    x = bf16_bits_to_f64(oracle.rms_norm(r, eps))
    got = np.mean(x * x, axis=1)
    assert np.all(np.abs(got / (ms / (ms + eps)) - 1.0) <= 2.0 ** -8)
    # every element is the nearest bf16 of its exact value: within half a bf16 ulp
    exact = rv / np.sqrt(ms + eps)[:, None]
    _, e = np.frexp(exact)
    assert np.all(np.abs(x - exact) <= np.ldexp(0.5, e - 8))
    # the sign of every element is kept and zeros stay zero
    assert np.array_equal(np.sign(x), np.sign(rv))


def test_chain_layer_feeds_the_next_layer():
    # chain_layer = rms_norm, then the layer with residual r: the output is the next residual
    import synth
    layer = synth.layer_to_numpy(synth.make_layer(2, 256, 128, 32, 6, 0, "cpu"))
    r = synth.bits16(synth.make_tokens(3, 256, 9, "cpu"))
    x, res = oracle.chain_layer(layer, r, 1e-6)
    assert np.array_equal(x, oracle.rms_norm(r, 1e-6))
    ref = oracle.moe_layer(layer, x, residual_bits=r)
    assert np.array_equal(res["y"], ref["y"]) and np.array_equal(res["ids"], ref["ids"])
