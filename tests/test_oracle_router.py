"""Pins for the oracle's router, top-k selection, weights and permutation (CPU only)."""

import math

import numpy as np
import pytest
import scipy.special

import oracle
from oracle.formats import f64_to_bf16_bits


def brute_topk(row, k):
    """Pick k times the largest remaining value, the lowest index on ties."""
    chosen = []
    for _ in range(k):
        best = -1
        for e, v in enumerate(row):
            if e in chosen:
                continue
            if best < 0 or v > row[best]:
                best = e
        chosen.append(best)
    return chosen


def test_router_logits_one_hot_tokens():
    rng = np.random.default_rng(0)
    E, H = 12, 64
    wr = (rng.standard_normal((E, H)) * 0.02).astype(np.float32)
    x = np.zeros((3, H))
    x[0, 5] = 1.0
    x[1, 7] = 2.0
    x[1, 60] = -1.0
    x[2, :] = 0.5
    lg = oracle.router_logits(f64_to_bf16_bits(x), wr)
    w64 = wr.astype(np.float64)
    assert lg.shape == (3, E)
    assert np.array_equal(lg[0], w64[:, 5])
    assert np.array_equal(lg[1], 2.0 * w64[:, 7] - w64[:, 60])
    assert np.allclose(lg[2], 0.5 * w64.sum(axis=1), rtol=1e-14, atol=0)


def test_topk_matches_brute_force_with_many_ties():
    rng = np.random.default_rng(1)
    T, E, k = 4000, 32, 6
    logits = rng.integers(0, 10, size=(T, E)).astype(np.float64)   # heavy ties
    logits[:1000] = rng.standard_normal((1000, E))                  # no ties
    ids = oracle.topk_select(logits, k)
    for t in range(T):
        assert ids[t].tolist() == brute_topk(logits[t].tolist(), k)


def test_topk_adversarial_cases():
    E, k = 16, 6
    assert oracle.topk_select(np.zeros((1, E)), k)[0].tolist() == [0, 1, 2, 3, 4, 5]
    row = np.zeros(E)
    row[[3, 9, 12]] = 2.0
    row[[1, 7, 8, 14]] = 1.0          # the 4 tied at rank 4..7 straddle k = 6
    assert oracle.topk_select(row[None], k)[0].tolist() == [3, 9, 12, 1, 7, 8]
    pm = np.full(E, -1.0)
    pm[[2, 5]] = -0.0
    pm[[4]] = 0.0
    # -0 and +0 compare equal: ties go to the lower index
    assert oracle.topk_select(pm[None], 3)[0].tolist() == [2, 4, 5]
    assert oracle.topk_select(np.arange(E, dtype=float)[None], E)[0].tolist() == list(range(E - 1, -1, -1))


def test_topk_non_finite_order():
    """Non-finite logits (the pages are silent): +inf ranks first, -inf below every
    finite value, NaN below everything; ties and NaNs go to the lower index, so the
    k ids are always distinct and in range."""
    nan, inf = float("nan"), float("inf")
    row = [1.0, nan, -inf, 3.0, inf, nan, -2.0, 3.0]
    assert oracle.topk_select(np.array([row]), 8)[0].tolist() == [4, 3, 7, 0, 6, 2, 1, 5]
    assert oracle.topk_select(np.full((1, 5), nan), 3)[0].tolist() == [0, 1, 2]
    both = [nan, -inf, nan, -inf]
    assert oracle.topk_select(np.array([both]), 4)[0].tolist() == [1, 3, 0, 2]


def test_weights_sum_to_one_and_are_ordered():
    rng = np.random.default_rng(2)
    T, E, k = 2000, 256, 6
    logits = rng.standard_normal((T, E)) * 3
    ids = oracle.topk_select(logits, k)
    w = oracle.topk_weights(logits, ids)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 4 * 2.0 ** -53 * k)
    assert np.all(np.diff(w, axis=1) <= 0)
    # equal to the full softmax renormalised over the selection
    full = scipy.special.softmax(logits, axis=1)
    sel = np.take_along_axis(full, ids, axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)


def test_weights_two_way_closed_form():
    l0, l1 = 1.25, -0.5
    w = oracle.topk_weights(np.array([[l0, l1]]), np.array([[0, 1]]))[0]
    assert math.isclose(w[0], 1.0 / (1.0 + math.exp(l1 - l0)), rel_tol=1e-15)
    assert math.isclose(w[1], 1.0 / (1.0 + math.exp(l0 - l1)), rel_tol=1e-15)
    # equal logits split evenly; a single expert gets weight exactly 1
    assert oracle.topk_weights(np.array([[3.0, 3.0, 3.0]]), np.array([[0, 1, 2]]))[0].tolist() == [1 / 3] * 3
    assert oracle.topk_weights(np.array([[7.0]]), np.array([[0]]))[0].tolist() == [1.0]


def brute_permute(ids, E):
    T, k = ids.shape
    buckets = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            buckets[int(ids[t, j])].append(t * k + j)
    counts = [len(b) for b in buckets]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    order = [p for b in buckets for p in b]
    return counts, offsets, order


@pytest.mark.parametrize("T,k,E", [(1, 6, 256), (4, 6, 32), (64, 6, 256), (37, 1, 5), (5, 3, 3), (0, 6, 32)])
def test_permute_matches_brute_force(T, k, E):
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), dtype=np.int64)
    counts, offsets, sorted_pairs, pair_pos = oracle.permute(ids, E)
    bc, bo, border = brute_permute(ids, E)
    assert counts.tolist() == bc and offsets.tolist() == bo and sorted_pairs.tolist() == border
    assert counts.sum() == T * k and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(pair_pos[sorted_pairs], np.arange(T * k))


def test_permute_all_tokens_one_expert():
    ids = np.full((9, 1), 3)
    counts, offsets, sp, pp = oracle.permute(ids, 4)
    assert counts.tolist() == [0, 0, 0, 9]
    assert offsets.tolist() == [0, 0, 0, 0, 9]
    assert sp.tolist() == list(range(9)) and pp.tolist() == list(range(9))
