"""Parity of the HIP path (through the C ABI) with the float64 oracle, on the
same seeded bytes.  Bit-exact for dequantised weights, expert ids and the
permutation; within the stated tolerances for floating-point outputs."""

import numpy as np
import pytest
import torch

import oracle
import synth
import bit_weight_only_moe_amd as moe
from tests.gpu_util import (DEV, TOL_EXPERT, TOL_LAYER, bits_of, check_decode_stages, near_tie_tokens,
                            normwise_err, ulp_bf16, y_diagnostics)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ dequant

def exhaustive_nvfp4(device):
    rows, cols = 256, 256
    i = np.arange(cols // 2)
    row_bytes = ((2 * i) % 16) | (((2 * i + 1) % 16) << 4)            # element c has code c % 16
    codes = np.broadcast_to(row_bytes.astype(np.uint8), (3, rows, cols // 2)).copy()
    sc = np.arange(256, dtype=np.uint8)
    sc[[0x7F, 0xFF]] = 0x38                                            # NaN codes are invalid input
    scales = np.broadcast_to(sc[:, None], (3, rows, cols // 16)).copy()
    ts = np.array([1.0, 2.0 ** -7, 0.0071234], dtype=np.float32)
    t = lambda a: torch.from_numpy(a).to(device)
    return {"fmt": 1, "num_experts": 3, "rows": rows, "cols": cols, "codes": t(codes), "scales": t(scales),
            "zeros": None, "tensor_scale": t(ts)}


def exhaustive_int4(device):
    rows, cols = 16, 1024
    i = np.arange(cols // 2)
    row_bytes = ((2 * i) % 16) | (((2 * i + 1) % 16) << 4)
    codes = np.broadcast_to(row_bytes.astype(np.uint8), (1, rows, cols // 2)).copy()
    zeros = np.broadcast_to(np.arange(16, dtype=np.uint8)[:, None], (1, rows, cols // 64)).copy()
    svals = np.array([1.0, -0.5, 0.0071234, 65504.0, 6.103515625e-05, 5.960464477539063e-08, 0.0123, -3.75,
                      0.005, 0.02, 1.5, 2.0 ** -10, 7.0, -0.0, 100.0, 0.333], dtype=np.float16)
    scales = np.broadcast_to(svals.view(np.uint16)[None, :], (1, rows, cols // 64)).copy()
    t = lambda a: torch.from_numpy(a).to(device)
    return {"fmt": 2, "num_experts": 1, "rows": rows, "cols": cols, "codes": t(codes),
            "scales": t(scales).view(torch.float16), "zeros": t(zeros), "tensor_scale": None}


def exhaustive_int4_sb(device):
    # every code against 16 scales x 16 biases (fp16 extremes, subnormals, signs, -0): rows r
    # takes bias r, group g scale g, so all 16 x 16 x 16 (code, scale, bias) combinations occur
    rows, cols = 16, 1024
    i = np.arange(cols // 2)
    row_bytes = ((2 * i) % 16) | (((2 * i + 1) % 16) << 4)
    codes = np.broadcast_to(row_bytes.astype(np.uint8), (1, rows, cols // 2)).copy()
    svals = np.array([1.0, -0.5, 0.0071234, 65504.0, 6.103515625e-05, 5.960464477539063e-08, 0.0123, -3.75,
                      0.005, 0.02, 1.5, 2.0 ** -10, 7.0, -0.0, 100.0, 0.333], dtype=np.float16)
    bvals = np.array([0.0, -1.25, 3.0, -65504.0, 5.960464477539063e-08, -6.0e-05, 0.1, -0.0, 1e-3, -7.5,
                      2048.0, 0.333, -0.0071234, 12.0, -1.0, 6.103515625e-05], dtype=np.float16)
    scales = np.broadcast_to(svals.view(np.uint16)[None, None, :], (1, rows, cols // 64)).copy()
    biases = np.broadcast_to(bvals.view(np.uint16)[None, :, None], (1, rows, cols // 64)).copy()
    t = lambda a: torch.from_numpy(a).to(device)
    return {"fmt": 3, "num_experts": 1, "rows": rows, "cols": cols, "codes": t(codes),
            "scales": t(scales).view(torch.float16), "zeros": None, "tensor_scale": None,
            "biases": t(biases).view(torch.float16)}


@pytest.mark.parametrize("which", ["nvfp4_exhaustive", "int4_exhaustive", "int4sb_exhaustive", "nvfp4_flint",
                                   "int4_flint", "int4sb_flint", "bf16_flint"])
def test_dequant_bit_exact(which):
    print("dequant", which, flush=True)
    if which == "nvfp4_exhaustive":
        mat = exhaustive_nvfp4(DEV)
    elif which == "int4_exhaustive":
        mat = exhaustive_int4(DEV)
    elif which == "int4sb_exhaustive":
        mat = exhaustive_int4_sb(DEV)
    else:
        fmt = {"nvfp4": 1, "int4": 2, "int4sb": 3, "bf16": 4}[which.split("_")[0]]
        mat = synth.make_matrix(fmt, 4, 768, 2048, seed=21, device=DEV, scale_range="full")
    host = synth.matrix_to_numpy(mat)
    for e in range(mat["num_experts"]):
        out = torch.empty((mat["rows"], mat["cols"]), dtype=torch.float32, device=DEV)
        moe.moe_dequant_w4(mat, e, out)
        sync()
        ref = oracle.dequant_matrix_f32(host, e)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (which, e)


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("T,E,k", [(4096, 256, 6), (37, 32, 8), (5, 1, 1), (64, 1024, 6), (50, 100, 6),
                                   (33, 200, 8), (9, 257, 6)])
def test_topk_softmax_bit_exact_ids(T, E, k):
    print("topk", T, E, k, flush=True)
    g = torch.Generator().manual_seed(T * 31 + E)
    lg = torch.randn((T, E), generator=g)
    half = T // 2
    lg[:half] = torch.randint(0, 12, (half, E), generator=g).float()   # many ties
    if T > 2:
        lg[1] = 0.0
        lg[2, ::2] = -0.0
    d_lg = lg.to(DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(d_lg, T, E, k, ids, w)
    sync()
    ref_ids = oracle.topk_select(lg.numpy().astype(np.float64), k)
    ref_w = oracle.topk_weights(lg.numpy().astype(np.float64), ref_ids)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=1e-7)


def test_topk_non_finite_logits():
    """NaN / inf logits: ids stay distinct and in range and follow the oracle's
    order (numbers first, +inf highest, NaN last, ties to the lower index)."""
    print("topk non-finite", flush=True)
    T, E, k = 6, 256, 6
    g = torch.Generator().manual_seed(5)
    lg = torch.randn((T, E), generator=g)
    lg[0] = float("nan")                       # every logit NaN
    lg[1, ::3] = float("nan")                  # some NaN
    lg[2, [7, 200]] = float("inf")
    lg[3] = float("-inf")
    lg[3, 250] = 1.0
    lg[4, :] = float("nan")
    lg[4, [9, 130]] = float("-inf")
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(lg.to(DEV), T, E, k, ids, w)
    sync()
    got = ids.cpu().numpy()
    assert ((got >= 0) & (got < E)).all()
    assert all(len(set(r)) == k for r in got.tolist())
    assert np.array_equal(got, oracle.topk_select(lg.numpy().astype(np.float64), k))


@pytest.mark.parametrize("T", [1, 5])
def test_layer_decode_router_ties(T):
    """Exactly tied logits spread over the expert range (the single-token top-k
    splits the experts into quarters and merges): ties go to the lower index."""
    print("router ties", T, flush=True)
    H, I, E, k = 256, 128, 256, 6
    layer = synth.make_layer(1, H, I, E, k, 11, DEV)
    wr = torch.zeros((E, H), dtype=torch.float32)
    for e in (250,):
        wr[e, 0] = 2.0
    for e in (200, 130, 70, 5):
        wr[e, 0] = 1.0
    layer["w_router"] = wr.to(DEV)
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    x[:, 0] = 1.0
    y, ids, w, ws = run_layer(layer, x, None, T)
    assert ids.cpu().numpy().tolist() == [[250, 5, 70, 130, 200, 0]] * T
    layer["w_router"] = torch.zeros((E, H), dtype=torch.float32, device=DEV)
    y, ids, w, ws = run_layer(layer, x, None, T)
    assert ids.cpu().numpy().tolist() == [list(range(k))] * T
    assert np.allclose(w.cpu().numpy(), 1.0 / k)


def test_layer_decode_non_finite_tokens():
    """Tokens holding inf / NaN must not disturb the finite tokens of the batch,
    and their expert ids stay valid (regression: an all-NaN logit row once
    produced expert -1)."""
    print("layer non-finite tokens", flush=True)
    H, I, E, k, T = 2048, 768, 256, 6, 4
    layer = synth.make_layer(1, H, I, E, k, 3, DEV)
    x = synth.make_tokens(T, H, 3, DEV)
    x[1] = float("nan")
    x[2, ::5] = float("inf")
    x[3, 100] = float("-inf")
    y, ids, w, ws = run_layer(layer, x, x, T)
    got = ids.cpu().numpy()
    assert ((got >= 0) & (got < E)).all()
    assert all(len(set(r)) == k for r in got.tolist())
    check_layer(layer, x, x, y, ids, w, tokens=[0], ws=ws)


@pytest.mark.parametrize("T,H,E", [(1, 2048, 256), (5, 2048, 256), (64, 2048, 256), (300, 2048, 256),
                                   (4096, 2048, 256), (300, 192, 100)])
def test_route_logits_and_ids(T, H, E):
    """Router logits within 2^-20 sum|x w| of fp64 (T >= 256 runs the matrix-core router with
    the weights split exactly into three bf16 parts), ids equal to the oracle's off near-ties."""
    print("route", T, H, E, flush=True)
    k = 6
    layer = synth.make_layer(1, H, 128, E, k, seed=30 + T, device=DEV, shared=False)
    x = synth.make_tokens(T, H, 30 + T, DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_route(x, layer["w_router"], T, H, E, k, lg, ids, w)
    sync()
    xb = bits_of(x)
    wr = layer["w_router"].cpu().numpy()
    ref_lg, ref_ids, _ = oracle.route(xb, wr, k)
    bound = 2.0 ** -20 * (np.abs(oracle.bf16_bits_to_f64(xb)) @ np.abs(wr.astype(np.float64)).T)
    assert np.all(np.abs(lg.cpu().numpy() - ref_lg) <= bound)
    gids = ids.cpu().numpy()
    # the GPU's own logits, ranked by the oracle, give the GPU's ids
    assert np.array_equal(oracle.topk_select(lg.cpu().numpy().astype(np.float64), k), gids)
    ties = near_tie_tokens(xb, wr, k)
    assert np.array_equal(gids[~ties], ref_ids[~ties])
    assert ties.sum() <= max(1, T // 500)


# ------------------------------------------------------------------ permute

# chunk scan shapes: 96 chunks in 4 groups; 5 chunks in 4 groups (last one
# empty); 64 chunks in one group (two batches); 24 chunks in 10 groups of an E
# that does not divide 1024 (empty groups at the end)
@pytest.mark.parametrize("T,k,E", [(1, 6, 256), (4, 6, 32), (64, 6, 256), (4096, 6, 256), (300, 1, 3),
                                   (77, 8, 1024), (200, 6, 256), (2048, 8, 1024), (1000, 6, 100)])
def test_permute_bit_exact(T, k, E):
    print("permute", T, k, E, flush=True)
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    H = 256
    x = synth.make_tokens(T, H, 40, DEV)
    d_ids = torch.from_numpy(ids).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=DEV)
    pp = torch.empty(T * k, dtype=torch.int32, device=DEV)
    xp = torch.empty((T * k, H), dtype=torch.bfloat16, device=DEV)
    nws = moe.moe_permute_workspace_size(T, k, E)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=DEV)
    moe.moe_permute(d_ids, T, k, E, counts, offsets, sp, pp, x, xp, H, ws, nws)
    sync()
    rc, ro, rsp, rpp = oracle.permute(ids, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sp.cpu().numpy(), rsp)
    assert np.array_equal(pp.cpu().numpy(), rpp)
    assert np.array_equal(bits_of(xp), bits_of(x)[rsp // k])


# ------------------------------------------------------------------ grouped FFN

FFN_CASES = [
    # fmt, H, I, E, k, T, seed
    (2, 256, 128, 32, 6, 4, 0),
    (1, 2048, 768, 256, 6, 5, 51),
    (2, 2048, 768, 256, 6, 3, 52),
    (1, 192, 320, 8, 3, 9, 53),       # K/32 not a multiple of 4: 2 lanes per row
    (2, 3840, 256, 16, 4, 3, 54),     # the largest K: pieces streamed in chunks
]
# every non-NaN e4m3 block scale (both signs, subnormals, 448) / signed, subnormal and zero fp16 scales
FFN_CASES_FULL = [(1, 2048, 768, 256, 6, 5, 55), (2, 2048, 768, 256, 6, 5, 56), (1, 192, 320, 8, 3, 9, 57),
                  (3, 2048, 768, 256, 6, 5, 58), (3, 192, 320, 8, 3, 9, 59)]
FFN_CASES = FFN_CASES + [(3, 2048, 768, 256, 6, 5, 60), (3, 256, 128, 32, 6, 4, 61),
                         # a dense FFN layer as the one-expert call (inter 3840 assumed; the pages give none)
                         (1, 2048, 3840, 1, 1, 4, 62), (2, 2048, 3840, 1, 1, 8, 63),
                         # BF16 weights (the 16-bit checkpoint)
                         (4, 2048, 768, 256, 6, 5, 64), (4, 192, 320, 8, 3, 9, 65)]


@pytest.mark.parametrize("fmt,H,I,E,k,T,seed,scales", [c + ("narrow",) for c in FFN_CASES] +
                         [c + ("full",) for c in FFN_CASES_FULL])
def test_grouped_ffn_gemv(fmt, H, I, E, k, T, seed, scales):
    print("grouped_ffn", fmt, H, I, E, k, T, seed, scales, flush=True)
    layer = synth.make_layer(fmt, H, I, E, k, seed, DEV, scale_range=scales)
    x = synth.make_tokens(T, H, seed, DEV)
    lg = synth.uniform_logits(T, E, seed, "cpu").numpy()
    ids = oracle.topk_select(lg.astype(np.float64), k)
    counts, offsets, sp, pp = oracle.permute(ids, E)
    n = T * k
    out = torch.empty((n, H), dtype=torch.float32, device=DEV)
    nws = moe.moe_grouped_ffn_workspace_size(E, H, I, n, moe.MOE_MODE_GEMV)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    d_off = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    d_sp = torch.from_numpy(sp.astype(np.int32)).to(DEV)
    moe.moe_grouped_w4a16_ffn(layer["experts"], E, H, I, x, d_sp, k, d_off, n, out, moe.MOE_MODE_GEMV, ws, nws)
    # the shared expert as E = 1, rows = tokens
    out_s = torch.empty((T, H), dtype=torch.float32, device=DEV)
    d_off_s = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    nws_s = moe.moe_grouped_ffn_workspace_size(1, H, I, T, moe.MOE_MODE_GEMV)
    ws_s = torch.empty(nws_s, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_w4a16_ffn(layer["shared"], 1, H, I, x, None, 1, d_off_s, T, out_s, moe.MOE_MODE_GEMV, ws_s,
                              nws_s)
    sync()
    host = synth.layer_to_numpy(layer, experts=set(ids.ravel().tolist()))
    xb = bits_of(x)
    ref = oracle.grouped_ffn(host["experts"], xb, offsets, sp, k)
    ref_s = oracle.grouped_ffn(host["shared"], xb, np.array([0, T]))
    assert normwise_err(out.cpu().numpy(), ref) <= TOL_EXPERT
    assert normwise_err(out_s.cpu().numpy(), ref_s) <= TOL_EXPERT


# ------------------------------------------------------------------ dense GEMV (output head)

DENSE_CASES = [
    # fmt, rows, cols, T, seed, scales, sampled: the 4-bit head over the 150,144-token vocabulary
    # (not a multiple of 256 rows): up to 7 tokens on the vector units, from 8 NVFP4 tokens on
    # the matrix cores (the last 256-column slice partial), INT4 in two batches of at most 8
    # tokens; other shapes take the runtime-shape kernel, or the matrix cores (NVFP4, from 8
    # tokens, cols a multiple of 256 up to 2048)
    (1, 150144, 2048, 1, 70, "narrow", True),
    (1, 150144, 2048, 5, 71, "full", True),
    (2, 150144, 2048, 11, 72, "narrow", True),
    (3, 150144, 2048, 2, 73, "full", True),
    (1, 1000, 3840, 3, 74, "narrow", False),
    (2, 777, 192, 9, 75, "full", False),
    (3, 33, 256, 1, 76, "narrow", False),
    (1, 100, 256, 9, 77, "full", False),
    (1, 600, 1024, 70, 78, "narrow", False),
    (1, 150144, 2048, 8, 79, "narrow", True),
]


@pytest.mark.parametrize("fmt,rows,cols,T,seed,scales,sampled", DENSE_CASES)
def test_dense_gemv(fmt, rows, cols, T, seed, scales, sampled):
    """Dense 4-bit GEMV against the oracle: every output within an fp32
    dot-product bound (2^-14 of sum |w x|) of the float64 value, on sampled
    rows at the head shape, on every row otherwise."""
    print("dense", fmt, rows, cols, T, seed, scales, flush=True)
    mat = synth.make_matrix(fmt, 2, rows, cols, seed, DEV, scale_range=scales)
    x = synth.make_tokens(T, cols, seed, DEV)
    out = torch.empty((T, rows), dtype=torch.float32, device=DEV)
    moe.moe_dense_w4a16_gemv(mat, 1, x, T, out)
    sync()
    rng = np.random.default_rng(seed)
    sel = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, 600, replace=False)])) if sampled \
        else np.arange(rows)
    host = synth.matrix_to_numpy(mat, experts={1})
    xb = bits_of(x)
    ref = oracle.dense_gemv(host, 1, xb, rows=sel)
    absw = np.abs(oracle.dequant_matrix(host, 1, sel))
    bound = 2.0 ** -14 * (np.abs(oracle.bf16_bits_to_f64(xb)) @ absw.T)
    got = out.cpu().numpy()[:, sel].astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    assert normwise_err(got, ref) <= 1e-5


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("T,k,H,shared,res", [(1, 6, 2048, True, False), (33, 6, 256, True, True),
                                             (7, 1, 64, False, True), (64, 8, 2048, False, False)])
def test_combine(T, k, H, shared, res):
    print("combine", T, k, H, shared, res, flush=True)
    g = torch.Generator().manual_seed(T * k + H)
    o = torch.randn((T * k, H), generator=g)
    perm = torch.randperm(T * k, generator=g)
    w = torch.softmax(torch.randn((T, k), generator=g), dim=1)
    osh = torch.randn((T, H), generator=g) if shared else None
    r = torch.randn((T, H), generator=g).to(torch.bfloat16) if res else None
    y = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    yf = torch.empty((T, H), dtype=torch.float32, device=DEV)
    d = lambda t: None if t is None else t.to(DEV)
    moe.moe_combine(d(o), d(perm.to(torch.int32)), d(w), d(osh), d(r), T, k, H, y, yf)
    sync()
    o_pairs = o.numpy().astype(np.float64)[perm.numpy()].reshape(T, k, H)
    ref = oracle.combine(o_pairs, w.numpy(), None if osh is None else osh.numpy().astype(np.float64),
                         None if r is None else bits_of(r))
    assert normwise_err(yf.cpu().numpy(), ref) <= 1e-6
    yb = oracle.bf16_bits_to_f64(bits_of(y))
    _, e = np.frexp(ref)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    assert np.all(np.abs(yb - ref) <= ulp)


# ------------------------------------------------------------------ whole layer

def run_layer(layer, x, residual, T):
    y = torch.empty_like(x)
    ids = torch.empty((T, layer["k"]), dtype=torch.int32, device=DEV)
    w = torch.empty((T, layer["k"]), dtype=torch.float32, device=DEV)
    L = moe.Layer(layer)
    nws = moe.moe_layer_decode_workspace_size(L, T)
    ws = torch.zeros(nws, dtype=torch.uint8, device=DEV)
    moe.moe_layer_decode(L, x, residual, T, y, ids, w, ws, nws)
    moe.moe_layer_decode(L, x, residual, T, y, ids, w, ws, nws)   # the workspace is reusable as left
    sync()
    H = layer["H"]
    nsync = 16 * (17 + (H + 31) // 32)   # ticket words at the start of the workspace
    tickets = ws[:4 * nsync].view(torch.int32).cpu().numpy()
    assert not tickets.any(), np.nonzero(tickets)   # every ticket counter left reset for the next call
    return y, ids, w, ws


def check_layer(layer, x, residual, y, ids, w, tokens=None, ws=None):
    """Ids bit-exact off near-ties, weights, the graded normwise bound, the
    elementwise diagnostic (every element within one bf16 ulp plus 2^-8 of
    its token's rms), and, on the fused path (T <= 64, ws given), the
    per-stage checks through the kernel's own h."""
    T = x.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    xb = bits_of(x)
    rb = None if residual is None else bits_of(residual)
    wr = layer["w_router"].cpu().numpy()
    ref_lg, ref_ids, _ = oracle.route(xb[tokens], wr, layer["k"])
    host = synth.layer_to_numpy(layer, experts=set(ref_ids.ravel().tolist()))
    ref = oracle.moe_layer(host, xb, residual_bits=rb, tokens=tokens)
    gids = ids.cpu().numpy()[tokens]
    ties = near_tie_tokens(xb[tokens], wr, layer["k"])
    assert ties.sum() <= 2, "too many near-tie tokens"
    ok = ~ties
    assert np.array_equal(gids[ok], ref["ids"][ok])
    assert np.allclose(w.cpu().numpy()[tokens][ok], ref["w"][ok], rtol=1e-5, atol=1e-7)
    yb = bits_of(y)[tokens]
    err = normwise_err(oracle.bf16_bits_to_f64(yb[ok]), ref["y"][ok])
    diag = y_diagnostics(yb[ok], ref["y"][ok])
    print("  normwise err %.3e  elementwise-diag frac %.2e  near-ties %d" % (err, diag, int(ties.sum())),
          flush=True)
    assert err <= TOL_LAYER
    assert diag == 0.0, "elementwise diagnostic: %.2e of the outputs outside ulp + 2^-8 rms" % diag
    if ws is not None and T <= 64:
        frac, cnt = check_decode_stages(layer, x, residual, y, ids, w, ws, tokens=tokens)
        print("  stages ok: h flips %.2e of %d" % (frac, cnt), flush=True)
    return err


LAYER_CASES = [
    # name, fmt, H, I, E, k, T, seed, residual
    ("tiny_int4_T4", 2, 256, 128, 32, 6, 4, 0, False),
    ("tiny_int4_T4_res", 2, 256, 128, 32, 6, 4, 0, True),
    ("flint_nvfp4_T1", 1, 2048, 768, 256, 6, 1, 1, False),
    ("flint_nvfp4_T4", 1, 2048, 768, 256, 6, 4, 6, True),
    ("flint_int4_T4", 2, 2048, 768, 256, 6, 4, 6, False),
    ("flint_nvfp4_T16", 1, 2048, 768, 256, 6, 16, 18, False),
    ("flint_int4_T16", 2, 2048, 768, 256, 6, 16, 18, True),
    ("tiny_nvfp4_T80_composed", 1, 256, 128, 32, 6, 80, 7, True),
    ("one_expert_k1", 1, 256, 128, 1, 1, 9, 8, False),
    ("k8_E16", 2, 256, 192, 16, 8, 13, 9, True),
    ("ragged_H192_I320", 1, 192, 320, 8, 3, 9, 10, True),
    ("flint_int4_T1", 2, 2048, 768, 256, 6, 1, 12, True),
    ("tiny_nvfp4_T1_k8", 1, 256, 128, 16, 8, 1, 13, True),
    ("tiny_int4_T1_k8", 2, 256, 128, 16, 8, 1, 14, False),
    # one token, 7 units of 18 rows per down block: the last block is partial
    ("ragged_H192_I320_T1", 1, 192, 320, 8, 6, 1, 15, True),
    ("ragged_int4_H192_I320_T1", 2, 192, 320, 8, 6, 1, 16, False),
    # more than 256 experts: the selection by wave maxima (one token: by the
    # whole block), grouping over up to 1024 experts, the largest k and T
    ("wide_E1024_k8_T1", 1, 256, 128, 1024, 8, 1, 17, True),
    ("wide_int4_E1024_k8_T5", 2, 256, 128, 1024, 8, 5, 19, False),
    ("wide_E300_T64", 1, 256, 128, 300, 6, 64, 20, True),
    ("wide_E1024_k8_T64", 1, 256, 128, 1024, 8, 64, 21, False),
    # the largest supported hidden size (3840 columns)
    ("big_H3840_T1", 1, 3840, 512, 64, 4, 1, 22, True),
    ("big_int4_H3840_T8", 2, 3840, 512, 64, 4, 8, 23, False),
    # INT4 with scale and bias per group of 64
    ("tiny_int4sb_T4", 3, 256, 128, 32, 6, 4, 24, True),
    ("flint_int4sb_T1", 3, 2048, 768, 256, 6, 1, 25, True),
    ("flint_int4sb_T4", 3, 2048, 768, 256, 6, 4, 26, False),
    ("flint_int4sb_T16", 3, 2048, 768, 256, 6, 16, 27, True),
    ("ragged_int4sb_H192_I320_T1", 3, 192, 320, 8, 6, 1, 28, False),
    # BF16 weights
    ("flint_bf16_T1", 4, 2048, 768, 256, 6, 1, 29, True),
    # several tokens on bf16 weights take the composed kernels (the fused
    # several-token kernels in this format are switched off after a memory
    # fault in a timed run whose cause is not found)
    ("flint_bf16_T4", 4, 2048, 768, 256, 6, 4, 30, False),
    ("flint_bf16_T16", 4, 2048, 768, 256, 6, 16, 31, True),
    ("tiny_bf16_T64", 4, 256, 128, 32, 6, 64, 32, False),
    ("ragged_bf16_H192_I320_T1", 4, 192, 320, 8, 6, 1, 33, True),
    # 2 to 4 tokens: each gate/up block groups the pairs itself (one-token
    # router batches), up to 1024 experts and k = 8
    ("wide_E1024_k8_T4", 1, 256, 128, 1024, 8, 4, 34, True),
    ("tiny_nvfp4_T3", 1, 256, 128, 32, 6, 3, 35, False),
    ("ragged_int4_H192_I320_T2", 2, 192, 320, 8, 6, 2, 36, True),
    # 2 to 4 tokens at the Flint shape: the down launch that combines in LDS
    ("flint_nvfp4_T2", 1, 2048, 768, 256, 6, 2, 37, True),
    ("flint_int4_T3", 2, 2048, 768, 256, 6, 3, 38, False),
    ("flint_int4sb_T2_k8", 3, 2048, 768, 256, 8, 2, 39, True),
    # 8 tokens with k = 8: 64 pairs, one per lane of the grouping wave
    ("wide_E1024_k8_T8", 1, 256, 128, 1024, 8, 8, 40, True),
    ("flint_int4sb_T8_k8", 3, 2048, 768, 256, 8, 8, 41, False),
]


@pytest.mark.parametrize("shared,I_shared,T", [(False, None, 1), (False, None, 4), (True, 256, 1), (True, 256, 5)])
def test_layer_decode_shared_variants(shared, I_shared, T):
    """No shared expert, or a shared expert wider than the routed ones (the
    single-token down kernel needs equal widths and the layer falls back)."""
    print("shared variants", shared, I_shared, T, flush=True)
    layer = synth.make_layer(1, 256, 128, 32, 6, 40 + T, DEV, shared=shared, I_shared=I_shared)
    x = synth.make_tokens(T, 256, 40 + T, DEV)
    y, ids, w, ws = run_layer(layer, x, x, T)
    check_layer(layer, x, x, y, ids, w, ws=ws)


@pytest.mark.parametrize("name,fmt,H,I,E,k,T,seed,res", LAYER_CASES)
def test_layer_decode(name, fmt, H, I, E, k, T, seed, res):
    print("layer", name, flush=True)
    layer = synth.make_layer(fmt, H, I, E, k, seed, DEV)
    x = synth.make_tokens(T, H, seed, DEV)
    residual = synth.make_tokens(T, H, seed + 1000, DEV) if res else None
    y, ids, w, ws = run_layer(layer, x, residual, T)
    check_layer(layer, x, residual, y, ids, w, ws=ws)


@pytest.mark.parametrize("fmt", [1, 2])
def test_layer_decode_T64_sampled(fmt):
    print("layer T64 sampled", fmt, flush=True)
    layer = synth.make_layer(fmt, 2048, 768, 256, 6, 66, DEV)
    x = synth.make_tokens(64, 2048, 66, DEV)
    y, ids, w, ws = run_layer(layer, x, x, 64)
    check_layer(layer, x, x, y, ids, w, tokens=[0, 17, 31, 40, 63], ws=ws)


@pytest.mark.parametrize("fmt,T", [(1, 1), (2, 1), (2, 4), (1, 16), (2, 16), (3, 1), (3, 16)])
def test_layer_decode_full_scale_range(fmt, T):
    """Flint-shaped layer whose block scales cover the whole format: every
    non-NaN e4m3 code (both signs, subnormals, up to 448) for NVFP4; signed,
    subnormal and zero fp16 scales for INT4."""
    print("layer full scales", fmt, T, flush=True)
    layer = synth.make_layer(fmt, 2048, 768, 256, 6, 200 + T, DEV, scale_range="full")
    x = synth.make_tokens(T, 2048, 200 + T, DEV)
    y, ids, w, ws = run_layer(layer, x, x, T)
    check_layer(layer, x, x, y, ids, w, ws=ws)


@pytest.mark.parametrize("fmt,T", [(1, 1), (2, 1), (1, 4), (2, 16), (1, 64)])
def test_workspace_reuse_with_new_routing(fmt, T):
    """A call on one workspace after a differently routed call gives the
    bits of a call on a fresh zeroed workspace (the blocks that take the
    last ticket must see this call's logits, ids, weights and outputs, not
    the previous call's)."""
    print("workspace reuse", fmt, T, flush=True)
    H, I, E, k = 2048, 768, 256, 6
    layer = synth.make_layer(fmt, H, I, E, k, 230 + T, DEV)
    x1 = synth.make_tokens(T, H, 231 + T, DEV)
    x2 = synth.make_tokens(T, H, 232 + T, DEV)
    L = moe.Layer(layer)
    nws = moe.moe_layer_decode_workspace_size(L, T)
    outs = []
    for fresh in (False, True):
        ws = torch.zeros(nws, dtype=torch.uint8, device=DEV)
        y = torch.empty_like(x2)
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        if not fresh:
            moe.moe_layer_decode(L, x1, x1, T, y, ids, w, ws, nws)
            sync()
            ids1 = ids.clone()
        moe.moe_layer_decode(L, x2, x2, T, y, ids, w, ws, nws)
        sync()
        outs.append((y, ids, w))
    assert not torch.equal(ids1, outs[0][1]), "the two inputs should route differently"
    (ya, ia, wa), (yb, ib, wb) = outs
    assert torch.equal(ia, ib) and torch.equal(wa, wb)
    assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


@pytest.mark.parametrize("fmt", [1, 2])
def test_chain_teacher_forced(fmt):
    """Three chained Flint-shaped layers at batch 8: x_l = rms_norm(r_l),
    r_{l+1} = layer_l(x_l, residual r_l).  Each step is checked against the
    oracle on the GPU's own inputs to that step (teacher forcing): the
    normalisation within one bf16 ulp, the layer with the layer checks."""
    print("chain", fmt, flush=True)
    H, I, E, k, T, NL, eps = 2048, 768, 256, 6, 8, 3, 1e-6
    r = synth.make_tokens(T, H, 4, DEV)
    prev_ids = None
    for l in range(NL):
        layer = synth.make_layer(fmt, H, I, E, k, synth.seed_of(4, l), DEV)
        x = torch.empty_like(r)
        moe.moe_rms_norm(r, T, H, eps, x)
        sync()
        rb = bits_of(r)
        rv = oracle.bf16_bits_to_f64(rb)
        exact = rv / np.sqrt(np.mean(rv * rv, axis=1, keepdims=True) + eps)
        xg = oracle.bf16_bits_to_f64(bits_of(x))
        assert np.all(np.abs(xg - exact) <= ulp_bf16(exact)), "layer %d: norm off by more than one ulp" % l
        flips = np.mean(bits_of(x) != oracle.rms_norm(rb, eps))
        assert flips <= 5e-3, flips
        y, ids, w, ws = run_layer(layer, x, r, T)
        print("  layer %d" % l, flush=True)
        check_layer(layer, x, r, y, ids, w, ws=ws)
        prev_ids = ids
        r = y
    assert prev_ids is not None


@pytest.mark.parametrize("fmt,T,NL,shape", [(1, 8, 3, "flint"), (2, 8, 2, "flint"), (1, 1, 2, "flint"),
                                            (1, 16, 2, "flint"), (2, 64, 2, "flint"), (1, 70, 2, "flint"),
                                            (2, 5, 2, "small"), (3, 16, 2, "flint"), (4, 1, 2, "small"),
                                            (4, 6, 2, "small")])
def test_decode_step_matches_calls_and_oracle(fmt, T, NL, shape):
    """moe_decode_step (one call for NL chained layers; each layer's first
    launch normalises its tokens itself, above 64 tokens the norm kernel
    does) equals the same moe_rms_norm + moe_layer_decode calls bit for bit,
    and every layer of it, fed the GPU's own residual (teacher forcing),
    passes the layer checks."""
    print("decode step", fmt, T, NL, shape, flush=True)
    H, I, E, k, eps = (2048, 768, 256, 6, 1e-6) if shape == "flint" else (256, 192, 16, 4, 1e-5)
    layers = [synth.make_layer(fmt, H, I, E, k, synth.seed_of(40, l), DEV) for l in range(NL)]
    ll = moe.LayerList(layers)
    r0 = synth.make_tokens(T, H, 41, DEV)
    nws = moe.moe_decode_step_workspace_size(ll, T, with_r_all=True)
    ws = torch.zeros(nws, dtype=torch.uint8, device=DEV)
    r_out = torch.empty_like(r0)
    r_all = torch.empty((NL, T, H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((NL, T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((NL, T, k), dtype=torch.float32, device=DEV)
    moe.moe_decode_step(ll, r0, T, eps, r_out, r_all, ids, w, ws, nws)
    # the same chain through the separate calls
    r = r0
    nws1 = moe.moe_layer_decode_workspace_size(ll.layers[0], T)
    ws1 = torch.zeros(nws1, dtype=torch.uint8, device=DEV)
    xs = []
    for l in range(NL):
        x = torch.empty_like(r)
        moe.moe_rms_norm(r, T, H, eps, x)
        y = torch.empty_like(r)
        moe.moe_layer_decode(ll.layers[l], x, r, T, y, None, None, ws1, nws1)
        xs.append(x)
        r = y
    sync()
    assert torch.equal(r.view(torch.int16), r_out.view(torch.int16))
    assert torch.equal(r_all[NL - 1].view(torch.int16), r_out.view(torch.int16))
    # teacher forcing: layer l on the GPU's r_l
    r = r0
    for l in range(NL):
        check_layer(layers[l], xs[l], r, r_all[l], ids[l], w[l], tokens=None if T <= 16 else [0, T // 3, T - 1])
        r = r_all[l]
    # a step without r_all gives the same result
    nws2 = moe.moe_decode_step_workspace_size(ll, T)
    ws2 = torch.zeros(nws2, dtype=torch.uint8, device=DEV)
    r_out2 = torch.empty_like(r0)
    moe.moe_decode_step(ll, r0, T, eps, r_out2, None, None, None, ws2, nws2)
    sync()
    assert torch.equal(r_out2.view(torch.int16), r_out.view(torch.int16))


def test_rms_norm_in_place_and_ranges():
    """The normalisation kernel in place (x == r), on rows of very
    different scales, against the oracle within one bf16 ulp."""
    print("rms norm", flush=True)
    T, H, eps = 37, 3840, 1e-5
    g = torch.Generator().manual_seed(12)
    r = (torch.randn((T, H), generator=g) * torch.exp2(torch.randint(-30, 30, (T, 1), generator=g).float()))
    r = r.to(torch.bfloat16).to(DEV)
    rb = bits_of(r)
    moe.moe_rms_norm(r, T, H, eps, r)
    sync()
    rv = oracle.bf16_bits_to_f64(rb)
    exact = rv / np.sqrt(np.mean(rv * rv, axis=1, keepdims=True) + eps)
    xg = oracle.bf16_bits_to_f64(bits_of(r))
    assert np.all(np.abs(xg - exact) <= ulp_bf16(exact))
    assert np.mean(bits_of(r) != oracle.rms_norm(rb, eps)) <= 5e-3


@pytest.mark.parametrize("T,E", [(1, 256), (7, 256), (64, 1024), (300, 256)])
def test_route_without_logits_buffer(T, E):
    """moe_route with logits_out NULL: the same ids and weights as with a
    logits buffer below 256 tokens (the same fp32 logits), and ids equal to
    the oracle's off near-ties at any size."""
    print("route no logits", T, E, flush=True)
    H, k = 2048, 6
    layer = synth.make_layer(1, H, 128, E, k, seed=60 + T, device=DEV, shared=False)
    x = synth.make_tokens(T, H, 60 + T, DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids_a = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w_a = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ids_b = torch.empty_like(ids_a)
    w_b = torch.empty_like(w_a)
    moe.moe_route(x, layer["w_router"], T, H, E, k, lg, ids_a, w_a)
    moe.moe_route(x, layer["w_router"], T, H, E, k, None, ids_b, w_b)
    sync()
    if T < 256:
        assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b)
    xb = bits_of(x)
    wr = layer["w_router"].cpu().numpy()
    _, ref_ids, ref_w = oracle.route(xb, wr, k)
    ties = near_tie_tokens(xb, wr, k)
    gids = ids_b.cpu().numpy()
    assert np.array_equal(gids[~ties], ref_ids[~ties])
    assert np.allclose(w_b.cpu().numpy()[~ties], ref_w[~ties], rtol=1e-5, atol=1e-7)


def test_layer_decode_deterministic_and_token_independent():
    print("determinism", flush=True)
    layer = synth.make_layer(1, 2048, 768, 256, 6, 70, DEV)
    x = synth.make_tokens(8, 2048, 70, DEV)
    y1, i1, _, _ = run_layer(layer, x, None, 8)
    y2, i2, _, _ = run_layer(layer, x, None, 8)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and torch.equal(i1, i2)
    # a single token alone gives the same routing and an output within tolerance
    y3, i3, _, _ = run_layer(layer, x[3:4].contiguous(), None, 1)
    assert torch.equal(i3[0], i1[3])
    a = y3[0].float().cpu().numpy().astype(np.float64)
    b = y1[3].float().cpu().numpy().astype(np.float64)
    assert np.linalg.norm(a - b) <= 1e-3 * np.linalg.norm(b)


@pytest.mark.parametrize("fmt,T", [(1, 2), (1, 6), (2, 16), (1, 64)])
def test_composed_calls_match_fused_layer(fmt, T):
    """route -> permute -> grouped FFN (routed, shared; GEMV mode) -> combine
    equals moe_layer_decode bit for bit for 2 <= T <= 64."""
    print("composed vs fused", fmt, T, flush=True)
    H, I, E, k = 2048, 768, 256, 6
    layer = synth.make_layer(fmt, H, I, E, k, 80 + T, DEV)
    x = synth.make_tokens(T, H, 80 + T, DEV)
    yf, idf, wf, _ = run_layer(layer, x, x, T)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_route(x, layer["w_router"], T, H, E, k, lg, ids, w)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=DEV)
    pp = torch.empty(T * k, dtype=torch.int32, device=DEV)
    nws = moe.moe_permute_workspace_size(T, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_permute(ids, T, k, E, counts, offsets, sp, pp, None, None, 0, ws, nws)
    out = torch.empty((T * k, H), dtype=torch.float32, device=DEV)
    nws = moe.moe_grouped_ffn_workspace_size(E, H, I, T * k)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_w4a16_ffn(layer["experts"], E, H, I, x, sp, k, offsets, T * k, out, moe.MOE_MODE_GEMV, ws, nws)
    out_s = torch.empty((T, H), dtype=torch.float32, device=DEV)
    off_s = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    nws = moe.moe_grouped_ffn_workspace_size(1, H, I, T)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_w4a16_ffn(layer["shared"], 1, H, I, x, None, 1, off_s, T, out_s, moe.MOE_MODE_GEMV, ws, nws)
    y = torch.empty_like(x)
    moe.moe_combine(out, pp, w, out_s, x, T, k, H, y)
    sync()
    assert torch.equal(ids, idf) and torch.equal(w, wf)
    assert torch.equal(y.view(torch.int16), yf.view(torch.int16))


@pytest.mark.parametrize("fmt,T", [(2, 4), (1, 1), (1, 16)])
def test_layer_decode_graph_capture_replays(fmt, T):
    """Replays of a captured layer call (the one-token path has its own down
    launch; 16 tokens use several router batches) equal the eager call."""
    print("graph capture", fmt, T, flush=True)
    H, I, E, k = 2048, 768, 256, 6
    layer = synth.make_layer(fmt, H, I, E, k, 90 + T, DEV)
    x = synth.make_tokens(T, H, 90, DEV)
    L = moe.Layer(layer)
    nws = moe.moe_layer_decode_workspace_size(L, T)
    ws = torch.zeros(nws, dtype=torch.uint8, device=DEV)
    y_eager = torch.empty_like(x)
    moe.moe_layer_decode(L, x, x, T, y_eager, None, None, ws, nws)
    sync()
    y = torch.empty_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.moe_layer_decode(L, x, x, T, y, None, None, ws, nws, stream=s)   # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_layer_decode(L, x, x, T, y, None, None, ws, nws, stream=s)
    for rep in range(4):
        y.zero_()
        junk = torch.randn(1000, device=DEV).sum()   # unrelated eager work between replays
        g.replay()
        sync()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), rep
        del junk


# ------------------------------------------------------------------ MFMA grouped FFN (prefill / large batch)

MFMA_CASES = [
    # fmt, H, I, E, k, T, seed, routing
    (2, 256, 128, 32, 6, 64, 100, "uniform"),
    (1, 256, 192, 8, 3, 300, 101, "zipf"),       # several 128-row tiles per expert, ragged tails
    (1, 256, 384, 16, 4, 200, 104, "zipf"),      # LDS-staged 128-row tiles with 64-row remainders
    (1, 2048, 768, 256, 6, 512, 102, "zipf"),
    (2, 2048, 768, 256, 6, 512, 103, "zipf"),
    # K above 2048 and I not a multiple of 128: the LDS-staged 128-row tile kernels, both formats
    (2, 3840, 256, 16, 4, 300, 105, "zipf"),
    (1, 3840, 512, 8, 2, 200, 106, "uniform"),
    (2, 256, 192, 8, 3, 300, 107, "zipf"),
    # 1024 experts, k = 8: the tile table's widest scan, most experts with one or no tile
    (1, 256, 128, 1024, 8, 300, 108, "uniform"),
]


MFMA_CASES_FULL = [
    (1, 2048, 768, 256, 6, 512, 109, "zipf"),
    (2, 2048, 768, 256, 6, 512, 110, "zipf"),
    (1, 256, 192, 8, 3, 300, 111, "uniform"),
]


def routed_rows(T, E, k, seed, routing):
    lg = (synth.zipf_logits(T, E, 1.1, seed, "cpu") if routing == "zipf" else synth.uniform_logits(T, E, seed, "cpu"))
    ids = oracle.topk_select(lg.numpy().astype(np.float64), k)
    return ids, oracle.permute(ids, E)


@pytest.mark.parametrize("fmt,H,I,E,k,T,seed,routing,scales", [c + ("narrow",) for c in MFMA_CASES] +
                         [c + ("full",) for c in MFMA_CASES_FULL])
def test_grouped_ffn_mfma(fmt, H, I, E, k, T, seed, routing, scales):
    """Matrix-core grouped FFN against the oracle: every row at the Flint
    shape (hidden 2048), sampled rows elsewhere; and against the GEMV path
    everywhere."""
    print("grouped_ffn mfma", fmt, H, I, E, k, T, seed, routing, scales, flush=True)
    layer = synth.make_layer(fmt, H, I, E, k, seed, DEV, scale_range=scales)
    x = synth.make_tokens(T, H, seed, DEV)
    ids, (counts, offsets, sp, pp) = routed_rows(T, E, k, seed, routing)
    n = T * k
    d_off = torch.from_numpy(offsets.astype(np.int32)).to(DEV)
    d_sp = torch.from_numpy(sp.astype(np.int32)).to(DEV)
    outs = {}
    for mode in (moe.MOE_MODE_MFMA, moe.MOE_MODE_GEMV):
        out = torch.empty((n, H), dtype=torch.float32, device=DEV)
        nws = moe.moe_grouped_ffn_workspace_size(E, H, I, n, mode)
        ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
        moe.moe_grouped_w4a16_ffn(layer["experts"], E, H, I, x, d_sp, k, d_off, n, out, mode, ws, nws)
        outs[mode] = out
    out_s = torch.empty((T, H), dtype=torch.float32, device=DEV)
    d_off_s = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    nws = moe.moe_grouped_ffn_workspace_size(1, H, I, T, moe.MOE_MODE_MFMA)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_w4a16_ffn(layer["shared"], 1, H, I, x, None, 1, d_off_s, T, out_s, moe.MOE_MODE_MFMA, ws, nws)
    sync()
    xb = bits_of(x)
    if H == 2048:
        # every row of the Flint-shaped case against the oracle
        host = synth.layer_to_numpy(layer, experts=set(ids.ravel().tolist()))
        ref = oracle.grouped_ffn(host["experts"], xb, offsets, sp, k)
        assert normwise_err(outs[moe.MOE_MODE_MFMA].cpu().numpy(), ref) <= TOL_EXPERT
    else:
        # sampled rows: the first and last rows of the three largest experts, and a spread of others
        big = np.argsort(-counts, kind="stable")[:3]
        rows = set()
        for e in big:
            rows |= {int(offsets[e]), int(offsets[e + 1]) - 1, int((offsets[e] + offsets[e + 1]) // 2)}
        rows |= set(np.linspace(0, n - 1, 24).astype(int).tolist())
        rows = np.array(sorted(rows))
        experts = set(int(np.searchsorted(offsets, r, side="right") - 1) for r in rows)
        host = synth.layer_to_numpy(layer, experts=experts)
        ref = np.zeros((len(rows), H))
        for i, r in enumerate(rows):
            e = int(np.searchsorted(offsets, r, side="right") - 1)
            ref[i] = oracle.expert_ffn(host["experts"], e, oracle.bf16_bits_to_f64(xb[[sp[r] // k]]))[0]
        got = outs[moe.MOE_MODE_MFMA].cpu().numpy()[rows]
        assert normwise_err(got, ref) <= TOL_EXPERT
    # MFMA and GEMV agree everywhere: each is within TOL_EXPERT of the exact
    # result (their h roundings flip independently), so within twice that
    assert normwise_err(outs[moe.MOE_MODE_MFMA].cpu().numpy(), outs[moe.MOE_MODE_GEMV].cpu().numpy()) <= 2 * TOL_EXPERT
    srows = np.arange(T) if H == 2048 else np.unique(np.linspace(0, T - 1, 12).astype(int))
    ref_s = oracle.expert_ffn(host["shared"], 0, oracle.bf16_bits_to_f64(xb[srows]))
    assert normwise_err(out_s.cpu().numpy()[srows], ref_s) <= TOL_EXPERT


def test_prefill_4096_zipf_sampled():
    """Flint-shaped prefill: 4096 tokens, Zipf(1.1) routing, NVFP4, composed
    route -> top-k on skewed logits -> permute -> MFMA grouped FFN (routed and
    shared) -> combine; sampled tokens against the oracle."""
    print("prefill 4096", flush=True)
    H, I, E, k, T = 2048, 768, 256, 6, 4096
    layer = synth.make_layer(1, H, I, E, k, 5, DEV)
    x = synth.make_tokens(T, H, 5, DEV)
    lg = synth.zipf_logits(T, E, 1.1, 5, DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    moe.moe_topk_softmax(lg, T, E, k, ids, w)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sp = torch.empty(T * k, dtype=torch.int32, device=DEV)
    pp = torch.empty(T * k, dtype=torch.int32, device=DEV)
    nws = moe.moe_permute_workspace_size(T, k, E)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_permute(ids, T, k, E, counts, offsets, sp, pp, None, None, 0, ws, nws)
    out = torch.empty((T * k, H), dtype=torch.float32, device=DEV)
    nws = moe.moe_grouped_ffn_workspace_size(E, H, I, T * k)
    ws = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_w4a16_ffn(layer["experts"], E, H, I, x, sp, k, offsets, T * k, out, moe.MOE_MODE_AUTO, ws, nws)
    out_s = torch.empty((T, H), dtype=torch.float32, device=DEV)
    off_s = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    nws = moe.moe_grouped_ffn_workspace_size(1, H, I, T)
    ws2 = torch.empty(nws, dtype=torch.uint8, device=DEV)
    moe.moe_grouped_w4a16_ffn(layer["shared"], 1, H, I, x, None, 1, off_s, T, out_s, moe.MOE_MODE_AUTO, ws2, nws)
    y = torch.empty_like(x)
    moe.moe_combine(out, pp, w, out_s, x, T, k, H, y)
    sync()
    # routing of the skewed logits: bit-exact ids for every token
    lg_np = lg.cpu().numpy()
    ref_ids = oracle.topk_select(lg_np.astype(np.float64), k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    c = counts.cpu().numpy()
    assert c.max() > 1000 and c.min() >= 1          # the skew the workload asks for
    tokens = np.unique(np.concatenate([np.linspace(0, T - 1, 10).astype(int), [1, 2, T - 2]]))
    host = synth.layer_to_numpy(layer, experts=set(ref_ids[tokens].ravel().tolist()))
    ref = oracle.moe_layer(host, bits_of(x), residual_bits=bits_of(x), logits=lg_np, tokens=tokens)
    err = normwise_err(oracle.bf16_bits_to_f64(bits_of(y)[tokens]), ref["y"])
    print("  prefill sampled normwise err %.3e" % err, flush=True)
    assert err <= TOL_LAYER


@pytest.mark.parametrize("fmt,T", [(2, 200), (1, 70), (1, 100), (3, 100), (4, 100)])
def test_layer_decode_large_batch_uses_grouped_gemm(fmt, T):
    """Above 64 tokens the layer is composed from the separate calls; 70 tokens
    (420 pairs, under two per expert) take the GEMV grouped FFN, 100 and 200
    the matrix-core one."""
    print("layer composed", fmt, T, flush=True)
    layer = synth.make_layer(fmt, 2048, 768, 256, 6, 110 + T, DEV)
    x = synth.make_tokens(T, 2048, 110 + T, DEV)
    y, ids, w, ws = run_layer(layer, x, x, T)
    check_layer(layer, x, x, y, ids, w, tokens=[0, T // 3, (2 * T) // 3, T - 1], ws=ws)
