"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (CPU only: no compute calls)."""

import ctypes
import os
import re

import pytest

import bit_weight_only_moe_amd as moe


def declared_functions(repo_root):
    src = open(os.path.join(repo_root, "include", "moe_w4a16.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(repo_root):
    names = declared_functions(repo_root)
    assert len(names) >= 12
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(moe.EXPORTED)


def test_abi_version_matches_header(repo_root):
    src = open(os.path.join(repo_root, "include", "moe_w4a16.h")).read()
    v = int(re.search(r"#define MOE_ABI_VERSION (\d+)", src).group(1))
    assert moe.moe_abi_version() == v


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced (validation fails first)


def fake_matrix(fmt=1, E=4, rows=128, cols=256, codes=FAKE, scales=FAKE):
    return {"fmt": fmt, "num_experts": E, "rows": rows, "cols": cols, "codes": codes, "scales": scales,
            "zeros": FAKE if fmt == 2 else None, "tensor_scale": FAKE if fmt == 1 else None,
            "biases": FAKE if fmt == 3 else None}


def fake_ffn(fmt=1, E=4, H=256, I=128):
    return {"gate": fake_matrix(fmt, E, I, H), "up": fake_matrix(fmt, E, I, H), "down": fake_matrix(fmt, E, H, I)}


def expect(code, fn, *args, **kw):
    with pytest.raises(moe.MoeError) as ei:
        fn(*args, **kw)
    assert ei.value.code == code, str(ei.value)
    return str(ei.value)


def test_route_validation():
    inv, uns = moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED
    expect(inv, moe.moe_route, FAKE, FAKE, -1, 256, 32, 6, FAKE, FAKE, FAKE)
    expect(inv, moe.moe_route, FAKE, FAKE, 4, 256, 32, 9, FAKE, FAKE, FAKE)      # k > 8
    expect(inv, moe.moe_route, FAKE, FAKE, 4, 256, 4, 5, FAKE, FAKE, FAKE)       # k > E
    expect(inv, moe.moe_route, FAKE, FAKE, 4, 256, 32, 0, FAKE, FAKE, FAKE)      # k < 1
    expect(uns, moe.moe_route, FAKE, FAKE, 4, 256, 1025, 6, FAKE, FAKE, FAKE)    # E > 1024
    expect(inv, moe.moe_route, FAKE, FAKE, 4, 200, 32, 6, FAKE, FAKE, FAKE)      # H % 64
    expect(inv, moe.moe_route, None, FAKE, 4, 256, 32, 6, FAKE, FAKE, FAKE)
    expect(inv, moe.moe_route, FAKE + 2, FAKE, 4, 256, 32, 6, FAKE, FAKE, FAKE)  # misaligned
    expect(inv, moe.moe_topk_softmax, None, 4, 32, 6, FAKE, FAKE)
    expect(uns, moe.moe_topk_softmax, FAKE, 4, 2048, 6, FAKE, FAKE)


def test_route_logits_out_is_optional():
    """logits_out may be NULL (the logits then stay on chip); shapes whose
    one-token batch does not fit 64 KB of LDS are rejected on the host."""
    uns = moe.MOE_ERR_UNSUPPORTED
    assert moe.moe_route(FAKE, FAKE, 0, 2048, 256, 6, None, FAKE, FAKE) == 0
    # 2*H + 4*E + 3328 > 65536: H = 30720, E = 1024
    msg = expect(uns, moe.moe_route, FAKE, FAKE, 4, 30720, 1024, 6, None, FAKE, FAKE)
    assert "logits_out" in msg
    # the same shape with a logits buffer is accepted (T = 0: nothing is launched)
    assert moe.moe_route(FAKE, FAKE, 0, 30720, 1024, 6, FAKE, FAKE, FAKE) == 0


def test_zero_tokens_is_a_noop_without_touching_the_gpu():
    assert moe.moe_topk_softmax(FAKE, 0, 32, 6, FAKE, FAKE) == 0
    assert moe.moe_route(FAKE, FAKE, 0, 256, 32, 6, FAKE, FAKE, FAKE) == 0
    assert moe.moe_combine(FAKE, FAKE, FAKE, None, None, 0, 6, 256, FAKE) == 0


def test_permute_validation():
    inv = moe.MOE_ERR_INVALID_ARG
    need = moe.moe_permute_workspace_size(64, 6, 256)
    assert need > 0
    expect(inv, moe.moe_permute, FAKE, 64, 6, 256, FAKE, FAKE, FAKE, FAKE, ws=FAKE, ws_bytes=need - 1)
    expect(inv, moe.moe_permute, FAKE, 64, 6, 256, None, FAKE, FAKE, FAKE, ws=FAKE, ws_bytes=need)
    expect(inv, moe.moe_permute, FAKE, 64, 6, 256, FAKE, FAKE, FAKE, FAKE, x=FAKE, x_perm=None, H=256,
           ws=FAKE, ws_bytes=need)


def test_grouped_ffn_validation():
    inv, uns = moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED
    f = fake_ffn()
    need = moe.moe_grouped_ffn_workspace_size(4, 256, 128, 24)
    expect(inv, moe.moe_grouped_w4a16_ffn, f, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE, ws_bytes=need - 1)
    expect(inv, moe.moe_grouped_w4a16_ffn, f, 4, 256, 192, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE, ws_bytes=need)
    expect(uns, moe.moe_grouped_w4a16_ffn, f, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, mode=7, ws=FAKE,
           ws_bytes=need)
    bad = fake_ffn()
    bad["up"]["fmt"] = 5
    expect(uns, moe.moe_grouped_w4a16_ffn, bad, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE, ws_bytes=need)
    mixed = fake_ffn()
    mixed["down"] = fake_matrix(2, 4, 256, 128)
    expect(inv, moe.moe_grouped_w4a16_ffn, mixed, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE, ws_bytes=need)
    noscale = fake_ffn()
    noscale["gate"]["tensor_scale"] = None
    expect(inv, moe.moe_grouped_w4a16_ffn, noscale, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE,
           ws_bytes=need)
    unaligned = fake_ffn()
    unaligned["down"]["codes"] = FAKE + 8
    expect(inv, moe.moe_grouped_w4a16_ffn, unaligned, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE,
           ws_bytes=need)
    # scale + bias INT4: needs its biases; the matrix-core mode does not take it
    sb = fake_ffn(fmt=3)
    need_sb = moe.moe_grouped_ffn_workspace_size(4, 256, 128, 24, moe.MOE_MODE_MFMA)
    msg = expect(uns, moe.moe_grouped_w4a16_ffn, sb, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, mode=moe.MOE_MODE_MFMA,
                 ws=FAKE, ws_bytes=need_sb)
    assert "scale+bias" in msg
    nob = fake_ffn(fmt=3)
    nob["down"]["biases"] = None
    expect(inv, moe.moe_grouped_w4a16_ffn, nob, 4, 256, 128, FAKE, FAKE, 6, FAKE, 24, FAKE, ws=FAKE, ws_bytes=need)
    # at most 3840 columns per matrix (the header's limit); 3840 itself passes validation
    need_w = moe.moe_grouped_ffn_workspace_size(4, 3904, 128, 24)
    msg = expect(uns, moe.moe_grouped_w4a16_ffn, fake_ffn(H=3904), 4, 3904, 128, FAKE, FAKE, 6, FAKE, 24, FAKE,
                 ws=FAKE, ws_bytes=need_w)
    assert "3840" in msg


def test_layer_decode_validation():
    inv = moe.MOE_ERR_INVALID_ARG
    layer = {"H": 256, "I": 128, "E": 4, "k": 2, "w_router": FAKE, "experts": fake_ffn(), "shared": fake_ffn(E=1)}
    need = moe.moe_layer_decode_workspace_size(layer, 8)
    assert need > 0
    expect(inv, moe.moe_layer_decode, layer, FAKE, None, 8, FAKE, ws=FAKE, ws_bytes=need - 1)
    expect(inv, moe.moe_layer_decode, layer, FAKE, None, 8, FAKE, ws=FAKE + 16, ws_bytes=need)   # not 256-aligned
    expect(inv, moe.moe_layer_decode, layer, FAKE, None, 8, FAKE, ids_out=FAKE, w_out=None, ws=FAKE, ws_bytes=need)
    bad_shared = dict(layer, shared=fake_ffn(fmt=2, E=1))
    expect(inv, moe.moe_layer_decode, bad_shared, FAKE, None, 8, FAKE, ws=FAKE, ws_bytes=need)
    bad_k = dict(layer, k=5)
    expect(inv, moe.moe_layer_decode, bad_k, FAKE, None, 8, FAKE, ws=FAKE, ws_bytes=need)
    assert moe.moe_layer_decode(layer, FAKE, None, 0, FAKE, ws=FAKE, ws_bytes=need) == 0
    assert "workspace" in moe.moe_last_error() or moe.moe_last_error() != ""


def test_layer_decode_noalloc_validation():
    """The static-scratch entry point rejects, on the host, what its array
    cannot hold: more than 64 tokens, or a layer whose workspace exceeds the
    array (before it touches any device)."""
    inv, uns = moe.MOE_ERR_INVALID_ARG, moe.MOE_ERR_UNSUPPORTED
    cap = moe.moe_layer_decode_noalloc_max_bytes()
    assert cap == 8 << 20
    layer = {"H": 256, "I": 128, "E": 4, "k": 2, "w_router": FAKE, "experts": fake_ffn(), "shared": fake_ffn(E=1)}
    assert moe.moe_layer_decode_noalloc(layer, FAKE, None, 0, FAKE) == 0
    expect(uns, moe.moe_layer_decode_noalloc, layer, FAKE, None, 65, FAKE)
    expect(inv, moe.moe_layer_decode_noalloc, layer, FAKE, None, -1, FAKE)
    expect(inv, moe.moe_layer_decode_noalloc, layer, FAKE, None, 4, FAKE, ids_out=FAKE, w_out=None)
    big = {"H": 3840, "I": 512, "E": 1024, "k": 8, "w_router": FAKE, "experts": fake_ffn(E=1024, H=3840, I=512),
           "shared": fake_ffn(E=1, H=3840, I=512)}
    assert moe.moe_layer_decode_workspace_size(big, 64) > cap
    msg = expect(uns, moe.moe_layer_decode_noalloc, big, FAKE, None, 64, FAKE)
    assert "scratch" in msg


def test_decode_step_validation():
    """One call for a chain of layers: every layer must share layer 0's shape and
    format (one workspace serves them all), and the usual argument checks run
    before anything is launched."""
    inv = moe.MOE_ERR_INVALID_ARG
    mk = lambda **kw: dict({"H": 256, "I": 128, "E": 4, "k": 2, "w_router": FAKE, "experts": fake_ffn(),
                            "shared": fake_ffn(E=1)}, **kw)
    layers = [mk(), mk(), mk()]
    need = moe.moe_decode_step_workspace_size(layers, 8)
    need_all = moe.moe_decode_step_workspace_size(layers, 8, with_r_all=True)
    assert need > need_all > 0
    assert moe.moe_decode_step(layers, FAKE, 0, 1e-6, FAKE, ws=FAKE, ws_bytes=need) == 0
    expect(inv, moe.moe_decode_step, layers, FAKE, 8, 1e-6, FAKE, ws=FAKE, ws_bytes=need - 1)
    expect(inv, moe.moe_decode_step, layers, FAKE, 8, -1.0, FAKE, ws=FAKE, ws_bytes=need)
    expect(inv, moe.moe_decode_step, layers, FAKE, 8, 1e-6, None, ws=FAKE, ws_bytes=need)
    expect(inv, moe.moe_decode_step, layers, FAKE, 8, 1e-6, FAKE, ids_out=FAKE, ws=FAKE, ws_bytes=need)
    odd = [mk(), mk(k=1), mk()]
    msg = expect(inv, moe.moe_decode_step, odd, FAKE, 8, 1e-6, FAKE, ws=FAKE, ws_bytes=need)
    assert "layer 1" in msg
    expect(inv, moe.moe_decode_step, [mk(), mk(shared=None)], FAKE, 8, 1e-6, FAKE, ws=FAKE, ws_bytes=need)


def test_bf16_layer_validation():
    """bf16 expert weights pass the layer calls' validation at any T (several
    tokens take the composed kernels); the usual argument checks apply."""
    inv = moe.MOE_ERR_INVALID_ARG
    bf = lambda: {"H": 256, "I": 128, "E": 4, "k": 2, "w_router": FAKE, "experts": fake_ffn(fmt=4),
                  "shared": fake_ffn(fmt=4, E=1)}
    for T in (1, 4, 64, 100):
        need = moe.moe_layer_decode_workspace_size(bf(), T)
        assert need > 0
        expect(inv, moe.moe_layer_decode, bf(), FAKE, None, T, FAKE, ws=FAKE, ws_bytes=need - 1)
    assert moe.moe_layer_decode(bf(), FAKE, None, 0, FAKE, ws=FAKE, ws_bytes=need) == 0
