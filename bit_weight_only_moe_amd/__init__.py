"""Python binding of libmoe_w4a16.so, the gfx950 W4A16 mixture-of-experts layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  The functions carry the C names (``moe_route``, ``moe_permute``,
``moe_grouped_w4a16_ffn``, ``moe_combine``, ``moe_layer_decode``, ...) and
take torch tensors (their device pointers are passed through) plus packed
weight dicts with keys ``fmt``, ``num_experts``, ``rows``, ``cols``,
``codes``, ``scales``, ``zeros``, ``tensor_scale`` and (scale + bias INT4)
``biases``.  Non-zero status codes
raise :class:`MoeError` with the library's message.

If the shared library has not been built, importing this package raises
ImportError: there is no fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4a16.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP = 0, -1, -2, -3
MOE_FMT_NVFP4, MOE_FMT_INT4_G64, MOE_FMT_INT4_SB, MOE_FMT_BF16 = 1, 2, 3, 4
MOE_MODE_AUTO, MOE_MODE_GEMV, MOE_MODE_MFMA = 0, 1, 2

EXPORTED = [
    "moe_abi_version", "moe_last_error", "moe_dequant_w4", "moe_route", "moe_topk_softmax",
    "moe_permute_workspace_size", "moe_permute", "moe_grouped_ffn_workspace_size",
    "moe_grouped_w4a16_ffn", "moe_combine", "moe_layer_decode_workspace_size", "moe_layer_decode",
    "moe_rms_norm", "moe_layer_decode_noalloc_max_bytes", "moe_layer_decode_noalloc", "moe_dense_w4a16_gemv",
    "moe_decode_step_workspace_size", "moe_decode_step",
]


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("status %d: %s" % (code, msg))
        self.code = code


class W4Matrix(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("num_experts", ctypes.c_int), ("rows", ctypes.c_int),
                ("cols", ctypes.c_int), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zeros", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class FfnWeights(ctypes.Structure):
    _fields_ = [("gate", W4Matrix), ("up", W4Matrix), ("down", W4Matrix)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int), ("I", ctypes.c_int), ("E", ctypes.c_int), ("k", ctypes.c_int),
                ("w_router", ctypes.c_void_p), ("experts", FfnWeights),
                ("shared", ctypes.POINTER(FfnWeights))]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libmoe_w4a16.so is not built (run __graft_entry__.build() or "
                          "python -m bit_weight_only_moe_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, Z, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    sig = {
        "moe_abi_version": (I, []),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_dequant_w4": (I, [ctypes.POINTER(W4Matrix), I, P, S]),
        "moe_route": (I, [P, P, I, I, I, I, P, P, P, S]),
        "moe_topk_softmax": (I, [P, I, I, I, P, P, S]),
        "moe_permute_workspace_size": (Z, [I, I, I]),
        "moe_permute": (I, [P, I, I, I, P, P, P, P, P, P, I, P, Z, S]),
        "moe_grouped_ffn_workspace_size": (Z, [I, I, I, I, I]),
        "moe_grouped_w4a16_ffn": (I, [ctypes.POINTER(FfnWeights), I, I, I, P, P, I, P, I, P, I, P, Z, S]),
        "moe_combine": (I, [P, P, P, P, P, I, I, I, P, P, S]),
        "moe_layer_decode_workspace_size": (Z, [ctypes.POINTER(LayerWeights), I]),
        "moe_layer_decode": (I, [ctypes.POINTER(LayerWeights), P, P, I, P, P, P, P, Z, S]),
        "moe_rms_norm": (I, [P, I, I, ctypes.c_float, P, S]),
        "moe_layer_decode_noalloc_max_bytes": (Z, []),
        "moe_dense_w4a16_gemv": (I, [ctypes.POINTER(W4Matrix), I, P, I, P, S]),
        "moe_decode_step_workspace_size": (Z, [ctypes.POINTER(LayerWeights), I, I, I]),
        "moe_decode_step": (I, [ctypes.POINTER(LayerWeights), I, P, I, ctypes.c_float, P, P, P, P, P, Z, S]),
        "moe_layer_decode_noalloc": (I, [ctypes.POINTER(LayerWeights), P, P, I, P, P, P, S]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, _lib.moe_last_error().decode())
    return rc


def moe_abi_version():
    return _lib.moe_abi_version()


def moe_last_error():
    return _lib.moe_last_error().decode()


def w4_matrix(m):
    """A moe_w4_matrix from a packed-weight dict (torch tensors on the device)."""
    return W4Matrix(int(m["fmt"]), int(m["num_experts"]), int(m["rows"]), int(m["cols"]),
                    _ptr(m["codes"]), _ptr(m["scales"]), _ptr(m.get("zeros")), _ptr(m.get("tensor_scale")),
                    _ptr(m.get("biases")))


def ffn_weights(f):
    return FfnWeights(w4_matrix(f["gate"]), w4_matrix(f["up"]), w4_matrix(f["down"]))


class Layer:
    """moe_layer_weights for a layer dict (H, I, E, k, w_router, experts, shared)."""

    def __init__(self, layer):
        self.layer = layer  # keeps the tensors alive
        self._shared = ffn_weights(layer["shared"]) if layer.get("shared") is not None else None
        self.c = LayerWeights(int(layer["H"]), int(layer["I"]), int(layer["E"]), int(layer["k"]),
                              _ptr(layer["w_router"]), ffn_weights(layer["experts"]),
                              ctypes.pointer(self._shared) if self._shared is not None else None)


def moe_dequant_w4(mat, expert, out, stream=None):
    m = w4_matrix(mat)
    return _check(_lib.moe_dequant_w4(ctypes.byref(m), int(expert), _ptr(out), _stream(stream)))


def moe_route(x, w_router, T, H, E, k, logits_out, topk_ids, topk_w, stream=None):
    return _check(_lib.moe_route(_ptr(x), _ptr(w_router), T, H, E, k, _ptr(logits_out), _ptr(topk_ids),
                                 _ptr(topk_w), _stream(stream)))


def moe_topk_softmax(logits, T, E, k, topk_ids, topk_w, stream=None):
    return _check(_lib.moe_topk_softmax(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_w), _stream(stream)))


def moe_permute_workspace_size(T, k, E):
    return _lib.moe_permute_workspace_size(T, k, E)


def moe_permute(topk_ids, T, k, E, counts, offsets, sorted_pairs, pair_pos, x=None, x_perm=None, H=0,
                ws=None, ws_bytes=0, stream=None):
    return _check(_lib.moe_permute(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sorted_pairs),
                                   _ptr(pair_pos), _ptr(x), _ptr(x_perm), H, _ptr(ws), ws_bytes, _stream(stream)))


def moe_grouped_ffn_workspace_size(E, H, I, total_rows, mode=MOE_MODE_AUTO):
    return _lib.moe_grouped_ffn_workspace_size(E, H, I, total_rows, mode)


def moe_grouped_w4a16_ffn(ffn, E, H, I, x, sorted_pairs, k, offsets, total_rows, out, mode=MOE_MODE_AUTO,
                          ws=None, ws_bytes=0, stream=None):
    w = ffn_weights(ffn) if isinstance(ffn, dict) else ffn
    return _check(_lib.moe_grouped_w4a16_ffn(ctypes.byref(w), E, H, I, _ptr(x), _ptr(sorted_pairs), k,
                                             _ptr(offsets), total_rows, _ptr(out), mode, _ptr(ws), ws_bytes,
                                             _stream(stream)))


def moe_combine(out_perm, pair_pos, topk_w, out_shared, residual, T, k, H, y, y_f32=None, stream=None):
    return _check(_lib.moe_combine(_ptr(out_perm), _ptr(pair_pos), _ptr(topk_w), _ptr(out_shared),
                                   _ptr(residual), T, k, H, _ptr(y), _ptr(y_f32), _stream(stream)))


def moe_layer_decode_workspace_size(layer, T):
    L = layer if isinstance(layer, Layer) else Layer(layer)
    return _lib.moe_layer_decode_workspace_size(ctypes.byref(L.c), T)


def moe_layer_decode(layer, x, residual, T, y, ids_out=None, w_out=None, ws=None, ws_bytes=0, stream=None):
    L = layer if isinstance(layer, Layer) else Layer(layer)
    return _check(_lib.moe_layer_decode(ctypes.byref(L.c), _ptr(x), _ptr(residual), T, _ptr(y), _ptr(ids_out),
                                        _ptr(w_out), _ptr(ws), ws_bytes, _stream(stream)))


def moe_rms_norm(r, T, H, eps, x, stream=None):
    return _check(_lib.moe_rms_norm(_ptr(r), T, H, float(eps), _ptr(x), _stream(stream)))


def moe_layer_decode_noalloc_max_bytes():
    return _lib.moe_layer_decode_noalloc_max_bytes()


def moe_layer_decode_noalloc(layer, x, residual, T, y, ids_out=None, w_out=None, stream=None):
    L = layer if isinstance(layer, Layer) else Layer(layer)
    return _check(_lib.moe_layer_decode_noalloc(ctypes.byref(L.c), _ptr(x), _ptr(residual), T, _ptr(y),
                                                _ptr(ids_out), _ptr(w_out), _stream(stream)))


def moe_dense_w4a16_gemv(mat, expert, x, T, out, stream=None):
    m = w4_matrix(mat)
    return _check(_lib.moe_dense_w4a16_gemv(ctypes.byref(m), int(expert), _ptr(x), T, _ptr(out), _stream(stream)))


class LayerList:
    """A host array of moe_layer_weights for moe_decode_step (keeps the layers alive)."""

    def __init__(self, layers):
        self.layers = [l if isinstance(l, Layer) else Layer(l) for l in layers]
        self.arr = (LayerWeights * len(self.layers))(*[l.c for l in self.layers])

    def __len__(self):
        return len(self.layers)


def moe_decode_step_workspace_size(layers, T, with_r_all=False):
    ll = layers if isinstance(layers, LayerList) else LayerList(layers)
    return _lib.moe_decode_step_workspace_size(ll.arr, len(ll), T, int(bool(with_r_all)))


def moe_decode_step(layers, r_in, T, eps, r_out, r_all=None, ids_out=None, w_out=None, ws=None, ws_bytes=0,
                    stream=None):
    ll = layers if isinstance(layers, LayerList) else LayerList(layers)
    return _check(_lib.moe_decode_step(ll.arr, len(ll), _ptr(r_in), T, float(eps), _ptr(r_out), _ptr(r_all),
                                       _ptr(ids_out), _ptr(w_out), _ptr(ws), ws_bytes, _stream(stream)))
