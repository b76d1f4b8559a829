"""Scalar, loop-by-loop evaluation of the MoE layer for tiny inputs.

A second, independently written form of the layer used only to cross-check
the vectorised oracle on tiny shapes (a handful of tokens).  It decodes
every number with Python's ``struct``/``math`` from the bit-level format
definitions and sums with plain Python floats (IEEE double), one element at
a time, so it shares no code path with numpy's vectorised one.
"""

import math
import struct


def bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def fp16(bits):
    return struct.unpack("<e", struct.pack("<H", int(bits) & 0xFFFF))[0]


def e2m1(n):
    sign = -1.0 if n & 8 else 1.0
    exp = (n >> 1) & 3
    man = n & 1
    if exp == 0:
        return sign * math.ldexp(man, -1)
    return sign * math.ldexp(2 + man, exp - 2)


def e4m3(b):
    sign = -1.0 if b & 0x80 else 1.0
    exp = (b >> 3) & 15
    man = b & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        return sign * math.ldexp(man, -9)
    return sign * math.ldexp(8 + man, exp - 10)


def round_bf16(v):
    if v == 0.0 or math.isinf(v) or math.isnan(v):
        return v
    m, e = math.frexp(v)
    q = max(e - 8, -133)
    r = round(math.ldexp(v, -q))          # Python rounds halves to even
    out = math.ldexp(r, q)
    if abs(out) > math.ldexp(2 ** 8 - 1, 120):
        return math.copysign(math.inf, v)
    return out


def weight(mat, e, r, c):
    byte = int(mat["codes"][e][r][c // 2])
    nib = (byte >> 4) if (c & 1) else (byte & 15)
    if mat["fmt"] == 1:
        ts = float(mat["tensor_scale"][e])
        return ts * e4m3(int(mat["scales"][e][r][c // 16])) * e2m1(nib)
    s = fp16(mat["scales"][e][r][c // 64])
    z = int(mat["zeros"][e][r][c // 64])
    return s * (nib - z)


def ffn(f, e, x):
    I = f["gate"]["rows"]
    H = f["gate"]["cols"]
    h = []
    for i in range(I):
        g = 0.0
        u = 0.0
        for c in range(H):
            g += weight(f["gate"], e, i, c) * x[c]
            u += weight(f["up"], e, i, c) * x[c]
        h.append(round_bf16(g / (1.0 + math.exp(-g)) * u))
    out = []
    for n in range(H):
        acc = 0.0
        for i in range(I):
            acc += weight(f["down"], e, n, i) * h[i]
        out.append(acc)
    return out


def layer(L, x_bits_rows, residual_rows=None):
    """Returns per token: (ids, weights, y list)."""
    E = L["w_router"].shape[0]
    H = L["w_router"].shape[1]
    k = L["k"]
    results = []
    for t, xb in enumerate(x_bits_rows):
        x = [bf16(b) for b in xb]
        logits = []
        for e in range(E):
            acc = 0.0
            for c in range(H):
                acc += float(L["w_router"][e][c]) * x[c]
            logits.append(acc)
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or logits[e] > logits[best]:
                    best = e
            chosen.append(best)
        top = max(logits[e] for e in chosen)
        ex = [math.exp(logits[e] - top) for e in chosen]
        tot = sum(ex)
        w = [v / tot for v in ex]
        y = [0.0] * H
        for j, e in enumerate(chosen):
            o = ffn(L["experts"], e, x)
            for n in range(H):
                y[n] += w[j] * o[n]
        if L.get("shared") is not None:
            o = ffn(L["shared"], 0, x)
            for n in range(H):
                y[n] += o[n]
        if residual_rows is not None:
            for n in range(H):
                y[n] += bf16(residual_rows[t][n])
        results.append((chosen, w, y))
    return results
