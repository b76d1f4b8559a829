"""Seeded synthetic inputs for the 4-bit weight-only MoE layer.

This module only draws random bytes and numbers in the canonical packed
layout and copies them between device and host.  It holds none of the
layer's arithmetic, so both the HIP path (through its tests and benchmark)
and the CPU oracle can consume the very same bytes.

Layout (row-major [out, in], groups along ``in``):
  codes  uint8 [E, rows, cols/2]     element 2i in the low nibble of byte i
  NVFP4  scales uint8 e4m3 [E, rows, cols/16], tensor_scale float32 [E]
  INT4   scales float16 [E, rows, cols/64], zeros uint8 [E, rows, cols/64]

Value recipes (no trained weights exist here; these stand in for them):
  tokens          bf16 ~ N(0, 1)
  router weights  fp32 ~ N(0, 0.02)
  NVFP4           codes uniform over all 16 nibbles; block scales uniform
                  over the 16 e4m3 codes 0x30..0x3F (values in [0.5, 2));
                  tensor scale ~ U(0.004, 0.008) per (expert, matrix)
  INT4 group 64   codes uniform; fp16 scale ~ U(0.005, 0.02); zero U{0..15}
  BF16 weights    bf16 ~ N(0, 0.02), about the RMS of the 4-bit recipes
  INT4 scale+bias codes uniform; fp16 scale ~ U(0.005, 0.02); fp16 bias =
                  -scale * U(6.5, 8.5) (groups roughly centred on zero, as a
                  min/max affine quantiser gives them)
  full-range scales (scale_range="full", for parity cases that cover the
                  whole of both scale formats):
                  NVFP4 block scales uniform over all 254 non-NaN e4m3 codes
                  (both signs, subnormals, up to 448) with the tensor scale
                  divided by 86 (the RMS of those 254 values is about 86
                  times that of the codes 0x30..0x3F), so the weight RMS
                  stays near 1/sqrt(H); INT4 fp16 scales with a random sign,
                  10% of them fp16 subnormals U(2**-24, 2**-14), 5% zeros
                  (signed), the rest U(0.005, 0.02); scale+bias INT4 draws its
                  scales so and its biases as -scale * U(6.5, 8.5) with 10% of
                  them fp16 subnormals of either sign
  routing logits  "uniform": fp32 ~ U(0, 1) i.i.d.;
                  "zipf": log p(rank(e)) + Gumbel(0, 1), p(r) ~ r**-s over
                  a seeded permutation of the experts (Gumbel-top-k draws k
                  experts without replacement with Zipf weights).
"""

import numpy as np
import torch

FMT_NVFP4 = 1
FMT_INT4_G64 = 2
FMT_INT4_SB = 3
FMT_BF16 = 4
FMT_NAMES = {"nvfp4": FMT_NVFP4, "int4": FMT_INT4_G64, "int4sb": FMT_INT4_SB, "bf16": FMT_BF16}


def seed_of(*keys):
    """A 63-bit torch seed derived from a tuple of non-negative integers."""
    s = np.random.SeedSequence([int(k) for k in keys]).generate_state(2, dtype=np.uint32)
    return int((int(s[0]) << 31) ^ int(s[1])) & ((1 << 63) - 1)


def _gen(device, *keys):
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(*keys))
    return g


def make_matrix(fmt, num_experts, rows, cols, seed, device="cpu", scale_range="narrow"):
    """One packed 4-bit matrix stack [num_experts, rows, cols]."""
    if cols % 64 or rows <= 0:
        raise ValueError("cols must be a multiple of 64")
    if scale_range not in ("narrow", "full"):
        raise ValueError("scale_range must be 'narrow' or 'full'")
    E = num_experts
    g = _gen(device, seed, 1)
    if fmt == FMT_BF16:
        w = torch.randn((E, rows, cols), dtype=torch.float32, device=device, generator=g) * 0.02
        return {"fmt": fmt, "num_experts": E, "rows": rows, "cols": cols, "codes": w.to(torch.bfloat16),
                "scales": None, "zeros": None, "tensor_scale": None}
    codes = torch.randint(0, 256, (E, rows, cols // 2), dtype=torch.uint8, device=device, generator=g)
    if fmt == FMT_NVFP4:
        if scale_range == "full":
            # 254 codes: 0x00..0x7E and 0x80..0xFE (0x7F and 0xFF are NaN)
            r = torch.randint(0, 254, (E, rows, cols // 16), dtype=torch.int32, device=device, generator=g)
            scales = (r + (r >= 127).to(torch.int32)).to(torch.uint8)
        else:
            scales = torch.randint(0x30, 0x40, (E, rows, cols // 16), dtype=torch.uint8, device=device, generator=g)
        ts = torch.rand((E,), dtype=torch.float32, device=device, generator=g) * 0.004 + 0.004
        if scale_range == "full":
            ts = ts / 86.0
        return {"fmt": fmt, "num_experts": E, "rows": rows, "cols": cols,
                "codes": codes, "scales": scales, "zeros": None, "tensor_scale": ts}
    if fmt == FMT_INT4_G64:
        shape = (E, rows, cols // 64)
        s = (torch.rand(shape, dtype=torch.float32, device=device, generator=g) * 0.015 + 0.005)
        zeros = torch.randint(0, 16, shape, dtype=torch.uint8, device=device, generator=g)
        if scale_range == "full":
            kind = torch.rand(shape, dtype=torch.float32, device=device, generator=g)
            sub = torch.exp2(torch.rand(shape, dtype=torch.float32, device=device, generator=g) * 10.0 - 24.0)
            s = torch.where(kind < 0.10, sub, s)
            s = torch.where((kind >= 0.10) & (kind < 0.15), torch.zeros_like(s), s)
            sign = torch.randint(0, 2, shape, dtype=torch.int32, device=device, generator=g) * 2 - 1
            s = s * sign.to(torch.float32)
        return {"fmt": fmt, "num_experts": E, "rows": rows, "cols": cols,
                "codes": codes, "scales": s.to(torch.float16), "zeros": zeros, "tensor_scale": None}
    if fmt == FMT_INT4_SB:
        shape = (E, rows, cols // 64)
        s = (torch.rand(shape, dtype=torch.float32, device=device, generator=g) * 0.015 + 0.005)
        if scale_range == "full":
            kind = torch.rand(shape, dtype=torch.float32, device=device, generator=g)
            sub = torch.exp2(torch.rand(shape, dtype=torch.float32, device=device, generator=g) * 10.0 - 24.0)
            s = torch.where(kind < 0.10, sub, s)
            s = torch.where((kind >= 0.10) & (kind < 0.15), torch.zeros_like(s), s)
            sign = torch.randint(0, 2, shape, dtype=torch.int32, device=device, generator=g) * 2 - 1
            s = s * sign.to(torch.float32)
        s = s.to(torch.float16).to(torch.float32)
        b = -s * (torch.rand(shape, dtype=torch.float32, device=device, generator=g) * 2.0 + 6.5)
        if scale_range == "full":
            kind = torch.rand(shape, dtype=torch.float32, device=device, generator=g)
            sub = torch.exp2(torch.rand(shape, dtype=torch.float32, device=device, generator=g) * 10.0 - 24.0)
            sign = torch.randint(0, 2, shape, dtype=torch.int32, device=device, generator=g) * 2 - 1
            b = torch.where(kind < 0.10, sub * sign.to(torch.float32), b)
        return {"fmt": fmt, "num_experts": E, "rows": rows, "cols": cols,
                "codes": codes, "scales": s.to(torch.float16), "zeros": None, "tensor_scale": None,
                "biases": b.to(torch.float16)}
    raise ValueError("unknown format %r" % (fmt,))


def make_ffn(fmt, num_experts, H, I, seed, device="cpu", scale_range="narrow"):
    """gate [I, H], up [I, H], down [H, I] for num_experts experts."""
    return {"gate": make_matrix(fmt, num_experts, I, H, seed_of(seed, 11), device, scale_range),
            "up": make_matrix(fmt, num_experts, I, H, seed_of(seed, 12), device, scale_range),
            "down": make_matrix(fmt, num_experts, H, I, seed_of(seed, 13), device, scale_range)}


def make_layer(fmt, H, I, E, k, seed, device="cpu", shared=True, I_shared=None, scale_range="narrow"):
    """Router, routed experts and (optionally) the shared expert of one layer."""
    g = _gen(device, seed, 2)
    w_router = torch.randn((E, H), dtype=torch.float32, device=device, generator=g) * 0.02
    return {"fmt": fmt, "H": H, "I": I, "E": E, "k": k,
            "w_router": w_router,
            "experts": make_ffn(fmt, E, H, I, seed_of(seed, 3), device, scale_range),
            "shared": make_ffn(fmt, 1, H, I_shared or I, seed_of(seed, 4), device, scale_range) if shared else None}


def make_tokens(T, H, seed, device="cpu"):
    """bf16 activations ~ N(0, 1), shape [T, H]."""
    g = _gen(device, seed, 5)
    return torch.randn((T, H), dtype=torch.float32, device=device, generator=g).to(torch.bfloat16)


def uniform_logits(T, E, seed, device="cpu"):
    g = _gen(device, seed, 6)
    return torch.rand((T, E), dtype=torch.float32, device=device, generator=g)


def zipf_logits(T, E, s, seed, device="cpu"):
    """log p(rank(e)) + Gumbel(0, 1) noise, p(r) proportional to r**-s."""
    rng = np.random.Generator(np.random.PCG64(seed_of(seed, 7)))
    perm = rng.permutation(E)
    rank = np.empty(E, dtype=np.int64)
    rank[perm] = np.arange(1, E + 1)
    logp = -s * np.log(rank.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    u = rng.random((T, E))
    gumbel = -np.log(-np.log(np.clip(u, 1e-300, 1.0)))
    return torch.from_numpy((logp[None, :] + gumbel).astype(np.float32)).to(device)


# ---------------------------------------------------------------- host copies

def bits16(t):
    """A bf16/fp16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _np_expert_slice(t, experts):
    if t is None:
        return None
    if experts is None:
        return bits16(t) if t.dtype in (torch.float16, torch.bfloat16) else t.detach().cpu().numpy()
    idx = sorted(int(e) for e in experts)
    if not idx:
        return {}
    sel = torch.as_tensor(idx, device=t.device, dtype=torch.long)
    sub = t.index_select(0, sel)
    arr = bits16(sub) if sub.dtype in (torch.float16, torch.bfloat16) else sub.cpu().numpy()
    return {e: arr[i] for i, e in enumerate(idx)}


def matrix_to_numpy(mat, experts=None):
    """Host copy of a packed matrix; with ``experts``, only those (a dict by id)."""
    out = {"fmt": mat["fmt"], "num_experts": mat["num_experts"], "rows": mat["rows"], "cols": mat["cols"]}
    for key in ("codes", "scales", "zeros", "tensor_scale", "biases"):
        out[key] = _np_expert_slice(mat.get(key), experts)
    return out


def ffn_to_numpy(ffn, experts=None):
    return {m: matrix_to_numpy(ffn[m], experts) for m in ("gate", "up", "down")}


def layer_to_numpy(layer, experts=None):
    return {"fmt": layer["fmt"], "H": layer["H"], "I": layer["I"], "E": layer["E"], "k": layer["k"],
            "w_router": layer["w_router"].detach().cpu().numpy(),
            "experts": ffn_to_numpy(layer["experts"], experts),
            "shared": None if layer["shared"] is None else ffn_to_numpy(layer["shared"])}


def matrix_bytes(fmt, rows, cols):
    """Bytes of one expert's packed matrix (codes + scales + zeros + tensor scale)."""
    n = rows * cols
    if fmt == FMT_NVFP4:
        return n // 2 + n // 16 + 4
    if fmt == FMT_INT4_SB:
        return n // 2 + 2 * (n // 64) + 2 * (n // 64)
    if fmt == FMT_BF16:
        return 2 * n
    return n // 2 + 2 * (n // 64) + n // 64


def expert_bytes(fmt, H, I):
    return 2 * matrix_bytes(fmt, I, H) + matrix_bytes(fmt, H, I)
