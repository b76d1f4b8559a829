"""Benchmark of the W4A16 MoE layer on one MI355X.

Default (``--workload all``): the headline is one Flint-shaped MoE decode
layer at batch 1 (hidden 2048, 256 experts top-6 + 1 shared expert, expert
inter 768, NVFP4 W4A16 weights, bf16 activations).  One step = one
moe_layer_decode call on one token: router GEMV, top-k + softmax, expert
grouping, gate/up + SwiGLU, down projection, shared expert and combine.
The same JSON line carries a ``sweep`` object with the rest of the metric:
decode at 1/4/16/64 tokens in the three 4-bit weight formats (NVFP4, INT4
with a zero point, INT4 with scale and bias) and in BF16 weights for
comparison, the 47-layer batch-8 chained decode
step, and the 4096-token Zipf(1.1) prefill in NVFP4 and zero-point INT4,
each with its roofline fraction and a short timing of the float64 CPU
oracle on a bounded sample of the same workload.

Decode steps rotate over independently seeded weight copies, enough that no
copy is read again within 512 MB (twice the ~256 MB memory-side cache) of
weight traffic, and every step gets fresh tokens; the memory-side cache is
flushed (a 1 GiB read) right before the timed replay.  K steps are captured
in one HIP graph; after a warm replay, further warm replays worth 50 ms,
the flush and the timed replay (between HIP events on the launch stream)
are queued back to back, so the timed steps start on a busy chip.

The sweep also carries the dense 4-bit output-head GEMV (150,144 x 2048,
1 and 8 tokens).  ``process_spread`` times the headline workload again in
fresh processes (``--spread-processes``, default 2).

Single workloads (``--workload``): decode_b1, decode_T4, decode_T16,
decode_T64 (with ``--fmt int4`` or ``--fmt int4sb`` for the other formats), chain_b8, prefill,
dense_head (``--tokens T``),
and hbm_copy: a plain 1 GiB device copy whose HBM counter readings calibrate
the traffic figures.

Prints ONE JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE decode tokens/s and weight HBM GB/s (% of peak), batch 1-64; prefill TFLOP/s"
H, I, E, K_TOP = 2048, 768, 256, 6
CHAIN_LAYERS, CHAIN_T, CHAIN_EPS = 47, 8, 1e-6
ROTATE_BYTES = 512e6      # no weight copy is read again within this much weight traffic
MAX_COPIES = 48           # about 33 GB of NVFP4 layer copies
WARM_MS = 50.0            # untimed graph replays queued right before the timed one

# HBM bytes per measured unit (one layer call; the 47-layer chained step; one head GEMV call;
# the prefill's grouped FFN, routed + shared) from two rocprofv3 --pmc runs of the same workload
# with the current kernels: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, the factors that make the
# counters read 1 GiB each for a plain 1 GiB device copy (profiles/hbm_traffic_counters.md).
# Workloads not listed report null.
TRAFFIC_BYTES = {
    ("decode_b1", "nvfp4"): 21.52e6,
    ("decode_T4", "nvfp4"): 68.6e6,
    ("decode_T16", "nvfp4"): 221.5e6,
    ("decode_T16", "int4"): 215.8e6,
    ("decode_T64", "nvfp4"): 559.8e6,
    ("chain_b8", "nvfp4"): 5.89e9,
    ("dense_head_T1", "nvfp4"): 173.7e6,
    ("dense_head_T8", "nvfp4"): 214.6e6,
    ("prefill", "nvfp4"): 1236.6e6,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="all")
    p.add_argument("--fmt", default="nvfp4", choices=["nvfp4", "int4", "int4sb", "bf16"])
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the headline's CPU oracle leg")
    p.add_argument("--sweep-cpu-seconds", type=float, default=3.0, help="time budget of each sweep entry's oracle leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--spread-processes", type=int, default=2,
                   help="fresh processes that time the headline workload again (0: none)")
    p.add_argument("--tokens", type=int, default=1, help="tokens of the dense_head workload")
    p.add_argument("--eager", action="store_true",
                   help="launch the K timed steps directly instead of replaying a captured graph (profiler runs)")
    return p.parse_args()


def host_cores():
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = None
    return len(os.sched_getaffinity(0)), blas


def cpu_entry(value, unit, sample):
    cores, blas = host_cores()
    return {"value": value, "unit": unit, "cores": cores, "blas_threads": blas, "kind": "oracle",
            "sample": sample + "; float64 numpy oracle as it stands (a correctness reference, not a tuned CPU MoE)"}


class Ctx:
    def __init__(self, args):
        import torch
        import bit_weight_only_moe_amd as moe
        import synth
        self.args, self.torch, self.moe, self.synth = args, torch, moe, synth
        self.dev = "cuda"
        self.stream = torch.cuda.Stream()
        self._flush = None
        self._copies = {}

    def _flush_buffers(self):
        t = self.torch
        if self._flush is None:
            self._flush = t.zeros(1 << 27, dtype=t.int64, device=self.dev)  # 1 GiB

    def _flush_async(self):
        """Read 1 GiB (a sum): evicts the memory-side cache and, unlike a copy, leaves no
        dirty lines whose write-back would slow the next steps (a 1 GiB copy cost the first
        three 16-token steps after it 15, 9 and 3 us)."""
        self._flush_buffers()
        self._flush_sum = self._flush.sum()

    def flush(self):
        """Evict the memory-side cache and wait."""
        t = self.torch
        with t.cuda.stream(self.stream):
            self._flush_async()
        t.cuda.synchronize()

    def copies(self, fmt_name, n):
        """n independently seeded Flint-shaped layers (created once per format, shared by the
        decode entries and the chain)."""
        have = self._copies.setdefault(fmt_name, [])
        fmt = self.synth.FMT_NAMES[fmt_name]
        while len(have) < n:
            l = len(have)
            layer = self.synth.make_layer(fmt, H, I, E, K_TOP, self.synth.seed_of(1, l), self.dev)
            have.append((layer, self.moe.Layer(layer)))
        return have[:n]

    def drop(self, fmt_name):
        self._copies.pop(fmt_name, None)
        self.torch.cuda.empty_cache()

    def timed(self, body, K, W):
        """W eager warm-up steps, K steps captured in one graph, one warm replay, then warm
        replays worth WARM_MS, a cache flush and the timed replay between events on the launch
        stream, queued together (with --eager: the K steps launched directly after a flush).
        Returns ms."""
        t, s = self.torch, self.stream
        t.cuda.synchronize()  # the inputs were made on the default stream; the steps run on s
        with t.cuda.stream(s):
            for i in range(W):
                body(i, s)
        t.cuda.synchronize()
        if self.args.eager:
            self.flush()
            ev0, ev1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            with t.cuda.stream(s):
                ev0.record(s)
                for i in range(K):
                    body(i, s)
                ev1.record(s)
            t.cuda.synchronize()
            return ev0.elapsed_time(ev1)
        g = t.cuda.CUDAGraph()
        with t.cuda.graph(g, stream=s):
            for i in range(K):
                body(i, s)
        ev0, ev1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        with t.cuda.stream(s):
            ev0.record(s)
            g.replay()
            ev1.record(s)
        t.cuda.synchronize()
        # warm replays worth >= WARM_MS of work, the cache flush and the timed replay, queued back
        # to back: the timed replay starts on a chip that has been busy for a while, not after an
        # idle gap (clocks ramp with load: 20 steps of 64 tokens ran 8% slower per step than 200
        # steps when timed after a single warm replay)
        n_warm = max(1, math.ceil(WARM_MS / max(ev0.elapsed_time(ev1), 1e-3)))
        with t.cuda.stream(s):
            for _ in range(n_warm):
                g.replay()
            self._flush_async()
            ev0.record(s)
            g.replay()
            ev1.record(s)
        t.cuda.synchronize()
        return ev0.elapsed_time(ev1)


def decode_entry(c, fmt_name, T, K, W, cpu_seconds):
    """K decode steps of one layer at T tokens, rotating over weight copies."""
    t, moe, synth = c.torch, c.moe, c.synth
    fmt = synth.FMT_NAMES[fmt_name]
    eb = synth.expert_bytes(fmt, H, I)
    exp_touched = E * (1.0 - (1.0 - K_TOP / E) ** T) + 1.0
    R = int(min(MAX_COPIES, max(K, math.ceil(ROTATE_BYTES / (exp_touched * eb)))))
    copies = c.copies(fmt_name, R)
    NX = max(K, W, 1)
    xs = [synth.make_tokens(T, H, synth.seed_of(2, T, i), c.dev) for i in range(NX)]
    ys = [t.empty_like(x) for x in xs]
    ids = [t.empty((T, K_TOP), dtype=t.int32, device=c.dev) for _ in range(NX)]
    ws_ = [t.empty((T, K_TOP), dtype=t.float32, device=c.dev) for _ in range(NX)]
    nws = moe.moe_layer_decode_workspace_size(copies[0][1], T)
    wsb = t.zeros(nws, dtype=t.uint8, device=c.dev)

    def step(i, s):
        moe.moe_layer_decode(copies[i % R][1], xs[i % NX], None, T, ys[i % NX], ids[i % NX], ws_[i % NX], wsb, nws,
                             stream=s)

    ms = c.timed(step, K, W)
    ms_step = ms / K
    touched = [len(np.unique(ids[i % NX].cpu().numpy())) + 1 for i in range(K)]
    bytes_step = eb * float(np.mean(touched))
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    wl = "decode_b1" if T == 1 else "decode_T%d" % T
    entry = {"workload": "moe_decode_layer T=%d %s H=2048 I=768 E=256 top6+1shared" % (T, fmt_name),
             "tokens_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step, "steps": K, "warmup": W,
             "weight_copies": R, "distinct_experts_per_step": float(np.mean(touched)),
             "expert_bytes_per_step": bytes_step, "router_bytes_per_step": E * H * 4,
             "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": gbs / HBM_PEAK_GBS, "traffic": TRAFFIC_BYTES.get((wl, fmt_name)),
                          "kernel": "moe_layer_decode (one layer call: %s), events on the launch stream"
                                    % ("k_layer_route_shared + k_layer_gateup + k_layer_down_t1" if T == 1 else
                                       "the composed kernels: router, top-k, permute, grouped GEMV gate/up and "
                                       "down for the routed and shared experts, k_combine" if fmt_name == "bf16" else
                                       "k_layer_route_shared + k_layer_gateup + k_layer_down_combine"
                                       + (" + k_combine" if T > 16 else "")),
                          "bytes": "expert weights of the distinct touched experts + shared expert, per call"},
             "cpu_baseline": None}
    if cpu_seconds > 0:
        import oracle
        # a few of the timed steps (step i ran on weight copy i % R); host copies of the experts
        # that the GPU or the oracle routes them to are made before the clock starts
        steps = list(range(min(NX, 8 if T <= 16 else 2)))
        need = {}
        for i in steps:
            r = i % R
            xb = synth.bits16(xs[i])
            _, oid, _ = oracle.route(xb, copies[r][0]["w_router"].cpu().numpy(), K_TOP)
            need.setdefault(r, set()).update(ids[i].cpu().numpy().ravel().tolist() + oid.ravel().tolist())
        hosts = {r: synth.layer_to_numpy(copies[r][0], experts=ex) for r, ex in need.items()}
        xbits = {i: synth.bits16(xs[i]) for i in steps}
        t0 = time.perf_counter()
        calls = 0
        while True:
            i = steps[calls % len(steps)]
            oracle.moe_layer(hosts[i % R], xbits[i])
            calls += 1
            if time.perf_counter() - t0 >= cpu_seconds or calls >= 64:
                break
        el = time.perf_counter() - t0
        entry["cpu_baseline"] = cpu_entry(calls * T / el, "tokens/s",
                                          "%d layer calls of this workload (T=%d, %s; %d distinct steps), %.1f s "
                                          "incl. dequantisation of the touched experts" % (calls, T, fmt_name,
                                                                                          len(steps), el))
    return entry


def chain_entry(c, fmt_name, K, W, cpu_seconds):
    """One decode step through 47 chained layers at batch 8: r_0 = tokens; per layer
    x_l = rms_norm(r_l), r_{l+1} = moe_layer_decode(x_l, residual = r_l), so every layer's
    routing depends on the layer before."""
    t, moe, synth = c.torch, c.moe, c.synth
    fmt = synth.FMT_NAMES[fmt_name]
    NL, T = CHAIN_LAYERS, CHAIN_T
    layers = c.copies(fmt_name, NL)
    NX = max(K, W, 1)
    r0 = [synth.make_tokens(T, H, synth.seed_of(4, i), c.dev) for i in range(NX)]
    ll = moe.LayerList([L for _, L in layers])
    r_out = t.empty((T, H), dtype=t.bfloat16, device=c.dev)
    ids_all = t.empty((NL, T, K_TOP), dtype=t.int32, device=c.dev)
    w_all = t.empty((NL, T, K_TOP), dtype=t.float32, device=c.dev)
    nws = moe.moe_decode_step_workspace_size(ll, T)
    wsb = t.zeros(nws, dtype=t.uint8, device=c.dev)
    ids = [ids_all[l] for l in range(NL)]

    def step(i, s):
        moe.moe_decode_step(ll, r0[i % NX], T, CHAIN_EPS, r_out, None, ids_all, w_all, wsb, nws, stream=s)

    ms = c.timed(step, K, W)
    ms_step = ms / K
    eb = synth.expert_bytes(fmt, H, I)
    bytes_step = sum((len(np.unique(ids[l].cpu().numpy())) + 1) * eb for l in range(NL))
    gbs = bytes_step / (ms_step * 1e-3) / 1e9
    entry = {"workload": "moe_decode_chain 47 layers T=8 %s H=2048 I=768 E=256 top6+1shared, rms-normalised "
                         "residual stream between layers" % fmt_name,
             "tokens_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step, "steps": K, "warmup": W,
             "expert_bytes_per_step": bytes_step, "resident_weight_bytes": NL * (E + 1) * eb,
             "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": gbs / HBM_PEAK_GBS, "traffic": TRAFFIC_BYTES.get(("chain_b8", fmt_name)),
                          "kernel": "moe_decode_step: 47 x (k_rms_norm + the three decode launches), one "
                                    "call per step, events on the launch stream"},
             "cpu_baseline": None}
    if cpu_seconds > 0:
        import oracle
        # the oracle's own chain from one step's input, layer by layer; each layer's host copy
        # (the experts the oracle routes to) is made off the clock
        r = synth.bits16(r0[0])
        el, nl = 0.0, 0
        while nl < NL and el < cpu_seconds:
            L = layers[nl][0]
            x = oracle.rms_norm(r, CHAIN_EPS)
            _, oid, _ = oracle.route(x, L["w_router"].cpu().numpy(), K_TOP)
            host = synth.layer_to_numpy(L, experts=set(oid.ravel().tolist()))
            t0 = time.perf_counter()
            _, res = oracle.chain_layer(host, r, CHAIN_EPS)
            el += time.perf_counter() - t0
            r = oracle.f64_to_bf16_bits(res["y_bf16"])
            nl += 1
        step_s = el / nl * NL
        entry["cpu_baseline"] = cpu_entry(T / step_s, "tokens/s",
                                          "%d of the 47 chained layers at T=8 (%s), %.1f s of oracle time, scaled "
                                          "to the 47-layer step" % (nl, fmt_name, el))
    return entry


def prefill_entry(c, fmt_name, K, W, cpu_seconds):
    """4096-token prefill of one Flint-shaped layer with Zipf(1.1) expert popularity."""
    t, moe, synth = c.torch, c.moe, c.synth
    fmt = synth.FMT_NAMES[fmt_name]
    T = 4096
    R = 2
    layers = [synth.make_layer(fmt, H, I, E, K_TOP, synth.seed_of(5, r), c.dev) for r in range(R)]
    x = synth.make_tokens(T, H, 5, c.dev)
    zl = synth.zipf_logits(T, E, 1.1, 5, c.dev)
    n = T * K_TOP
    lg = t.empty((T, E), dtype=t.float32, device=c.dev)
    ids = t.empty((T, K_TOP), dtype=t.int32, device=c.dev)
    w = t.empty((T, K_TOP), dtype=t.float32, device=c.dev)
    counts = t.empty(E, dtype=t.int32, device=c.dev)
    offsets = t.empty(E + 1, dtype=t.int32, device=c.dev)
    sp = t.empty(n, dtype=t.int32, device=c.dev)
    pp = t.empty(n, dtype=t.int32, device=c.dev)
    pws_n = moe.moe_permute_workspace_size(T, K_TOP, E)
    pws = t.empty(pws_n, dtype=t.uint8, device=c.dev)
    out = t.empty((n, H), dtype=t.float32, device=c.dev)
    out_s = t.empty((T, H), dtype=t.float32, device=c.dev)
    off_s = t.tensor([0, T], dtype=t.int32, device=c.dev)
    gws_n = max(moe.moe_grouped_ffn_workspace_size(E, H, I, n), moe.moe_grouped_ffn_workspace_size(1, H, I, T))
    gws = t.empty(gws_n, dtype=t.uint8, device=c.dev)
    gws_s = t.empty(gws_n, dtype=t.uint8, device=c.dev)
    y = t.empty_like(x)
    f_routed = [moe.ffn_weights(l["experts"]) for l in layers]
    f_shared = [moe.ffn_weights(l["shared"]) for l in layers]
    # The shared expert needs no routing: its grouped FFN runs on a side stream (own
    # workspace), forked after the top-k, alongside the permute kernels, which leave most
    # of the chip idle, and the start of the routed FFN; both join before the combine.
    side = t.cuda.Stream()

    def shared_ffn(i, s):
        side.wait_stream(s)
        moe.moe_grouped_w4a16_ffn(f_shared[i % R], 1, H, I, x, None, 1, off_s, T, out_s, moe.MOE_MODE_AUTO, gws_s,
                                  gws_n, stream=side)

    def routed_ffn(i, s):
        moe.moe_grouped_w4a16_ffn(f_routed[i % R], E, H, I, x, sp, K_TOP, offsets, n, out, moe.MOE_MODE_AUTO, gws,
                                  gws_n, stream=s)

    def step(i, s):
        L = layers[i % R]
        moe.moe_route(x, L["w_router"], T, H, E, K_TOP, lg, ids, w, stream=s)  # router GEMM (timed)
        moe.moe_topk_softmax(zl, T, E, K_TOP, ids, w, stream=s)             # the skewed logits route
        shared_ffn(i, s)
        moe.moe_permute(ids, T, K_TOP, E, counts, offsets, sp, pp, None, None, 0, pws, pws_n, stream=s)
        routed_ffn(i, s)
        s.wait_stream(side)
        moe.moe_combine(out, pp, w, out_s, x, T, K_TOP, H, y, stream=s)

    def ffn_pair(i, s):
        shared_ffn(i, s)
        routed_ffn(i, s)
        s.wait_stream(side)

    ms = c.timed(step, K, W)
    ms_ffn = c.timed(ffn_pair, K, W)
    flops = 6.0 * (n + T) * H * I
    cnt = counts.cpu().numpy()
    ffn_tf = flops / (ms_ffn / K * 1e-3) / 1e12
    entry = {"workload": "moe_prefill T=4096 %s H=2048 I=768 E=256 top6+1shared zipf1.1" % fmt_name,
             "tflops": flops / (ms / K * 1e-3) / 1e12, "tokens_per_s": T * K / (ms * 1e-3),
             "ms_per_step": ms / K, "ffn_ms": ms_ffn / K, "steps": K, "warmup": W, "expert_gflop": flops / 1e9,
             "max_rows_per_expert": int(cnt.max()), "min_rows_per_expert": int(cnt.min()),
             "roofline": {"bound": "mfma", "achieved": ffn_tf, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": ffn_tf / MFMA_BF16_PEAK_TFLOPS, "traffic": TRAFFIC_BYTES.get(("prefill", fmt_name)),
                          "kernel": "moe_grouped_w4a16_ffn routed + shared (%s gate/up and down), events on the "
                                    "launch stream" % ("k_mfma_bl" if fmt == 1 else "k_mfma_bd")},
             "cpu_baseline": None}
    if cpu_seconds > 0:
        import oracle
        lg_np = zl.cpu().numpy()
        ids_np = oracle.topk_select(lg_np.astype(np.float64), K_TOP)
        xb = synth.bits16(x)
        n_tok = 32
        toks = np.arange(n_tok)
        host = synth.layer_to_numpy(layers[0], experts=set(ids_np[toks].ravel().tolist()))
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.moe_layer(host, xb, residual_bits=xb, logits=lg_np, tokens=toks)
            done += 1
            if time.perf_counter() - t0 >= cpu_seconds:
                break
        el = time.perf_counter() - t0
        f = 6.0 * (n_tok * K_TOP + n_tok) * H * I * done
        entry["cpu_baseline"] = cpu_entry(f / el / 1e12, "TFLOP/s",
                                          "%d oracle runs over the first 32 of the 4096 Zipf-routed tokens (%s), "
                                          "%.1f s incl. dequantisation of their experts" % (done, fmt_name, el))
    return entry


def dense_entry(c, fmt_name, T, K, W, cpu_seconds, rows=150144):
    """The 4-bit output head: out[T, 150144] = W x over hidden 2048, one matrix
    per step, rotating over copies of more than 512 MB in all."""
    t, moe, synth = c.torch, c.moe, c.synth
    fmt = synth.FMT_NAMES[fmt_name]
    mb = synth.matrix_bytes(fmt, rows, H)
    R = max(2, math.ceil(ROTATE_BYTES / mb))
    mats = [synth.make_matrix(fmt, 1, rows, H, synth.seed_of(6, r), c.dev) for r in range(R)]
    NX = max(K, W, 1)
    xs = [synth.make_tokens(T, H, synth.seed_of(7, T, i), c.dev) for i in range(NX)]
    out = t.empty((T, rows), dtype=t.float32, device=c.dev)

    def step(i, s):
        moe.moe_dense_w4a16_gemv(mats[i % R], 0, xs[i % NX], T, out, stream=s)

    ms = c.timed(step, K, W)
    ms_step = ms / K
    gbs = mb * ((T + 63) // 64) / (ms_step * 1e-3) / 1e9  # algorithmic: the matrix once per 64 tokens
    entry = {"workload": "dense_w4a16_gemv output head %d x 2048 T=%d %s" % (rows, T, fmt_name),
             "tokens_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step, "steps": K, "warmup": W,
             "weight_copies": R, "matrix_bytes": mb,
             "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": gbs / HBM_PEAK_GBS, "traffic": TRAFFIC_BYTES.get(("dense_head_T%d" % T, fmt_name)),
                          "kernel": "%s (one call), events on the launch stream"
                                    % ("k_mfma_bl dense form" if (T >= 8 and fmt == 1) else "k_dense_gemv"),
                          "bytes": "the packed matrix once per 64 tokens"},
             "cpu_baseline": None}
    if cpu_seconds > 0:
        import oracle
        host = synth.matrix_to_numpy(mats[0])
        xb = synth.bits16(xs[0])
        n = 4096
        t0 = time.perf_counter()
        done = 0
        while True:
            oracle.dense_gemv(host, 0, xb, rows=np.arange(done * n % rows, done * n % rows + n) % rows)
            done += 1
            if time.perf_counter() - t0 >= cpu_seconds:
                break
        el = time.perf_counter() - t0
        full_s = el / (done * n) * rows
        entry["cpu_baseline"] = cpu_entry(T / full_s, "tokens/s",
                                          "%d oracle runs over 4096 of the 150,144 rows (%s, T=%d), %.1f s incl. "
                                          "dequantisation, scaled to the full head" % (done, fmt_name, T, el))
    return entry


def copy_line(c, args):
    """A plain device copy of 1 GiB (torch's copy kernel): 1 GiB read + 1 GiB written per step."""
    t = c.torch
    n = 1 << 30
    src = t.empty(n, dtype=t.uint8, device="cuda")
    dst = t.empty_like(src)
    src.fill_(1)
    K, W = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
    for _ in range(W):
        with t.cuda.stream(c.stream):
            dst.copy_(src)
    t.cuda.synchronize()
    ev0, ev1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
    with t.cuda.stream(c.stream):
        ev0.record(c.stream)
        for _ in range(K):
            dst.copy_(src)
        ev1.record(c.stream)
    t.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    gbs = 2.0 * n * K / (ms * 1e-3) / 1e9
    return {"metric": "device copy GB/s (read + write)", "value": gbs, "unit": "GB/s", "n_gpus": 1,
            "steps": K, "warmup": W, "ms_per_step": ms / K, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
            "config": {"workload": "hbm_copy 1 GiB", "bytes_read_per_step": n, "bytes_written_per_step": n},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "torch copy"},
            "cpu_baseline": None}


def line_from(entry, fmt_name, value_key, unit, K, W):
    cfg = {k: v for k, v in entry.items() if k not in ("roofline", "cpu_baseline", "ms_per_step", "steps", "warmup")}
    return {"metric": METRIC, "value": entry[value_key], "unit": unit, "n_gpus": 1, "steps": K, "warmup": W,
            "ms_per_step": entry["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "%s/bf16 act/fp32 acc" % ("w16(bf16)" if fmt_name == "bf16" else "w4(%s)" % fmt_name),
            "data": "synthetic", "config": cfg,
            "roofline": entry["roofline"], "cpu_baseline": entry["cpu_baseline"]}


def process_spread(args, head_ms, K, W):
    """The headline workload timed again in fresh processes, each with its own
    weight copies and tokens: the spread between processes, next to the one in
    this process."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--workload", "decode_b1", "--fmt", "nvfp4",
           "--steps", str(K), "--warmup", str(W), "--no-cpu-baseline"]
    vals = [head_ms]
    for _ in range(args.spread_processes):
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
        if r.returncode != 0 or not lines:
            return {"error": "a spread process failed (exit %d)" % r.returncode, "ms_per_step": vals}
        vals.append(json.loads(lines[-1])["ms_per_step"])
    med = float(np.median(vals))
    return {"processes": len(vals), "ms_per_step": vals, "median_ms": med,
            "spread": (max(vals) - min(vals)) / med}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    c = Ctx(args)
    K, W = max(1, args.steps), max(0, args.warmup)
    cpu = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    scpu = 0.0 if args.no_cpu_baseline else args.sweep_cpu_seconds
    wl = args.workload
    decode_T = {"decode_b1": 1, "decode_T4": 4, "decode_T16": 16, "decode_T64": 64}
    Kc, Wc = max(1, min(K, 10)), max(1, min(W, 3))       # the chain and prefill steps are long
    if wl == "hbm_copy":
        print(json.dumps(copy_line(c, args)))
        return
    if wl in decode_T:
        e = decode_entry(c, args.fmt, decode_T[wl], K, W, cpu)
        print(json.dumps(line_from(e, args.fmt, "tokens_per_s", "tokens/s", K, W)))
        return
    if wl == "dense_head":
        e = dense_entry(c, args.fmt, args.tokens, K, W, cpu)
        print(json.dumps(line_from(e, args.fmt, "tokens_per_s", "tokens/s", K, W)))
        return
    if wl == "chain_b8":
        e = chain_entry(c, args.fmt, Kc, Wc, cpu)
        print(json.dumps(line_from(e, args.fmt, "tokens_per_s", "tokens/s", Kc, Wc)))
        return
    if wl == "prefill":
        e = prefill_entry(c, args.fmt, Kc, Wc, cpu)
        out = line_from(e, args.fmt, "tflops", "TFLOP/s", Kc, Wc)
        out["dtype"] = "w4(%s)/bf16 mfma/fp32 acc" % args.fmt
        print(json.dumps(out))
        return
    if wl != "all":
        print("unknown workload %s" % wl, file=sys.stderr)
        sys.exit(2)
    # the headline, then the rest of the metric
    head = decode_entry(c, "nvfp4", 1, K, W, cpu)
    sweep = {}
    t_start = time.perf_counter()
    for fmt_name in ("nvfp4", "int4", "int4sb", "bf16"):
        for T in (1, 4, 16, 64):
            if fmt_name == "nvfp4" and T == 1:
                continue
            sweep["decode_T%d_%s" % (T, fmt_name)] = decode_entry(c, fmt_name, T, K, W, scpu)
            print("[bench] decode T=%d %s done (%.0f s)" % (T, fmt_name, time.perf_counter() - t_start),
                  file=sys.stderr, flush=True)
        if fmt_name == "nvfp4":
            sweep["chain_b8_nvfp4"] = chain_entry(c, "nvfp4", Kc, Wc, scpu)
            print("[bench] chain done (%.0f s)" % (time.perf_counter() - t_start), file=sys.stderr, flush=True)
        c.drop(fmt_name)
        if fmt_name in ("int4sb", "bf16"):
            continue       # the matrix-core grouped GEMM takes NVFP4 and zero-point INT4 only
        sweep["prefill_%s" % fmt_name] = prefill_entry(c, fmt_name, Kc, Wc, scpu)
        c.torch.cuda.empty_cache()
        print("[bench] prefill %s done (%.0f s)" % (fmt_name, time.perf_counter() - t_start), file=sys.stderr,
              flush=True)
    for T in (1, 8):
        sweep["dense_head_T%d_nvfp4" % T] = dense_entry(c, "nvfp4", T, K, W, scpu)
        print("[bench] dense head T=%d done (%.0f s)" % (T, time.perf_counter() - t_start), file=sys.stderr,
              flush=True)
    out = line_from(head, "nvfp4", "tokens_per_s", "tokens/s", K, W)
    if args.spread_processes > 0:
        out["process_spread"] = process_spread(args, out["ms_per_step"], K, W)
        print("[bench] process spread done (%.0f s)" % (time.perf_counter() - t_start), file=sys.stderr, flush=True)
    out["sweep"] = sweep
    print(json.dumps(out))


if __name__ == "__main__":
    main()
