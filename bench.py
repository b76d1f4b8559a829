"""Benchmark of the W4A16 MoE layer on one MI355X.

Default workload: one Flint-shaped MoE decode layer at batch 1 (hidden 2048,
256 experts top-6 + 1 shared expert, expert inter 768, NVFP4 W4A16 weights,
bf16 activations).  One step = one moe_layer_decode call on one token: router
GEMV, top-k + softmax, expert grouping, gate/up + SwiGLU, down projection,
shared expert and combine.  Steps rotate over independently seeded weight
copies (more than twice the size of the on-die caches) and fresh tokens, so
weights stream from HBM; K steps are captured in one HIP graph and replayed.

Other workloads (--workload): decode batch sweep (decode_T4, decode_T16,
decode_T64, with --fmt int4), the 47-layer batch-8 chain (chain_b8), the
4096-token prefill (prefill), and hbm_copy: a plain 1 GiB device copy whose
HBM counter readings calibrate the traffic figures of the others.

Prints ONE JSON line (rank 0).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# HBM bytes per measured unit (one layer call; the prefill's grouped FFN) from two rocprofv3
# --pmc runs of the same workload with the current kernels: FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0,
# the factors that make the counters read 1 GiB each for a plain 1 GiB device copy
# (profiles/hbm_traffic_counters.md).  Workloads not listed report null.
TRAFFIC_BYTES = {
    ("decode_b1", "nvfp4"): 21.75e6,
    ("decode_T16", "nvfp4"): 222.9e6,
    ("prefill", "nvfp4"): 1239.0e6,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_b1")
    p.add_argument("--fmt", default="nvfp4", choices=["nvfp4", "int4"])
    p.add_argument("--copies", type=int, default=8, help="independently seeded weight copies to rotate over")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the CPU oracle leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_weight_only_moe_amd as moe
    import synth

    dev = "cuda"
    fmt = synth.FMT_NAMES[args.fmt]
    workload = args.workload
    if workload == "prefill":
        return bench_prefill(args, fmt)
    if workload == "chain_b8":
        return bench_chain(args, fmt)
    if workload == "hbm_copy":
        return bench_copy(args)
    T = {"decode_b1": 1, "decode_T4": 4, "decode_T16": 16, "decode_T64": 64}.get(workload)
    if T is None:
        print("unknown workload %s" % workload, file=sys.stderr)
        sys.exit(2)
    H, I, E, k = 2048, 768, 256, 6
    R = max(1, args.copies)
    K, W = args.steps, args.warmup

    layers = [synth.make_layer(fmt, H, I, E, k, synth.seed_of(1, r), dev) for r in range(R)]
    Ls = [moe.Layer(l) for l in layers]
    NX = max(K, W, 1)
    xs = [synth.make_tokens(T, H, synth.seed_of(2, i), dev) for i in range(NX)]
    ys = [torch.empty_like(x) for x in xs]
    ids = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(NX)]
    ws_ = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in range(NX)]
    nws = moe.moe_layer_decode_workspace_size(Ls[0], T)
    wsb = torch.zeros(nws, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream()

    def step(i, s):
        moe.moe_layer_decode(Ls[i % R], xs[i % NX], None, T, ys[i % NX], ids[i % NX], ws_[i % NX], wsb, nws, stream=s)

    with torch.cuda.stream(stream):
        for i in range(W):
            step(i, stream)
    torch.cuda.synchronize()

    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(K):
                step(i, stream)
        graph.replay()              # untimed warm replay
        torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                step(i, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    ms_per_step = ms / K

    # algorithmic bytes: distinct touched experts (from the realised routing) + shared expert
    eb = synth.expert_bytes(fmt, H, I)
    touched = []
    for i in range(K):
        touched.append(len(np.unique(ids[i % NX].cpu().numpy())) + 1)
    bytes_per_step = eb * float(np.mean(touched))
    router_bytes = E * H * 4
    achieved_gbs = bytes_per_step / (ms_per_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        sample_layers = 2
        hosts = []
        for r in range(sample_layers):
            used = set()
            for i in range(r, min(NX, 64), R):
                used |= set(ids[i].cpu().numpy().ravel().tolist())
            hosts.append(synth.layer_to_numpy(layers[r], experts=used))
        # the steps r, r+R, ... ran on weight copy r: their experts are in the host copy
        xs_bits = []
        for r in range(sample_layers):
            for i in range(r, min(NX, 64), R):
                xs_bits.append((r, synth.bits16(xs[i])))
        import oracle
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            blas_threads = 1
        t0 = time.perf_counter()
        n_tok = 0
        j = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            r, xbits = xs_bits[j % len(xs_bits)]
            oracle.moe_layer(hosts[r], xbits)
            n_tok += xbits.shape[0]
            j += 1
        el = time.perf_counter() - t0
        cpu = {"value": n_tok / el, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
               "sample": "%d layer calls of the same workload (T=%d, %s, %d of %d weight copies), "
                         "%.1f s of float64 numpy oracle incl. dequantisation of the touched experts"
                         % (j, T, args.fmt, sample_layers, R, el)}

    out = {
        "metric": "MoE decode tokens/s and weight HBM GB/s (% of peak), batch 1-64; prefill TFLOP/s",
        "value": T * K / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "w4(%s)/bf16 act/fp32 acc" % args.fmt,
        "data": "synthetic",
        "config": {"workload": "moe_decode_layer T=%d %s H=2048 I=768 E=256 top6+1shared" % (T, args.fmt),
                   "tokens_per_step": T, "weight_copies": R, "graph": graph is not None,
                   "expert_bytes_per_step": bytes_per_step, "router_bytes_per_step": router_bytes,
                   "distinct_experts_per_step": float(np.mean(touched))},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": TRAFFIC_BYTES.get((workload, args.fmt)),
                     "kernel": "moe_layer_decode: k_layer_route_shared + k_layer_gateup + %s "
                               "(one layer call, events on the launch stream)"
                               % ("k_layer_down_t1" if T == 1 else "k_layer_down_combine"),
                     "bytes": "expert weights of the distinct touched experts + shared expert, per call"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def timed_graph(torch, stream, body, K, W, use_graph=True):
    """Warm up W eager steps, capture K steps in one graph, time one replay
    (or, without a graph, time K eager steps)."""
    with torch.cuda.stream(stream):
        for i in range(W):
            body(i, stream)
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(K):
                body(i, stream)
        graph.replay()
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(K):
                body(i, stream)
        ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1)


def bench_copy(args):
    """A plain device copy of 1 GiB (torch's copy kernel): 1 GiB read + 1 GiB written per step."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    K, W = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
    stream = torch.cuda.Stream()
    for _ in range(W):
        with torch.cuda.stream(stream):
            dst.copy_(src)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(K):
            dst.copy_(src)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    gbs = 2.0 * n * K / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": "device copy GB/s (read + write)", "value": gbs, "unit": "GB/s", "n_gpus": 1,
                      "steps": K, "warmup": W, "ms_per_step": ms / K, "higher_is_better": True,
                      "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
                      "config": {"workload": "hbm_copy 1 GiB", "bytes_read_per_step": n,
                                 "bytes_written_per_step": n},
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "torch copy"},
                      "cpu_baseline": None}))


def bench_prefill(args, fmt):
    """4096-token prefill of one Flint-shaped layer with Zipf(1.1) expert popularity."""
    import torch
    import bit_weight_only_moe_amd as moe
    import synth
    dev = "cuda"
    H, I, E, k, T = 2048, 768, 256, 6, 4096
    R = max(1, min(args.copies, 2))
    K, W = max(1, min(args.steps, 10)), max(1, min(args.warmup, 2))
    layers = [synth.make_layer(fmt, H, I, E, k, synth.seed_of(5, r), dev) for r in range(R)]
    x = synth.make_tokens(T, H, 5, dev)
    zl = synth.zipf_logits(T, E, 1.1, 5, dev)
    n = T * k
    lg = torch.empty((T, E), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sp = torch.empty(n, dtype=torch.int32, device=dev)
    pp = torch.empty(n, dtype=torch.int32, device=dev)
    pws_n = moe.moe_permute_workspace_size(T, k, E)
    pws = torch.empty(pws_n, dtype=torch.uint8, device=dev)
    out = torch.empty((n, H), dtype=torch.float32, device=dev)
    out_s = torch.empty((T, H), dtype=torch.float32, device=dev)
    off_s = torch.tensor([0, T], dtype=torch.int32, device=dev)
    gws_n = max(moe.moe_grouped_ffn_workspace_size(E, H, I, n), moe.moe_grouped_ffn_workspace_size(1, H, I, T))
    gws = torch.empty(gws_n, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    f_routed = [moe.ffn_weights(l["experts"]) for l in layers]
    f_shared = [moe.ffn_weights(l["shared"]) for l in layers]

    # The shared expert needs no routing: its grouped FFN runs on a side stream
    # (own workspace), forked after the top-k, alongside the permute kernels,
    # which leave most of the chip idle, and the start of the routed FFN; both
    # join before the combine.  (Forked before the router it slows the router
    # about as much as it gains; forked before the top-k it slows the top-k.)
    side = torch.cuda.Stream()
    gws_s = torch.empty(gws_n, dtype=torch.uint8, device=dev)

    def shared_ffn(i, s):
        side.wait_stream(s)
        moe.moe_grouped_w4a16_ffn(f_shared[i % R], 1, H, I, x, None, 1, off_s, T, out_s, moe.MOE_MODE_AUTO, gws_s,
                                  gws_n, stream=side)

    def routed_ffn(i, s):
        moe.moe_grouped_w4a16_ffn(f_routed[i % R], E, H, I, x, sp, k, offsets, n, out, moe.MOE_MODE_AUTO, gws,
                                  gws_n, stream=s)

    def step(i, s):
        L = layers[i % R]
        moe.moe_route(x, L["w_router"], T, H, E, k, lg, ids, w, stream=s)   # router GEMM (timed; skewed logits route)
        moe.moe_topk_softmax(zl, T, E, k, ids, w, stream=s)
        shared_ffn(i, s)
        moe.moe_permute(ids, T, k, E, counts, offsets, sp, pp, None, None, 0, pws, pws_n, stream=s)
        routed_ffn(i, s)
        s.wait_stream(side)
        moe.moe_combine(out, pp, w, out_s, x, T, k, H, y, stream=s)

    def ffn_pair(i, s):
        shared_ffn(i, s)
        routed_ffn(i, s)
        s.wait_stream(side)

    stream = torch.cuda.Stream()
    ms = timed_graph(torch, stream, step, K, W, not args.no_graph)
    # the grouped FFN alone (routed + shared), timed the same way
    ms_ffn = timed_graph(torch, stream, ffn_pair, K, W, not args.no_graph)
    flops = 6.0 * (n + T) * H * I
    c = counts.cpu().numpy()
    out_line = {
        "metric": "MoE decode tokens/s and weight HBM GB/s (% of peak), batch 1-64; prefill TFLOP/s",
        "value": flops / (ms / K * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "w4(%s)/bf16 mfma/fp32 acc" % args.fmt, "data": "synthetic",
        "config": {"workload": "moe_prefill T=4096 %s H=2048 I=768 E=256 top6+1shared zipf1.1" % args.fmt,
                   "expert_gflop": flops / 1e9, "tokens_per_s": T * K / (ms * 1e-3),
                   "max_rows_per_expert": int(c.max()), "min_rows_per_expert": int(c.min()), "weight_copies": R},
        "roofline": {"bound": "mfma", "achieved": flops / (ms_ffn / K * 1e-3) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / (ms_ffn / K * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": TRAFFIC_BYTES.get(("prefill", args.fmt)),
                     "kernel": "moe_grouped_w4a16_ffn routed + shared: k_tile_table, %s gate/up, %s down"
                               % (("k_mfma_bl",) * 2 if fmt == 1 else ("k_mfma_bd",) * 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(out_line))


def bench_chain(args, fmt):
    """One decode step through 47 chained MoE layers at batch 8.

    Layer l adds its MoE output to the residual stream r: r_{l+1} = r_l + MoE_l(x_l).
    In the model x_l is the normalised residual; the normalisation is outside the
    MoE layer, so each layer reads a seeded unit-scale stand-in x_l and the chain
    runs through the residual (without it, SwiGLU's roughly quadratic growth would
    overflow bf16 within a few layers)."""
    import torch
    import bit_weight_only_moe_amd as moe
    import synth
    dev = "cuda"
    H, I, E, k, T, NL = 2048, 768, 256, 6, 8, 47
    K, W = max(1, min(args.steps, 20)), max(1, min(args.warmup, 3))
    layers = [synth.make_layer(fmt, H, I, E, k, synth.seed_of(4, l), dev) for l in range(NL)]
    Ls = [moe.Layer(l) for l in layers]
    xin = [synth.make_tokens(T, H, synth.seed_of(5, l), dev) for l in range(NL)]
    rs = [synth.make_tokens(T, H, 4, dev)] + [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    ids = [torch.empty((T, k), dtype=torch.int32, device=dev) for _ in range(NL)]
    ws_ = [torch.empty((T, k), dtype=torch.float32, device=dev) for _ in range(NL)]
    nws = moe.moe_layer_decode_workspace_size(Ls[0], T)
    wsb = torch.zeros(nws, dtype=torch.uint8, device=dev)

    def step(i, s):
        for l in range(NL):
            moe.moe_layer_decode(Ls[l], xin[l], rs[l], T, rs[l + 1], ids[l], ws_[l], wsb, nws, stream=s)

    stream = torch.cuda.Stream()
    ms = timed_graph(torch, stream, step, K, W)
    eb = synth.expert_bytes(fmt, H, I)
    bytes_step = sum((len(np.unique(ids[l].cpu().numpy())) + 1) * eb for l in range(NL))
    gbs = bytes_step / (ms / K * 1e-3) / 1e9
    out_line = {
        "metric": "MoE decode tokens/s and weight HBM GB/s (% of peak), batch 1-64; prefill TFLOP/s",
        "value": T * K / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": ms / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "w4(%s)/bf16 act/fp32 acc" % args.fmt, "data": "synthetic",
        "config": {"workload": "moe_decode_chain 47 layers T=8 %s H=2048 I=768 E=256 top6+1shared" % args.fmt,
                   "expert_bytes_per_step": bytes_step, "resident_weight_bytes": NL * (E + 1) * eb},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "kernel": "47 x moe_layer_decode"},
        "cpu_baseline": None,
    }
    print(json.dumps(out_line))


if __name__ == "__main__":
    main()
