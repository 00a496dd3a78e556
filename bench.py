#!/usr/bin/env python3
"""Benchmark of the routed-expert FFN hot path on one MI355X.

Workload: a decode layer shaped like a 35B-A3B hybrid MoE (hidden 2048, 256
experts, top-8 softmax gating plus one always-on shared expert, expert FFN
512, gate/up Q4_K, down Q6_K), one token per step.  A step is one pass of the
whole hot path (router logits, top-k gating and expert lists, q8_K of x,
gate/up dequant-dot, SwiGLU, q8_K(h), down dequant-dot, weighted combine with
the shared expert) over one token.  Steps cycle through `--layers` distinct
synthetic layers resident in HBM, so, as in a real decoder stack, a step's
weights were last touched many steps earlier and stream from HBM rather than
from the 256 MB Infinity Cache.  The layers are captured as HIP graphs (per-layer
graphs as in the Strata summary's execution paragraph, and one graph for the
whole cycle, the way a decode step runs the stack) and replayed.

Output: one JSON line (metric, value = MoE-layer tokens/s, roofline of the
expert FFN, cpu_baseline = the CPU oracle on the host cores).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode B=1, verify B=4)"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle sample time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def build_layers(cfg, L, device):
    """Layer 0 from the numpy generator (the parity-tested one); layers 1..L-1
    from the same recipe drawn with torch's seeded device generator."""
    import torch
    from quantized_moe_expert_router_amd import moeq
    from quantized_moe_expert_router_amd import synthetic as syn

    layers = []
    lay0 = syn.gen_layer(cfg)
    dl0 = moeq.DeviceLayer(lay0, device=device)
    layers.append(dict(w_router=dl0.w_router, desc=dl0.ffn_desc(1), keep=dl0))
    gen = torch.Generator(device=device)
    for l in range(1, L):
        gen.manual_seed(cfg.seed * 1000 + l)
        keep = []

        def packed(fmt, rows, cols, n):
            aos = syn.gen_weight_blocks_device(fmt, rows * n, cols, gen, device)
            p = moeq.moeq_pack_experts(fmt, aos, n, rows, cols)
            keep.append(p)
            return p, moeq.moeq_packed_bytes(fmt, rows, cols)

        def table(fmt, rows, cols):
            p, pb = packed(fmt, rows, cols, cfg.E)
            t = torch.arange(cfg.E, dtype=torch.int64, device=device) * pb + p.data_ptr()
            keep.append(t)
            return t

        g, u, d = table(cfg.fmt_gate, cfg.F, cfg.H), table(cfg.fmt_up, cfg.F, cfg.H), table(cfg.fmt_down, cfg.H, cfg.F)
        sg, _ = packed(cfg.sh_fmt_gate, cfg.F_shared, cfg.H, 1)
        su, _ = packed(cfg.sh_fmt_up, cfg.F_shared, cfg.H, 1)
        sd, _ = packed(cfg.sh_fmt_down, cfg.H, cfg.F_shared, 1)
        wr = torch.randn((cfg.E, cfg.H), generator=gen, device=device, dtype=torch.float32) * 0.02
        desc = moeq.FfnDesc()
        desc.T, desc.H, desc.F, desc.E, desc.k = 1, cfg.H, cfg.F, cfg.E, cfg.k
        desc.fmt_gate, desc.fmt_up, desc.fmt_down = cfg.fmt_gate, cfg.fmt_up, cfg.fmt_down
        desc.gate, desc.up, desc.down = g.data_ptr(), u.data_ptr(), d.data_ptr()
        desc.F_shared = cfg.F_shared
        desc.sh_fmt_gate, desc.sh_fmt_up, desc.sh_fmt_down = cfg.sh_fmt_gate, cfg.sh_fmt_up, cfg.sh_fmt_down
        desc.sh_gate, desc.sh_up, desc.sh_down = sg.data_ptr(), su.data_ptr(), sd.data_ptr()
        layers.append(dict(w_router=wr, desc=desc, keep=keep))
    torch.cuda.synchronize()
    return layers


def cpu_baseline(cfg, seconds):
    """The CPU oracle, as it stands, on a bounded sample of decode tokens of layer 0."""
    import numpy as np
    import oracle
    from quantized_moe_expert_router_amd import synthetic as syn

    lay = syn.gen_layer(cfg)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))

    def run(n, seed):
        x = syn.gen_x(cfg, seed, 0, T=n)
        t0 = time.perf_counter()
        _, ids, w = oracle.route(x, lay.w_router, lay.bias, cfg.k, cfg.gating)
        oracle.expert_ffn(lay, ids, w, list(range(n)), x=x)
        return time.perf_counter() - t0

    probe = max(threads, 8)
    tp = run(probe, 4242)
    n = int(max(probe, min(20000, probe * seconds / max(tp, 1e-3))))
    dt = run(n, 4343)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d decode tokens (route + expert FFN) of the 2048x256x8+shared layer, %.1f s wall, "
                      "OpenMP over tokens" % (n, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from quantized_moe_expert_router_amd import moeq
    from quantized_moe_expert_router_amd import synthetic as syn

    dev = "cuda:0"
    torch.cuda.set_device(0)
    cfg = syn.CONFIGS["decode"]
    L = args.layers
    t_setup = time.time()
    layers = build_layers(cfg, L, dev)
    rng = np.random.default_rng(7)
    xs = [torch.from_numpy(rng.standard_normal((1, cfg.H)).astype(np.float32)).to(dev) for _ in range(L)]
    route_out = moeq.RouteOut(1, cfg.E, cfg.k, dev)
    route_ws = torch.empty(max(256, moeq.moeq_route_workspace(1, cfg.H, cfg.E, cfg.k, cfg.gating)),
                           dtype=torch.uint8, device=dev)
    xq = torch.empty((1, cfg.H // 256 * moeq.Q8K_BYTES), dtype=torch.uint8, device=dev)
    ffn_ws = torch.empty(moeq.moeq_expert_ffn_workspace(layers[0]["desc"]), dtype=torch.uint8, device=dev)
    y = torch.empty((1, cfg.H), dtype=torch.float32, device=dev)

    rdesc = moeq.RouteDesc(1, cfg.H, cfg.E, cfg.k, cfg.gating, 1.0)
    layer_ws = torch.empty(moeq.moeq_moe_layer_workspace(rdesc, layers[0]["desc"]), dtype=torch.uint8,
                           device=dev)

    def layer_step(l, stream=None):
        lay = layers[l]
        moeq.moeq_moe_layer(rdesc, lay["desc"], xs[l], lay["w_router"], None, route_out, None, y, layer_ws,
                            stream)

    def ffn_only(l, stream=None):
        lay = layers[l]
        moeq.moeq_expert_ffn(lay["desc"], xq, route_out.ids, route_out.w, route_out.offsets, route_out.pairs,
                             route_out.active, None, y, ffn_ws, stream)

    # Eager warm-up of every layer, then HIP graphs: one per layer and one for
    # the whole cycle of L layers (a decode step through the stack).
    for l in range(L):
        layer_step(l)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    graphs = []
    with torch.cuda.stream(stream):
        for l in range(L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                layer_step(l, stream)
            graphs.append(g)
        cycle = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cycle, stream=stream):
            for l in range(L):
                layer_step(l, stream)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    def run_steps(n):
        for _ in range(n // L):
            cycle.replay()
        for l in range(n % L):
            graphs[l].replay()

    # ---- timed region: exactly `steps` whole layers (value)
    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_per_step = dt * 1e3 / args.steps
    tokens_per_s = args.steps / dt

    # ---- expert FFN launches timed with HIP events on their stream, GPU kept
    # busy ahead of them so host launch overhead is hidden.
    cur = torch.cuda.current_stream()
    n_ev = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    moeq.moeq_route(xs[0], layers[0]["w_router"], None, cfg.k, cfg.gating, out=route_out, ws=route_ws,
                    x_q8K=xq)                # routing of layer 0 feeds every timed launch
    torch.cuda.synchronize()
    # calibrate a GPU busy-wait long enough for the host to enqueue all launches
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(cur)
    torch.cuda._sleep(1_000_000)
    c1.record(cur)
    torch.cuda.synchronize()
    per_cycle_ms = max(c0.elapsed_time(c1), 1e-3) / 1_000_000
    torch.cuda._sleep(int(min(2e9, (0.1 + n_ev * 50e-6) * 1e3 / per_cycle_ms)))
    for i in range(n_ev):
        starts[i].record(cur)
        ffn_only(i % L)
        ends[i].record(cur)
    torch.cuda.synchronize()
    ffn_us = float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e3

    # Algorithmic bytes of one expert FFN launch: the weights of the 8 selected
    # experts and the shared one, read once, plus q8_K(x) in and y out.
    eb = syn.expert_bytes(cfg)
    sb = syn.shared_bytes(cfg)
    ffn_bytes = cfg.k * eb + sb + cfg.H // 256 * 292 + cfg.H * 4
    layer_bytes = ffn_bytes + cfg.E * cfg.H * 4 + cfg.H * 4
    achieved = ffn_bytes / (ffn_us * 1e-6) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-dot/f64-combine (Q4_K,Q6_K x q8_K)",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": 1, "H": cfg.H, "E": cfg.E, "k": cfg.k, "F": cfg.F,
                   "shared_F": cfg.F_shared, "gate_up": "Q4_K", "down": "Q6_K", "layers_cycled": L,
                   "layer_bytes": layer_bytes, "parallelism": "single GPU"},
        "layer_hbm_gbs": layer_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "kernel": "expert FFN (gate/up GEMV + down GEMV)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "bytes_per_launch": ffn_bytes, "avg_launch_us": ffn_us},
        "cpu_baseline": cpu,
        "setup_s": setup_s,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
