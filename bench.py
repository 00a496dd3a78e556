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
expert FFN, cpu_baseline = the CPU oracle on the host cores), with the 4-token
verify, 16-token chunk and 8192-token prefill layers measured beside it.
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
    ap.add_argument("--no-verify", action="store_true", help="skip the verify (4-token) measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill measurement")
    ap.add_argument("--no-chunk", action="store_true", help="skip the 16-token chunk measurement")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a device copy of this many MiB (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench "
                         "into profiles/decode_ffn_hbm_traffic.json")
    return ap.parse_args()


KERNEL_SOURCES = ["common.hpp", "formats.hpp", "topk.hpp", "one_token.hpp", "ffn_gemv.hip", "route.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_ffn_hbm_traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_moe_expert_router_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per expert-FFN launch from the committed counter summary,
    or None when the kernels changed since the counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    return t["traffic_bytes_per_ffn"] if t.get("source_hash") == kernel_source_hash() else None


def summarize_pmc(fetch_dir, write_dir, calib_mib):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode layer's gate/up
    and down launches, scaled by what the same counters read for the copy of
    known size, summed per expert-FFN launch."""
    import csv
    import glob

    def load(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(f)) if r.get("Counter_Name") == counter]
        return rows

    out = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        rows = load(d, counter)
        per = {}
        for r in rows:
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        copy = [v for n, vs in per.items() if "copy" in n.lower() for v in vs]
        copy_kib = max(copy) if copy else None
        factor = (calib_mib * 1024.0 / copy_kib) if copy_kib else 1.0

        def med(key):
            vs = sorted(v for n, vv in per.items() if key in n for v in vv)
            return vs[len(vs) // 2] * factor if vs else None

        out[counter] = {"gateup_kib": med("k_gateup1<1, 1, 0>"), "down_kib": med("k_down_rows1"),
                        "logits_kib": med("k_logits"), "copy_kib_raw": copy_kib, "scale": factor}
    f, w = out["FETCH_SIZE"], out["WRITE_SIZE"]
    traffic = (f["gateup_kib"] + f["down_kib"] + w["gateup_kib"] + w["down_kib"]) * 1024.0
    res = {"source_hash": kernel_source_hash(), "calib_copy_mib": calib_mib, "counters": out,
           "traffic_bytes_per_ffn": traffic,
           "note": "median per dispatch of the expert-FFN-only launches (k_gateup1 with given ids, then k_down_rows1) "
                   "over 32 cycled layers"}
    json.dump(res, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(res, indent=1))


def build_layers(cfg, L, device, T):
    """Layer 0 from the numpy generator (the parity-tested one); layers 1..L-1
    from the same recipe drawn with torch's seeded device generator."""
    import torch
    from quantized_moe_expert_router_amd import moeq
    from quantized_moe_expert_router_amd import synthetic as syn

    layers = []
    lay0 = syn.gen_layer(cfg)
    dl0 = moeq.DeviceLayer(lay0, device=device)
    layers.append(dict(w_router=dl0.w_router, bias=dl0.bias, desc=dl0.ffn_desc(T), keep=dl0))
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
        wr = torch.randn((cfg.E, cfg.H), generator=gen, device=device, dtype=torch.float32) * 0.02
        desc = moeq.FfnDesc()
        desc.T, desc.H, desc.F, desc.E, desc.k = T, cfg.H, cfg.F, cfg.E, cfg.k
        desc.fmt_gate, desc.fmt_up, desc.fmt_down = cfg.fmt_gate, cfg.fmt_up, cfg.fmt_down
        desc.gate, desc.up, desc.down = g.data_ptr(), u.data_ptr(), d.data_ptr()
        if cfg.shared:
            sg, _ = packed(cfg.sh_fmt_gate, cfg.F_shared, cfg.H, 1)
            su, _ = packed(cfg.sh_fmt_up, cfg.F_shared, cfg.H, 1)
            sd, _ = packed(cfg.sh_fmt_down, cfg.H, cfg.F_shared, 1)
            desc.F_shared = cfg.F_shared
            desc.sh_fmt_gate, desc.sh_fmt_up, desc.sh_fmt_down = cfg.sh_fmt_gate, cfg.sh_fmt_up, cfg.sh_fmt_down
            desc.sh_gate, desc.sh_up, desc.sh_down = sg.data_ptr(), su.data_ptr(), sd.data_ptr()
        layers.append(dict(w_router=wr, bias=dl0.bias, desc=desc, keep=keep))
    torch.cuda.synchronize()
    return layers


class LayerCycle:
    """L synthetic layers of one shape with T tokens each, their per-layer HIP
    graphs and one graph for the whole cycle; run(n) replays exactly n layer
    steps (one step = the whole hot path of one layer over its T tokens)."""

    def __init__(self, cfg, T, L, device):
        import numpy as np
        import torch
        from quantized_moe_expert_router_amd import moeq
        self.cfg, self.T, self.L = cfg, T, L
        self.layers = build_layers(cfg, L, device, T)
        rng = np.random.default_rng(7)
        self.xs = [torch.from_numpy(rng.standard_normal((T, cfg.H)).astype(np.float32)).to(device)
                   for _ in range(L)]
        self.route_out = moeq.RouteOut(T, cfg.E, cfg.k, device)
        self.y = torch.empty((T, cfg.H), dtype=torch.float32, device=device)
        self.rdesc = moeq.RouteDesc(T, cfg.H, cfg.E, cfg.k, cfg.gating, 1.0)
        self.ws = torch.empty(moeq.moeq_moe_layer_workspace(self.rdesc, self.layers[0]["desc"]), dtype=torch.uint8,
                              device=device)
        for l in range(L):
            self.step(l)
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        self.graphs = []
        with torch.cuda.stream(stream):
            for l in range(L):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    self.step(l, stream)
                self.graphs.append(g)
            self.cycle = torch.cuda.CUDAGraph()
            with torch.cuda.graph(self.cycle, stream=stream):
                for l in range(L):
                    self.step(l, stream)
        torch.cuda.synchronize()

    def step(self, l, stream=None):
        from quantized_moe_expert_router_amd import moeq
        lay = self.layers[l]
        moeq.moeq_moe_layer(self.rdesc, lay["desc"], self.xs[l], lay["w_router"], lay["bias"], self.route_out, None,
                            self.y, self.ws, stream)

    def run(self, n):
        for _ in range(n // self.L):
            self.cycle.replay()
        for l in range(n % self.L):
            self.graphs[l].replay()

    def time(self, steps, warmup):
        import torch
        self.run(warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.run(steps)
        torch.cuda.synchronize()
        return time.perf_counter() - t0


def ffn_event_us(cyc, n_ev):
    """Mean duration of expert-FFN-only launches (moeq_expert_ffn on the routing
    of layer 0, weights cycling over the layers), timed with HIP events on the
    launch stream while a GPU busy-wait ahead of them hides host launch time."""
    import numpy as np
    import torch
    from quantized_moe_expert_router_amd import moeq
    cfg, T, L = cyc.cfg, cyc.T, cyc.L
    dev = cyc.y.device
    route_ws = torch.empty(max(256, moeq.moeq_route_workspace(T, cfg.H, cfg.E, cfg.k, cfg.gating)),
                           dtype=torch.uint8, device=dev)
    xq = torch.empty((T, cfg.H // 256 * moeq.Q8K_BYTES), dtype=torch.uint8, device=dev)
    ffn_ws = torch.empty(moeq.moeq_expert_ffn_workspace(cyc.layers[0]["desc"]), dtype=torch.uint8, device=dev)
    ro = cyc.route_out
    moeq.moeq_route(cyc.xs[0], cyc.layers[0]["w_router"], cyc.layers[0]["bias"], cfg.k, cfg.gating, out=ro,
                    ws=route_ws, x_q8K=xq)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(cur)
    torch.cuda._sleep(1_000_000)
    c1.record(cur)
    torch.cuda.synchronize()
    per_cycle_ms = max(c0.elapsed_time(c1), 1e-3) / 1_000_000
    torch.cuda._sleep(int(min(2e9, (0.1 + n_ev * 50e-6) * 1e3 / per_cycle_ms)))
    for i in range(n_ev):
        lay = cyc.layers[i % L]
        starts[i].record(cur)
        moeq.moeq_expert_ffn(lay["desc"], xq, ro.ids, ro.w, ro.offsets, ro.pairs, ro.active, None, cyc.y,
                             ffn_ws, None)
        ends[i].record(cur)
    torch.cuda.synchronize()
    return float(np.mean([s.elapsed_time(e) for s, e in zip(starts, ends)])) * 1e3


INT8_PEAK_TOPS = 5000.0


def secondary(name, L, steps, warmup, dev):
    """Whole-layer throughput of another workload (layers cycled so weights
    stream from HBM), its expert-FFN launch time, and the FFN's roofline
    figures: HBM GB/s over the union's weights, and int8-MFMA fraction of the
    useful integer work (2 ops per weight x activation product)."""
    import torch
    from quantized_moe_expert_router_amd import synthetic as syn
    cfg = syn.CONFIGS[name]
    cyc = LayerCycle(cfg, cfg.T, L, dev)
    dt = cyc.time(steps, warmup)
    ms = dt * 1e3 / steps
    ids = cyc.route_out.ids.cpu().numpy()
    union = len(set(ids.reshape(-1).tolist()))
    ffn_us = ffn_event_us(cyc, max(steps, 8))
    w_bytes = union * syn.expert_bytes(cfg) + (syn.shared_bytes(cfg) if cfg.shared else 0)
    layer_bytes = w_bytes + cfg.E * cfg.H * 4 + 2 * cfg.T * cfg.H * 4
    pairs = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    Fs = cfg.F_shared if cfg.shared else cfg.F
    ops = 2 * 3 * cfg.H * (cfg.T * cfg.k * cfg.F + (cfg.T * Fs if cfg.shared else 0))
    out = {"workload": cfg.name, "T": cfg.T, "tokens_per_s": cfg.T * steps / dt, "ms_per_step": ms,
           "layers_cycled": L, "union": union, "pairs": pairs, "layer_hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
           "ffn_us": ffn_us, "ffn_weight_gbs": w_bytes / (ffn_us * 1e-6) / 1e9,
           "ffn_int8_tops": ops / (ffn_us * 1e-6) / 1e12,
           "ffn_int8_mfma_frac": ops / (ffn_us * 1e-6) / 1e12 / INT8_PEAK_TOPS}
    del cyc
    torch.cuda.empty_cache()
    return out


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
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.calib_copy_mib or 256)
        return
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
    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    cfg = syn.CONFIGS["decode"]
    L = args.layers
    t_setup = time.time()
    cyc = LayerCycle(cfg, 1, L, dev)
    setup_s = time.time() - t_setup

    # ---- timed region: exactly `steps` whole layers (value)
    dt = cyc.time(args.steps, args.warmup)
    ms_per_step = dt * 1e3 / args.steps
    tokens_per_s = args.steps / dt

    # ---- expert FFN launches timed with HIP events on their stream
    ffn_us = ffn_event_us(cyc, args.steps)

    # Algorithmic bytes of one expert FFN launch: the weights of the 8 selected
    # experts and the shared one, read once, plus q8_K(x) in and y out.
    eb = syn.expert_bytes(cfg)
    sb = syn.shared_bytes(cfg)
    ffn_bytes = cfg.k * eb + sb + cfg.H // 256 * 292 + cfg.H * 4
    layer_bytes = ffn_bytes + cfg.E * cfg.H * 4 + cfg.H * 4
    achieved = ffn_bytes / (ffn_us * 1e-6) / 1e9
    del cyc
    torch.cuda.empty_cache()

    # ---- secondary: MTP verify rows (4 tokens per step, union of experts)
    verify = None
    if not args.no_verify:
        verify = secondary("verify", max(4, L // 4), max(8, args.steps // 4), max(4, args.warmup // 4), dev)
    # ---- secondary: 16-token chunk (sigmoid top-6, Q2_K/Q4_K experts, Q8_0 shared expert)
    chunk = None
    if not args.no_chunk:
        chunk = secondary("chunk16", max(4, L // 4), max(8, args.steps // 4), max(4, args.warmup // 4), dev)
    # ---- secondary: 8192-token prefill chunk (int8 MFMA grouped GEMM)
    prefill = None
    if not args.no_prefill:
        prefill = secondary("prefill", 2, args.prefill_steps, 2, dev)

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
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "bytes_per_launch": ffn_bytes, "avg_launch_us": ffn_us},
        "cpu_baseline": cpu,
        "verify_b4": verify,
        "chunk16_b16": chunk,
        "prefill_8192": prefill,
        "setup_s": setup_s,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
