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
from the 256 MB Infinity Cache.  The timed steps are one moeq_moe_stack call
(the MoE blocks of a decode step on a pre-norm residual stream: each layer
routes and runs on the RMS norm of the stream and adds its output to it, so
every layer's routing follows from the previous layers' outputs) captured as
a HIP graph and replayed; the same steps as single-layer calls on fixed
inputs, and as one single-layer graph each (per Strata summary's execution
paragraph), are reported beside it.

Output: one JSON line (metric, value = MoE-layer tokens/s, roofline of the
expert FFN, cpu_baseline = the CPU oracle on the host cores), with the 4-token
verify, 16-token chunk and 8192-token prefill layers measured beside it, and
the measured ceilings (a 4 GiB streaming read, an int8 MFMA loop) that the
rooflines are also read against.
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
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU oracle time over all layer shapes (all cores and one core)")
    ap.add_argument("--cpu-child", nargs=3, metavar=("CONFIG", "THREADS", "SECONDS"), help=argparse.SUPPRESS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="skip the verify (4-token) measurement")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8192-token prefill measurement")
    ap.add_argument("--no-chunk", action="store_true", help="skip the 16-token chunk measurement")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured HBM and int8-MFMA ceilings")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a device copy of this many MiB (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench "
                         "into profiles/decode_ffn_hbm_traffic.json")
    return ap.parse_args()


# the sources of the two launches the traffic counters measure (k_gateup1 with
# ids given, k_down_rows1)
KERNEL_SOURCES = ["common.hpp", "formats.hpp", "topk.hpp", "one_token.hpp", "ffn_gemv.hip", "launch.hpp"]
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


def build_layers(cfg, L, device, T, aux):
    """Layer 0 from the numpy generator (the parity-tested one); layers 1..L-1
    from the same recipe drawn with torch's seeded device generator.  Every
    layer's FFN gets the auxiliary stream `aux` (for a shared expert that runs
    apart from the routed launches)."""
    import torch
    from quantized_moe_expert_router_amd import moeq
    from quantized_moe_expert_router_amd import synthetic as syn

    layers = []
    lay0 = syn.gen_layer(cfg)
    dl0 = moeq.DeviceLayer(lay0, device=device)
    layers.append(dict(w_router=dl0.w_router, bias=dl0.bias, desc=dl0.ffn_desc(T, aux=aux), keep=dl0))
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
        aux.attach(desc)
        layers.append(dict(w_router=wr, bias=dl0.bias, desc=desc, keep=keep))
    torch.cuda.synchronize()
    return layers


class LayerCycle:
    """L synthetic layers of one shape with T tokens each.  A layer step is the
    whole hot path of one layer over its T tokens (one moeq_moe_layer call).

    time(steps, warmup) captures one HIP graph of exactly `steps` layer steps,
    layer (first + i) mod L for step i, and times one replay of it.  The
    warm-up before it replays max(warmup, L) steps, so every timed layer was
    last touched at least L - 1 layer steps earlier: with L layers whose
    weights together exceed the 256 MB Infinity Cache, each step streams its
    weights from HBM, as in a decoder stack.  The timed figure does not
    depend on how `steps` relates to L.  time_per_layer_graphs() times the
    same steps as one single-layer graph launch each (a graph per layer, as
    the Strata summary's execution paragraph describes)."""

    def __init__(self, cfg, T, L, device):
        import numpy as np
        import torch
        from quantized_moe_expert_router_amd import moeq
        self.cfg, self.T, self.L = cfg, T, L
        self.aux = moeq.AuxStream(device)
        self.layers = build_layers(cfg, L, device, T, self.aux)
        rng = np.random.default_rng(7)
        self.xs = [torch.from_numpy(rng.standard_normal((T, cfg.H)).astype(np.float32)).to(device)
                   for _ in range(L)]
        # RMS-norm gains of the stack's layers (around one)
        self.norm_w = [torch.from_numpy((1.0 + 0.1 * rng.standard_normal(cfg.H)).astype(np.float32)).to(device)
                       for _ in range(L)]
        # no logits output: the hot path needs ids, weights and lists only (from
        # 257 tokens the router then runs its approximate contraction with
        # exact rescoring)
        self.route_out = moeq.RouteOut(T, cfg.E, cfg.k, device, with_logits=False)
        self.y = torch.empty((T, cfg.H), dtype=torch.float32, device=device)
        self.rdesc = moeq.RouteDesc(T, cfg.H, cfg.E, cfg.k, cfg.gating, 1.0)
        self.ws = torch.empty(moeq.moeq_moe_layer_workspace(self.rdesc, self.layers[0]["desc"]), dtype=torch.uint8,
                              device=device)
        for l in range(L):
            self.step(l)
        torch.cuda.synchronize()
        self.stream = torch.cuda.Stream()
        self.graphs = [self.capture(l, 1) for l in range(L)]
        torch.cuda.synchronize()

    def step(self, l, stream=None):
        from quantized_moe_expert_router_amd import moeq
        lay = self.layers[l]
        moeq.moeq_moe_layer(self.rdesc, lay["desc"], self.xs[l], lay["w_router"], lay["bias"], self.route_out, None,
                            self.y, self.ws, stream)

    def capture(self, first, n):
        """One graph of n layer steps: layers first, first+1, ... (mod L)."""
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    self.step((first + i) % self.L, self.stream)
        return g

    def time(self, steps, warmup):
        import torch
        wsteps = max(warmup, self.L)
        gw = self.capture(0, wsteps)
        gt = self.capture(wsteps % self.L, steps)
        torch.cuda.synchronize()
        gw.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gt.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del gw, gt
        return dt, wsteps

    def capture_stack(self, first, n, y, out, ws):
        """One graph of one stack call over n layers (first, first+1, ... mod L)
        on the residual stream y (y = x, then y += MoE_l(RMSNorm_l(y)) per
        layer)."""
        import torch
        from quantized_moe_expert_router_amd import moeq
        idx = [(first + i) % self.L for i in range(n)]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            with torch.cuda.graph(g, stream=self.stream):
                moeq.moeq_moe_stack(self.rdesc, [self.layers[l]["desc"] for l in idx],
                                    [self.layers[l]["w_router"] for l in idx], [self.layers[l]["bias"] for l in idx],
                                    self.xs[first], out, y, ws, self.stream,
                                    norm_ws=[self.norm_w[l] for l in idx], norm_eps=NORM_EPS)
        return g

    def time_stack(self, steps, warmup):
        """The decode step as one stack call (moeq_moe_stack) of exactly
        `steps` layers, after a warm-up stack of max(warmup, L) layers."""
        import torch
        from quantized_moe_expert_router_amd import moeq
        wsteps = max(warmup, self.L)
        n = max(wsteps, steps)
        y = torch.empty_like(self.xs[0])
        out = moeq.StackOut(n, self.T, self.cfg.E, self.cfg.k, y.device)
        descs = [self.layers[i % self.L]["desc"] for i in range(min(n, self.L))]
        ws = torch.empty(moeq.moeq_moe_stack_workspace(self.rdesc, descs), dtype=torch.uint8, device=y.device)
        gw = self.capture_stack(0, wsteps, y, out, ws)
        gt = self.capture_stack(wsteps % self.L, steps, y, out, ws)
        torch.cuda.synchronize()
        gw.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gt.replay()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del gw, gt
        if not bool(torch.isfinite(y).all()):
            raise RuntimeError("the residual stream is not finite after the timed stack")
        return dt, wsteps

    def time_per_layer_graphs(self, steps, warmup):
        import torch
        wsteps = max(warmup, self.L)
        for i in range(wsteps):
            self.graphs[i % self.L].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.graphs[(wsteps + i) % self.L].replay()
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
NORM_EPS = 1e-6
CEIL_READ_BYTES = 4 << 30
CEIL_READ_BLOCKS = 1 << 19
CEIL_MFMA_BLOCKS = 4096
CEIL_MFMA_ITERS = 2000


def measure_ceilings(dev, reps=10):
    """Measured ceilings of the two rooflines, read beside the nominal peaks:
    a streaming read of a 4 GiB buffer with the plain 16-byte global loads the
    kernels use (GB/s), and a register-only loop of independent int8 MFMAs
    (TOPS).  Each is the median of `reps` launches timed with HIP events on
    the stream they run on, after two untimed ones."""
    import numpy as np
    import torch
    from quantized_moe_expert_router_amd import moeq
    st = torch.cuda.current_stream()
    buf = torch.zeros(CEIL_READ_BYTES, dtype=torch.uint8, device=dev)
    sums = torch.empty(CEIL_READ_BLOCKS, dtype=torch.int64, device=dev)
    flags = torch.empty(4 * CEIL_MFMA_BLOCKS, dtype=torch.int32, device=dev)
    L = moeq.lib()
    sp = st.cuda_stream

    def read():
        moeq._check("moeq_ceiling_read", L.moeq_ceiling_read(buf.data_ptr(), CEIL_READ_BYTES, CEIL_READ_BLOCKS,
                                                             sums.data_ptr(), sp))

    def mfma():
        moeq._check("moeq_ceiling_mfma_i8", L.moeq_ceiling_mfma_i8(CEIL_MFMA_ITERS, CEIL_MFMA_BLOCKS,
                                                                   flags.data_ptr(), sp))

    def median_ms(fn):
        fn()
        fn()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    t_read = median_ms(read)
    t_mfma = median_ms(mfma)
    assert int(sums.sum().item()) == 0, "ceiling read: the zero buffer summed to a nonzero value"
    assert bool((flags == 128 * CEIL_MFMA_ITERS).all().item()), "ceiling MFMA loop: wrong step count"
    ops = CEIL_MFMA_BLOCKS * 4 * CEIL_MFMA_ITERS * 4 * 2 * 32 * 32 * 32
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read": {"value": CEIL_READ_BYTES / (t_read * 1e-3) / 1e9, "unit": "GB/s",
                         "bytes": CEIL_READ_BYTES, "launch_us": t_read * 1e3,
                         "kernel": "moeq_ceiling_read: plain 16-byte global loads, grid-stride, "
                                   "%d workgroups x 256 threads, 4 loads in flight per thread" % CEIL_READ_BLOCKS},
            "int8_mfma": {"value": ops / (t_mfma * 1e-3) / 1e12, "unit": "TOPS", "ops": ops,
                          "launch_us": t_mfma * 1e3,
                          "kernel": "moeq_ceiling_mfma_i8: 4 independent v_mfma_i32_32x32x32_i8 chains per wave, "
                                    "%d workgroups x 4 waves, %d steps" % (CEIL_MFMA_BLOCKS, CEIL_MFMA_ITERS)}}


def layer_bytes_of(cfg, union):
    """Algorithmic bytes of one layer step: the weights of the experts in the
    union (each read once) and of the shared expert, the router weights, x in
    and y out."""
    from quantized_moe_expert_router_amd import synthetic as syn
    w_bytes = union * syn.expert_bytes(cfg) + (syn.shared_bytes(cfg) if cfg.shared else 0)
    return w_bytes, w_bytes + cfg.E * cfg.H * 4 + 2 * cfg.T * cfg.H * 4


def secondary(name, L, steps, warmup, dev):
    """Whole-layer throughput of another workload (layers cycled so weights
    stream from HBM), its expert-FFN launch time, and the FFN's roofline
    figures: HBM GB/s over the union's weights, and int8-MFMA fraction of the
    useful integer work (2 ops per weight x activation product)."""
    import torch
    from quantized_moe_expert_router_amd import synthetic as syn
    cfg = syn.CONFIGS[name]
    cyc = LayerCycle(cfg, cfg.T, L, dev)
    dt, _ = cyc.time(steps, warmup)
    ms = dt * 1e3 / steps
    ids = cyc.route_out.ids.cpu().numpy()
    union = len(set(ids.reshape(-1).tolist()))
    ffn_us = ffn_event_us(cyc, max(steps, 8))
    w_bytes, layer_bytes = layer_bytes_of(cfg, union)
    pairs = cfg.T * cfg.k + (cfg.T if cfg.shared else 0)
    Fs = cfg.F_shared if cfg.shared else cfg.F
    ops = 2 * 3 * cfg.H * (cfg.T * cfg.k * cfg.F + (cfg.T * Fs if cfg.shared else 0))
    out = {"workload": cfg.name, "T": cfg.T, "tokens_per_s": cfg.T * steps / dt, "ms_per_step": ms,
           "steps": steps, "layers_cycled": L, "union": union, "pairs": pairs,
           "layer_hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
           "ffn_us": ffn_us, "ffn_weight_gbs": w_bytes / (ffn_us * 1e-6) / 1e9,
           "ffn_int8_tops": ops / (ffn_us * 1e-6) / 1e12,
           "ffn_int8_mfma_frac": ops / (ffn_us * 1e-6) / 1e12 / INT8_PEAK_TOPS}
    del cyc
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_child(name, threads, seconds):
    """Child process (OMP_NUM_THREADS = threads): the CPU oracle, as it stands,
    on a bounded sample of tokens of the named layer shape (router + expert
    FFN, the sample's tokens in one oracle call; tokens are independent rows,
    so a decode shape's sample is a batch of decode tokens).  Prints one JSON
    object."""
    import numpy as np
    import oracle
    from quantized_moe_expert_router_amd import synthetic as syn

    cfg = syn.CONFIGS[name]
    lay = syn.gen_layer(cfg, T=1)

    def run(n, seed):
        x = syn.gen_x(cfg, seed, 0, T=n)
        t0 = time.perf_counter()
        _, ids, w = oracle.route(x, lay.w_router, lay.bias, cfg.k, cfg.gating)
        oracle.expert_ffn(lay, ids, w, list(range(n)), x=x)
        return time.perf_counter() - t0

    n = 1
    dt = run(n, 4242)
    for it in range(3):
        if dt >= seconds / 2:
            break
        n = min(1 << 16, max(n * 2, int(n * seconds / max(dt, 1e-4))))
        dt = run(n, 4343 + it)
    print(json.dumps({"tokens": n, "seconds": dt, "tokens_per_s": n / dt}), flush=True)


def cpu_baseline(seconds):
    """The CPU oracle on the host cores: every layer shape, on all cores and on
    one core, each on a bounded sample of its tokens (a child process per run,
    so OpenMP takes the stated thread count)."""
    import subprocess
    from quantized_moe_expert_router_amd import synthetic as syn
    all_threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    per = {}
    per_run = seconds / (2 * len(syn.CONFIG_ORDER))
    for name in syn.CONFIG_ORDER:
        cfg = syn.CONFIGS[name]
        row = {"workload": cfg.name}
        for label, th in (("all_cores", all_threads), ("one_core", 1)):
            env = dict(os.environ, OMP_NUM_THREADS=str(th))
            r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-child", name, str(th),
                                str(per_run)], capture_output=True, text=True, env=env, timeout=600)
            if r.returncode != 0:
                raise RuntimeError("CPU oracle run failed for %s: %s" % (name, r.stderr[-2000:]))
            res = json.loads(r.stdout.strip().splitlines()[-1])
            row[label] = {"tokens_per_s": res["tokens_per_s"], "tokens": res["tokens"],
                          "seconds": res["seconds"], "threads": th}
        per[name] = row
    d = per["decode"]["all_cores"]
    return {"value": d["tokens_per_s"], "unit": "tokens/s", "cores": all_threads, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": "%d decode tokens (router + expert FFN) of the hidden-2048, 256-expert top-8 + shared layer, "
                      "%.2f s wall on %d OpenMP threads; per_config: every layer shape on all cores and on one "
                      "core, a sample of its tokens each" % (d["tokens"], d["seconds"], all_threads),
            "per_config": per}


def main():
    args = parse()
    if args.cpu_child:
        cpu_child(args.cpu_child[0], int(args.cpu_child[1]), float(args.cpu_child[2]))
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.calib_copy_mib or 256)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch
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

    # ---- timed region: the decode step as one stack call of exactly `steps`
    # layers on the residual stream (value)
    dt, wsteps = cyc.time_stack(args.steps, args.warmup)
    ms_per_step = dt * 1e3 / args.steps
    tokens_per_s = args.steps / dt
    # ---- secondaries: the same steps as single-layer calls in one graph, and
    # as one single-layer graph launch each
    dt_lc, _ = cyc.time(args.steps, args.warmup)
    dt_pl = cyc.time_per_layer_graphs(args.steps, args.warmup)

    # ---- expert FFN launches timed with HIP events on their stream
    ffn_us = ffn_event_us(cyc, max(args.steps, 32))

    # Algorithmic bytes of one expert FFN launch: the weights of the 8 selected
    # experts and the shared one, read once, plus q8_K(x) in and y out.
    eb = syn.expert_bytes(cfg)
    sb = syn.shared_bytes(cfg)
    ffn_bytes = cfg.k * eb + sb + cfg.H // 256 * 292 + cfg.H * 4
    layer_bytes = ffn_bytes + cfg.E * cfg.H * 4 + cfg.H * 4
    achieved = ffn_bytes / (ffn_us * 1e-6) / 1e9
    del cyc
    torch.cuda.empty_cache()

    sub_steps = max(8, args.steps // 4)
    sub_warm = max(4, args.warmup // 4)
    # ---- secondary: MTP verify rows (4 tokens per step, union of experts)
    verify = None
    if not args.no_verify:
        verify = secondary("verify", max(4, L // 4), sub_steps, sub_warm, dev)
    # ---- secondary: 16-token chunk (sigmoid top-6, Q2_K/Q4_K experts, Q8_0 shared expert)
    chunk = None
    if not args.no_chunk:
        chunk = secondary("chunk16", max(4, L // 4), sub_steps, sub_warm, dev)
    # ---- secondary: 8192-token prefill chunk (int8 MFMA grouped GEMM)
    prefill = None
    if not args.no_prefill:
        prefill = secondary("prefill", 2, args.prefill_steps, 2, dev)

    ceil = None
    if not args.no_ceilings:
        ceil = measure_ceilings(dev)
        if prefill is not None:
            prefill["ffn_int8_frac_of_measured"] = prefill["ffn_int8_tops"] / ceil["int8_mfma"]["value"]
        for sec in (verify, chunk):
            if sec is not None:
                sec["ffn_weight_frac_of_measured"] = sec["ffn_weight_gbs"] / ceil["hbm_read"]["value"]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)

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
                   "layer_bytes": layer_bytes, "parallelism": "single GPU",
                   "timing": "one HIP graph of one moeq_moe_stack call over exactly `steps` layers cycling the "
                             "layers on a pre-norm residual stream, after a warm-up stack of %d layers (at least "
                             "one whole cycle)" % wsteps},
        "layer_hbm_gbs": layer_bytes / (ms_per_step * 1e-3) / 1e9,
        "layer_calls_graph": {"tokens_per_s": args.steps / dt_lc, "ms_per_step": dt_lc * 1e3 / args.steps,
                              "note": "the same layer steps as moeq_moe_layer calls on fixed per-layer inputs "
                                      "in one graph"},
        "per_layer_graphs": {"tokens_per_s": args.steps / dt_pl, "ms_per_step": dt_pl * 1e3 / args.steps,
                             "note": "the same layer steps, one single-layer graph launch each"},
        "roofline": {"bound": "hbm", "kernel": "expert FFN (gate/up GEMV + down GEMV)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "bytes_per_launch": ffn_bytes, "avg_launch_us": ffn_us,
                     "frac_of_measured": achieved / ceil["hbm_read"]["value"] if ceil else None},
        "ceilings": ceil,
        "cpu_baseline": cpu,
        "verify_b4": verify,
        "chunk16_b16": chunk,
        "prefill_8192": prefill,
        "setup_s": setup_s,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
