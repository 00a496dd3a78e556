"""moeq_moe_layer_noalloc (static per-GPU workspace) against moeq_moe_layer
(caller workspace), both through the C ABI: the same kernels run, so every
output must be identical.  Two calls in a row on the static workspace, the
second with a smaller input (it finds the first call's contents there)."""
import numpy as np
import pytest
import torch

from guards import GuardedAlloc
from quantized_moe_expert_router_amd import moeq
from quantized_moe_expert_router_amd import synthetic as syn

pytestmark = pytest.mark.gpu


def _outputs(ga, T, cfg, tag):
    out = moeq.RouteOut(T, cfg.E, cfg.k, "cuda")
    out.logits = ga.empty((T, cfg.E), torch.float64, tag + " logits")
    out.ids = ga.empty((T, cfg.k), torch.int32, tag + " ids")
    out.w = ga.empty((T, cfg.k), torch.float32, tag + " w")
    out.offsets = ga.empty(cfg.E + 1, torch.int32, tag + " offsets")
    out.pairs = ga.empty(max(1, T * cfg.k), torch.int32, tag + " pairs")
    out.active = ga.empty(1 + min(cfg.E, T * cfg.k), torch.int32, tag + " active")
    y = ga.empty((T, cfg.H), torch.float32, tag + " y")
    return out, y


def _host(out, y, T, k):
    act = out.active.cpu().numpy()
    return dict(logits=out.logits.cpu().numpy(), ids=out.ids.cpu().numpy(), w=out.w.cpu().numpy(),
                offsets=out.offsets.cpu().numpy(), pairs=out.pairs.cpu().numpy()[:T * k],
                active=act[:1 + act[0]], y=y.cpu().numpy())


def _run_both(name, stream):
    cfg = syn.CONFIGS[name]
    layer = syn.gen_layer(cfg)
    dl = moeq.DeviceLayer(layer)
    aux = moeq.AuxStream()
    fdesc = dl.ffn_desc(cfg.T, aux=aux)
    rdesc = moeq.RouteDesc(cfg.T, cfg.H, cfg.E, cfg.k, cfg.gating, 1.0)
    assert 0 < moeq.moeq_moe_layer_workspace(rdesc, fdesc) <= moeq.NOALLOC_MAX_BYTES
    x = torch.from_numpy(layer.x).cuda()
    ga = GuardedAlloc()
    o_ref, y_ref = _outputs(ga, cfg.T, cfg, "ref")
    o_st, y_st = _outputs(ga, cfg.T, cfg, "noalloc")
    ws = ga.empty(moeq.moeq_moe_layer_workspace(rdesc, fdesc), torch.uint8, "ws")
    with torch.cuda.stream(stream):
        moeq.moeq_moe_layer(rdesc, fdesc, x, dl.w_router, dl.bias, o_ref, None, y_ref, ws, stream)
        moeq.moeq_moe_layer_noalloc(rdesc, fdesc, x, dl.w_router, dl.bias, o_st, None, y_st, stream)
    torch.cuda.synchronize()
    ga.check(name)
    a, b = _host(o_ref, y_ref, cfg.T, cfg.k), _host(o_st, y_st, cfg.T, cfg.k)
    for key in a:
        assert np.array_equal(a[key], b[key]), (name, key)
    assert np.isfinite(b["y"]).all() and np.abs(b["y"]).max() > 0
    return b


def test_noalloc_matches_layer_call_twice_shrinking():
    stream = torch.cuda.Stream()
    print("[gpu-case] noalloc chunk16 then decode", flush=True)
    _run_both("chunk16", stream)        # 16 tokens, MFMA tiles, shared expert on the auxiliary stream
    _run_both("decode", stream)         # then one token: the one-token kernels on the same static workspace


def test_noalloc_rejects_beyond_static_limit():
    cfg = syn.CONFIGS["prefill"]
    f = moeq.FfnDesc()
    f.T, f.H, f.F, f.E, f.k = cfg.T, cfg.H, cfg.F, cfg.E, cfg.k
    f.fmt_gate = f.fmt_up = f.fmt_down = moeq.Q4_K
    f.gate = f.up = f.down = 0x1000
    r = moeq.RouteDesc(cfg.T, cfg.H, cfg.E, cfg.k, cfg.gating, 1.0)
    assert moeq.moeq_moe_layer_workspace(r, f) > moeq.NOALLOC_MAX_BYTES
    y = torch.full((4,), 7.0, device="cuda")
    rc = moeq.lib().moeq_moe_layer_noalloc(moeq.ctypes.byref(r), moeq.ctypes.byref(f), 0x1000, 0x1000, None, None,
                                           0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, y.data_ptr(), None)
    assert rc == moeq.MOEQ_E_STATIC_LIMIT
    torch.cuda.synchronize()
    assert (y.cpu().numpy() == 7.0).all()
