"""Host-side checks of the C ABI: the library loads without a GPU, exports
every symbol include/moeq.h declares, and rejects bad arguments before any
launch (no compute calls here)."""
import ctypes
import os
import re

import pytest

from quantized_moe_expert_router_amd import moeq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "moeq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moeq_[a-zA-Z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    syms = _declared_symbols()
    assert len(syms) >= 10
    L = moeq.lib()
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(moeq.SYMBOLS)


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert moeq.status_string(st) != "unknown status"
    assert moeq.status_string(7) == "unknown status"


def test_packed_bytes_and_workspace_queries():
    assert moeq.moeq_packed_bytes(moeq.Q4_K, 512, 2048) == 512 * 8 * 144
    assert moeq.moeq_packed_bytes(moeq.Q6_K, 2048, 512) == 2048 * 2 * 210
    # Q2_K is laid out in 2688-byte 32-row units: one row pads to a unit (256-byte aligned total)
    assert moeq.moeq_packed_bytes(moeq.Q2_K, 1, 256) == 2816
    assert moeq.moeq_packed_bytes(moeq.Q2_K, 1536, 4096) == 1536 * 16 * 84
    # Q3_K planes 64 + 32 + 16 + 2 B per super-block, Q5_K 128 + 32 + 16, each 256-byte aligned
    assert moeq.moeq_packed_bytes(moeq.Q3_K, 512, 2048) == 4096 * (64 + 32 + 16 + 2)
    assert moeq.moeq_packed_bytes(moeq.Q5_K, 512, 2048) == 4096 * (128 + 32 + 16)
    assert moeq.moeq_packed_bytes(moeq.Q3_K, 1, 256) == 4 * 256
    assert moeq.moeq_packed_bytes(moeq.Q4_0, 512, 2048) == 4096 * (128 + 16)
    assert moeq.moeq_packed_bytes(moeq.Q5_1, 512, 2048) == 4096 * (128 + 64)
    assert moeq.moeq_packed_bytes(99, 1, 256) == 0
    assert moeq.moeq_packed_bytes(moeq.Q4_K, 1, 100) == 0
    assert moeq.moeq_route_workspace(1, 2048, 256, 8, 0) > 0


def _desc(**kw):
    d = moeq.FfnDesc()
    d.T, d.H, d.F, d.E, d.k = 1, 2048, 512, 256, 8
    d.fmt_gate = d.fmt_up = moeq.Q4_K
    d.fmt_down = moeq.Q6_K
    d.gate = d.up = d.down = 0x1000
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,status", [
    (dict(H=2000), moeq.MOEQ_E_INVALID),
    (dict(F=300), moeq.MOEQ_E_INVALID),
    (dict(k=0), moeq.MOEQ_E_INVALID),
    (dict(k=33), moeq.MOEQ_E_INVALID),
    (dict(E=4097), moeq.MOEQ_E_INVALID),
    (dict(fmt_down=99), moeq.MOEQ_E_UNSUPPORTED),
    (dict(fmt_up=moeq.Q2_K), moeq.MOEQ_E_UNSUPPORTED),
    (dict(gate=0), moeq.MOEQ_E_INVALID),
    (dict(sh_gate=0x2000, F_shared=512, sh_fmt_gate=1, sh_fmt_up=1, sh_fmt_down=1), moeq.MOEQ_E_INVALID),
    (dict(path=5), moeq.MOEQ_E_INVALID),
    (dict(accumulate=2), moeq.MOEQ_E_INVALID),
    (dict(H=256 * 40), moeq.MOEQ_E_UNSUPPORTED),
    (dict(aux_stream=0x3000), moeq.MOEQ_E_INVALID),            # auxiliary stream without its events
    (dict(aux_fork=0x3000, aux_join=0x4000), moeq.MOEQ_E_INVALID),
])
def test_ffn_rejects_bad_descriptors(kw, status):
    d = _desc(**kw)
    L = moeq.lib()
    assert L.moeq_expert_ffn_workspace(ctypes.byref(d)) == 0
    rc = L.moeq_expert_ffn(ctypes.byref(d), 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 0x1000, 0x100000,
                           1 << 30, None)
    assert rc == status


def test_ffn_rejects_small_or_misaligned_workspace_and_null_inputs():
    d = _desc()
    L = moeq.lib()
    need = L.moeq_expert_ffn_workspace(ctypes.byref(d))
    assert need > 0
    args = [0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None, 0x1000]
    assert L.moeq_expert_ffn(ctypes.byref(d), *args, 0x100000, need - 1, None) == moeq.MOEQ_E_WORKSPACE
    assert L.moeq_expert_ffn(ctypes.byref(d), *args, 0x100010, need, None) == moeq.MOEQ_E_INVALID
    bad = list(args)
    bad[0] = None
    assert L.moeq_expert_ffn(ctypes.byref(d), *bad, 0x100000, need, None) == moeq.MOEQ_E_INVALID
    # T == 0 is a valid no-op
    d0 = _desc(T=0)
    assert L.moeq_expert_ffn(ctypes.byref(d0), None, None, None, None, None, None, None, None, None, 0, None) == 0
    bad = list(args)
    bad[1] = None                                               # topk_ids is required
    assert L.moeq_expert_ffn(ctypes.byref(d), *bad, 0x100000, need, None) == moeq.MOEQ_E_INVALID


def test_layer_call_validation():
    L = moeq.lib()
    f = _desc()
    r = moeq.RouteDesc(1, 2048, 256, 8, 0, 1.0)
    need = L.moeq_moe_layer_workspace(ctypes.byref(r), ctypes.byref(f))
    assert need >= L.moeq_expert_ffn_workspace(ctypes.byref(f))
    ptrs = [0x1000] * 11
    ptrs[2] = None                                              # no bias
    assert L.moeq_moe_layer(ctypes.byref(r), ctypes.byref(f), *ptrs, 0x100000, need - 1, None) == \
        moeq.MOEQ_E_WORKSPACE
    r2 = moeq.RouteDesc(1, 2048, 256, 6, 0, 1.0)               # k disagrees with the FFN descriptor
    assert L.moeq_moe_layer_workspace(ctypes.byref(r2), ctypes.byref(f)) == 0
    assert L.moeq_moe_layer(ctypes.byref(r2), ctypes.byref(f), *ptrs, 0x100000, 1 << 30, None) == \
        moeq.MOEQ_E_INVALID


def test_route_and_quantize_validation():
    L = moeq.lib()
    d = moeq.RouteDesc(4, 2048, 256, 8, 0, 1.0)
    ws = L.moeq_route_workspace(ctypes.byref(d))
    ok = dict(x=0x1000, w=0x2000, b=None, lg=None, ids=0x3000, tw=0x4000, off=0x5000, pairs=0x6000, act=0x7000,
              xq=None)

    def call(desc, ws_bytes=ws, wsp=0x100000, **over):
        a = dict(ok, **over)
        return L.moeq_route(ctypes.byref(desc), a["x"], a["w"], a["b"], a["lg"], a["ids"], a["tw"], a["off"],
                            a["pairs"], a["act"], a["xq"], wsp, ws_bytes, None)

    assert call(d, ws_bytes=ws - 1) == moeq.MOEQ_E_WORKSPACE
    assert call(d, x=0x1004) == moeq.MOEQ_E_INVALID            # x must be 16-byte aligned
    assert call(d, ids=None) == moeq.MOEQ_E_INVALID
    assert call(d, xq=0x8002) == moeq.MOEQ_E_INVALID           # q8_K output must be 4-byte aligned
    assert call(moeq.RouteDesc(4, 2048, 256, 0, 0, 1.0)) == moeq.MOEQ_E_INVALID
    assert call(moeq.RouteDesc(4, 2048, 4, 5, 0, 1.0)) == moeq.MOEQ_E_INVALID
    assert call(moeq.RouteDesc(4, 2046, 256, 8, 0, 1.0)) == moeq.MOEQ_E_INVALID
    assert call(moeq.RouteDesc(4, 2048, 256, 8, 3, 1.0)) == moeq.MOEQ_E_UNSUPPORTED
    assert L.moeq_quantize_q8K(0x1000, 2, 300, 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_quantize_q8K(None, 2, 256, 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_quantize_q8K(0x1004, 2, 256, 0x2000, None) == moeq.MOEQ_E_INVALID   # x 16-byte aligned
    assert L.moeq_quantize_q8K(0x1000, 0, 256, 0x2000, None) == 0
    assert L.moeq_pack_experts(99, 0x1000, 1, 1, 256, 0x2000, None) == moeq.MOEQ_E_UNSUPPORTED
    assert L.moeq_pack_experts(1, 0x1000, 1, 1, 256, 0x2010, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_debug_subdots(1, 0x1000, 1, 300, 0x2000, 1, 0x3000, None) == moeq.MOEQ_E_INVALID


def test_noalloc_layer_rejects_requests_beyond_its_static_workspace():
    # the 8192-token prefill layer needs far more than the 32 MiB static
    # workspace: rejected on the host before any device call
    L = moeq.lib()
    f = _desc(T=8192, H=2048, F=512, E=512, k=10, fmt_down=moeq.Q4_K)
    r = moeq.RouteDesc(8192, 2048, 512, 10, 0, 1.0)
    assert L.moeq_moe_layer_workspace(ctypes.byref(r), ctypes.byref(f)) > moeq.NOALLOC_MAX_BYTES
    ptrs = [0x1000] * 12
    ptrs[2] = ptrs[3] = None
    assert L.moeq_moe_layer_noalloc(ctypes.byref(r), ctypes.byref(f), *ptrs, None) == moeq.MOEQ_E_STATIC_LIMIT
    r2 = moeq.RouteDesc(8192, 2048, 512, 6, 0, 1.0)            # descriptors that disagree
    assert L.moeq_moe_layer_noalloc(ctypes.byref(r2), ctypes.byref(f), *ptrs, None) == moeq.MOEQ_E_INVALID
    assert moeq.status_string(moeq.MOEQ_E_STATIC_LIMIT) != "unknown status"


def test_stack_call_validation():
    L = moeq.lib()
    r = moeq.RouteDesc(1, 2048, 256, 8, 0, 1.0)
    fs = moeq._ffn_array([_desc(), _desc()])
    one = L.moeq_moe_layer_workspace(ctypes.byref(r), ctypes.byref(_desc()))
    need = L.moeq_moe_stack_workspace(ctypes.byref(r), fs, 2)
    assert need == one + 2048 * 4                                   # plus the normalised rows
    assert L.moeq_moe_stack_workspace(ctypes.byref(r), fs, 0) == 0
    bad = moeq._ffn_array([_desc(), _desc(accumulate=1)])          # layers of a stack do not accumulate
    assert L.moeq_moe_stack_workspace(ctypes.byref(r), bad, 2) == 0
    wr = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    args = [0x1000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, None, 0x8000]
    eps = ctypes.c_float(1e-5)

    def call(rd=r, wrs=wr, nw=None, e=eps, ws_bytes=need):
        return L.moeq_moe_stack(ctypes.byref(rd), fs, 2, wrs, None, nw, e, *args, 0x100000, ws_bytes, None)

    assert call(ws_bytes=need - 1) == moeq.MOEQ_E_WORKSPACE
    assert call(wrs=(ctypes.c_void_p * 2)(0x1000, 0x2004)) == moeq.MOEQ_E_INVALID   # router weights 16-byte aligned
    assert call(rd=moeq.RouteDesc(1, 2048, 256, 6, 0, 1.0)) == moeq.MOEQ_E_INVALID  # k disagrees with f
    assert call(nw=(ctypes.c_void_p * 2)(None, 0x2008)) == moeq.MOEQ_E_INVALID     # norm gains 16-byte aligned
    for e in (-1.0, float("inf"), float("nan")):
        assert call(e=ctypes.c_float(e)) == moeq.MOEQ_E_INVALID


def test_rms_norm_validation():
    L = moeq.lib()
    e = ctypes.c_float(1e-6)
    assert L.moeq_rms_norm(0x1000, 2, 300, None, e, 0x2000, None) == moeq.MOEQ_E_INVALID    # H % 256
    assert L.moeq_rms_norm(0x1000, -1, 256, None, e, 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_rms_norm(None, 2, 256, None, e, 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_rms_norm(0x1004, 2, 256, None, e, 0x2000, None) == moeq.MOEQ_E_INVALID  # x 16-byte aligned
    assert L.moeq_rms_norm(0x1000, 2, 256, 0x3004, e, 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_rms_norm(0x1000, 2, 256, None, ctypes.c_float(-1e-6), 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_rms_norm(0x1000, 2, 256, None, ctypes.c_float(float("nan")), 0x2000, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_rms_norm(None, 0, 256, None, e, None, None) == 0                        # T == 0: no-op


def test_ceiling_calls_validation():
    L = moeq.lib()
    ok = 0x100000
    assert L.moeq_ceiling_read(None, 1 << 20, 64, ok, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_ceiling_read(ok, 1 << 20, 64, None, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_ceiling_read(ok + 8, 1 << 20, 64, ok, None) == moeq.MOEQ_E_INVALID     # buffer 16-byte aligned
    assert L.moeq_ceiling_read(ok, 1 << 20, 64, ok + 4, None) == moeq.MOEQ_E_INVALID     # sums 8-byte aligned
    for nbytes in (0, -16, 24):
        assert L.moeq_ceiling_read(ok, nbytes, 64, ok, None) == moeq.MOEQ_E_INVALID
    for nb in (0, -1, (1 << 22) + 1):
        assert L.moeq_ceiling_read(ok, 1 << 20, nb, ok, None) == moeq.MOEQ_E_INVALID
        assert L.moeq_ceiling_mfma_i8(4, nb, ok, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_ceiling_mfma_i8(0, 64, ok, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_ceiling_mfma_i8(4, 64, None, None) == moeq.MOEQ_E_INVALID
    assert L.moeq_ceiling_mfma_i8(4, 64, ok + 2, None) == moeq.MOEQ_E_INVALID
