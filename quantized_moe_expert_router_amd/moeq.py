"""Thin ctypes binding of libmoeq.so (declared in include/moeq.h).

Argument marshalling only: every step of the routed-expert FFN runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the stream.
The library must be built (quantized_moe_expert_router_amd.build); there is
no fallback path: a missing library or a failing call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq.so")

MOEQ_OK, MOEQ_E_INVALID, MOEQ_E_UNSUPPORTED, MOEQ_E_WORKSPACE, MOEQ_E_HIP = 0, -1, -2, -3, -4
MOEQ_E_STATIC_LIMIT = -5
NOALLOC_MAX_BYTES = 32 << 20
Q4_K, Q6_K, Q2_K, Q8_0, Q3_K, Q5_K, Q4_0, Q5_1 = 1, 2, 3, 4, 5, 6, 7, 8
SOFTMAX_TOPK, SOFTMAX_ALL, SIGMOID_TOPK = 0, 1, 2
PATH_AUTO, PATH_GEMV, PATH_MFMA = 0, 1, 2
Q8K_BYTES = 292
SUBBLOCK = {Q4_K: 32, Q6_K: 16, Q2_K: 16, Q8_0: 32, Q3_K: 16, Q5_K: 32, Q4_0: 32, Q5_1: 32}

SYMBOLS = ["moeq_status_string", "moeq_quantize_q8K", "moeq_route_workspace", "moeq_route",
           "moeq_packed_bytes", "moeq_pack_experts", "moeq_expert_ffn_workspace", "moeq_expert_ffn",
           "moeq_moe_layer_workspace", "moeq_moe_layer", "moeq_ffn_h_view", "moeq_debug_subdots",
           "moeq_moe_layer_noalloc", "moeq_debug_mfma_sums", "moeq_moe_stack_workspace", "moeq_moe_stack",
           "moeq_rms_norm", "moeq_ceiling_read", "moeq_ceiling_mfma_i8"]


class MoeqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %d (%s)" % (fn, status, status_string(status)))
        self.status = status


class RouteDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int32), ("gating", ctypes.c_int32), ("scale", ctypes.c_float)]


class FfnDesc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("F", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int32), ("fmt_gate", ctypes.c_int32), ("fmt_up", ctypes.c_int32),
                ("fmt_down", ctypes.c_int32), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("F_shared", ctypes.c_int64), ("sh_fmt_gate", ctypes.c_int32),
                ("sh_fmt_up", ctypes.c_int32), ("sh_fmt_down", ctypes.c_int32), ("sh_gate", ctypes.c_void_p),
                ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p), ("path", ctypes.c_int32),
                ("accumulate", ctypes.c_int32), ("aux_stream", ctypes.c_void_p), ("aux_fork", ctypes.c_void_p),
                ("aux_join", ctypes.c_void_p)]


class AuxStream:
    """A caller-owned auxiliary stream (default priority) and the two events
    moeq_ffn_desc.aux_* take: a shared expert launched apart from the routed
    launches runs there, forked from and joined back into the call's stream.
    Calls that may run concurrently need one each."""

    def __init__(self, device=None):
        self.stream = torch.cuda.Stream(device=device)
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        self.fork.record(self.stream)          # torch creates an event at its first record
        self.join.record(self.stream)
        torch.cuda.synchronize(device)

    def attach(self, desc: "FfnDesc") -> "FfnDesc":
        """Put the stream and event handles into desc; desc keeps this object
        alive (torch destroys an event with its Python object, which would
        leave the descriptor with dangling handles)."""
        desc.aux_stream = self.stream.cuda_stream
        desc.aux_fork = self.fork.cuda_event
        desc.aux_join = self.join.cuda_event
        desc._aux_owner = self
        return desc


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoeq.so is not built: run quantized_moe_expert_router_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.moeq_status_string.restype = ctypes.c_char_p
        L.moeq_status_string.argtypes = [ctypes.c_int]
        L.moeq_quantize_q8K.argtypes = [vp, i64, i64, vp, vp]
        L.moeq_route_workspace.restype = sz
        L.moeq_route_workspace.argtypes = [ctypes.POINTER(RouteDesc)]
        L.moeq_route.argtypes = [ctypes.POINTER(RouteDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moeq_packed_bytes.restype = sz
        L.moeq_packed_bytes.argtypes = [i32, i64, i64]
        L.moeq_pack_experts.argtypes = [i32, vp, i64, i64, i64, vp, vp]
        L.moeq_expert_ffn_workspace.restype = sz
        L.moeq_expert_ffn_workspace.argtypes = [ctypes.POINTER(FfnDesc)]
        L.moeq_expert_ffn.argtypes = [ctypes.POINTER(FfnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moeq_moe_layer_workspace.restype = sz
        L.moeq_moe_layer_workspace.argtypes = [ctypes.POINTER(RouteDesc), ctypes.POINTER(FfnDesc)]
        L.moeq_moe_layer.argtypes = [ctypes.POINTER(RouteDesc), ctypes.POINTER(FfnDesc), vp, vp, vp, vp, vp, vp,
                                     vp, vp, vp, vp, vp, vp, sz, vp]
        L.moeq_moe_stack_workspace.restype = sz
        L.moeq_moe_stack_workspace.argtypes = [ctypes.POINTER(RouteDesc), ctypes.POINTER(FfnDesc), i64]
        L.moeq_moe_stack.argtypes = [ctypes.POINTER(RouteDesc), ctypes.POINTER(FfnDesc), i64, vp, vp, vp,
                                     ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moeq_rms_norm.argtypes = [vp, i64, i64, vp, ctypes.c_float, vp, vp]
        L.moeq_moe_layer_noalloc.argtypes = [ctypes.POINTER(RouteDesc), ctypes.POINTER(FfnDesc), vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp, vp]
        L.moeq_ffn_h_view.argtypes = [ctypes.POINTER(FfnDesc), vp, sz, ctypes.POINTER(vp), ctypes.POINTER(vp)]
        L.moeq_debug_subdots.argtypes = [i32, vp, i64, i64, vp, i64, vp, vp]
        L.moeq_debug_mfma_sums.argtypes = [i32, vp, i64, i64, vp, i64, vp, vp]
        L.moeq_ceiling_read.argtypes = [vp, i64, i32, vp, vp]
        L.moeq_ceiling_mfma_i8.argtypes = [i64, i32, vp, vp]
        for s in ("moeq_quantize_q8K", "moeq_route", "moeq_pack_experts", "moeq_expert_ffn", "moeq_moe_layer",
                  "moeq_ffn_h_view", "moeq_debug_subdots", "moeq_moe_layer_noalloc", "moeq_debug_mfma_sums",
                  "moeq_moe_stack", "moeq_rms_norm", "moeq_ceiling_read", "moeq_ceiling_mfma_i8"):
            getattr(L, s).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moeq_status_string(status).decode()


def _check(fn: str, rc: int) -> None:
    if rc != MOEQ_OK:
        raise MoeqError(fn, rc)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s CUDA tensor" % (name, dtype))


# ------------------------------------------------------------------ entry points

def moeq_quantize_q8K(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """q8_K blocks (uint8 [rows, cols/256*292]) of fp32 x [rows, cols]."""
    _need(x, torch.float32, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols // 256 * Q8K_BYTES), dtype=torch.uint8, device=x.device)
    _check("moeq_quantize_q8K", lib().moeq_quantize_q8K(_ptr(x), rows, cols, _ptr(out), _stream(stream)))
    return out


class RouteOut:
    def __init__(self, T, E, k, device, with_logits=True):
        self.logits = torch.empty((T, E), dtype=torch.float64, device=device) if with_logits else None
        self.ids = torch.empty((T, k), dtype=torch.int32, device=device)
        self.w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=device)
        self.pairs = torch.empty(max(1, T * k), dtype=torch.int32, device=device)
        self.active = torch.empty(1 + min(E, T * k), dtype=torch.int32, device=device)


def moeq_route_workspace(T: int, H: int, E: int, k: int, gating: int, scale: float = 1.0) -> int:
    d = RouteDesc(T, H, E, k, gating, scale)
    return lib().moeq_route_workspace(ctypes.byref(d))


def moeq_route(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], k: int, gating: int,
               scale: float = 1.0, out: Optional[RouteOut] = None, ws: Optional[torch.Tensor] = None,
               stream=None, x_q8K: Optional[torch.Tensor] = None) -> RouteOut:
    """Router + top-k + lists; with x_q8K given, the same launch also writes q8_K(x)."""
    _need(x, torch.float32, "x")
    _need(w_router, torch.float32, "w_router")
    if bias is not None:
        _need(bias, torch.float32, "bias")
    T, H = x.shape
    E = w_router.shape[0]
    d = RouteDesc(T, H, E, k, gating, scale)
    if out is None:
        out = RouteOut(T, E, k, x.device)
    nws = lib().moeq_route_workspace(ctypes.byref(d))
    if ws is None:
        ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=x.device)
    rc = lib().moeq_route(ctypes.byref(d), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(out.logits), _ptr(out.ids),
                          _ptr(out.w), _ptr(out.offsets), _ptr(out.pairs), _ptr(out.active), _ptr(x_q8K),
                          _ptr(ws), ws.numel(), _stream(stream))
    _check("moeq_route", rc)
    return out


def moeq_packed_bytes(fmt: int, rows: int, cols: int) -> int:
    return lib().moeq_packed_bytes(fmt, rows, cols)


def moeq_pack_experts(fmt: int, aos: torch.Tensor, n_mats: int, rows: int, cols: int,
                      packed: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Repack n_mats exchange-format matrices (uint8, back to back) into the packed form."""
    if not aos.is_cuda or aos.dtype != torch.uint8:
        raise ValueError("aos must be a uint8 CUDA tensor")
    pb = moeq_packed_bytes(fmt, rows, cols)
    if pb == 0:
        raise MoeqError("moeq_packed_bytes", MOEQ_E_UNSUPPORTED)
    if packed is None:
        packed = torch.empty(n_mats * pb, dtype=torch.uint8, device=aos.device)
    _check("moeq_pack_experts", lib().moeq_pack_experts(fmt, _ptr(aos), n_mats, rows, cols, _ptr(packed),
                                                        _stream(stream)))
    return packed


def moeq_expert_ffn_workspace(desc: FfnDesc) -> int:
    return lib().moeq_expert_ffn_workspace(ctypes.byref(desc))


def moeq_expert_ffn(desc: FfnDesc, x_q8K: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                    expert_offsets: torch.Tensor, pairs: torch.Tensor, active: torch.Tensor,
                    shared_scale: Optional[torch.Tensor], y: torch.Tensor, ws: torch.Tensor,
                    stream=None) -> torch.Tensor:
    rc = lib().moeq_expert_ffn(ctypes.byref(desc), _ptr(x_q8K), _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets),
                               _ptr(pairs), _ptr(active), _ptr(shared_scale), _ptr(y), _ptr(ws), ws.numel(),
                               _stream(stream))
    _check("moeq_expert_ffn", rc)
    return y


def moeq_moe_layer_workspace(rdesc: RouteDesc, fdesc: FfnDesc) -> int:
    return lib().moeq_moe_layer_workspace(ctypes.byref(rdesc), ctypes.byref(fdesc))


def moeq_moe_layer(rdesc: RouteDesc, fdesc: FfnDesc, x: torch.Tensor, w_router: torch.Tensor,
                   bias: Optional[torch.Tensor], out: "RouteOut", shared_scale: Optional[torch.Tensor],
                   y: torch.Tensor, ws: torch.Tensor, stream=None) -> torch.Tensor:
    """The whole layer (route, q8_K(x), expert FFN) in one library call."""
    rc = lib().moeq_moe_layer(ctypes.byref(rdesc), ctypes.byref(fdesc), _ptr(x), _ptr(w_router), _ptr(bias),
                              _ptr(out.logits), _ptr(out.ids), _ptr(out.w), _ptr(out.offsets), _ptr(out.pairs),
                              _ptr(out.active), _ptr(shared_scale), _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    _check("moeq_moe_layer", rc)
    return y


def moeq_moe_layer_noalloc(rdesc: RouteDesc, fdesc: FfnDesc, x: torch.Tensor, w_router: torch.Tensor,
                           bias: Optional[torch.Tensor], out: "RouteOut", shared_scale: Optional[torch.Tensor],
                           y: torch.Tensor, stream=None) -> torch.Tensor:
    """The whole layer with the library's static per-GPU workspace (no
    workspace argument; calls on one GPU must not overlap)."""
    rc = lib().moeq_moe_layer_noalloc(ctypes.byref(rdesc), ctypes.byref(fdesc), _ptr(x), _ptr(w_router), _ptr(bias),
                                      _ptr(out.logits), _ptr(out.ids), _ptr(out.w), _ptr(out.offsets),
                                      _ptr(out.pairs), _ptr(out.active), _ptr(shared_scale), _ptr(y),
                                      _stream(stream))
    _check("moeq_moe_layer_noalloc", rc)
    return y


class StackOut:
    """Per-layer routing outputs of a stack of L layers ([L, ...] each)."""

    def __init__(self, L, T, E, k, device):
        self.L, self.T, self.E, self.k = L, T, E, k
        self.ids = torch.empty((L, T, k), dtype=torch.int32, device=device)
        self.w = torch.empty((L, T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty((L, E + 1), dtype=torch.int32, device=device)
        self.pairs = torch.empty((L, max(1, T * k)), dtype=torch.int32, device=device)
        self.active = torch.empty((L, 1 + min(E, T * k)), dtype=torch.int32, device=device)


def _ffn_array(fdescs: Sequence[FfnDesc]):
    arr = (FfnDesc * len(fdescs))()
    for i, d in enumerate(fdescs):
        ctypes.memmove(ctypes.byref(arr[i]), ctypes.byref(d), ctypes.sizeof(FfnDesc))
    return arr


def moeq_moe_stack_workspace(rdesc: RouteDesc, fdescs: Sequence[FfnDesc]) -> int:
    return lib().moeq_moe_stack_workspace(ctypes.byref(rdesc), _ffn_array(fdescs), len(fdescs))


def moeq_moe_stack(rdesc: RouteDesc, fdescs: Sequence[FfnDesc], w_routers: Sequence[torch.Tensor],
                   biases: Optional[Sequence[Optional[torch.Tensor]]], x: torch.Tensor, out: StackOut,
                   y: torch.Tensor, ws: torch.Tensor, stream=None,
                   shared_scales: Optional[Sequence[Optional[torch.Tensor]]] = None,
                   norm_ws: Optional[Sequence[Optional[torch.Tensor]]] = None, norm_eps: float = 1e-6) -> torch.Tensor:
    """L layers on a pre-norm residual stream in one library call:
    y = x, then y += MoE_l(RMSNorm_l(y)) for every layer."""
    L = len(fdescs)
    arr = _ffn_array(fdescs)
    wr = (ctypes.c_void_p * L)(*[_ptr(w) for w in w_routers])
    bs = None if biases is None else (ctypes.c_void_p * L)(*[_ptr(b) for b in biases])
    nw = None if norm_ws is None else (ctypes.c_void_p * L)(*[_ptr(g) for g in norm_ws])
    ss = None if shared_scales is None else (ctypes.c_void_p * L)(*[_ptr(t) for t in shared_scales])
    rc = lib().moeq_moe_stack(ctypes.byref(rdesc), arr, L, wr, bs, nw, ctypes.c_float(norm_eps), _ptr(x),
                              _ptr(out.ids), _ptr(out.w), _ptr(out.offsets), _ptr(out.pairs), _ptr(out.active), ss,
                              _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    _check("moeq_moe_stack", rc)
    return y


def moeq_rms_norm(x: torch.Tensor, gamma: Optional[torch.Tensor], eps: float, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """RMS pre-norm of the rows of x (fp32 [T, H]); gamma fp32 [H] or None."""
    _need(x, torch.float32, "x")
    if gamma is not None:
        _need(gamma, torch.float32, "gamma")
    T, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check("moeq_rms_norm", lib().moeq_rms_norm(_ptr(x), T, H, _ptr(gamma), ctypes.c_float(eps), _ptr(out),
                                                _stream(stream)))
    return out


def moeq_ffn_h_view(desc: FfnDesc, ws: torch.Tensor):
    """(routed, shared) q8_K(h) byte views into ws after moeq_expert_ffn."""
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    _check("moeq_ffn_h_view", lib().moeq_ffn_h_view(ctypes.byref(desc), _ptr(ws), ws.numel(), ctypes.byref(a),
                                                    ctypes.byref(b)))
    base = ws.data_ptr()
    nr = desc.T * desc.k * (desc.F // 256) * Q8K_BYTES
    routed = ws[a.value - base: a.value - base + nr].view(desc.T * desc.k, -1) if nr else None
    shared = None
    if b.value:
        ns = desc.T * (desc.F_shared // 256) * Q8K_BYTES
        shared = ws[b.value - base: b.value - base + ns].view(desc.T, -1)
    return routed, shared


def moeq_debug_subdots(fmt: int, packed_w: torch.Tensor, rows: int, cols: int, x_q8K: torch.Tensor,
                       stream=None) -> torch.Tensor:
    n_x = x_q8K.shape[0]
    out = torch.empty((n_x, rows, cols // SUBBLOCK[fmt]), dtype=torch.int32, device=packed_w.device)
    _check("moeq_debug_subdots", lib().moeq_debug_subdots(fmt, _ptr(packed_w), rows, cols, _ptr(x_q8K), n_x,
                                                          _ptr(out), _stream(stream)))
    return out


def moeq_debug_mfma_sums(fmt: int, packed_w: torch.Tensor, rows: int, cols: int, x_q8K: torch.Tensor,
                         stream=None) -> torch.Tensor:
    """int32 [n_x, rows, cols/256, 8]: the MFMA tiles' exact integer parts of
    every super-block term (S1, S2 for the K-quants; the 32-block sums for Q8_0)."""
    n_x = x_q8K.shape[0]
    out = torch.empty((n_x, rows, cols // 256, 8), dtype=torch.int32, device=packed_w.device)
    _check("moeq_debug_mfma_sums", lib().moeq_debug_mfma_sums(fmt, _ptr(packed_w), rows, cols, _ptr(x_q8K), n_x,
                                                              _ptr(out), _stream(stream)))
    return out


def moeq_ceiling_read(buf: torch.Tensor, n_blocks: int, stream=None) -> torch.Tensor:
    """uint64 [n_blocks] partial sums (as int64) of the 32-bit words of buf,
    read once by the streaming-read ceiling kernel."""
    out = torch.empty(n_blocks, dtype=torch.int64, device=buf.device)
    _check("moeq_ceiling_read", lib().moeq_ceiling_read(_ptr(buf), buf.numel() * buf.element_size(), n_blocks,
                                                        _ptr(out), _stream(stream)))
    return out


def moeq_ceiling_mfma_i8(iters: int, n_blocks: int, device, stream=None) -> torch.Tensor:
    """int32 [4 * n_blocks]: 128 * iters (mod 2^32) per wave of the int8 MFMA
    loop ceiling kernel."""
    out = torch.empty(4 * n_blocks, dtype=torch.int32, device=device)
    _check("moeq_ceiling_mfma_i8", lib().moeq_ceiling_mfma_i8(iters, n_blocks, _ptr(out), _stream(stream)))
    return out


# ------------------------------------------------------------------ device layer

class DeviceLayer:
    """One MoE layer's weights on the device: packed expert matrices, the
    per-expert pointer tables the FFN takes, router weights and bias.

    `layer` is a synthetic LayerData (numpy exchange-format bytes).  `present`
    marks experts resident in this instance (others get NULL pointers).
    fused_gate_up: take each expert's gate and up as one fused exchange tensor
    [2F, H] (gate rows, then up rows), packed as two matrices per expert.
    """

    def __init__(self, layer, device="cuda", present: Optional[Sequence[bool]] = None, stream=None,
                 fused_gate_up: bool = False):
        cfg = layer.cfg
        self.cfg = cfg
        self.device = device
        self.w_router = torch.from_numpy(layer.w_router).to(device)
        self.bias = None if layer.bias is None else torch.from_numpy(layer.bias).to(device)
        E = cfg.E
        have = [layer.gate[e] is not None and (present is None or present[e]) for e in range(E)]
        self.present = have
        self._bufs: List[torch.Tensor] = []

        def pack_all(mats, fmt, rows, cols):
            idx = [e for e in range(E) if have[e]]
            ptrs = torch.zeros(E, dtype=torch.int64)
            if idx:
                import numpy as np
                aos = torch.from_numpy(np.ascontiguousarray(np.stack([mats[e] for e in idx]))).to(device)
                packed = moeq_pack_experts(fmt, aos, len(idx), rows, cols, stream=stream)
                pb = moeq_packed_bytes(fmt, rows, cols)
                self._bufs.append(packed)
                for n, e in enumerate(idx):
                    ptrs[e] = packed.data_ptr() + n * pb
                del aos
            t = ptrs.to(device)
            self._bufs.append(t)
            return t

        if fused_gate_up:
            # one exchange tensor [2F, H] per expert is two [F, H] matrices back
            # to back: one pack call with two matrices per expert
            import numpy as np
            idx = [e for e in range(E) if have[e]]
            gp, up = torch.zeros(E, dtype=torch.int64), torch.zeros(E, dtype=torch.int64)
            if idx:
                fused = np.stack([np.concatenate([layer.gate[e], layer.up[e]]) for e in idx])
                aos = torch.from_numpy(np.ascontiguousarray(fused)).to(device)
                packed = moeq_pack_experts(cfg.fmt_gate, aos, 2 * len(idx), cfg.F, cfg.H, stream=stream)
                pb = moeq_packed_bytes(cfg.fmt_gate, cfg.F, cfg.H)
                self._bufs.append(packed)
                for n, e in enumerate(idx):
                    gp[e] = packed.data_ptr() + 2 * n * pb
                    up[e] = packed.data_ptr() + (2 * n + 1) * pb
                del aos
            self.gate_ptrs, self.up_ptrs = gp.to(device), up.to(device)
            self._bufs += [self.gate_ptrs, self.up_ptrs]
        else:
            self.gate_ptrs = pack_all(layer.gate, cfg.fmt_gate, cfg.F, cfg.H)
            self.up_ptrs = pack_all(layer.up, cfg.fmt_up, cfg.F, cfg.H)
        self.down_ptrs = pack_all(layer.down, cfg.fmt_down, cfg.H, cfg.F)
        self.sh = None
        if cfg.shared and layer.sh_gate is not None:
            def pack1(m, fmt, rows, cols):
                aos = torch.from_numpy(m.reshape(-1)).to(device)
                p = moeq_pack_experts(fmt, aos, 1, rows, cols, stream=stream)
                self._bufs.append(p)
                return p
            self.sh = (pack1(layer.sh_gate, cfg.sh_fmt_gate, cfg.F_shared, cfg.H),
                       pack1(layer.sh_up, cfg.sh_fmt_up, cfg.F_shared, cfg.H),
                       pack1(layer.sh_down, cfg.sh_fmt_down, cfg.H, cfg.F_shared))

    def ffn_desc(self, T: int, path: int = PATH_AUTO, accumulate: int = 0, shared: bool = True,
                 aux: Optional[AuxStream] = None) -> FfnDesc:
        c = self.cfg
        d = FfnDesc()
        d.T, d.H, d.F, d.E, d.k = T, c.H, c.F, c.E, c.k
        d.fmt_gate, d.fmt_up, d.fmt_down = c.fmt_gate, c.fmt_up, c.fmt_down
        d.gate, d.up, d.down = self.gate_ptrs.data_ptr(), self.up_ptrs.data_ptr(), self.down_ptrs.data_ptr()
        if self.sh is not None and shared:
            d.F_shared = c.F_shared
            d.sh_fmt_gate, d.sh_fmt_up, d.sh_fmt_down = c.sh_fmt_gate, c.sh_fmt_up, c.sh_fmt_down
            d.sh_gate, d.sh_up, d.sh_down = (p.data_ptr() for p in self.sh)
        d.path, d.accumulate = path, accumulate
        if aux is not None:
            aux.attach(d)
        return d


class LayerRunner:
    """Preallocated buffers for route -> quantize -> ffn of one layer shape.

    forward() enqueues the library calls on the current stream and allocates
    nothing (all buffers are made here).  With `aux`, a shared expert that
    runs apart from the routed launches goes to that auxiliary stream.
    """

    def __init__(self, dl: DeviceLayer, T: int, path: int = PATH_AUTO, shared_scale: Optional[torch.Tensor] = None,
                 aux: Optional[AuxStream] = None):
        c = dl.cfg
        self.dl, self.T = dl, T
        dev = dl.w_router.device
        self.route_out = RouteOut(T, c.E, c.k, dev)
        self.route_ws = torch.empty(max(256, moeq_route_workspace(T, c.H, c.E, c.k, c.gating)), dtype=torch.uint8,
                                    device=dev)
        self.xq = torch.empty((T, c.H // 256 * Q8K_BYTES), dtype=torch.uint8, device=dev)
        self.aux = aux
        self.desc = dl.ffn_desc(T, path=path, aux=aux)
        n = moeq_expert_ffn_workspace(self.desc)
        if n == 0:
            raise MoeqError("moeq_expert_ffn_workspace", MOEQ_E_UNSUPPORTED)
        self.ffn_ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.y = torch.empty((T, c.H), dtype=torch.float32, device=dev)
        self.shared_scale = shared_scale
        self.layer_ws = None

    def route(self, x: torch.Tensor, stream=None, with_q8K: bool = True):
        c = self.dl.cfg
        return moeq_route(x, self.dl.w_router, self.dl.bias, c.k, c.gating, out=self.route_out, ws=self.route_ws,
                          stream=stream, x_q8K=self.xq if with_q8K else None)

    def forward(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        """route (+ q8_K(x) in the same launch) then the expert FFN."""
        self.route(x, stream)
        return self.ffn(stream)

    def ffn(self, stream=None) -> torch.Tensor:
        r = self.route_out
        return moeq_expert_ffn(self.desc, self.xq, r.ids, r.w, r.offsets, r.pairs, r.active, self.shared_scale,
                               self.y, self.ffn_ws, stream)

    def layer(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        """The fused whole-layer call (moeq_moe_layer)."""
        c = self.dl.cfg
        if self.layer_ws is None:
            self.rdesc = RouteDesc(self.T, c.H, c.E, c.k, c.gating, 1.0)
            n = moeq_moe_layer_workspace(self.rdesc, self.desc)
            if n == 0:
                raise MoeqError("moeq_moe_layer_workspace", MOEQ_E_UNSUPPORTED)
            self.layer_ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        return moeq_moe_layer(self.rdesc, self.desc, x, self.dl.w_router, self.dl.bias, self.route_out,
                              self.shared_scale, self.y, self.layer_ws, stream)

    def layer_h_view(self):
        """q8_K(h) views after layer(): the FFN region sits at the start of the layer workspace."""
        return moeq_ffn_h_view(self.desc, self.layer_ws)
