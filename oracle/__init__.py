"""CPU oracle of the routed-expert FFN (ctypes binding of moe_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and never calls it; the library never calls it either.

The C source is plain scalar code in fp64 (see the header of moe_oracle.c for
what each function computes and which passage of the pages it follows).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        L.orc_half_to_double.restype = dbl
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_block_codes.argtypes = [i32, vp, vp, vp, vp, vp, vp]
        L.orc_dequant_row.argtypes = [i32, vp, i64, vp]
        L.orc_quantize_q8K.argtypes = [vp, i64, i64, vp]
        L.orc_quantize_q8K.restype = None
        L.orc_dequant_q8K_row.argtypes = [vp, i64, vp]
        L.orc_dequant_q8K_row.restype = None
        L.orc_rms_norm.argtypes = [vp, i64, i64, vp, dbl, vp]
        L.orc_rms_norm.restype = None
        L.orc_route.argtypes = [i64, i64, i64, i32, i32, dbl, vp, vp, vp, vp, vp, vp]
        L.orc_lists.argtypes = [i64, i32, i64, vp, vp, vp, vp]
        L.orc_lists.restype = None
        L.orc_subdots.argtypes = [i32, vp, i64, i64, vp, i64, vp]
        L.orc_scales_matrix.argtypes = [i32, vp, i64, i64, vp, vp]
        L.orc_dot_intform.argtypes = [i32, vp, i64, vp]
        L.orc_dot_intform.restype = dbl
        L.orc_matvec.argtypes = [i32, vp, i64, i64, vp, vp]
        L.orc_expert_ffn.argtypes = ([i64, i64, i64, i64, i32, i32, i32, i32, vp, vp, vp,
                                      i64, i32, i32, i32, vp, vp, vp,
                                      vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp])
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


SUBBLOCK = {1: 32, 2: 16, 3: 16, 4: 32, 5: 16, 6: 32, 7: 32, 8: 32}
BLOCK_W = {1: 256, 2: 256, 3: 256, 4: 32, 5: 256, 6: 256, 7: 32, 8: 32}
BLOCK_B = {1: 144, 2: 210, 3: 84, 4: 34, 5: 110, 6: 176, 7: 18, 8: 24}


def half_to_double(h: int) -> float:
    return lib().orc_half_to_double(h)


def block_codes(fmt: int, block: np.ndarray):
    """(d, dmin, sc[n_sub], m[n_sub], q[n_weights]) of one block."""
    b = _c(block, np.uint8)
    d = np.zeros(1, np.float64)
    dm = np.zeros(1, np.float64)
    sc = np.zeros(16, np.int32)
    m = np.zeros(16, np.int32)
    q = np.zeros(256, np.int32)
    if lib().orc_block_codes(fmt, _p(b), _p(d), _p(dm), _p(sc), _p(m), _p(q)):
        raise ValueError("bad format")
    nsub = BLOCK_W[fmt] // SUBBLOCK[fmt]
    return float(d[0]), float(dm[0]), sc[:nsub].copy(), m[:nsub].copy(), q[:BLOCK_W[fmt]].copy()


def dequant_row(fmt: int, row: np.ndarray, cols: int) -> np.ndarray:
    r = _c(row, np.uint8)
    out = np.zeros(cols, np.float64)
    if lib().orc_dequant_row(fmt, _p(r), cols, _p(out)):
        raise ValueError("bad row")
    return out


def dequant_matrix(fmt: int, W: np.ndarray, rows: int, cols: int) -> np.ndarray:
    W = _c(W, np.uint8).reshape(rows, -1)
    return np.stack([dequant_row(fmt, W[r], cols) for r in range(rows)])


def quantize_q8K(x: np.ndarray) -> np.ndarray:
    """q8_K bytes [rows, cols/256*292] of fp32 x [rows, cols]."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None]
    rows, cols = x.shape
    if cols % 256:
        raise ValueError("cols % 256")
    out = np.zeros((rows, cols // 256 * 292), np.uint8)
    lib().orc_quantize_q8K(_p(x), rows, cols, _p(out))
    return out


def rms_norm(x: np.ndarray, gamma: Optional[np.ndarray], eps: float) -> np.ndarray:
    """RMS pre-norm of the rows of fp32 x [rows, cols]: fl32((x * r) * gamma),
    r = 1 / sqrt(mean(x^2) + eps) in fp64 (the input of each MoE block of a
    pre-norm residual stack)."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None]
    rows, cols = x.shape
    g = None if gamma is None else _c(gamma, np.float32).reshape(cols)
    out = np.zeros((rows, cols), np.float32)
    lib().orc_rms_norm(_p(x), rows, cols, _p(g), float(eps), _p(out))
    return out


def dequant_q8K(q: np.ndarray, cols: int) -> np.ndarray:
    q = _c(q, np.uint8).reshape(-1, cols // 256 * 292)
    out = np.zeros((q.shape[0], cols), np.float64)
    for r in range(q.shape[0]):
        lib().orc_dequant_q8K_row(_p(q[r]), cols, _p(out[r]))
    return out


def route(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray], k: int, gating: int,
          scale: float = 1.0):
    """(logits fp64 [T,E], ids int32 [T,k], w fp32 [T,k])."""
    x = _c(x, np.float32)
    W = _c(w_router, np.float32)
    T, H = x.shape
    E = W.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    logits = np.zeros((T, E), np.float64)
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    if lib().orc_route(T, H, E, k, gating, scale, _p(x), _p(W), _p(b), _p(logits), _p(ids), _p(w)):
        raise ValueError("orc_route failed")
    return logits, ids, w


def lists(ids: np.ndarray, E: int):
    """(offsets [E+1], pairs [T*k], active [1+n]) of the routed pairs."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    off = np.zeros(E + 1, np.int32)
    pairs = np.zeros(T * k, np.int32)
    active = np.zeros(1 + E, np.int32)
    lib().orc_lists(T, k, E, _p(ids), _p(off), _p(pairs), _p(active))
    return off, pairs, active[:1 + active[0]].copy()


def subdots(fmt: int, W: np.ndarray, rows: int, cols: int, xq: np.ndarray) -> np.ndarray:
    """Exact int32 sub-block dots [n_x, rows, cols/subblock]."""
    W = _c(W, np.uint8)
    xq = _c(xq, np.uint8).reshape(-1, cols // 256 * 292)
    n_x = xq.shape[0]
    out = np.zeros((n_x, rows, cols // SUBBLOCK[fmt]), np.int32)
    if lib().orc_subdots(fmt, _p(W), rows, cols, _p(xq), n_x, _p(out)):
        raise ValueError("orc_subdots failed")
    return out


def scales_matrix(fmt: int, W: np.ndarray, rows: int, cols: int):
    """(sc, m) int32 [rows, blocks per row, sub-blocks per block]: the decoded
    sub-block scales and mins of every block."""
    W = _c(W, np.uint8)
    nblk = cols // BLOCK_W[fmt]
    sc = np.zeros((rows, nblk, 16), np.int32)
    m = np.zeros((rows, nblk, 16), np.int32)
    if lib().orc_scales_matrix(fmt, _p(W), rows, cols, _p(sc), _p(m)):
        raise ValueError("orc_scales_matrix failed")
    nsub = BLOCK_W[fmt] // SUBBLOCK[fmt]
    return sc[:, :, :nsub].copy(), m[:, :, :nsub].copy()


def dot_intform(fmt: int, wrow: np.ndarray, cols: int, xq_row: np.ndarray) -> float:
    return lib().orc_dot_intform(fmt, _p(_c(wrow, np.uint8)), cols, _p(_c(xq_row, np.uint8)))


def matvec(fmt: int, W: np.ndarray, rows: int, cols: int, v: np.ndarray) -> np.ndarray:
    W = _c(W, np.uint8)
    v = _c(v, np.float64)
    out = np.zeros(rows, np.float64)
    if lib().orc_matvec(fmt, _p(W), rows, cols, _p(v), _p(out)):
        raise ValueError("orc_matvec failed")
    return out


class FFNResult:
    def __init__(self, y, hq, g, u, h):
        self.y, self.hq, self.g, self.u, self.h = y, hq, g, u, h


def expert_ffn(layer, ids: np.ndarray, w: np.ndarray, sel: Sequence[int],
               shared_scale: Optional[np.ndarray] = None, x: Optional[np.ndarray] = None,
               present: Optional[Sequence[bool]] = None, diag: bool = False) -> FFNResult:
    """Oracle FFN for the tokens in `sel` of a synthetic layer (quantized_moe_expert_router_amd.synthetic.LayerData).

    present[e] False (or a None matrix) marks expert e as not resident.
    Returns y [n, H] fp32, hq [n, k+1, Fmax/256*292] bytes, and optionally
    g/u [n, k+1, Fmax] fp64 and h [n, k+1, Fmax] fp32.
    """
    cfg = layer.cfg
    L = lib()
    x = _c(layer.x if x is None else x, np.float32)
    T, H = x.shape
    E, k, F = cfg.E, ids.shape[1], cfg.F
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    keep: List[np.ndarray] = []

    def arr(mats):
        a = (ctypes.c_void_p * E)()
        for e in range(E):
            m = mats[e]
            if m is None or (present is not None and not present[e]):
                a[e] = None
            else:
                mm = _c(m, np.uint8)
                keep.append(mm)
                a[e] = mm.ctypes.data
        return a

    ga, ua, da = arr(layer.gate), arr(layer.up), arr(layer.down)
    Fs = cfg.F_shared if cfg.shared else 0
    sh = [None if m is None else _c(m, np.uint8) for m in (layer.sh_gate, layer.sh_up, layer.sh_down)]
    Fmax = max(F, Fs)
    sel = np.ascontiguousarray(sel, dtype=np.int64)
    n = len(sel)
    y = np.zeros((n, H), np.float32)
    hq = np.zeros((n, k + 1, Fmax // 256 * 292), np.uint8)
    g = u = h = None
    if diag:
        g = np.zeros((n, k + 1, Fmax), np.float64)
        u = np.zeros((n, k + 1, Fmax), np.float64)
        h = np.zeros((n, k + 1, Fmax), np.float32)
    ss = None if shared_scale is None else _c(shared_scale, np.float32)
    rc = L.orc_expert_ffn(T, H, F, E, k, cfg.fmt_gate, cfg.fmt_up, cfg.fmt_down,
                          ctypes.cast(ga, ctypes.c_void_p), ctypes.cast(ua, ctypes.c_void_p),
                          ctypes.cast(da, ctypes.c_void_p),
                          Fs, cfg.sh_fmt_gate, cfg.sh_fmt_up, cfg.sh_fmt_down,
                          _p(sh[0]), _p(sh[1]), _p(sh[2]),
                          _p(x), _p(ids), _p(w), _p(ss), _p(sel), n,
                          _p(y), _p(hq), _p(g), _p(u), _p(h))
    if rc:
        raise ValueError("orc_expert_ffn failed")
    return FFNResult(y, hq, g, u, h)
