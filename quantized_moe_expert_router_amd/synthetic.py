"""Seeded synthetic inputs for the routed-expert FFN: layer shapes, activations,
router weights, and expert weight blocks in the exchange (AoS) byte format.

This module holds no arithmetic of the method.  It draws random numbers and
places them into buffers; both the CPU oracle and the HIP path consume what it
produces.  Weight blocks are produced as uniformly random bytes, which makes
every quant code, scale code and min code uniform over its full range, and
then the fp16 super-scale fields are overwritten with draws from the stated
ranges.  The only layout knowledge needed for that is where each fp16 field
sits inside a block and how long a block is.

Shapes follow the workloads the pages describe: a Qwen3.6-35B-A3B-like decode
layer (top-8 of 256 plus a shared expert, Pulsar README, 'What it does today'
model table), MTP verify rows (Pulsar README, ThinkingCap paragraph: verify
rows share one weight read), a DeepSeek-V4-Flash-like 16-token chunk (top-6 of
256 plus shared, same table; batched 16-token chunks in the DeepSeek-V4-Flash
paragraph) and a Strata-like 8192-token prefill chunk (Strata summary:
48 layers x 512 experts, about 10 active, chunked prefill up to 8192 tokens).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

# Format ids (same values as the C header's moeq_wfmt).
Q4_K, Q6_K, Q2_K, Q8_0, Q3_K, Q5_K, Q4_0, Q5_1 = 1, 2, 3, 4, 5, 6, 7, 8
FMT_NAMES = {Q4_K: "Q4_K", Q6_K: "Q6_K", Q2_K: "Q2_K", Q8_0: "Q8_0", Q3_K: "Q3_K", Q5_K: "Q5_K", Q4_0: "Q4_0",
             Q5_1: "Q5_1"}

# Gating ids (same values as moeq_gating).
SOFTMAX_TOPK, SOFTMAX_ALL, SIGMOID_TOPK = 0, 1, 2

# Bytes per block and weights per block of each exchange format.
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q2_K: 84, Q8_0: 34, Q3_K: 110, Q5_K: 176, Q4_0: 18, Q5_1: 24}
BLOCK_WEIGHTS = {Q4_K: 256, Q6_K: 256, Q2_K: 256, Q8_0: 32, Q3_K: 256, Q5_K: 256, Q4_0: 32, Q5_1: 32}
Q8K_BLOCK_BYTES = 292

# Byte offsets of fp16 scale fields inside a block, with the draw range of each:
# value = fp16(mult * U[1,2) * base).
_FP16_FIELDS = {
    Q4_K: [(0, 1.0, 1e-4), (2, 7.5, 1e-4)],    # d, dmin
    Q2_K: [(0, 1.0, 1e-3), (2, 1.5, 1e-3)],    # d, dmin
    Q6_K: [(0, 1.0, 1e-5)],                    # d
    Q8_0: [(0, 1.0, 1e-4)],                    # d
    Q3_K: [(0, 1.0, 3e-4)],                    # d
    Q5_K: [(0, 1.0, 5e-5), (2, 7.5, 5e-5)],    # d, dmin
    Q4_0: [(0, 1.0, 5e-3)],                    # d
    Q5_1: [(0, 1.0, 2e-3), (2, -16.0, 2e-3)],  # d, m (negative: the block's values centre on zero)
}

# Stream roles, mixed into the seed so every tensor has an independent stream.
ROLE_X, ROLE_ROUTER, ROLE_BIAS, ROLE_OUTLIER, ROLE_ZIPF = 1, 2, 3, 4, 5
ROLE_GATE, ROLE_UP, ROLE_DOWN = 10, 11, 12
ROLE_SH_GATE, ROLE_SH_UP, ROLE_SH_DOWN = 20, 21, 22


def matrix_bytes(fmt: int, rows: int, cols: int) -> int:
    """Exchange-format size of a [rows, cols] matrix (rows of blocks)."""
    if cols % BLOCK_WEIGHTS[fmt]:
        raise ValueError("cols must be a multiple of the block width")
    return rows * (cols // BLOCK_WEIGHTS[fmt]) * BLOCK_BYTES[fmt]


def rng_for(seed: int, layer: int, role: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, layer, role, index]))


def gen_weight_blocks(fmt: int, rows: int, cols: int, rng: np.random.Generator) -> np.ndarray:
    """[rows, bytes_per_row] uint8: random codes, fp16 scales from their ranges."""
    bb = BLOCK_BYTES[fmt]
    nblk = rows * (cols // BLOCK_WEIGHTS[fmt])
    raw = rng.integers(0, 256, size=nblk * bb, dtype=np.uint8)
    blocks = raw.reshape(nblk, bb)
    for off, mult, base in _FP16_FIELDS[fmt]:
        u = rng.random(nblk) + 1.0
        h = (mult * u * base).astype(np.float16)
        blocks[:, off:off + 2] = h.view(np.uint8).reshape(nblk, 2)
    return raw.reshape(rows, -1)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    seed: int
    T: int
    H: int
    E: int
    k: int
    F: int
    gating: int
    fmt_gate: int
    fmt_up: int
    fmt_down: int
    shared: bool = False
    F_shared: int = 0
    sh_fmt_gate: int = 0
    sh_fmt_up: int = 0
    sh_fmt_down: int = 0
    outlier_p: float = 0.0        # Bernoulli mask probability for x outliers
    outlier_mult: float = 1.0
    zipf_s: float = 0.0           # >0: per-expert logit bias from a Zipf popularity law
    zipf_beta: float = 0.5

    def nb(self, n: int) -> int:
        return n // 256


# The five layer shapes.  Names say what the layer is shaped like.
CONFIGS: Dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny_h512_e16_top2_q4k", 101, T=1, H=512, E=16, k=2, F=256,
                        gating=SOFTMAX_TOPK, fmt_gate=Q4_K, fmt_up=Q4_K, fmt_down=Q4_K),
    "decode": LayerConfig("decode_35b_a3b_h2048_e256_top8_shared", 102, T=1, H=2048, E=256, k=8,
                          F=512, gating=SOFTMAX_TOPK, fmt_gate=Q4_K, fmt_up=Q4_K, fmt_down=Q6_K,
                          shared=True, F_shared=512, sh_fmt_gate=Q4_K, sh_fmt_up=Q4_K,
                          sh_fmt_down=Q6_K),
    "verify": LayerConfig("verify4_h4096_e192_top8_q2k", 103, T=4, H=4096, E=192, k=8, F=1536,
                          gating=SOFTMAX_TOPK, fmt_gate=Q2_K, fmt_up=Q2_K, fmt_down=Q2_K),
    "chunk16": LayerConfig("chunk16_dsv4flash_h4096_e256_top6_sigmoid_shared", 104, T=16, H=4096,
                           E=256, k=6, F=2048, gating=SIGMOID_TOPK, fmt_gate=Q2_K, fmt_up=Q2_K,
                           fmt_down=Q4_K, shared=True, F_shared=2048, sh_fmt_gate=Q8_0,
                           sh_fmt_up=Q8_0, sh_fmt_down=Q8_0, outlier_p=0.01, outlier_mult=20.0),
    "prefill": LayerConfig("prefill8192_strata_h2048_e512_top10_shared_zipf", 105, T=8192, H=2048,
                           E=512, k=10, F=512, gating=SOFTMAX_TOPK, fmt_gate=Q4_K, fmt_up=Q4_K,
                           fmt_down=Q4_K, shared=True, F_shared=512, sh_fmt_gate=Q4_K,
                           sh_fmt_up=Q4_K, sh_fmt_down=Q4_K, zipf_s=1.1),
}
CONFIG_ORDER = ["tiny", "decode", "verify", "chunk16", "prefill"]


@dataclasses.dataclass
class LayerData:
    cfg: LayerConfig
    x: np.ndarray                       # fp32 [T, H]
    w_router: np.ndarray                # fp32 [E, H]
    bias: Optional[np.ndarray]          # fp32 [E] or None
    gate: List[Optional[np.ndarray]]    # per expert uint8 [F, bytes_per_row] (None = absent)
    up: List[Optional[np.ndarray]]
    down: List[Optional[np.ndarray]]    # per expert uint8 [H, bytes_per_row]
    sh_gate: Optional[np.ndarray] = None
    sh_up: Optional[np.ndarray] = None
    sh_down: Optional[np.ndarray] = None


def gen_x(cfg: LayerConfig, seed: int, layer: int = 0, T: Optional[int] = None) -> np.ndarray:
    T = cfg.T if T is None else T
    r = rng_for(seed, layer, ROLE_X)
    x = r.standard_normal((T, cfg.H)).astype(np.float32)
    if cfg.outlier_p > 0:
        ro = rng_for(seed, layer, ROLE_OUTLIER)
        mask = ro.random((T, cfg.H)) < cfg.outlier_p
        x = np.where(mask, x * np.float32(cfg.outlier_mult), x).astype(np.float32)
    return x


def gen_router(cfg: LayerConfig, seed: int, layer: int = 0) -> np.ndarray:
    r = rng_for(seed, layer, ROLE_ROUTER)
    return (r.standard_normal((cfg.E, cfg.H)) * 0.02).astype(np.float32)


def gen_bias(cfg: LayerConfig, seed: int, layer: int = 0) -> Optional[np.ndarray]:
    """Per-expert logit bias that skews expert popularity like a Zipf law.

    Popularity p_e is proportional to rank_e^-s with ranks from a seeded
    permutation; the bias is beta * sigma_logit * ln(p_e / p_max) with
    sigma_logit = 0.02 * sqrt(H), the spread of the router logits.
    """
    if cfg.zipf_s <= 0:
        return None
    r = rng_for(seed, layer, ROLE_ZIPF)
    rank = r.permutation(cfg.E).astype(np.float64) + 1.0
    sigma = 0.02 * math.sqrt(cfg.H)
    b = cfg.zipf_beta * sigma * (-cfg.zipf_s) * np.log(rank)   # ln(p_e/p_max) = -s ln(rank)
    return b.astype(np.float32)


def gen_expert(cfg: LayerConfig, seed: int, layer: int, e: int):
    g = gen_weight_blocks(cfg.fmt_gate, cfg.F, cfg.H, rng_for(seed, layer, ROLE_GATE, e))
    u = gen_weight_blocks(cfg.fmt_up, cfg.F, cfg.H, rng_for(seed, layer, ROLE_UP, e))
    d = gen_weight_blocks(cfg.fmt_down, cfg.H, cfg.F, rng_for(seed, layer, ROLE_DOWN, e))
    return g, u, d


def gen_shared(cfg: LayerConfig, seed: int, layer: int):
    if not cfg.shared:
        return None, None, None
    Fs = cfg.F_shared
    g = gen_weight_blocks(cfg.sh_fmt_gate, Fs, cfg.H, rng_for(seed, layer, ROLE_SH_GATE))
    u = gen_weight_blocks(cfg.sh_fmt_up, Fs, cfg.H, rng_for(seed, layer, ROLE_SH_UP))
    d = gen_weight_blocks(cfg.sh_fmt_down, cfg.H, Fs, rng_for(seed, layer, ROLE_SH_DOWN))
    return g, u, d


def gen_layer(cfg: LayerConfig, seed: Optional[int] = None, layer: int = 0,
              experts: Optional[List[int]] = None, T: Optional[int] = None) -> LayerData:
    """Build one synthetic layer.  `experts` limits which experts are generated
    (others are None); every expert's bytes depend only on (seed, layer, e)."""
    seed = cfg.seed if seed is None else seed
    want = range(cfg.E) if experts is None else experts
    gate: List[Optional[np.ndarray]] = [None] * cfg.E
    up: List[Optional[np.ndarray]] = [None] * cfg.E
    down: List[Optional[np.ndarray]] = [None] * cfg.E
    for e in want:
        gate[e], up[e], down[e] = gen_expert(cfg, seed, layer, e)
    sg, su, sd = gen_shared(cfg, seed, layer)
    return LayerData(cfg=cfg, x=gen_x(cfg, seed, layer, T), w_router=gen_router(cfg, seed, layer),
                     bias=gen_bias(cfg, seed, layer), gate=gate, up=up, down=down,
                     sh_gate=sg, sh_up=su, sh_down=sd)


def expert_bytes(cfg: LayerConfig) -> int:
    return (matrix_bytes(cfg.fmt_gate, cfg.F, cfg.H) + matrix_bytes(cfg.fmt_up, cfg.F, cfg.H)
            + matrix_bytes(cfg.fmt_down, cfg.H, cfg.F))


def shared_bytes(cfg: LayerConfig) -> int:
    if not cfg.shared:
        return 0
    Fs = cfg.F_shared
    return (matrix_bytes(cfg.sh_fmt_gate, Fs, cfg.H) + matrix_bytes(cfg.sh_fmt_up, Fs, cfg.H)
            + matrix_bytes(cfg.sh_fmt_down, cfg.H, Fs))


def gen_weight_blocks_device(fmt: int, rows: int, cols: int, generator, device) -> "torch.Tensor":
    """The same recipe as gen_weight_blocks (uniform random bytes, fp16 scale
    fields drawn from their ranges) drawn with torch's seeded device generator;
    used to fill many layers quickly.  Returns uint8 [rows * bytes_per_row]."""
    import torch
    bb = BLOCK_BYTES[fmt]
    nblk = rows * (cols // BLOCK_WEIGHTS[fmt])
    raw = torch.randint(0, 256, (nblk, bb), dtype=torch.uint8, device=device, generator=generator)
    for off, mult, base in _FP16_FIELDS[fmt]:
        u = torch.rand(nblk, dtype=torch.float64, device=device, generator=generator) + 1.0
        h = (mult * u * base).to(torch.float16)
        raw[:, off:off + 2] = h.view(torch.uint8).view(nblk, 2)
    return raw.reshape(-1)
