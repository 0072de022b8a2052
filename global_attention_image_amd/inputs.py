"""Seeded synthetic inputs and workload geometry for hierarchical local attention.

This module is shared by the tests, the benchmark and the oracle's callers.  It holds
no arithmetic of the method itself: only the workload table, the seeded random draws
and the float32 -> bfloat16 round-to-nearest-even input rounding.

Workloads stand in for the pages' FLUX generation runs at 2K-8K (UltraGen [it] §3,
[es] §4): activations are not available, so Q, K, V are iid N(0, 1) at the same token
shapes.  The token geometry (16 pixels per latent token per axis) follows the token
counts quoted in UltraGen [es] §1 (a 4K image is 65 536 tokens).

Citation keys: [UltraGen/<lang> §n] is the gist.science summary page "UltraGen:
Efficient Ultra-High-Resolution Image Generation with Hierarchical Local Attention"
in the named language edition (it, fr, es, ar, ko), section n of its technical summary.
"""
from __future__ import annotations

from dataclasses import dataclass, asdict, replace
import math

import numpy as np


@dataclass(frozen=True)
class Geometry:
    """One attention problem.

    Tensors are token-major ``[B, L, heads, head_dim]`` with ``L = T + N + M``: rows
    ``0..T-1`` are text tokens (none unless T > 0), then the hi-res tokens of an ``H x W``
    grid in raster order, then the low-res guide tokens of an ``H_lr x W_lr`` grid in
    raster order.
    """

    B: int
    heads: int
    head_dim: int
    H: int
    W: int
    w: int
    H_lr: int
    W_lr: int
    rho: int = 4
    theta: float = 10000.0
    name: str = "custom"
    # mask options: neighbourhood radius in windows (1 = clipped 3x3) and which guide
    # tokens a hi-res query sees (0 = all; 1 = those whose scaled position lies in the
    # query's own window; 2 = those lying in the query's neighbourhood of windows)
    radius: int = 1
    guide_mode: int = 0
    # text tokens at the front of the joint sequence (text | hi | guide)
    T: int = 0

    @property
    def N(self) -> int:
        return self.H * self.W

    @property
    def M(self) -> int:
        return self.H_lr * self.W_lr

    @property
    def L(self) -> int:
        return self.T + self.N + self.M

    @property
    def n_windows(self) -> int:
        return (self.H // self.w) * (self.W // self.w)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def shape(self) -> tuple:
        return (self.B, self.L, self.heads, self.head_dim)

    def with_(self, **kw) -> "Geometry":
        return replace(self, **kw)

    def as_dict(self) -> dict:
        return asdict(self)


# The five workloads.  Seeds are the position in this list.
CONFIGS = {
    "tiny": Geometry(B=1, heads=2, head_dim=64, H=32, W=32, w=8, H_lr=8, W_lr=8, name="tiny"),
    "2k": Geometry(B=1, heads=24, head_dim=128, H=128, W=128, w=16, H_lr=32, W_lr=32, name="2k"),
    "4k": Geometry(B=1, heads=24, head_dim=128, H=256, W=256, w=16, H_lr=64, W_lr=64, name="4k"),
    "nonsquare": Geometry(B=2, heads=24, head_dim=128, H=256, W=128, w=16, H_lr=64, W_lr=32,
                          name="nonsquare"),
    "8k": Geometry(B=1, heads=24, head_dim=128, H=512, W=512, w=16, H_lr=128, W_lr=128, name="8k"),
}
CONFIG_SEEDS = {name: i for i, name in enumerate(CONFIGS)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs must be finite (the generators only produce finite normals).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


CHUNK = 1 << 22  # elements per independently seeded stream


def _threads() -> int:
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16_bits(shape, seed: int, tensor: int) -> np.ndarray:
    """iid N(0, 1) float32 rounded to bfloat16 bits, C order, reproducible in parallel.

    Element block c (CHUNK elements, C order) of tensor index ``tensor`` is drawn from
    ``numpy.random.default_rng([seed, tensor, c]).standard_normal(..., dtype=float32)``,
    so the values do not depend on the number of worker threads.
    """
    from concurrent.futures import ThreadPoolExecutor

    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def work(c):
        s = c * CHUNK
        e = min(n, s + CHUNK)
        x = np.random.default_rng([seed, tensor, c]).standard_normal(e - s, dtype=np.float32)
        out[s:e] = f32_to_bf16_bits(x)

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


def make_qkv_bits(geom: Geometry, seed: int):
    """Q, K, V as bfloat16 bit patterns, shape ``[B, L, heads, head_dim]``.

    Recipe: iid N(0, 1) float32 in C order, tensor index 0, 1, 2 for Q, K, V, drawn per
    block of CHUNK elements from ``default_rng([seed, tensor, block])`` and rounded to
    bfloat16 (round to nearest even).
    """
    return tuple(normal_bf16_bits(geom.shape(), seed, t) for t in range(3))


def make_config_inputs(name: str):
    """(geometry, q_bits, k_bits, v_bits) for a named workload with its fixed seed."""
    geom = CONFIGS[name]
    return (geom,) + make_qkv_bits(geom, CONFIG_SEEDS[name])


def _axis_neighbour_sum(n: int, r: int) -> int:
    """Sum over n positions of the number of positions within distance r (clipped)."""
    return sum(min(n - 1, i + r) - max(0, i - r) + 1 for i in range(n))


def _guide_cells_per_window(geom: Geometry):
    """[n_wy, n_wx] count of guide cells whose scaled position lies in each window."""
    a, b = geom.H // geom.w, geom.W // geom.w
    cy = np.zeros(a, dtype=np.int64)
    cx = np.zeros(b, dtype=np.int64)
    for i in range(geom.H_lr):
        if geom.rho * i < geom.H:
            cy[(geom.rho * i) // geom.w] += 1
    for j in range(geom.W_lr):
        if geom.rho * j < geom.W:
            cx[(geom.rho * j) // geom.w] += 1
    return cy[:, None] * cx[None, :]


def algorithmic_pairs(geom: Geometry) -> dict:
    """Unmasked (query, key) pairs per (batch, head), by term.

    Geometry bookkeeping for throughput figures: along an axis of n windows the clipped
    neighbour counts within radius r sum to sum_i (min(n-1, i+r) - max(0, i-r) + 1)
    (3n - 2 for r = 1); the local pairs are that product times w^4.
    """
    a, b = geom.H // geom.w, geom.W // geom.w
    r = geom.radius
    local = _axis_neighbour_sum(a, r) * _axis_neighbour_sum(b, r) * geom.w ** 4
    if geom.guide_mode == 0:
        hi_lr = geom.N * geom.M
    else:
        g = _guide_cells_per_window(geom)
        if geom.guide_mode == 2:
            # guide cells of every window within radius r, per query window
            pad = np.pad(g, r)
            g = sum(pad[dy:dy + a, dx:dx + b] for dy in range(2 * r + 1) for dx in range(2 * r + 1))
        hi_lr = int(g.sum()) * geom.w * geom.w
    lr_lr = geom.M * geom.M
    # text: text queries see every key; every other query also sees every text key
    text = geom.T * geom.L + (geom.N + geom.M) * geom.T
    return {"local": local, "hi_lr": hi_lr, "lr_lr": lr_lr, "text": text,
            "total": local + hi_lr + lr_lr + text}


def algorithmic_flops(geom: Geometry) -> dict:
    """Matrix FLOPs of the unmasked pairs: 4 * head_dim per pair (QK^T and PV), all (b, h)."""
    p = algorithmic_pairs(geom)
    f = 4 * geom.head_dim * geom.B * geom.heads
    hi_text = geom.N * geom.T
    lr_text = geom.M * geom.T
    return {"hi": f * (p["local"] + p["hi_lr"] + hi_text), "lr": f * (p["lr_lr"] + lr_text),
            "text": f * geom.T * geom.L, "total": f * p["total"]}
