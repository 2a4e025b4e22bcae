"""Seeded synthetic workloads for the hierarchical local attention path.

This module holds the workload shapes and the seeded input generator that both
the CPU oracle and the GPU library are fed from.  It contains none of the
method's arithmetic: only shapes and random draws, rounded to the storage type.

Shapes follow the token grids the UltraGen pages work at (1K = 64x64 latent
tokens, 4K = 256x256, 8K = 512x512, l = 16, rho = 4; "UltraGen: Efficient
Ultra-High-Resolution Image Generation with Hierarchical Local Attention",
papernotes.org notes, sections 关键设计 1 and 2).  Head count, head size, text
length and the ragged 250x380 grid are the evaluation shapes chosen for this
library; the pages do not state them.  The values stand in for real MMDiT
activations, which need trained weights: Q, K, V are independent N(0, 1) draws.

Recipe: for workload ``cfg_id``, tensor ``t`` (Q=0, K=1, V=2, and for the
backward the output gradient dO=3) and head ``h``,
``numpy.random.default_rng([2026, cfg_id, t, h]).standard_normal((L, D))`` in
float64, rounded to float32 (round-to-nearest-even), then for bf16 workloads
rounded again to bfloat16 (round-to-nearest-even on the float32 bits), then
multiplied by the tensor's scale (a power of two, so exact).
"""
from __future__ import annotations

import concurrent.futures as _cf
from dataclasses import dataclass, asdict

import numpy as np

Q, K, V, DO = 0, 1, 2, 3


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    hr_h: int
    hr_w: int
    lr_h: int
    lr_w: int
    n_text: int
    heads: int
    head_dim: int
    dtype: str            # "f32" or "bf16"
    window: int = 16
    radius: int = 1
    rho: int = 4
    rope_theta: float = 10000.0
    batch: int = 1
    q_scale: float = 1.0  # power of two; 8 gives peaked softmax rows
    lr_mode: int = 0      # 0: HR queries see every LR token; 1: corresponding LR windows only

    @property
    def n_hr(self) -> int:
        return self.hr_h * self.hr_w

    @property
    def n_lr(self) -> int:
        return self.lr_h * self.lr_w

    @property
    def seq_len(self) -> int:
        return self.n_text + self.n_hr + self.n_lr

    def shape(self):
        return (self.batch, self.seq_len, self.heads, self.head_dim)

    def as_dict(self):
        return asdict(self)

    def with_(self, **kw) -> "Workload":
        d = asdict(self)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # tiny fp32: 32x32 HR (2x2 windows), 8x8 LR, 16 text, 2 heads, D=64
    "tiny": Workload("tiny", 0, 32, 32, 8, 8, 16, 2, 64, "f32"),
    # 1K-equivalent: 64x64 HR, 16x16 LR, 512 text, 24 heads, D=128
    "1k": Workload("1k", 1, 64, 64, 16, 16, 512, 24, 128, "bf16"),
    "2k": Workload("2k", 2, 128, 128, 32, 32, 512, 24, 128, "bf16"),
    # headline: 256x256 HR = 65,536 tokens, 64x64 LR, 512 text
    "4k": Workload("4k", 3, 256, 256, 64, 64, 512, 24, 128, "bf16"),
    "8k": Workload("8k", 4, 512, 512, 128, 128, 512, 24, 128, "bf16"),
    # ragged: partial edge windows (ceil partition), LR 63x95
    "ragged": Workload("ragged", 5, 250, 380, 63, 95, 512, 24, 128, "bf16"),
    # small cases where the window mask bites and tails are ragged
    "tiny_masked": Workload("tiny_masked", 6, 48, 48, 12, 12, 16, 2, 64, "f32"),
    "small_ragged": Workload("small_ragged", 7, 40, 56, 10, 14, 40, 3, 128, "bf16"),
    "small_d64": Workload("small_d64", 8, 48, 40, 12, 10, 24, 2, 64, "bf16"),
    "small_ragged_f32": Workload("small_ragged_f32", 9, 37, 45, 10, 12, 9, 2, 64, "f32"),
    # corresponding-LR variant (each HR window sees the LR anchors of its
    # neighbourhood only); LR grids that overhang the HR grid put anchors
    # outside every window
    "4k_corr": Workload("4k_corr", 10, 256, 256, 64, 64, 512, 24, 128, "bf16", lr_mode=1),
    "small_ragged_corr": Workload("small_ragged_corr", 11, 40, 56, 10, 14, 40, 3, 128, "bf16", lr_mode=1),
    "tiny_masked_corr": Workload("tiny_masked_corr", 12, 48, 48, 12, 12, 16, 2, 64, "f32", lr_mode=1),
    "ragged_corr_f32": Workload("ragged_corr_f32", 13, 37, 45, 11, 13, 9, 2, 64, "f32", lr_mode=1),
    # two images of 8 heads: batch*heads = 16, so the work queues group each
    # head's long items on one XCD; ragged 72x88 grid
    "ragged_b2": Workload("ragged_b2", 14, 72, 88, 18, 22, 64, 8, 128, "bf16", batch=2),
    # the 4K layer with head_dim 64 (the D = 64 kernels at full size) and with
    # radius 2 (5x5 windows: 25 HR ranges per query tile)
    "4k_d64": Workload("4k_d64", 15, 256, 256, 64, 64, 512, 24, 64, "bf16"),
    "4k_r2": Workload("4k_r2", 16, 256, 256, 64, 64, 512, 24, 128, "bf16", radius=2),
    # fp32 with head_dim 128 (the fp32 D = 128 attention kernel), ragged grid
    "small_f32_d128": Workload("small_f32_d128", 17, 40, 56, 10, 14, 40, 3, 128, "f32"),
}


def _round_f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (inputs finite)."""
    u = x32.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _scale(w: Workload, tensor: int) -> float:
    return w.q_scale if tensor == Q else 1.0


def head_storage(w: Workload, tensor: int, head: int, batch: int = 0) -> np.ndarray:
    """One head's [L, D] block in storage form: uint16 bf16 bits or float32."""
    seed = [2026, w.cfg_id, tensor, head] if batch == 0 else [2026, w.cfg_id, tensor, head, batch]
    x = np.random.default_rng(seed).standard_normal((w.seq_len, w.head_dim))
    x32 = x.astype(np.float32) * np.float32(_scale(w, tensor))
    if w.dtype == "f32":
        return x32
    return _round_f32_to_bf16_bits(x32)


def head_f64(w: Workload, tensor: int, head: int, batch: int = 0) -> np.ndarray:
    """Exact float64 values of one head's stored [L, D] block."""
    s = head_storage(w, tensor, head, batch)
    if w.dtype == "f32":
        return s.astype(np.float64)
    return bf16_bits_to_f64(s)


def tensor_storage(w: Workload, tensor: int, threads: int = 8) -> np.ndarray:
    """Whole [B, L, Hh, D] tensor in storage form (uint16 bf16 bits or float32)."""
    dt = np.float32 if w.dtype == "f32" else np.uint16
    out = np.empty(w.shape(), dtype=dt)
    jobs = [(b, h) for b in range(w.batch) for h in range(w.heads)]

    def fill(bh):
        b, h = bh
        out[b, :, h, :] = head_storage(w, tensor, h, b)

    with _cf.ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, jobs))
    return out


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.astype(np.float64) if dtype == "f32" else bf16_bits_to_f64(a)


# --------------------------------------------------------------------------
# Warm-start latents: channels-last [B, H, W, C] latent grids (C = 64 as in
# FLUX's packed latent tokens; the pages do not state it).  x_lr and the noise
# X_T are independent N(0, 1) draws, seeded [2026, cfg_id, 10 or 11, batch].
# --------------------------------------------------------------------------
WARM_LR, WARM_NOISE = 10, 11


@dataclass(frozen=True)
class WarmWorkload:
    name: str
    cfg_id: int
    batch: int
    hr_h: int
    hr_w: int
    lr_h: int
    lr_w: int
    channels: int
    rho: int
    dtype: str
    alpha: float = 0.6    # t / T
    sharpen: float = 0.5

    def with_(self, **kw) -> "WarmWorkload":
        d = asdict(self)
        d.update(kw)
        return WarmWorkload(**d)


WARM_WORKLOADS = {
    "warm_tiny": WarmWorkload("warm_tiny", 30, 1, 40, 36, 10, 9, 8, 4, "f32"),
    "warm_ragged": WarmWorkload("warm_ragged", 31, 2, 250, 380, 63, 95, 64, 4, "bf16"),
    "warm_4k": WarmWorkload("warm_4k", 32, 1, 256, 256, 64, 64, 64, 4, "bf16"),
    "warm_4k_b16": WarmWorkload("warm_4k_b16", 33, 16, 256, 256, 64, 64, 64, 4, "bf16"),
}


def warm_storage(w: WarmWorkload, tensor: int) -> np.ndarray:
    """x_lr [B, h, w, C] (tensor WARM_LR) or noise [B, H, W, C] (WARM_NOISE) in
    storage form (float32, or uint16 bf16 bits)."""
    hh, ww = (w.lr_h, w.lr_w) if tensor == WARM_LR else (w.hr_h, w.hr_w)
    out = []
    for b in range(w.batch):
        x = np.random.default_rng([2026, w.cfg_id, tensor, b]).standard_normal((hh, ww, w.channels))
        x32 = x.astype(np.float32)
        out.append(x32 if w.dtype == "f32" else _round_f32_to_bf16_bits(x32))
    return np.stack(out)


def warm_f64(w: WarmWorkload, tensor: int) -> np.ndarray:
    a = warm_storage(w, tensor)
    return a.astype(np.float64) if w.dtype == "f32" else bf16_bits_to_f64(a)
