"""Seeded synthetic inputs for fused linear cross-entropy (FLCE).

This module is shared by the oracle's tests, the GPU parity tests, ``bench.py``
and ``smoke()``.  It draws random numbers and rounds them to the storage dtype;
it holds none of the method's arithmetic (no logits, softcap, softmax or
gradients), so it can serve both sides without coupling them.

Workloads stand in for the pages' runs, which use randomly initialised models at
real lm_head dimensions and no dataset:

* Liger-Kernel commit e6a81bb0c3 ("Muse Glimmer" support), section "Memory":
  hidden 6656, vocab 202048, bf16, random init.
* Liger-Kernel commit 40a9d8a61b ("DeepSeek-V3" support), section "Memory":
  hidden 7168, vocab 129280, bf16, random init, batch 1 x seq 8192 and
  4 x 8192.

Recipe (each config has its own seed, values drawn in this order):

1. ``h = standard_normal((N, H), float32)``
2. ``W = 0.02 * standard_normal((V, H), float32)`` (0.02 is a standard
   deviation, the usual ``initializer_range``)
3. bf16 configs: both rounded to bf16 with round-to-nearest-even on the fp32
   bit pattern; fp32 configs keep the fp32 values.
4. labels: ``integers(0, V, N)`` (uniform) or a Zipf(s) law truncated to
   ranks 1..V with token id = rank - 1, drawn by inverse CDF.
5. ignore mask: exactly ``round(f * N)`` rows, either chosen uniformly without
   replacement, or as one padding run at the tail of each sequence.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

IGNORE_INDEX = -100

# Rows of W drawn per call; drawing in blocks yields the same stream as one
# call (checked in tests/test_synth.py) and bounds host memory.
_W_BLOCK_ROWS = 8192


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str            # "bf16" or "f32"
    N: int
    H: int
    V: int
    ignore_frac: float
    labels: str           # "uniform" or "zipf"
    softcap_T: float      # <= 0: no softcap
    multiplier: float
    reduction: str        # "mean" or "sum"
    seed: int
    zipf_s: float = 1.1
    seq_len: Optional[int] = None   # tail padding runs per sequence when set
    ignore_layout: str = "random"   # "random" or "tail"

    @property
    def n_ignored(self) -> int:
        return int(round(self.ignore_frac * self.N))

    @property
    def n_valid(self) -> int:
        return self.N - self.n_ignored


# The five workloads: a small fp32 case the oracle finishes in seconds, then
# the bf16 lm_head shapes.  Muse-Glimmer-shaped (c4) is the headline workload.
CONFIGS = {
    "c1": Config("c1", "f32", 256, 128, 1024, 0.10, "uniform", 0.0, 1.0, "mean", 1001),
    "c2": Config("c2", "bf16", 4096, 4096, 128256, 0.05, "uniform", 0.0, 1.0, "mean", 1002),
    "c3": Config("c3", "bf16", 8192, 7168, 129280, 0.05, "zipf", 0.0, 1.0, "mean", 1003),
    "c4": Config("c4", "bf16", 8192, 6656, 202048, 0.05, "uniform", 30.0, 0.5, "mean", 1004),
    "c5": Config("c5", "bf16", 32768, 7168, 129280, 0.20, "zipf", 30.0, 1.0, "sum", 1005,
                 seq_len=8192, ignore_layout="tail"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_labels(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """Truncated Zipf over ranks 1..V, P(k) proportional to k**-s, token id = k-1."""
    k = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-s))
    cdf /= cdf[-1]
    u = rng.random(n)
    ids = np.searchsorted(cdf, u, side="right")
    return np.minimum(ids, V - 1).astype(np.int64)


def tail_run_lengths(total: int, n_seq: int) -> list:
    """Split ``total`` ignored rows over ``n_seq`` sequences, shorter runs first."""
    base, extra = divmod(total, n_seq)
    return [base + (1 if i >= n_seq - extra else 0) for i in range(n_seq)]


@dataclasses.dataclass
class Case:
    """One seeded input set.  ``h``/``W`` hold the storage dtype's values:
    uint16 bf16 bit patterns for bf16, float32 for f32."""
    cfg: Config
    h: np.ndarray
    W: np.ndarray
    labels: np.ndarray

    def h_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.h) if self.cfg.dtype == "bf16" else self.h

    def W_f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.W) if self.cfg.dtype == "bf16" else self.W

    def digest(self) -> str:
        m = hashlib.sha256()
        for a in (self.h, self.W, self.labels):
            m.update(np.ascontiguousarray(a).view(np.uint8))
        return m.hexdigest()[:16]


def _draw_matrix(rng, rows, cols, scale, dtype, block_rows=_W_BLOCK_ROWS):
    out = np.empty((rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[r0:r1] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out


def make_case(cfg: Config, *, N: Optional[int] = None, H: Optional[int] = None,
              V: Optional[int] = None, seed: Optional[int] = None) -> Case:
    """Draw the inputs of ``cfg`` (sizes and seed may be overridden for small
    parity shapes; the recipe stays the same)."""
    N = cfg.N if N is None else N
    H = cfg.H if H is None else H
    V = cfg.V if V is None else V
    cfg = dataclasses.replace(cfg, N=N, H=H, V=V, seed=cfg.seed if seed is None else seed)
    rng = np.random.default_rng(cfg.seed)
    h = _draw_matrix(rng, N, H, 1.0, cfg.dtype)
    W = _draw_matrix(rng, V, H, 0.02, cfg.dtype)
    if cfg.labels == "uniform":
        labels = rng.integers(0, V, N, dtype=np.int64)
    elif cfg.labels == "zipf":
        labels = zipf_labels(rng, N, V, cfg.zipf_s)
    else:
        raise ValueError(cfg.labels)
    n_ign = cfg.n_ignored
    if n_ign:
        if cfg.ignore_layout == "random":
            idx = rng.choice(N, size=n_ign, replace=False)
            labels[idx] = IGNORE_INDEX
        elif cfg.ignore_layout == "tail":
            S = min(cfg.seq_len or N, N)
            n_seq = max(1, N // S)
            for i, L in enumerate(tail_run_lengths(n_ign, n_seq)):
                end = (i + 1) * S
                labels[end - L:end] = IGNORE_INDEX
        else:
            raise ValueError(cfg.ignore_layout)
    return Case(cfg, h, W, labels)


def small_config(base: str = "c1", **kw) -> Config:
    """A config with the recipe of ``base`` and overridden fields."""
    return dataclasses.replace(CONFIGS[base], **kw)
