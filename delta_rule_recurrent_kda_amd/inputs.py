"""Seeded synthetic inputs for the KDA forward scan.

This module only draws random numbers and lays them out; it holds none of the
scan's arithmetic, so both the fp64 oracle and the HIP path can consume it.

Token stream (Chimera, arXiv 2607.28611, Sec. 3 "KDA" paragraph and the
explainer's "One stream, three mechanisms" section): a text prefix followed by
visual tokens in temporal-major raster order, position (i, j, k) of a (T, H, W)
latent grid going to index m = i*H*W + j*W + k, an image being a one-frame grid.
Samples are packed back to back with no padding and addressed by ``cu_seqlens``.

Draws (all in fp64, token order, one generator per (tensor, head) slice so any
slice can be regenerated alone):
  q, k ~ N(0, 1)^d, each (token, head) vector L2-normalised before the cast
  v    ~ N(0, 1)^d
  log_alpha = -U(lo, hi) per key channel
  beta = sigmoid(N(0, 1))
then one cast to the storage dtype by round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

TENSOR_ID = {"q": 1, "k": 2, "v": 3, "log_alpha": 4, "beta": 5}


# ----------------------------------------------------------------------------
# bf16 storage: round-to-nearest-even from fp64, carried as uint16 bit patterns
# ----------------------------------------------------------------------------
def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even); return uint16 bits.

    The fp32 cast is exact enough everywhere except where it lands exactly on a
    bf16 halfway point; there the fp64 value decides the direction (a plain
    second rounding would round an inexact tie to even instead).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    bits = f.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    out = ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    ties = np.flatnonzero((bits & np.uint32(0xFFFF)) == np.uint32(0x8000))
    if ties.size:
        xf, ff = x.reshape(-1)[ties], f.reshape(-1)[ties].astype(np.float64)
        hi = (bits.reshape(-1)[ties] >> np.uint32(16)).astype(np.uint16)
        o = out.reshape(-1)
        o[ties] = np.where(np.abs(xf) > np.abs(ff), hi + np.uint16(1),
                           np.where(np.abs(xf) < np.abs(ff), hi, o[ties]))
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def raster_index(i: int, j: int, k: int, H: int, W: int) -> int:
    """Temporal-major raster position of latent (i, j, k) in a (T, H, W) grid."""
    return i * H * W + j * W + k


# ----------------------------------------------------------------------------
# problem description
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class KdaSpec:
    name: str
    seq_lens: Tuple[int, ...]
    heads: int
    dk: int
    dv: int
    dtype: str                      # "f32" or "bf16"
    log_alpha_range: Tuple[float, float]
    seed: int                       # first word of every generator key
    text_tokens: Tuple[int, ...] = ()
    grid: Optional[Tuple[int, int, int]] = None   # (T, H, W) of the visual part

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def head_tokens(self) -> int:
        return self.total_tokens * self.heads

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)]).astype(np.int32)


def _packed_lengths_seed_rule() -> Tuple[int, List[int]]:
    """Eight sample lengths U[512, 4096] whose total is about 16K tokens.

    Draw integers(512, 4097, 8) from default_rng(s) for s = 1001, 1002, ... and
    keep the first draw whose total lies in [15360, 17408].
    """
    for s in range(1001, 2001):
        lens = np.random.default_rng(s).integers(512, 4097, 8)
        if 15360 <= int(lens.sum()) <= 17408:
            return s, [int(x) for x in lens]
    raise RuntimeError("no seed found")


def config(cfg: int) -> KdaSpec:
    """The five named workloads (tiny fp32 case, packed batch, image, 5 s clip, 30 s clip)."""
    if cfg == 0:
        return KdaSpec("tiny-f32-d64", (1024,), 1, 64, 64, "f32", (0.001, 0.1), 0,
                       text_tokens=(64,), grid=(4, 8, 30))
    if cfg == 1:
        _, lens = _packed_lengths_seed_rule()
        return KdaSpec("packed8-bf16-d128", tuple(lens), 16, 128, 128, "bf16", (0.001, 0.1), 1,
                       text_tokens=(128,) * 8)
    if cfg == 2:
        return KdaSpec("image4x4352-bf16-d128", (4352,) * 4, 16, 128, 128, "bf16", (0.0005, 0.05), 2,
                       text_tokens=(256,) * 4, grid=(1, 64, 64))
    if cfg == 3:
        return KdaSpec("clip5s-33272-bf16-d128", (512 + 21 * 30 * 52,), 16, 128, 128, "bf16",
                       (0.0005, 0.05), 3, text_tokens=(512,), grid=(21, 30, 52))
    if cfg == 4:
        return KdaSpec("clip30s-189272-bf16-d128", (512 + 121 * 30 * 52,), 16, 128, 128, "bf16",
                       (0.0005, 0.05), 4, text_tokens=(512,), grid=(121, 30, 52))
    raise ValueError(f"unknown config {cfg}")


def custom(seq_lens: Sequence[int], heads: int, d: int, dtype: str = "bf16",
           log_alpha_range=(0.001, 0.1), seed: int = 100, dv: Optional[int] = None) -> KdaSpec:
    return KdaSpec(f"custom-{seed}", tuple(int(x) for x in seq_lens), heads, d,
                   d if dv is None else dv, dtype, tuple(log_alpha_range), seed)


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------
def _rng(spec: KdaSpec, tensor: str, head: int) -> np.random.Generator:
    return np.random.default_rng([spec.seed, TENSOR_ID[tensor], head])


def draw_head(spec: KdaSpec, tensor: str, head: int) -> np.ndarray:
    """fp64 draw of one (tensor, head) slice over all T tokens, token order."""
    T, rng = spec.total_tokens, _rng(spec, tensor, head)
    if tensor in ("q", "k"):
        x = rng.standard_normal((T, spec.dk))
        n = np.linalg.norm(x, axis=1, keepdims=True)
        return x / np.where(n == 0, 1.0, n)
    if tensor == "v":
        return rng.standard_normal((T, spec.dv))
    if tensor == "log_alpha":
        lo, hi = spec.log_alpha_range
        return -rng.uniform(lo, hi, (T, spec.dk))
    if tensor == "beta":
        return 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    raise ValueError(tensor)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    raise ValueError(dtype)


def generate(spec: KdaSpec, heads: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Stored-dtype arrays q, k, log_alpha: [T, H, dk]; v: [T, H, dv]; beta: [T, H].

    bf16 tensors are uint16 bit patterns. ``heads`` restricts which head slices
    are drawn (others stay zero) so that large workloads can be sampled cheaply.
    """
    T, H = spec.total_tokens, spec.heads
    store = np.float32 if spec.dtype == "f32" else np.uint16
    out = {
        "q": np.zeros((T, H, spec.dk), store),
        "k": np.zeros((T, H, spec.dk), store),
        "v": np.zeros((T, H, spec.dv), store),
        "log_alpha": np.zeros((T, H, spec.dk), store),
        "beta": np.zeros((T, H), store),
    }
    jobs = [(name, h) for h in (range(H) if heads is None else heads) for name in out]

    def fill(job):
        name, h = job
        out[name][:, h] = _cast(draw_head(spec, name, h), spec.dtype)

    if len(jobs) > 1 and spec.total_tokens * spec.dk > 1 << 16:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, jobs))
    else:
        for job in jobs:
            fill(job)
    out["cu_seqlens"] = spec.cu_seqlens()
    return out


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of a stored-dtype array."""
    if dtype == "f32":
        return arr.astype(np.float64)
    return bf16_bits_to_f64(arr)
