"""Seeded synthetic inputs for the dense attention forward.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It only draws and shapes random numbers; it holds none of the
attention arithmetic (no products, no softmax, no reductions).

Input recipe (the pages benchmark attention on iid Gaussian Q/K/V tensors of
shape [B, H, S, D]; "Learning FlashAttention the Hard Way - Part 2", the
SDPA_P / SDPA_L definitions, and "B200 Attention Kernel from Scratch to
Near-SOTA in 60 Diagrams", Chapter 14 - Persistent, for the hd128 shapes):

* ``numpy.random.default_rng(seed)`` (PCG64) draws float32 standard normals for
  q, then k, then v, each of shape [B, H, S, D];
* each tensor is rounded to the working dtype (fp16 or bf16) with
  round-to-nearest-even by ``torch.Tensor.to``;
* both the oracle and the GPU path consume exactly these rounded tensors.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, dtype and the seed of its inputs."""

    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    @property
    def flops(self) -> int:
        """Algorithmic FLOP of one forward: 2·S·S·D for Q·Kᵀ plus 2·S·S·D for P·V, per (b, h)."""
        return 4 * self.B * self.H * self.S * self.S * self.D

    @property
    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: read Q, K, V once, write O once, write the fp32 LSE."""
        elem = 2
        return 4 * self.B * self.H * self.S * self.D * elem + 4 * self.B * self.H * self.S

    def as_dict(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "S": self.S, "D": self.D,
                "dtype": self.dtype, "causal": False, "scale": self.scale, "seed": self.seed,
                "layout": "BHSD"}


# The five problems: the small fp16 listing case and the fp16 benchmark case of
# "Learning FlashAttention the Hard Way - Part 2" (SDPA_L, SDPA_P), and three
# hd128 bf16 cases at S = 4K / 8K / 16K with 16384 tokens each.
WORKLOADS = [
    Workload("b1_h4_s128_d64_fp16", 1, 4, 128, 64, "fp16", 1),
    Workload("b1_h8_s4096_d64_fp16", 1, 8, 4096, 64, "fp16", 2),
    Workload("b4_h16_s4096_d128_bf16", 4, 16, 4096, 128, "bf16", 3),
    Workload("b2_h16_s8192_d128_bf16", 2, 16, 8192, 128, "bf16", 4),
    Workload("b1_h16_s16384_d128_bf16", 1, 16, 16384, 128, "bf16", 5),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DTYPES[dtype])


def gaussian_qkv(B: int, H: int, S: int, D: int, dtype: str, seed: int):
    """iid N(0, 1) q, k, v of shape [B, H, S, D], drawn in that order, rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def workload_qkv(w: Workload):
    return gaussian_qkv(w.B, w.H, w.S, w.D, w.dtype, w.seed)


def forced_rebase_qkv(seed: int = 11, B: int = 1, H: int = 1, S: int = 1024, D: int = 64,
                      dtype: str = "bf16", boost: float = 4.0):
    """Inputs whose running row maximum jumps in the second half of the keys.

    Q and K are N(0, 1); keys S/2 .. S-1 are multiplied by ``boost`` so that
    the per-row maximum of the scores grows by several log2 units part-way
    through the key loop (this is what exercises a threshold-guarded rescale).
    V is uniform on (-1, 1) so that peaked rows keep |O| small.
    """
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    k[:, :, S // 2:, :] *= np.float32(boost)
    v = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def tile_signature_v(B: int, H: int, S: int, D: int, dtype: str, tile: int):
    """V whose row j is the one-hot vector e_{(j // tile) mod D} (scaled by 1).

    With Q = 0 every key gets the same weight, so output column c equals the
    fraction of keys whose tile index is congruent to c modulo D.  A K/V tile
    that is skipped, duplicated or read stale moves some column by about
    tile / S.
    """
    v = np.zeros((B, H, S, D), dtype=np.float32)
    j = np.arange(S)
    v[:, :, j, (j // tile) % D] = 1.0
    return _round(v, dtype)


def uniform_qkv(B: int, H: int, S: int, D: int, dtype: str, seed: int, lo: float = -1.0,
                hi: float = 1.0):
    rng = np.random.default_rng(seed)
    shape = (B, H, S, D)
    out = [rng.uniform(lo, hi, size=shape).astype(np.float32) for _ in range(3)]
    return tuple(_round(x, dtype) for x in out)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact decode of an fp16/bf16 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
