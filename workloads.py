"""Seeded synthetic inputs for exact attention, shared by the GPU path's tests,
the benchmark and the oracle checks.

This module holds no attention arithmetic: it only draws random tensors, applies
the outlier recipe and casts to the storage dtype.  Both sides of every parity
check receive exactly the same dtype-rounded tensors; the oracle upcasts them to
float64 without further rounding.

Recipe (one workload per configuration id k):
  * a CPU ``torch.Generator`` seeded with ``k`` (or an explicit seed);
  * draw order Q, K, V, then dO when the workload has a backward pass, each
    i.i.d. N(0, 1) in float32 with shape [B, H, N, d];
  * when ``outlier_frac > 0``: for every (b, h) in row-major order draw a
    ``randperm(N)`` from the same generator and multiply the first
    floor(outlier_frac * N) selected K rows by 8 (a power of two, so the scaling
    is exact in every storage dtype and only the rounding of the cast remains);
  * cast to the storage dtype on the CPU (round-to-nearest-even).

The shapes are those of the typical sequence lengths (1K-8K, and 16K for long
context) and head dimensions (64-128) named by the CMU 11-868 FlashAttention
notes (quidproquo.cc), section "The scenario", slide page 5.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    dtype: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    backward: bool
    outlier_frac: float = 0.0

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]


def default_scale(d: int) -> float:
    """1/sqrt(d), rounded to float32 so both sides use the identical value."""
    return float(np.float32(1.0 / math.sqrt(d)))


WORKLOADS = {
    1: Workload(1, "fwd_fp32_B1_H1_N128_d64", "fp32", 1, 1, 128, 64, False, False),
    2: Workload(2, "fwd_bf16_B8_H16_N1024_d64", "bf16", 8, 16, 1024, 64, False, False),
    3: Workload(3, "fwdbwd_fp16_B4_H16_N2048_d64", "fp16", 4, 16, 2048, 64, False, True),
    4: Workload(4, "fwdbwd_causal_bf16_B2_H16_N4096_d128_koutliers", "bf16", 2, 16, 4096, 128,
                True, True, 0.05),
    5: Workload(5, "fwdbwd_causal_bf16_B1_H32_N16384_d128", "bf16", 1, 32, 16384, 128, True, True),
}


def draw(B: int, H: int, N: int, d: int, dtype: str, seed: int, with_do: bool = True,
         outlier_frac: float = 0.0, outlier_mult: float = 8.0) -> dict:
    """Draw Q, K, V (and dO) per the recipe above; returns CPU tensors in ``dtype``."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=gen, dtype=torch.float32)
    k = torch.randn(shape, generator=gen, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, dtype=torch.float32)
    do = torch.randn(shape, generator=gen, dtype=torch.float32) if with_do else None
    n_out = int(math.floor(outlier_frac * N))
    if n_out > 0:
        for b in range(B):
            for h in range(H):
                idx = torch.randperm(N, generator=gen)[:n_out]
                k[b, h, idx] *= outlier_mult
    td = DTYPES[dtype]
    out = {"q": q.to(td), "k": k.to(td), "v": v.to(td)}
    if do is not None:
        out["do"] = do.to(td)
    return out


def workload_inputs(cid: int) -> dict:
    """Inputs of configuration ``cid`` with its own seed (the id)."""
    w = WORKLOADS[cid]
    return draw(w.B, w.H, w.N, w.d, w.dtype, seed=cid, with_do=w.backward,
                outlier_frac=w.outlier_frac)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of a dtype-rounded tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


# Split-K decode (Lecture 9 notes §9.8: one new token against the whole cache;
# CMU 11-868 notes, slide pages 57-60: contexts up to 128K).  A head layout of
# 32 heads of d = 128, one query per sequence, a 128K-token cache.
@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    dtype: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    Hkv: int = 0      # key/value heads (0: as many as query heads)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]


DECODE_WORKLOAD = DecodeWorkload("decode_bf16_B1_H32_Nq1_Nk131072_d128", "bf16", 1, 32, 1,
                                 131072, 128, True, 106)
# The same with grouped key/value heads: 32 query heads share 4 key/value heads
# (groups of 8), the case the CMU notes' GQA packing addresses.
DECODE_WORKLOAD_GQA = DecodeWorkload("decode_gqa8_bf16_B1_H32_Hkv4_Nq1_Nk131072_d128", "bf16", 1,
                                     32, 1, 131072, 128, True, 107, Hkv=4)


def draw_decode(B: int, H: int, nq: int, nk: int, d: int, dtype: str, seed: int,
                hkv: int | None = None) -> dict:
    """Q [B, H, nq, d], then K and V [B, hkv, nk, d] (hkv = H unless given), i.i.d.
    N(0, 1) from one CPU generator seeded with ``seed`` (draw order Q, K, V), cast to
    ``dtype`` (RNE)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    hkv = H if hkv is None else hkv
    out = {}
    for name, h, n in (("q", H, nq), ("k", hkv, nk), ("v", hkv, nk)):
        out[name] = torch.randn((B, h, n, d), generator=gen, dtype=torch.float32).to(DTYPES[dtype])
    return out


def draw_signs(d: int, seed: int) -> torch.Tensor:
    """Random signs (+1 / -1, float32 [d]) for the FP8 path's Hadamard rotation."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randint(0, 2, (d,), generator=gen).to(torch.float32) * 2 - 1
