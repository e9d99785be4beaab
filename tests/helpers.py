"""Shared helpers for the parity tests: GPU gating, tolerance rules, reporting."""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

# Mantissa bits (explicit) of each storage dtype.
_MANT = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


def require_gpu():
    """Skip when no GPU is visible.  With a GPU present, a missing library fails."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import exact_io_aware_forward_amd as fa
    fa.load_library()   # raises (the test fails) if libfa.so was not built


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half the spacing of `dtype` numbers at |x| (0 where x == 0)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if dtype == torch.float16:
        e = np.maximum(e, -14.0)
    return np.where(ax > 0, 2.0 ** (e - _MANT[dtype]) / 2, 0.0)


def o_tolerance(o_ref: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Element-wise bound on |O_gpu - O_ref|.

    fp32: 1e-5 max-abs.  fp16/bf16: 1e-2 plus half an ulp of the output dtype at
    O_ref, because the output itself is rounded to that dtype once (the literal
    1e-2 alone is below bf16's spacing for |O| >= 2, see
    tests/test_tolerance_reading.py)."""
    if dtype == torch.float32:
        return np.full(o_ref.shape, 1e-5)
    return 1e-2 + half_ulp(o_ref, dtype)


LSE_TOL = {torch.float32: 1e-5, torch.float16: 1e-3, torch.bfloat16: 1e-3}
GRAD_REL_FRO = 5e-2


def rel_fro(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_F / ||ref||_F, with the denominator floored at an RMS of 1e-3.

    The floor only matters where the exact gradient is (nearly) zero, e.g. N = 1,
    where dS = A (dA - D) vanishes identically and a relative error is undefined;
    there the bound becomes an absolute RMS error of 5e-5."""
    floor = 1e-3 * math.sqrt(ref.size)
    return float(np.linalg.norm((x - ref).ravel()) / max(np.linalg.norm(ref.ravel()), floor))


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, dtype, label=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    tol = o_tolerance(o_ref, dtype)
    bad = err > tol
    lerr = np.abs(np.asarray(lse_gpu, np.float64) - lse_ref)
    print(f"[{label}] O max-abs {err.max():.3e} (worst slack {(err - tol).max():.3e}), "
          f"LSE max-abs {lerr.max():.3e}", file=sys.stderr, flush=True)
    assert np.isfinite(o_gpu).all(), f"{label}: non-finite O"
    assert not bad.any(), f"{label}: {bad.sum()} O elements out of tolerance, max err {err.max()}"
    assert lerr.max() <= LSE_TOL[dtype], f"{label}: LSE max-abs {lerr.max()}"


def check_grads(g_gpu: dict, g_ref: dict, label=""):
    msgs = []
    for name in ("dq", "dk", "dv"):
        r = rel_fro(np.asarray(g_gpu[name], np.float64), g_ref[name])
        msgs.append(f"{name} {r:.3e}")
        assert np.isfinite(g_gpu[name]).all(), f"{label}: non-finite {name}"
        assert r <= GRAD_REL_FRO, f"{label}: {name} relative Frobenius error {r}"
    print(f"[{label}] grads rel-Fro: " + ", ".join(msgs), file=sys.stderr, flush=True)


def announce(label: str):
    """Print the case name before a GPU step, so a fault names its case."""
    print(f"== GPU case: {label}", file=sys.stderr, flush=True)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def score_shift(q_a, k_a, q_b, k_b, scale, causal):
    """delta_i = max over the keys j visible to query i of
    |scale * (q_a_i . k_a_j - q_b_i . k_b_j)|: how far apart two sets of scores
    (e.g. from two E4M3 code sets of the same rotated Q and K) lie, per row."""
    ds = np.abs(scale * (q_a @ k_a.T - q_b @ k_b.T))
    if causal:
        n = ds.shape[0]
        ds = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], ds, 0.0)
    return ds.max(axis=1)


def fp8_tolerances(o_ref, dtype, delta, v):
    """Element-wise bounds on |O_gpu - O_ref| and |LSE_gpu - LSE_ref| when the GPU
    forms its scores from codes that may differ from the reference's, with the
    per-row score shift delta (score_shift): a shift of at most delta in every
    score of a row changes each softmax weight by a factor in [e^-2delta,
    e^2delta], so O moves by at most (e^(2 delta) - 1) max_j |V_j| and LSE by at
    most delta (tests/test_oracle_fp8_pins.py checks both on the oracle).  Added
    to the 16-bit rule of o_tolerance and LSE_TOL."""
    vmax = np.abs(v).max()
    o_tol = o_tolerance(o_ref, dtype) + (np.expm1(2 * delta) * vmax)[:, None]
    return o_tol, LSE_TOL[dtype] + delta


# Accumulation precision of gfx950's E4M3 matrix instruction: its fp32 result
# differs from the exact sum of the 64 exact products by up to 2^-11.7 of the
# sum of their magnitudes (worst of 300 sums measured against exact CPU sums,
# uniform, Gaussian, outlier and cancelling operands; the 16-bit instructions
# accumulate in fp32).  2^-11 leaves a margin.
EPS_FP8_ACC = 2.0 ** -11


def fp8_acc_shift(q, k, scale, causal):
    """Per-row bound on the score error of the E4M3 product: EPS_FP8_ACC times
    scale * sum_c |q_ic k_jc|, maximised over the visible keys j."""
    mag = scale * (np.abs(q) @ np.abs(k).T)
    if causal:
        n = mag.shape[0]
        mag = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], mag, 0.0)
    return EPS_FP8_ACC * mag.max(axis=1)
