"""Float64 CPU oracle for the FP8 forward with incoherent processing.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
It imports nothing from the HIP path and shares no code with it.

What the pages fix (CMU 11-868 FlashAttention notes at quidproquo.cc,
"FlashAttention-3: asynchrony and FP8 on Hopper", slide page 24): FP8 scores
suffer from outliers, and the remedy is to multiply Q and K by one and the same
random orthogonal Hadamard matrix J.  Since (QJ)(KJ)^T = QK^T the product is
unchanged, while a large entry is spread over all coordinates; the slide reports
2.6x lower quantisation error on data with simulated outliers.

Readings where the pages are silent:

* J = diag(s) H / sqrt(d), where H is the d x d Sylvester Hadamard matrix
  (H_1 = [1], H_2n = [[H, H], [H, -H]]), d a power of two, and s is a vector of
  random signs that the caller draws and passes in.  J is orthogonal.
* The FP8 format is E4M3 without infinities: 4 exponent bits (bias 7), 3
  mantissa bits, largest finite value 448 = 1.75 * 2^8, smallest normal 2^-6,
  subnormals m * 2^-9.  Rounding is to nearest, ties to even, and values beyond
  448 in magnitude saturate to +-448.
* Scales are per row (per query and per key): a row's largest magnitude maps to
  448 (an all-zero row keeps scale 1 and quantises to zeros).
* Only Q and K go through FP8.  V, the probabilities and the remaining steps are
  those of the 16-bit path, so after dequantisation the oracle is the plain
  definition of ``attention.forward_head`` applied to the dequantised Q J and K J.
"""
from __future__ import annotations

import numpy as np

from .attention import forward_head

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
E4M3_MANTISSA_BITS = 3


def sylvester_hadamard(d: int) -> np.ndarray:
    """The d x d Sylvester Hadamard matrix, entries +-1, d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation(signs: np.ndarray) -> np.ndarray:
    """J = diag(signs) H / sqrt(d): the random orthogonal Hadamard matrix."""
    s = np.asarray(signs, dtype=np.float64)
    if s.ndim != 1 or not np.all(np.abs(s) == 1.0):
        raise ValueError("signs must be a vector of +-1")
    d = s.shape[0]
    return s[:, None] * sylvester_hadamard(d) / np.sqrt(d)


def round_e4m3(x: np.ndarray) -> np.ndarray:
    """Round every value to the nearest E4M3 value (ties to even), saturating at
    +-448.  Returns the rounded values as float64."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    # Spacing of the E4M3 values around |x|: 2^(e - 3) in the binade [2^e, 2^(e+1)),
    # and the subnormal step below the smallest normal.
    _, e2 = np.frexp(np.where(ax > 0, ax, 1.0))     # ax = m * 2^e2 with m in [0.5, 1)
    ulp = np.ldexp(1.0, e2 - 1 - E4M3_MANTISSA_BITS)
    ulp = np.where(ax < E4M3_MIN_NORMAL, E4M3_SUBNORMAL_STEP, ulp)
    r = np.round(ax / ulp) * ulp                    # np.round: half to even
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def quantize_rows(x: np.ndarray):
    """Per-row E4M3 quantisation: returns (codes as float64 values on the E4M3
    grid, scales) with x ~= codes * scales[:, None]."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    scales = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return round_e4m3(x / scales[..., None]), scales


def dequantized_rotated(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """x J, quantised per row to E4M3 and scaled back."""
    codes, scales = quantize_rows(np.asarray(x, np.float64) @ rotation(signs))
    return codes * scales[..., None]


def fp8_scores(q, k, signs, scale: float) -> np.ndarray:
    """scale * deq(Q J) deq(K J)^T, the scores the FP8 path forms."""
    return scale * (dequantized_rotated(q, signs) @ dequantized_rotated(k, signs).T)


def fp8_forward_head(q, k, v, causal: bool, scale: float, signs):
    """(O, LSE) of one head with Q and K rotated by J and quantised to E4M3."""
    return forward_head(dequantized_rotated(q, signs), dequantized_rotated(k, signs),
                        np.asarray(v, np.float64), causal, scale)
