"""Why the bf16 output tolerance is read as 1e-2 plus half an ulp of the output.

The N=4096, d=128, causal bf16 workload multiplies 5% of the K rows by 8, which
makes many attention rows nearly one-hot, so |O| reaches about 4-4.5.  Near 4 the
bf16 spacing is 2^-5 = 0.03125, so even the exact float64 output, rounded once
to bf16, misses a literal max-abs bound of 1e-2.  No kernel can beat that
rounding; the element-wise rule |O_gpu - O_ref| <= 1e-2 + ulp(O_ref)/2 keeps the
1e-2 budget for the kernel's own error and adds only the unavoidable output
rounding.
"""
import numpy as np
import torch

import oracle
import workloads


def half_ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7) / 2, 0.0)


def test_exactly_rounded_output_fails_the_literal_bound_at_the_outlier_workload():
    w = workloads.WORKLOADS[4]
    x = workloads.workload_inputs(4)
    q, k, v = (workloads.to_f64(x[n][0, 0]) for n in "qkv")
    o, _ = oracle.forward_head(q, k, v, True, w.scale)
    o_bf16 = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    err = np.abs(o_bf16 - o)
    assert err.max() > 1e-2                       # the literal reading fails ...
    assert (err <= 1e-2 + half_ulp_bf16(o)).all()  # ... the relaxed one holds


def test_lse_needs_the_unrounded_denominator_at_the_outlier_workload():
    """The kernels normalise O by the sum of the probabilities as rounded for P V,
    but take LSE from a separate fp32 sum of the unrounded ones.  This pins why:
    at the same workload, an LSE formed from the rounded (bf16) probabilities
    would miss the 1e-3 LSE bound on some rows, while the fp32 sum is exact to
    ~1e-7 relative."""
    w = workloads.WORKLOADS[4]
    x = workloads.workload_inputs(4)
    q, k = (workloads.to_f64(x[n][0, 0]) for n in "qk")
    _, lse = oracle.forward_head(q, k, workloads.to_f64(x["v"][0, 0]), True, w.scale)
    n = q.shape[0]
    s = (q @ k.T) * w.scale
    s[np.triu_indices(n, 1)] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p_rounded = torch.from_numpy(p).to(torch.bfloat16).double().numpy()
    lse_rounded = m[:, 0] + np.log(p_rounded.sum(axis=1))
    lse_fp32_sum = m[:, 0] + np.log(p.astype(np.float32).sum(axis=1, dtype=np.float32))
    assert np.abs(lse_rounded - lse).max() > 1e-3
    assert np.abs(lse_fp32_sum - lse).max() < 1e-5
