"""GPU parity of the FP8 input stage (fa_fp8_quantize_rows through the C ABI)
against the float64 oracle (``oracle/fp8.py``) on the same seeded inputs.

A code is a rounding decision.  The kernel takes it on an fp32 transform, the
oracle on the exact one, so where the exact value lies within fp32 rounding of
a midpoint between two E4M3 values either neighbour is correct: each GPU code
must lie between the oracle's codes for the exact value moved down and up by a
bound on the fp32 error, and at least 99.9 % of codes must equal the oracle's
exactly.  Without rotation and with a scale of exactly 1 the decision is exact,
and every code must match, ties included.

Covered: both 16-bit dtypes, d = 64 and 128, one row, ragged row counts,
outlier channels, all-zero rows, rows so small that 448 / amax would
overflow in fp32, the E4M3 value set and every midpoint, no rotation, and the causal N=4096 d=128 bf16 shape (Q and K, K with 5 % rows x8)
at full size on sampled rows.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_forward_amd as fa
import workloads
from helpers import announce, require_gpu
from oracle import fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def decode_codes(codes):
    return codes.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def check_rows(x, signs, codes, scales, label):
    """Compare GPU codes and scales for rows x ([rows, d], the 16-bit input) with
    the oracle's decision, allowing the neighbour code within the fp32 bound."""
    x64 = x.double().numpy().reshape(-1, x.shape[-1])
    d = x64.shape[1]
    y = x64 @ fp8.rotation(signs) if signs is not None else x64
    amax = np.abs(y).max(axis=1)
    scale = np.where(amax > 0, amax / 448.0, 1.0)
    t = y / scale[:, None]
    # fp32 error of the transform: at most log2(d) + 1 roundings of partial sums
    # bounded by sum|x| / sqrt(d); in code units, times 448 / amax.  Plus the
    # relative roundings of the scale and the division.
    growth = np.abs(x64).sum(axis=1) / math.sqrt(d) / np.where(amax > 0, amax, 1.0)
    rel = 1e-6 + (math.log2(d) + 2) * 2.0 ** -24 * growth if signs is not None \
        else np.full_like(amax, 1e-6)
    band = rel[:, None] * (np.abs(t) + 448.0 * (signs is not None))
    lo, hi = fp8.round_e4m3(t - band), fp8.round_e4m3(t + band)
    want = fp8.round_e4m3(t)
    got = decode_codes(codes).reshape(-1, d)
    s_got = scales.cpu().double().numpy().reshape(-1)
    assert np.isfinite(got).all(), f"{label}: NaN codes"
    # fp32 scales of tiny rows are subnormal: allow one step of the subnormal grid.
    assert (np.abs(s_got - scale) <= 4 * rel * scale + 2.0 ** -149).all(), f"{label}: scales"
    inside = (got >= lo) & (got <= hi)
    assert inside.all(), f"{label}: {(~inside).sum()} codes outside the rounding band"
    exact = (got == want).mean()
    print(f"[{label}] codes equal to the oracle's: {exact:.6f}", flush=True)
    assert exact >= 0.999, label


def signs_for(d, seed):
    return np.random.default_rng(seed).choice([-1.0, 1.0], size=d)


@pytest.mark.parametrize("rows", [1, 7, 333])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_rotate_quantize_matches_oracle(dtype, d, rows):
    gen = torch.Generator().manual_seed(900 + rows + d)
    x = torch.randn((rows, d), generator=gen)
    x[:, [3, d // 2 + 1]] *= 20                           # outlier channels
    if rows > 5:
        x[5] = 0.0                                        # an all-zero row
    x = x.to(workloads.DTYPES[dtype])
    s = signs_for(d, rows)
    announce(f"fp8 rotate+quantize {dtype} d={d} rows={rows}")
    codes, scales = fa.fp8_quantize_rows(x.cuda(), torch.tensor(s, dtype=torch.float32).cuda())
    torch.cuda.synchronize()
    check_rows(x, s, codes, scales, f"{dtype} d={d} rows={rows}")
    if rows > 5:
        # zero codes (the sign flips may make them negative zeros, byte 0x80)
        assert scales[5].item() == 1.0 and (decode_codes(codes[5]) == 0).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_unrotated_rounding_is_exact_on_every_value_and_midpoint(dtype):
    # Every non-negative E4M3 value (subnormals m * 2^-9, normals (1 + f/8) * 2^(E-7)
    # up to 448) and every midpoint, both signs, in rows led by 448 so that each
    # row's scale is 1: the kernel's code for every entry is then an exact
    # round-to-nearest-even.
    vals = np.array([m * 2.0 ** -9 for m in range(8)] +
                    [(1 + f / 8) * 2.0 ** (E - 7) for E in range(1, 16) for f in range(8)][:-1])
    assert len(vals) == 127 and vals[-1] == 448.0
    mids = (vals[:-1] + vals[1:]) / 2
    entries = np.concatenate([vals, mids, -vals[1:], -mids])
    d = 128
    per_row = d - 1
    n = -(-len(entries) // per_row)
    buf = np.zeros((n, d))
    buf[:, 0] = 448.0
    buf[:, 1:].flat[:len(entries)] = entries
    x = torch.tensor(buf).to(workloads.DTYPES[dtype])
    assert np.array_equal(x.double().numpy(), buf)        # exact in the 16-bit input
    announce(f"fp8 unrotated exact rounding {dtype}")
    codes, scales = fa.fp8_quantize_rows(x.cuda())
    torch.cuda.synchronize()
    assert (scales.cpu() == 1.0).all()
    np.testing.assert_array_equal(decode_codes(codes), fp8.round_e4m3(buf))


@pytest.mark.parametrize("rotate", [False, True])
def test_tiny_rows_get_finite_codes(rotate):
    # Rows whose largest magnitude lies below 448 / FLT_MAX (about 1.3e-36), where
    # 448 / amax would overflow to inf: the kernel scales such rows by an exact
    # power of two first, so their codes are the same decisions as for any row.
    gen = torch.Generator().manual_seed(41)
    x = torch.randn((24, 128), generator=gen) * 1e-37
    x[5] *= 1e4          # amax around 4e-33: below 2^-100, 448 / amax still finite
    x[7] = 0.0
    x[9, 17] = 3e-38     # one entry only
    x = x.to(torch.bfloat16)
    s = signs_for(128, 41) if rotate else None
    announce(f"fp8 tiny rows rotate={rotate}")
    codes, scales = fa.fp8_quantize_rows(
        x.cuda(), torch.tensor(s, dtype=torch.float32).cuda() if rotate else None)
    torch.cuda.synchronize()
    check_rows(x, s, codes, scales, f"tiny rows rotate={rotate}")
    assert (decode_codes(codes[7]) == 0).all() and scales[7].item() == 1.0


def test_unrotated_random_rows_match_oracle():
    gen = torch.Generator().manual_seed(31)
    x = (torch.randn((500, 64), generator=gen) * 3).to(torch.bfloat16)
    announce("fp8 unrotated random")
    codes, scales = fa.fp8_quantize_rows(x.cuda())
    torch.cuda.synchronize()
    check_rows(x, None, codes, scales, "unrotated bf16 d=64")


def test_full_size_q_and_k_sampled_rows():
    # The causal N=4096 d=128 bf16 shape: Q and K of B=2, H=16 (K with 5 % of its
    # rows scaled x8) as 131072 rows each; the oracle on 3000 sampled rows.
    w = workloads.WORKLOADS[4]
    x = workloads.workload_inputs(4)
    s = signs_for(w.d, 4)
    sg = torch.tensor(s, dtype=torch.float32).cuda()
    pick = np.random.default_rng(4).choice(w.B * w.H * w.N, size=3000, replace=False)
    for name in ("q", "k"):
        announce(f"fp8 full size {name} {w.name}")
        codes, scales = fa.fp8_quantize_rows(x[name].cuda(), sg)
        torch.cuda.synchronize()
        rows = x[name].reshape(-1, w.d)[pick]
        check_rows(rows, s, codes.reshape(-1, w.d)[pick.tolist()],
                   scales.reshape(-1)[pick.tolist()], f"full size {name}")
        assert torch.isfinite(scales).all() and (scales > 0).all()


def test_binding_checks_and_empty_input():
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    codes, scales = fa.fp8_quantize_rows(x)
    assert codes.shape == (0, 128) and scales.shape == (0,)
    y = torch.ones((4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.fp8_quantize_rows(y, torch.ones(128))                       # signs on the host
    with pytest.raises(ValueError):
        fa.fp8_quantize_rows(y, torch.ones(64, device="cuda"))        # wrong length
    with pytest.raises(fa.FAError):
        fa.fp8_quantize_rows(torch.ones((4, 96), dtype=torch.bfloat16, device="cuda"))
