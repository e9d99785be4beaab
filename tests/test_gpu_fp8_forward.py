"""GPU parity of the FP8 forward (fa_forward_fp8 through the C ABI) against the
float64 oracle, on the same seeded inputs.

Two comparisons:
  1. the attention kernel on its own inputs: O and LSE against the oracle's plain
     forward on exactly the values the kernel reads (the E4M3 codes times their
     row scales for Q J and K J, V as given).  The E4M3 matrix instruction sums
     its products with less than fp32 precision (helpers.EPS_FP8_ACC), so the
     scores may differ by up to that accumulation bound per row
     (helpers.fp8_acc_shift); the 16-bit rule (|dO| <= 1e-2 + half an ulp,
     |dLSE| <= 1e-3) is widened by that shift's effect on the softmax
     (helpers.fp8_tolerances, pinned in tests/test_oracle_fp8_pins.py).
  2. the FP8 path end to end (rotation and quantisation on the GPU, then the
     kernel) against oracle.fp8.fp8_forward_head, whose rounding decisions are
     taken in float64: the shift adds the score difference between the two code
     sets (helpers.score_shift).

Cases: both 16-bit V types, d = 64 and 128, causal and not, N = 1, ragged
tails, several tiles, keys with outlier rows, and the causal N=4096 d=128 bf16
shape with 5 % of K rows x8 on every head.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_forward_amd as fa
import workloads
from helpers import (announce, fp8_acc_shift, fp8_tolerances, require_gpu, score_shift, to64)
from oracle import attention as plain
from oracle import fp8

pytestmark = pytest.mark.gpu

DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def deq(codes, scales):
    c = codes.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return c * scales.cpu().double().numpy()[..., None]


def run(x, signs, causal, scale):
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    sg = torch.tensor(signs, dtype=torch.float32).cuda()
    o, lse, (qc, qs, kc, ks) = fa.fp8_attention(q, k, v, sg, causal, scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), deq(qc, qs), deq(kc, ks)


def check_heads(x, signs, causal, scale, dtype, label, heads=None, end_to_end=True):
    o, lse, qd, kd = run(x, signs, causal, scale)
    B, H = x["q"].shape[:2]
    worst = 0.0
    for bh in (range(B * H) if heads is None else heads):
        b, h = divmod(bh, H)
        v = to64(x["v"][b, h])
        tag = f"{label} b={b} h={h}"
        # 1. the kernel on the values it reads
        o_ref, l_ref = plain.forward_head(qd[b, h], kd[b, h], v, causal, scale)
        acc = fp8_acc_shift(qd[b, h], kd[b, h], scale, causal)
        o_tol, l_tol = fp8_tolerances(o_ref, dtype, acc, v)
        o_got, l_got = to64(o[b, h]), lse[b, h].double().numpy()
        assert np.isfinite(o_got).all(), f"{tag}: non-finite O"
        err, lerr = np.abs(o_got - o_ref), np.abs(l_got - l_ref)
        assert (err <= o_tol).all(), f"{tag} (its codes): O max err {err.max()}"
        assert (lerr <= l_tol).all(), f"{tag} (its codes): LSE max err {lerr.max()}"
        print(f"[{tag}] its codes: O max-abs {err.max():.3e}, LSE max-abs {lerr.max():.3e} "
              f"(accumulation shift up to {acc.max():.3e})", flush=True)
        if not end_to_end:
            continue
        # 2. end to end against the float64 FP8 oracle
        q, k = to64(x["q"][b, h]), to64(x["k"][b, h])
        o_e, l_e = fp8.fp8_forward_head(q, k, v, causal, scale, signs)
        qo, ko = fp8.dequantized_rotated(q, signs), fp8.dequantized_rotated(k, signs)
        delta = score_shift(qd[b, h], kd[b, h], qo, ko, scale, causal) + acc
        o_tol, l_tol = fp8_tolerances(o_e, dtype, delta, v)
        err = np.abs(to64(o[b, h]) - o_e)
        assert (err <= o_tol).all(), f"{tag}: end-to-end O, max err {err.max()}"
        assert (np.abs(lse[b, h].double().numpy() - l_e) <= l_tol).all(), f"{tag}: end-to-end LSE"
        worst = max(worst, float(delta.max()))
    print(f"[{label}] largest per-row score shift between GPU and oracle codes: {worst:.3e}",
          flush=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_small_shapes(dtype, d, causal):
    for i, n in enumerate([1, 17, 64, 100, 300]):
        x = workloads.draw(1, 2, n, d, dtype, seed=400 + i, with_do=False)
        signs = np.random.default_rng(400 + i).choice([-1.0, 1.0], size=d)
        announce(f"fp8 forward {dtype} d={d} causal={causal} N={n}")
        check_heads(x, signs, causal, workloads.default_scale(d), DT[dtype],
                    f"fp8 {dtype} d={d} causal={causal} N={n}")


def test_outlier_keys_and_scale():
    x = workloads.draw(1, 3, 777, 128, "bf16", seed=411, with_do=False, outlier_frac=0.05)
    signs = np.random.default_rng(411).choice([-1.0, 1.0], size=128)
    announce("fp8 forward outliers N=777")
    check_heads(x, signs, True, 0.3, torch.bfloat16, "fp8 outliers N=777 scale=0.3")


def test_causal_n4096_every_head():
    # The N=4096 d=128 causal bf16 shape with 5 % of the K rows x8.
    w = workloads.WORKLOADS[4]
    x = workloads.workload_inputs(4)
    x = {n: x[n] for n in ("q", "k", "v")}
    signs = np.random.default_rng(4).choice([-1.0, 1.0], size=w.d)
    announce(f"fp8 forward {w.name}")
    check_heads(x, signs, True, w.scale, w.torch_dtype, "fp8 " + w.name)


def test_binding_and_abi_checks():
    x = workloads.draw(1, 1, 64, 64, "bf16", seed=5, with_do=False)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    qc, qs = fa.fp8_quantize_rows(q)
    kc, ks = fa.fp8_quantize_rows(k)
    with pytest.raises(ValueError):
        fa.forward_fp8(qc, qs, kc, ks.cpu(), v)                      # scales on the host
    with pytest.raises(ValueError):
        fa.forward_fp8(qc.view(torch.int8), qs, kc, ks, v)           # not uint8 codes
    with pytest.raises(fa.FAError) as e:
        fa.forward_fp8(qc, qs, kc, ks, v, scale=-1.0)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
