"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded, dtype-rounded inputs.

Small shapes cover several tiles, ragged tails (N not a multiple of any tile),
N = 1, both head dimensions, causal and not, every dtype; the five workloads run
at their full sizes in the launch configuration the benchmark times, with the
oracle evaluated on sampled heads (every row of those heads), plus invariants
checked on every head.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_forward_amd as fa
import oracle
import workloads
from helpers import (announce, check_forward, check_grads, require_gpu, to64)

pytestmark = pytest.mark.gpu

DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def gpu_inputs(x):
    return {k: v.to("cuda") for k, v in x.items()}


def oracle_heads(x, heads, causal, scale, backward):
    """Oracle results for the listed flat head indices (b*H + h)."""
    B, H = x["q"].shape[:2]
    out = []
    for bh in heads:
        b, h = divmod(int(bh), H)
        q, k, v = (to64(x[n][b, h]) for n in ("q", "k", "v"))
        o, lse = oracle.forward_head(q, k, v, causal, scale)
        g = oracle.backward_head(q, k, v, to64(x["do"][b, h]), causal, scale) if backward else None
        out.append((b, h, o, lse, g))
    return out


def run_and_check(x, dtype, causal, scale, heads, backward, label):
    xs = gpu_inputs(x)
    announce(f"{label} forward")
    o, lse = fa.forward(xs["q"], xs["k"], xs["v"], causal, scale)
    torch.cuda.synchronize()
    grads = None
    if backward:
        announce(f"{label} backward")
        grads = fa.backward(xs["q"], xs["k"], xs["v"], o, xs["do"], lse, causal, scale)
        torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    g_c = [t.cpu() for t in grads] if backward else None
    for b, h, o_ref, lse_ref, g_ref in oracle_heads(x, heads, causal, scale, backward):
        tag = f"{label} b={b} h={h}"
        check_forward(to64(o_c[b, h]), lse_c[b, h].numpy(), o_ref, lse_ref, dtype, tag)
        if backward:
            check_grads({"dq": to64(g_c[0][b, h]), "dk": to64(g_c[1][b, h]),
                         "dv": to64(g_c[2][b, h])}, g_ref, tag)
    return o_c, lse_c, g_c


# ------------------------------------------------------------------ small shapes

SMALL_N = [1, 17, 64, 100, 129, 256, 300]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_small_forward(dtype, d, causal):
    for i, n in enumerate(SMALL_N):
        x = workloads.draw(1, 2, n, d, dtype, seed=100 + i, with_do=False)
        run_and_check(x, DT[dtype], causal, workloads.default_scale(d), [0, 1], False,
                      f"fwd {dtype} d={d} causal={causal} N={n}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_small_backward(dtype, d, causal):
    for i, n in enumerate(SMALL_N):
        x = workloads.draw(1, 2, n, d, dtype, seed=200 + i, with_do=True)
        run_and_check(x, DT[dtype], causal, workloads.default_scale(d), [0, 1], True,
                      f"fwdbwd {dtype} d={d} causal={causal} N={n}")


def test_scale_is_honoured():
    x = workloads.draw(1, 2, 150, 64, "bf16", seed=7, with_do=True)
    run_and_check(x, torch.bfloat16, True, 0.37, [0, 1], True, "scale=0.37")


def test_outlier_keys_small():
    x = workloads.draw(1, 2, 333, 128, "bf16", seed=8, with_do=True, outlier_frac=0.05)
    run_and_check(x, torch.bfloat16, True, workloads.default_scale(128), [0, 1], True,
                  "outliers N=333")


# ------------------------------------------------------------------ full workloads

SAMPLED_HEADS = {1: [0], 2: [0, 37, 74, 127], 3: [0, 21, 42, 63], 4: [0, 31], 5: [17]}


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload(cid):
    w = workloads.WORKLOADS[cid]
    x = workloads.workload_inputs(cid)
    o, lse, g = run_and_check(x, w.torch_dtype, w.causal, w.scale, SAMPLED_HEADS[cid], w.backward,
                              f"workload {cid} {w.name}")
    # Invariants on every head (hold at any size): finite outputs; the rows of
    # dS sum to zero, so sum over keys of dK vanishes; rows of A sum to one, so
    # the sum over keys of dV equals the sum over queries of dO.
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    if w.backward:
        dq, dk, dv = (t.double() for t in g)
        assert all(torch.isfinite(t).all() for t in (dq, dk, dv))
        do = x["do"].double()
        sk = dk.sum(dim=2).norm(dim=-1) / dk.norm(dim=(-2, -1)).clamp_min(1e-30)
        sv = (dv.sum(dim=2) - do.sum(dim=2)).norm(dim=-1) / do.sum(dim=2).norm(dim=-1)
        assert float(sk.max()) < 5e-2, float(sk.max())
        assert float(sv.max()) < 5e-2, float(sv.max())


# ------------------------------------------------------------------ tile map

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 127, 128, 129, 300, 1000, 4096])
def test_tile_map_bit_exact(n, causal):
    x = workloads.draw(1, 3, n, 64, "bf16", seed=300 + n, with_do=False)
    xs = gpu_inputs(x)
    announce(f"blockmap N={n} causal={causal}")
    o_m, l_m, codes = fa.forward_blockmap(xs["q"], xs["k"], xs["v"], causal)
    o, l = fa.forward(xs["q"], xs["k"], xs["v"], causal)
    torch.cuda.synchronize()
    br, bc = fa.tile_config(0, 64, torch.bfloat16)
    ref = oracle.tile_map(n, br, bc, causal)
    got = codes.cpu().numpy()
    for h in range(3):
        np.testing.assert_array_equal(got[0, h], ref)
    assert torch.equal(o_m, o) and torch.equal(l_m, l)   # same computation, bit for bit


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 127, 128, 129, 300, 1000, 4096])
def test_backward_tile_maps_bit_exact(n, causal):
    x = workloads.draw(1, 2, n, 64, "bf16", seed=700 + n, with_do=True)
    xs = gpu_inputs(x)
    announce(f"backward blockmap N={n} causal={causal}")
    o, l = fa.forward(xs["q"], xs["k"], xs["v"], causal)
    dq_m, dk_m, dv_m, c1, c2 = fa.backward_blockmap(xs["q"], xs["k"], xs["v"], o, xs["do"], l,
                                                    causal)
    dq, dk, dv = fa.backward(xs["q"], xs["k"], xs["v"], o, xs["do"], l, causal)
    torch.cuda.synchronize()
    br1, bc1 = fa.tile_config(1, 64, torch.bfloat16)
    br2, bc2 = fa.tile_config(2, 64, torch.bfloat16)
    # The dK/dV kernel stores its map key tile major: the transpose of the
    # (query tile, key tile) map over its own tile shape.
    ref1 = oracle.tile_map(n, br1, bc1, causal).T
    ref2 = oracle.tile_map(n, br2, bc2, causal)
    got1, got2 = c1.cpu().numpy(), c2.cpu().numpy()
    for h in range(2):
        np.testing.assert_array_equal(got1[0, h], ref1)
        np.testing.assert_array_equal(got2[0, h], ref2)
    assert torch.equal(dq_m, dq) and torch.equal(dk_m, dk) and torch.equal(dv_m, dv)


# ------------------------------------------------------------------ determinism

def test_runs_are_bitwise_deterministic():
    x = gpu_inputs(workloads.draw(2, 4, 777, 128, "bf16", seed=9, with_do=True))
    announce("determinism")
    res = []
    for _ in range(2):
        o, lse = fa.forward(x["q"], x["k"], x["v"], True)
        dq, dk, dv = fa.backward(x["q"], x["k"], x["v"], o, x["do"], lse, True)
        res.append((o, lse, dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_unsupported_returns_error_without_launch():
    x = gpu_inputs(workloads.draw(1, 1, 64, 64, "fp32", seed=1, with_do=True))
    with pytest.raises(fa.FAError) as e:
        fa.backward(x["q"], x["k"], x["v"], x["q"], x["do"],
                    torch.zeros(1, 1, 64, device="cuda"), False)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
