"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on the
same seeded, dtype-rounded inputs.

Small shapes cover several tiles, ragged tails (N not a multiple of any tile),
N = 1, both head dimensions, causal and not, every dtype; the five workloads run
at their full sizes in the launch configuration the benchmark times, with every
head compared against the oracle (at N = 16384 on sampled query rows for the
forward and on four whole heads for the gradients), plus invariants checked on
every head; NaN and infinite inputs propagate to the oracle's positions.
"""
import functools

import numpy as np
import pytest
import torch

import exact_io_aware_forward_amd as fa
import oracle
import workloads
from helpers import (GRAD_REL_FRO, LSE_TOL, announce, check_forward, check_grads, o_tolerance,
                     rel_fro, require_gpu, to64)

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

SMALL_N = [1, 17, 64, 100, 129, 256, 300, 600]   # 600: a ragged second 512-row forward tile


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


def random_shapes(count, seed):
    """Seeded (B, H, N, d, dtype, causal) draws: N spans one to a dozen 64-key tiles and
    ragged ends, so the forward's and dQ's 256-row workgroups see partial blocks,
    waves past the last row and every ring stage."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        out.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 800)),
                    int(rng.choice([64, 128])), str(rng.choice(["fp16", "bf16"])),
                    bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", random_shapes(12, 2026))
def test_random_shapes_forward_backward(case):
    B, H, n, d, dtype, causal = case
    x = workloads.draw(B, H, n, d, dtype, seed=900 + n, with_do=True)
    run_and_check(x, DT[dtype], causal, workloads.default_scale(d), list(range(B * H)), True,
                  f"random B={B} H={H} N={n} d={d} {dtype} causal={causal}")


def test_scale_is_honoured():
    x = workloads.draw(1, 2, 150, 64, "bf16", seed=7, with_do=True)
    run_and_check(x, torch.bfloat16, True, 0.37, [0, 1], True, "scale=0.37")


def test_outlier_keys_small():
    x = workloads.draw(1, 2, 333, 128, "bf16", seed=8, with_do=True, outlier_frac=0.05)
    run_and_check(x, torch.bfloat16, True, workloads.default_scale(128), [0, 1], True,
                  "outliers N=333")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_scores_growing_across_key_tiles(dtype, causal):
    # Each 64-key tile's scores lie ~20 exp2 units above the previous tile's, so
    # the forward's running max trails the true one by up to the lazy-rescale
    # threshold and the unnormalised probabilities reach ~2^20 between rescales
    # (bf16; fp16 rescales every tile).  The oracle forms the softmax directly.
    n, d = 700, 64
    scale = workloads.default_scale(d)
    c = scale * np.log2(np.e)
    g = torch.Generator().manual_seed(21)
    q = 0.5 * torch.randn(1, 2, n, d, generator=g)
    k = 0.5 * torch.randn(1, 2, n, d, generator=g)
    v = torch.randn(1, 2, n, d, generator=g)
    q[..., 0] = 4.0
    k[..., 0] = (20.0 * (torch.arange(n) // 64).float() + 2.0 * torch.randn(n, generator=g)) / (4.0 * c)
    x = {"q": q.to(DT[dtype]), "k": k.to(DT[dtype]), "v": v.to(DT[dtype])}
    run_and_check(x, DT[dtype], causal, scale, [0, 1], False, f"growing scores {dtype} causal={causal}")


# ------------------------------------------------------------------ full workloads
# Every head of every workload is compared with the oracle element by element,
# in the launch configuration the benchmark times.  At N = 16384 the forward is
# compared on a seeded sample of query rows of every head (four rows in every
# 256-row query tile, the tile's first and last row among them, so every
# workgroup of the forward grid is checked), and the gradients, which need
# whole heads, on four heads including the first and the last.

@functools.lru_cache(maxsize=1)
def workload_run(cid):
    """GPU forward (+ backward) of workload `cid` on its seeded inputs, copied
    back to the host.  Cached, so the several tests of one workload share a run."""
    w = workloads.WORKLOADS[cid]
    x = workloads.workload_inputs(cid)
    xs = gpu_inputs(x)
    announce(f"workload {cid} {w.name} forward")
    o, lse = fa.forward(xs["q"], xs["k"], xs["v"], w.causal, w.scale)
    torch.cuda.synchronize()
    g = None
    if w.backward:
        announce(f"workload {cid} {w.name} backward")
        g = fa.backward(xs["q"], xs["k"], xs["v"], o, xs["do"], lse, w.causal, w.scale)
        torch.cuda.synchronize()
        g = [t.cpu() for t in g]
    o, lse = o.cpu(), lse.cpu()
    del xs
    torch.cuda.empty_cache()
    return x, o, lse, g


def check_invariants(x, o, lse, g):
    """Properties that hold at any size, on every head: finite outputs; the rows
    of dS sum to zero, so the sum over keys of dK vanishes; the rows of A sum to
    one, so the sum over keys of dV equals the sum over queries of dO."""
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    if g is not None:
        dq, dk, dv = (t.double() for t in g)
        assert all(torch.isfinite(t).all() for t in (dq, dk, dv))
        do = x["do"].double()
        sk = dk.sum(dim=2).norm(dim=-1) / dk.norm(dim=(-2, -1)).clamp_min(1e-30)
        sv = (dv.sum(dim=2) - do.sum(dim=2)).norm(dim=-1) / do.sum(dim=2).norm(dim=-1)
        assert float(sk.max()) < 5e-2, float(sk.max())
        assert float(sv.max()) < 5e-2, float(sv.max())


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_workload(cid):
    """Workloads 1-4: O and LSE element by element and dQ, dK, dV per head on
    every head."""
    w = workloads.WORKLOADS[cid]
    x, o, lse, g = workload_run(cid)
    B, H = w.B, w.H
    for bh in range(B * H):
        b, h = divmod(bh, H)
        q, k, v = (to64(x[n][b, h]) for n in ("q", "k", "v"))
        o_ref, lse_ref = oracle.forward_head(q, k, v, w.causal, w.scale)
        tag = f"workload {cid} b={b} h={h}"
        check_forward(to64(o[b, h]), lse[b, h].numpy(), o_ref, lse_ref, w.torch_dtype, tag)
        if w.backward:
            g_ref = oracle.backward_head(q, k, v, to64(x["do"][b, h]), w.causal, w.scale)
            check_grads({"dq": to64(g[0][b, h]), "dk": to64(g[1][b, h]),
                         "dv": to64(g[2][b, h])}, g_ref, tag)
    check_invariants(x, o, lse, g)


def long_context_rows(n, br, per_tile, seed):
    """Sorted query rows: in every br-row tile its first and last row and
    per_tile - 2 distinct seeded rows between them."""
    rng = np.random.default_rng(seed)
    rows = []
    for t0 in range(0, n, br):
        t1 = min(n, t0 + br) - 1
        inner = rng.choice(np.arange(t0 + 1, t1), size=per_tile - 2, replace=False)
        rows.extend([t0, t1, *inner.tolist()])
    return np.unique(np.asarray(rows))


def test_workload_5_forward_every_head():
    """N = 16384: O and LSE of every head on 256 sampled query rows spanning all
    64 query tiles."""
    w = workloads.WORKLOADS[5]
    x, o, lse, g = workload_run(5)
    br, _ = fa.tile_config(0, w.d, w.torch_dtype)
    rows = long_context_rows(w.N, br, 4, seed=5)
    assert rows.size >= 256
    k_all, v_all = x["k"], x["v"]
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        q, k, v = (to64(t[b, h]) for t in (x["q"], k_all, v_all))
        o_ref, lse_ref = oracle.forward_head(q, k, v, True, w.scale, rows=rows)
        check_forward(to64(o[b, h])[rows], lse[b, h].numpy()[rows], o_ref, lse_ref,
                      w.torch_dtype, f"workload 5 b={b} h={h} rows={rows.size}")
    check_invariants(x, o, lse, g)


@pytest.mark.parametrize("h", [0, 9, 22, 31])
def test_workload_5_gradients(h):
    """N = 16384: dQ, dK, dV of whole heads against the oracle."""
    w = workloads.WORKLOADS[5]
    x, o, lse, g = workload_run(5)
    q, k, v, do = (to64(x[n][0, h]) for n in ("q", "k", "v", "do"))
    g_ref = oracle.backward_head(q, k, v, do, True, w.scale)
    check_grads({"dq": to64(g[0][0, h]), "dk": to64(g[1][0, h]), "dv": to64(g[2][0, h])}, g_ref,
                f"workload 5 h={h}")


# ------------------------------------------------------------------ non-finite inputs
# A NaN or an infinity in the inputs propagates as in the plain definition: the
# outputs that are NaN (or infinite) are exactly the oracle's, and the finite
# ones meet the usual tolerance.  Causal cases plant values only in Q and K,
# whose masked scores both sides exclude; a NaN in V or dO reaches, through
# 0 * NaN, outputs that a masked key cannot influence in exact arithmetic, and
# the two sides evaluate different sets of such products (the kernels skip
# tiles above the diagonal, a dense product does not), so those are tested
# without the mask.

NONFINITE = {
    "q_nan": ("q", (0, 5, 3), float("nan")),
    "k_nan": ("k", (0, 40, 7), float("nan")),
    "k_posinf": ("k", (1, 70, 2), float("inf")),
    "k_neginf": ("k", (1, 33, 9), float("-inf")),
    "v_nan": ("v", (0, 90, 11), float("nan")),
    "do_nan": ("do", (1, 17, 5), float("nan")),
}


def plant(x, case):
    name, (h, r, c), val = NONFINITE[case]
    x = {k: t.clone() for k, t in x.items()}
    x[name][0, h, r, c] = val
    return x


def compare_nonfinite(got, ref, tol, label):
    got = np.asarray(got, np.float64)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref), err_msg=f"{label}: NaN positions")
    np.testing.assert_array_equal(np.isposinf(got), np.isposinf(ref), err_msg=f"{label}: +inf")
    np.testing.assert_array_equal(np.isneginf(got), np.isneginf(ref), err_msg=f"{label}: -inf")
    fin = np.isfinite(ref)
    if tol is not None and fin.any():
        assert (np.abs(got[fin] - ref[fin]) <= tol[fin]).all(), f"{label}: finite values"
    return int((~fin).sum())


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("case,causal", [(c, m) for c in ("q_nan", "k_nan", "k_posinf", "k_neginf")
                                         for m in (False, True)] + [("v_nan", False)])
def test_nonfinite_forward(case, causal, dtype):
    n, d = 150, 64
    x = plant(workloads.draw(1, 2, n, d, dtype, seed=31, with_do=False), case)
    xs = gpu_inputs(x)
    announce(f"nonfinite forward {case} {dtype} causal={causal}")
    o, lse = fa.forward(xs["q"], xs["k"], xs["v"], causal)
    torch.cuda.synchronize()
    scale = workloads.default_scale(d)
    bad = 0
    for h in range(2):
        q, k, v = (to64(x[m][0, h]) for m in ("q", "k", "v"))
        o_ref, lse_ref = oracle.forward_head(q, k, v, causal, scale)
        tag = f"{case} {dtype} causal={causal} h={h}"
        bad += compare_nonfinite(to64(o[0, h]), o_ref, o_tolerance(o_ref, DT[dtype]), tag + " O")
        bad += compare_nonfinite(lse[0, h].double().cpu().numpy(), lse_ref,
                                 np.full(lse_ref.shape, LSE_TOL[DT[dtype]]), tag + " LSE")
    assert bad > 0   # the planted value reached the outputs


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("case", ["q_nan", "k_nan", "v_nan", "do_nan"])
def test_nonfinite_backward(case, dtype):
    n, d = 150, 64
    x = plant(workloads.draw(1, 2, n, d, dtype, seed=32, with_do=True), case)
    xs = gpu_inputs(x)
    announce(f"nonfinite backward {case} {dtype}")
    o, lse = fa.forward(xs["q"], xs["k"], xs["v"], False)
    dq, dk, dv = fa.backward(xs["q"], xs["k"], xs["v"], o, xs["do"], lse, False)
    torch.cuda.synchronize()
    scale = workloads.default_scale(d)
    bad = 0
    for h in range(2):
        q, k, v, do = (to64(x[m][0, h]) for m in ("q", "k", "v", "do"))
        g_ref = oracle.backward_head(q, k, v, do, False, scale)
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            got, ref = to64(t[0, h]), g_ref[name]
            bad += compare_nonfinite(got, ref, None, f"{case} {dtype} h={h} {name}")
            fin = np.isfinite(ref)
            if fin.any():
                assert rel_fro(got[fin], ref[fin]) <= GRAD_REL_FRO, f"{case} {name}"
    assert bad > 0


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
    br, bc = fa.tile_config(0 if causal else 3, 64, torch.bfloat16)
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


@pytest.mark.parametrize("d", [64, 128])
def test_backward_stages_compose_the_backward(d):
    """fa_backward is dQ (which also forms D and LSE*log2e) then dK/dV: the same
    two stages run one by one give bitwise the same gradients, and so does the
    workspace they leave.  Running the standalone preprocess, dK/dV, then dQ
    also matches: dQ bitwise (it forms its own D), dK/dV within the rounding of
    D's different summation order."""
    x = gpu_inputs(workloads.draw(2, 4, 777, d, "bf16", seed=11, with_do=True))
    announce(f"backward stages d={d}")
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o, lse = fa.forward(q, k, v, True)
    ws_ref = fa.new_workspace(q)
    ref = fa.backward(q, k, v, o, do, lse, True, workspace=ws_ref)
    ws = torch.full_like(ws_ref, float("nan"))
    got = tuple(torch.empty_like(t) for t in ref)
    for s in (fa.BWD_DQ, fa.BWD_DKDV):
        fa.backward_stage(s, q, k, v, o, do, lse, *got, ws, True)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    assert torch.equal(ws_ref, ws)
    ws3 = torch.full_like(ws_ref, float("nan"))
    got3 = tuple(torch.empty_like(t) for t in ref)
    for s in (fa.BWD_PREPROCESS, fa.BWD_DKDV, fa.BWD_DQ):
        fa.backward_stage(s, q, k, v, o, do, lse, *got3, ws3, True)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got3[0])
    for a, b in zip(ref[1:], got3[1:]):
        assert rel_fro(to64(b), to64(a)) < 1e-3
    rows = ws_ref.numel() // 2
    assert torch.allclose(ws3[:rows], ws_ref[:rows], rtol=1e-5, atol=1e-5)
    assert torch.equal(ws3[rows:], ws_ref[rows:])


def test_unsupported_returns_error_without_launch():
    x = gpu_inputs(workloads.draw(1, 1, 64, 64, "fp32", seed=1, with_do=True))
    with pytest.raises(fa.FAError) as e:
        fa.backward(x["q"], x["k"], x["v"], x["q"], x["do"],
                    torch.zeros(1, 1, 64, device="cuda"), False)
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
