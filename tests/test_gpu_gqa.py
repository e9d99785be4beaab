"""GPU parity of grouped key/value heads in the forward and backward passes
(fa_forward_gqa, fa_backward_gqa through the C ABI) against the float64 oracle.

Query heads h*g .. h*g+g-1 share key/value head h; dK and dV of a shared head
are the sums over its group.  Covered: g = 2, 4, 8, ragged N, both head
dimensions, causal and not, both 16-bit dtypes; forward output and dQ bitwise
equal to multi-head attention over repeated key/value heads (the same
arithmetic); deterministic reruns; the dK/dV group split in all three of its forms (none,
one query head per workgroup, several heads per part); eight seeded random shapes with N over
several query tiles.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_forward_amd as fa
import oracle
import workloads
from helpers import announce, check_forward, check_grads, require_gpu, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def draw_gqa(B, H, hkv, N, d, dtype, seed):
    gen = torch.Generator().manual_seed(seed)
    dt = workloads.DTYPES[dtype]
    q = torch.randn((B, H, N, d), generator=gen).to(dt)
    k = torch.randn((B, hkv, N, d), generator=gen).to(dt)
    v = torch.randn((B, hkv, N, d), generator=gen).to(dt)
    do = torch.randn((B, H, N, d), generator=gen).to(dt)
    return q, k, v, do


@pytest.mark.parametrize("hkv", [1, 2, 4])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,N", [(64, 1), (64, 100), (128, 65), (128, 300)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_grouped_forward_backward(hkv, causal, d, N, dtype):
    B, H = 2, 8
    q, k, v, do = draw_gqa(B, H, hkv, N, d, dtype, seed=500 + hkv + N + d)
    scale = workloads.default_scale(d)
    label = f"gqa {dtype} H={H} Hkv={hkv} N={N} d={d} causal={causal}"
    qg, kg, vg, dog = (t.to("cuda") for t in (q, k, v, do))
    announce(label)
    o, lse = fa.forward(qg, kg, vg, causal, scale)
    dq, dk, dv = fa.backward(qg, kg, vg, o, dog, lse, causal, scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), causal, scale)
    g_ref = oracle.backward(to64(q), to64(k), to64(v), to64(do), causal, scale)
    for b in range(B):
        for h in range(H):
            check_forward(to64(o[b, h]), lse[b, h].cpu().numpy(), o_ref[b, h], lse_ref[b, h],
                          q.dtype, f"{label} b={b} h={h}")
        for hk in range(hkv):
            check_grads({"dq": to64(dq[b, hk * (H // hkv)]), "dk": to64(dk[b, hk]),
                         "dv": to64(dv[b, hk])},
                        {"dq": g_ref["dq"][b, hk * (H // hkv)], "dk": g_ref["dk"][b, hk],
                         "dv": g_ref["dv"][b, hk]}, f"{label} b={b} kv={hk}")
    for b in range(B):
        for h in range(H):
            from helpers import rel_fro
            assert rel_fro(to64(dq[b, h]), g_ref["dq"][b, h]) <= 5e-2


def random_gqa_shapes(count, seed):
    """Seeded (H, Hkv, N, d, dtype, causal) draws with N over several 256-row
    workgroups and ragged ends."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        H = int(rng.choice([4, 8]))
        hkv = int(rng.choice([h for h in (1, 2, 4) if H % h == 0 and h < H]))
        out.append((H, hkv, int(rng.integers(200, 900)), int(rng.choice([64, 128])),
                    str(rng.choice(["fp16", "bf16"])), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", random_gqa_shapes(8, 77))
def test_random_grouped_shapes(case):
    H, hkv, N, d, dtype, causal = case
    q, k, v, do = draw_gqa(1, H, hkv, N, d, dtype, seed=1300 + N)
    scale = workloads.default_scale(d)
    label = f"random gqa {dtype} H={H} Hkv={hkv} N={N} d={d} causal={causal}"
    qg, kg, vg, dog = (t.to("cuda") for t in (q, k, v, do))
    announce(label)
    o, lse = fa.forward(qg, kg, vg, causal, scale)
    dq, dk, dv = fa.backward(qg, kg, vg, o, dog, lse, causal, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), causal, scale)
    g_ref = oracle.backward(to64(q), to64(k), to64(v), to64(do), causal, scale)
    for h in range(H):
        check_forward(to64(o[0, h]), lse[0, h].cpu().numpy(), o_ref[0, h], lse_ref[0, h],
                      q.dtype, f"{label} h={h}")
        hk = h // (H // hkv)
        check_grads({"dq": to64(dq[0, h]), "dk": to64(dk[0, hk]), "dv": to64(dv[0, hk])},
                    {"dq": g_ref["dq"][0, h], "dk": g_ref["dk"][0, hk], "dv": g_ref["dv"][0, hk]},
                    f"{label} h={h} kv={hk}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_grouped_forward_two_row_blocks_per_wave(dtype):
    # d = 64 without the causal mask: 512-row workgroups (two 32-row blocks per
    # wave), here three of them per head with a ragged last one.
    B, H, hkv, N, d = 1, 4, 2, 1100, 64
    assert fa.tile_config(3, d, workloads.DTYPES[dtype])[0] == 512
    q, k, v, _ = draw_gqa(B, H, hkv, N, d, dtype, seed=901)
    scale = workloads.default_scale(d)
    label = f"gqa two-block forward {dtype} N={N}"
    announce(label)
    o, lse = fa.forward(q.to("cuda"), k.to("cuda"), v.to("cuda"), False, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), False, scale)
    for h in range(H):
        check_forward(to64(o[0, h]), lse[0, h].cpu().numpy(), o_ref[0, h], lse_ref[0, h],
                      q.dtype, f"{label} h={h}")


def test_grouped_forward_and_dq_equal_repeated_heads_bitwise():
    B, H, hkv, N, d = 1, 8, 2, 1000, 128
    q, k, v, do = (t.to("cuda") for t in draw_gqa(B, H, hkv, N, d, "bf16", seed=9))
    kr = k.repeat_interleave(H // hkv, dim=1).contiguous()
    vr = v.repeat_interleave(H // hkv, dim=1).contiguous()
    announce("gqa vs repeated heads")
    o1, l1 = fa.forward(q, k, v, True)
    o2, l2 = fa.forward(q, kr, vr, True)
    dq1, dk1, dv1 = fa.backward(q, k, v, o1, do, l1, True)
    dq2, dk2, dv2 = fa.backward(q, kr, vr, o2, do, l2, True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(dq1, dq2)
    # shared heads: the group's sum (one rounding) against per-head gradients summed
    g = H // hkv
    ref_k = dk2.float().view(B, hkv, g, N, d).sum(2)
    ref_v = dv2.float().view(B, hkv, g, N, d).sum(2)
    for got, ref in ((dk1.float(), ref_k), (dv1.float(), ref_v)):
        assert ((got - ref).norm() / ref.norm()).item() <= 1e-2


def test_grouped_backward_is_deterministic():
    q, k, v, do = (t.to("cuda") for t in draw_gqa(2, 8, 2, 700, 64, "fp16", seed=3))
    announce("gqa determinism")
    o, l = fa.forward(q, k, v, True)
    a = fa.backward(q, k, v, o, do, l, True)
    b = fa.backward(q, k, v, o, do, l, True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_forward_fp32(causal):
    B, H, hkv, N, d = 1, 4, 2, 150, 64
    q, k, v, _ = draw_gqa(B, H, hkv, N, d, "fp32", seed=21)
    announce(f"gqa fp32 forward causal={causal}")
    o, lse = fa.forward(q.to("cuda"), k.to("cuda"), v.to("cuda"), causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.forward(to64(q), to64(k), to64(v), causal, workloads.default_scale(d))
    for h in range(H):
        check_forward(to64(o[0, h]), lse[0, h].cpu().numpy(), o_ref[0, h], lse_ref[0, h],
                      torch.float32, f"gqa fp32 h={h}")


def test_grouped_full_size_causal_outlier_shape():
    # The N=4096, d=128 causal bf16 shape (K with 5% rows x8) with 16 query heads
    # on 4 key/value heads; the oracle on key/value head 1 and its 4 query heads.
    B, H, hkv, N, d = 1, 16, 4, 4096, 128
    x = workloads.draw(B, H, N, d, "bf16", seed=44, with_do=True, outlier_frac=0.05)
    q, do = x["q"], x["do"]
    k, v = x["k"][:, :hkv].contiguous(), x["v"][:, :hkv].contiguous()
    scale = workloads.default_scale(d)
    qg, kg, vg, dog = (t.to("cuda") for t in (q, k, v, do))
    announce("gqa full size N=4096 H=16 Hkv=4")
    o, lse = fa.forward(qg, kg, vg, True, scale)
    dq, dk, dv = fa.backward(qg, kg, vg, o, dog, lse, True, scale)
    torch.cuda.synchronize()
    g = H // hkv
    kh, vh = to64(k[0, 1]), to64(v[0, 1])
    dk_ref, dv_ref = np.zeros_like(kh), np.zeros_like(vh)
    for h in range(g, 2 * g):
        qh, doh = to64(q[0, h]), to64(do[0, h])
        o_ref, lse_ref = oracle.forward_head(qh, kh, vh, True, scale)
        check_forward(to64(o[0, h]), lse[0, h].cpu().numpy(), o_ref, lse_ref, q.dtype,
                      f"gqa full size h={h}")
        gr = oracle.backward_head(qh, kh, vh, doh, True, scale)
        from helpers import rel_fro
        assert rel_fro(to64(dq[0, h]), gr["dq"]) <= 5e-2
        dk_ref += gr["dk"]
        dv_ref += gr["dv"]
    check_grads({"dq": to64(dq[0, g]), "dk": to64(dk[0, 1]), "dv": to64(dv[0, 1])},
                {"dq": oracle.backward_head(to64(q[0, g]), kh, vh, to64(do[0, g]), True,
                                            scale)["dq"], "dk": dk_ref, "dv": dv_ref},
                "gqa full size kv=1")


def _group_split(B, H, hkv, N, d):
    # The split count the library chose, read back from the workspace size it
    # asks for: D and LSE rows (padded to 4 floats), then 2 * splits * B * hkv * N * d
    # fp32 partials; a workspace of just the rows means one workgroup per group.
    lib = fa.load_library()
    floats = lib.fa_backward_gqa_workspace_size(B, H, hkv, N, d) // 4
    rows = (2 * B * H * N + 3) & ~3
    if floats == 2 * B * H * N:
        return 1
    return (floats - rows) // (2 * B * hkv * N * d)


@pytest.mark.parametrize("B,H,hkv,N,d,causal,splits", [
    (4, 16, 2, 2000, 64, False, 4),     # 4 workgroups of 2 query heads per group
    (4, 16, 2, 2000, 64, True, 4),
    (4, 16, 2, 4000, 128, True, 2),     # 2 workgroups of 4 query heads per group
])
def test_grouped_backward_partial_group_split(B, H, hkv, N, d, causal, splits):
    # Grids with fewer than 512 dK/dV workgroups split each group over several
    # workgroups that write fp32 partial sums, reduced in a fixed order.  Here the
    # split is partial (1 < splits < g), so each workgroup still walks several
    # query heads and the ragged last key tile is masked.
    g = H // hkv
    assert _group_split(B, H, hkv, N, d) == splits and 1 < splits < g
    q, k, v, do = draw_gqa(B, H, hkv, N, d, "bf16", seed=500 + N + splits + int(causal))
    scale = workloads.default_scale(d)
    qg, kg, vg, dog = (t.to("cuda") for t in (q, k, v, do))
    announce(f"gqa partial split B={B} H={H} Hkv={hkv} N={N} d={d} causal={causal}")
    o, lse = fa.forward(qg, kg, vg, causal, scale)
    dq, dk, dv = fa.backward(qg, kg, vg, o, dog, lse, causal, scale)
    torch.cuda.synchronize()
    checked = [(0, 1), (B - 1, 0)] if N <= 2000 else [(B - 1, 1)]
    for b, kv in checked:
        kh, vh = to64(k[b, kv]), to64(v[b, kv])
        dk_ref, dv_ref = np.zeros_like(kh), np.zeros_like(vh)
        for h in range(kv * g, (kv + 1) * g):
            qh, doh = to64(q[b, h]), to64(do[b, h])
            gr = oracle.backward_head(qh, kh, vh, doh, causal, scale)
            dk_ref += gr["dk"]
            dv_ref += gr["dv"]
            if h == kv * g + g - 1:
                o_ref, lse_ref = oracle.forward_head(qh, kh, vh, causal, scale)
                check_forward(to64(o[b, h]), lse[b, h].cpu().numpy(), o_ref, lse_ref, q.dtype,
                              f"gqa partial split b={b} h={h}")
                dq_ref = gr["dq"]
        check_grads({"dq": to64(dq[b, (kv + 1) * g - 1]), "dk": to64(dk[b, kv]),
                     "dv": to64(dv[b, kv])}, {"dq": dq_ref, "dk": dk_ref, "dv": dv_ref},
                    f"gqa partial split b={b} kv={kv}")
