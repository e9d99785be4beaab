"""GPU parity of the split-K decode path (through the C ABI) against the float64
oracle's decode on the same seeded, dtype-rounded inputs.

Small shapes cover one key, ragged cache lengths (not a multiple of the 32-key
tile), a single query and full 32-query blocks, both head dimensions, causal
and not, both 16-bit dtypes, the default slice count and explicit ones (one
slice, more slices than the default, more than there are tiles); keys with 8x
outlier rows exercise the running-max rescaling.  The decode workload (32
heads, one query, a 128K-token cache) runs at full size in the launch
configuration the benchmark times, checked against the oracle on every head.
"""
import numpy as np
import pytest
import torch

import exact_io_aware_forward_amd as fa
import oracle
import workloads
from helpers import announce, check_forward, require_gpu, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_decode_case(x, causal, scale, num_splits, label, heads=None):
    xs = {k: v.to("cuda") for k, v in x.items()}
    announce(label)
    o, lse = fa.decode(xs["q"], xs["k"], xs["v"], causal, scale, num_splits=num_splits)
    torch.cuda.synchronize()
    o_c, lse_c = o.cpu(), lse.cpu()
    B, H = x["q"].shape[:2]
    g = H // x["k"].shape[1]           # query heads per key/value head
    for bh in (range(B * H) if heads is None else heads):
        b, h = divmod(bh, H)
        o_ref, lse_ref = oracle.decode_head(to64(x["q"][b, h]), to64(x["k"][b, h // g]),
                                            to64(x["v"][b, h // g]), causal, scale)
        check_forward(to64(o_c[b, h]), lse_c[b, h].numpy(), o_ref, lse_ref,
                      x["q"].dtype, f"{label} b={b} h={h}")
    return o_c, lse_c


SHAPES = [(1, 1), (1, 31), (1, 33), (3, 200), (32, 32), (32, 1000), (7, 1029)]


@pytest.mark.parametrize("nq,nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_small_decode(dtype, d, causal, nq, nk):
    x = workloads.draw_decode(2, 2, nq, nk, d, dtype, seed=1000 + nq * 7 + nk)
    run_decode_case(x, causal, workloads.default_scale(d), 0,
                    f"decode {dtype} d={d} causal={causal} Nq={nq} Nk={nk}")


@pytest.mark.parametrize("num_splits", [1, 2, 3, 5, 13, 1000])
def test_decode_any_slice_count(num_splits):
    x = workloads.draw_decode(1, 3, 5, 2000, 128, "bf16", seed=77)
    run_decode_case(x, True, workloads.default_scale(128), num_splits,
                    f"decode splits={num_splits}")


def test_decode_outlier_keys_rescale():
    x = workloads.draw_decode(1, 4, 9, 3000, 128, "bf16", seed=5)
    gen = torch.Generator().manual_seed(55)
    for h in range(4):
        rows = torch.randperm(3000, generator=gen)[:150]
        x["k"][0, h, rows] = (x["k"][0, h, rows].float() * 8).to(torch.bfloat16)
    run_decode_case(x, True, workloads.default_scale(128), 0, "decode outlier keys")


def test_decode_stages_equal_the_whole_call():
    x = workloads.draw_decode(2, 3, 4, 777, 64, "fp16", seed=9)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    scale = workloads.default_scale(64)
    announce("decode stages")
    o1, l1 = fa.decode(q, k, v, True, scale, num_splits=3)
    ws = fa.new_decode_workspace(q, k, 3)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    fa.decode_stage(fa.DEC_SPLIT, q, k, v, None, None, True, scale, 3, ws)
    fa.decode_stage(fa.DEC_COMBINE, q, k, v, o2, l2, True, scale, 3, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_workload_full_size():
    w = workloads.DECODE_WORKLOAD
    x = workloads.draw_decode(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed)
    assert fa.decode_num_splits(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d) == 8
    run_decode_case(x, w.causal, w.scale, 0, w.name)
    # one slice per head (32 workgroups) gives the same answer
    run_decode_case(x, w.causal, w.scale, 1, w.name + " one slice", heads=[0, 13, 31])


@pytest.mark.parametrize("num_splits", [1, 4])
@pytest.mark.parametrize("row", [5, 21])
def test_decode_nan_query_row_stays_in_its_row(row, num_splits):
    # 32 query rows per head: rows r and r + 16 share a column of the kernel's
    # row-sum products, so a NaN in one must not reach the other.  NaN
    # positions and every finite value are compared with the oracle.
    x = workloads.draw_decode(1, 2, 32, 300, 64, "bf16", seed=12)
    x["q"][0, 1, row, 3] = float("nan")
    xs = {k: v.to("cuda") for k, v in x.items()}
    announce(f"decode NaN in query row {row} splits={num_splits}")
    o, lse = fa.decode(xs["q"], xs["k"], xs["v"], True, workloads.default_scale(64),
                       num_splits=num_splits)
    torch.cuda.synchronize()
    for h in range(2):
        o_ref, lse_ref = oracle.decode_head(to64(x["q"][0, h]), to64(x["k"][0, h]),
                                            to64(x["v"][0, h]), True, workloads.default_scale(64))
        got_o, got_l = to64(o[0, h].cpu()), lse[0, h].double().cpu().numpy()
        np.testing.assert_array_equal(np.isnan(got_o), np.isnan(o_ref))
        np.testing.assert_array_equal(np.isnan(got_l), np.isnan(lse_ref))
        assert np.isnan(o_ref).any() == (h == 1)
        fin = np.isfinite(lse_ref)
        check_forward(got_o[fin], got_l[fin], o_ref[fin], lse_ref[fin], torch.bfloat16,
                      f"decode NaN row {row} h={h}")


def test_decode_is_deterministic():
    x = workloads.draw_decode(1, 8, 3, 5000, 128, "bf16", seed=3)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    announce("decode determinism")
    a = fa.decode(q, k, v, True)
    b = fa.decode(q, k, v, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("hkv,nq", [(1, 1), (1, 4), (2, 1), (2, 3), (2, 8), (4, 16), (8, 2)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d,nk", [(64, 77), (128, 1000)])
def test_grouped_kv_heads_decode(hkv, nq, causal, d, nk):
    # 8 query heads over hkv key/value heads: g = 8 / hkv heads per group, g * nq
    # packed query rows (up to 32) against each key/value head's cache.
    x = workloads.draw_decode(2, 8, nq, nk, d, "bf16", seed=300 + hkv * 10 + nq, hkv=hkv)
    run_decode_case(x, causal, workloads.default_scale(d), 0,
                    f"decode gqa hkv={hkv} Nq={nq} causal={causal} d={d} Nk={nk}")


def test_grouped_decode_equals_repeated_cache():
    # Packing g query heads on one key/value head gives what separate heads over
    # copies of that cache give (within rounding of the partial sums).
    x = workloads.draw_decode(1, 8, 2, 3000, 128, "fp16", seed=41, hkv=2)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    announce("decode gqa vs repeated cache")
    o1, l1 = fa.decode(q, k, v, True)
    o2, l2 = fa.decode(q, k.repeat_interleave(4, dim=1).contiguous(),
                       v.repeat_interleave(4, dim=1).contiguous(), True)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-3
    assert (l1 - l2).abs().max().item() <= 1e-5


def test_grouped_decode_workload_full_size():
    w = workloads.DECODE_WORKLOAD_GQA
    x = workloads.draw_decode(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, hkv=w.kv_heads)
    assert fa.decode_num_splits(w.B, w.H, w.kv_heads, w.Nq, w.Nk, w.d) == 64
    run_decode_case(x, w.causal, w.scale, 0, w.name)


def test_binding_rejects_wrong_outputs_before_launch():
    x = workloads.draw_decode(1, 2, 1, 64, 64, "bf16", seed=1)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    with pytest.raises(ValueError):
        fa.decode(q, k, v, out=torch.empty((1, 2, 2, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.decode(q, k, v, lse=torch.empty((1, 2, 2), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.decode(q, k, v, workspace=torch.empty(1 << 16, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.forward(q, k, v, out=torch.empty((1, 2, 2, 64), dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("nk", [100, 5000])
def test_single_slice_direct_path_equals_the_two_kernel_path(nk):
    # One slice: the whole call writes O and LSE from the split kernel; the
    # stage path runs the split kernel into the workspace and then the combine.
    x = workloads.draw_decode(2, 4, 3, nk, 128, "bf16", seed=71, hkv=2)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    scale = workloads.default_scale(128)
    announce(f"decode direct path nk={nk}")
    o1, l1 = fa.decode(q, k, v, True, scale, num_splits=1)
    ws = fa.new_decode_workspace(q, k, 1)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    fa.decode_stage(fa.DEC_SPLIT, q, k, v, None, None, True, scale, 1, ws)
    fa.decode_stage(fa.DEC_COMBINE, q, k, v, o2, l2, True, scale, 1, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_binding_rejects_host_buffers_before_launch():
    # A host tensor's address must never reach a kernel: LSE and workspace
    # tensors on the CPU are refused by the binding before any call into the
    # library, in every entry point that takes them.
    x = workloads.draw(1, 2, 64, 64, "bf16", seed=2, with_do=True)
    q, k, v, do = (x[n].to("cuda") for n in ("q", "k", "v", "do"))
    announce("binding host-buffer rejection")
    o, lse = fa.forward(q, k, v, True)
    ws = fa.new_workspace(q)
    host_lse = lse.cpu()
    host_ws = ws.cpu()
    with pytest.raises(ValueError):
        fa.forward(q, k, v, True, lse=torch.empty((1, 2, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, do, host_lse, True)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, do, lse, True, workspace=host_ws)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    with pytest.raises(ValueError):
        fa.backward_stage(fa.BWD_PREPROCESS, q, k, v, o, do, lse, dq, dk, dv, host_ws, True)
    with pytest.raises(ValueError):
        fa.backward_stage(fa.BWD_PREPROCESS, q, k, v, o, do, host_lse, dq, dk, dv, ws, True)
    qd = q[:, :, :1].contiguous()
    with pytest.raises(ValueError):
        fa.decode(qd, k, v, workspace=fa.new_decode_workspace(qd, k).cpu())
    with pytest.raises(ValueError):
        fa.decode(qd, k, v, lse=torch.empty((1, 2, 1), dtype=torch.float32))
    # the GPU buffers themselves still work
    fa.backward(q, k, v, o, do, lse, True, workspace=ws)
    torch.cuda.synchronize()
