"""Race check: the FA_DEBUG_SYNC build of the library (libfa_debugsync.so), whose
kernels drain every outstanding buffer-to-LDS copy, load and LDS access at
each workgroup barrier, must give outputs bitwise equal to the production
build's on the same inputs.  An LDS race in production (a copy landing in a
buffer still being read, a read of a tile not yet published) would show up as
a difference, since the drained schedule has no copy in flight across any
barrier.  Covered: the causal N=4096 d=128 bf16 shape (forward and backward,
every head), ragged shapes at both head dimensions with and without the causal
mask, grouped heads with a split dK/dV pass, and a split-K decode.
"""
import pytest
import torch

import exact_io_aware_forward_amd as fa
import workloads
from helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def debug_lib():
    return fa.open_library(fa.DEBUG_SYNC_LIB_PATH)


def run_both(debug_lib, monkeypatch, fn):
    prod = fn()
    torch.cuda.synchronize()
    with monkeypatch.context() as m:
        m.setattr(fa, "_lib", debug_lib)
        dbg = fn()
        torch.cuda.synchronize()
    return prod, dbg


def assert_bitwise(prod, dbg, label):
    for i, (a, b) in enumerate(zip(prod, dbg)):
        assert torch.equal(a, b), f"{label}: output {i} differs from the drained build"


@pytest.mark.parametrize("case", ["causal_bf16_B2_H16_N4096_d128", "fp16_B2_H4_N1000_d64",
                                  "causal_bf16_B1_H4_N777_d64", "fp16_B1_H2_N1500_d128"])
def test_forward_backward_bitwise_equal(debug_lib, monkeypatch, case):
    if case == "causal_bf16_B2_H16_N4096_d128":
        x = workloads.workload_inputs(4)
        causal, scale = True, workloads.WORKLOADS[4].scale
    elif case == "fp16_B2_H4_N1000_d64":
        x = workloads.draw(2, 4, 1000, 64, "fp16", seed=61, with_do=True)
        causal, scale = False, workloads.default_scale(64)
    elif case == "causal_bf16_B1_H4_N777_d64":
        x = workloads.draw(1, 4, 777, 64, "bf16", seed=64, with_do=True)
        causal, scale = True, workloads.default_scale(64)
    else:
        x = workloads.draw(1, 2, 1500, 128, "fp16", seed=65, with_do=True)
        causal, scale = False, workloads.default_scale(128)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))

    def fn():
        o, lse = fa.forward(q, k, v, causal, scale)
        return (o, lse, *fa.backward(q, k, v, o, do, lse, causal, scale))

    announce(f"debug-sync bitwise {case}")
    prod, dbg = run_both(debug_lib, monkeypatch, fn)
    assert_bitwise(prod, dbg, case)


def test_grouped_split_backward_bitwise_equal(debug_lib, monkeypatch):
    x = workloads.draw(1, 8, 700, 128, "bf16", seed=62, with_do=True)
    q, do = x["q"].cuda(), x["do"].cuda()
    k, v = x["k"][:, :2].contiguous().cuda(), x["v"][:, :2].contiguous().cuda()

    def fn():
        o, lse = fa.forward(q, k, v, True)
        return (o, lse, *fa.backward(q, k, v, o, do, lse, True))

    announce("debug-sync bitwise grouped backward")
    prod, dbg = run_both(debug_lib, monkeypatch, fn)
    assert_bitwise(prod, dbg, "grouped")


def test_decode_bitwise_equal(debug_lib, monkeypatch):
    x = workloads.draw_decode(1, 8, 3, 5000, 128, "bf16", seed=63, hkv=2)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))

    def fn():
        return fa.decode(q, k, v, True, num_splits=7)

    announce("debug-sync bitwise decode")
    prod, dbg = run_both(debug_lib, monkeypatch, fn)
    assert_bitwise(prod, dbg, "decode")
