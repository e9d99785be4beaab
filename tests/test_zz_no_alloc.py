"""fa_backward_noalloc, the entry point that allocates nothing: its dQ, dK, dV
must equal fa_backward's (same kernels, same inputs: bitwise) on two calls in a
row on one device, the second with a smaller input, so the shared static
scratch array keeps no state that changes a later result; plus the size limit
and a caller-provided output set (no allocation in the binding either)."""
import pytest
import torch

import exact_io_aware_forward_amd as fa
import workloads
from helpers import announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def inputs(B, H, N, d, dtype, seed, causal):
    x = workloads.draw(B, H, N, d, dtype, seed=seed, with_do=True)
    q, k, v, do = (x[n].cuda() for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal)
    return q, k, v, o, do, lse


@pytest.mark.parametrize("causal", [True, False])
def test_two_calls_match_the_workspace_entry_point(causal):
    # First the N=4096 d=128 bf16 shape (B*H*N = 131072 rows), then a smaller,
    # ragged fp16 d=64 input.
    for shape in ((2, 16, 4096, 128, "bf16", 71), (1, 3, 333, 64, "fp16", 72)):
        q, k, v, o, do, lse = inputs(*shape[:5], shape[5], causal)
        announce(f"noalloc backward {shape} causal={causal}")
        ref = fa.backward(q, k, v, o, do, lse, causal)
        got = fa.backward_noalloc(q, k, v, o, do, lse, causal)
        torch.cuda.synchronize()
        for a, b, name in zip(got, ref, ("dq", "dk", "dv")):
            assert torch.equal(a, b), f"{shape}: {name} differs from fa_backward"


def test_largest_accepted_input_and_caller_outputs():
    # B*H*N = 2^20 rows exactly fills the 8 MiB array.
    q, k, v, o, do, lse = inputs(1, 256, 4096, 64, "bf16", 73, True)
    assert q.shape[0] * q.shape[1] * q.shape[2] == 1 << 20
    out = tuple(torch.empty_like(t) for t in (q, k, v))
    announce("noalloc backward at the size limit")
    fa.backward_noalloc(q, k, v, o, do, lse, True, out=out)
    ref = fa.backward(q, k, v, o, do, lse, True)
    torch.cuda.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(a, b)


def test_too_large_is_refused_before_launch():
    q = torch.zeros((1, 1, (1 << 20) + 32, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(q.shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FAError) as e:
        fa.backward_noalloc(q, q, q, q, q, lse, False)
    assert e.value.status == fa.FA_ERR_WORKSPACE
