"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph on ROCm).

Every entry point only enqueues kernels on the caller's stream: it allocates,
frees and synchronises nothing and records no memset, so a caller can capture
a whole decode step or forward + backward once and replay it as one submission
(the remedy for dispatch overhead in the Lecture 9 notes, section 9.8).  Each
graph is replayed several times, with eager work and synchronisations in
between, and every replay is checked bitwise against the eager result.
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


def test_decode_graph_replays_match_eager():
    x = workloads.draw_decode(1, 8, 1, 5000, 128, "bf16", seed=61, hkv=2)
    q, k, v = (x[n].to("cuda") for n in ("q", "k", "v"))
    ws = fa.new_decode_workspace(q, k)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    announce("decode graph")
    o_ref, lse_ref = fa.decode(q, k, v, True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        fa.decode(q, k, v, True, workspace=ws, out=o, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.decode(q, k, v, True, workspace=ws, out=o, lse=lse)
    for rep in range(3):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay {rep}"
        fa.decode(q, k, v, False)              # eager work between replays
        torch.cuda.synchronize()


def test_forward_backward_graph_replays_match_eager():
    x = workloads.draw(1, 4, 700, 128, "bf16", seed=62, with_do=True)
    q, k, v, do = (x[n].to("cuda") for n in ("q", "k", "v", "do"))
    announce("forward backward graph")
    o_ref, lse_ref = fa.forward(q, k, v, True)
    g_ref = fa.backward(q, k, v, o_ref, do, lse_ref, True)
    torch.cuda.synchronize()
    o, lse = torch.empty_like(q), torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = fa.new_workspace(q)

    def step():
        fa.forward(q, k, v, True, out=o, lse=lse)
        fa.backward(q, k, v, o, do, lse, True, workspace=ws, out=(dq, dk, dv))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for t in (o, lse, dq, dk, dv):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay {rep}"
        assert all(torch.equal(a, b) for a, b in zip((dq, dk, dv), g_ref)), f"replay {rep}"
        fa.forward(q, k, v, False)
        torch.cuda.synchronize()


def test_fp8_input_stage_graph_replays_match_eager():
    # Q and K of one step rotated and quantised inside one captured graph.
    x = workloads.draw(1, 4, 1000, 128, "bf16", seed=63, with_do=False)
    q, k = x["q"].to("cuda"), x["k"].to("cuda")
    signs = workloads.draw_signs(128, 63).to("cuda")
    announce("fp8 input stage graph")
    ref = [fa.fp8_quantize_rows(t, signs) for t in (q, k)]
    torch.cuda.synchronize()
    outs = [(torch.empty(t.shape, dtype=torch.uint8, device="cuda"),
             torch.empty(t.shape[:-1], dtype=torch.float32, device="cuda")) for t in (q, k)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        for t, (c, s) in zip((q, k), outs):
            fa.fp8_quantize_rows(t, signs, c, s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t, (c, s) in zip((q, k), outs):
            fa.fp8_quantize_rows(t, signs, c, s)
    for rep in range(3):
        for c, s in outs:
            c.zero_()
            s.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (c, s), (cr, sr) in zip(outs, ref):
            assert torch.equal(c, cr) and torch.equal(s, sr), f"replay {rep}"
        fa.fp8_quantize_rows(q, None)          # eager work between replays
        torch.cuda.synchronize()
