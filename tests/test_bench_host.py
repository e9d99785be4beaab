"""Host-side logic of bench.py (no GPU): the work model, the count of visited
tiles behind the executed-FLOP figures, and the single-GPU guard."""
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 127, 128, 129, 300, 1000, 4096])
@pytest.mark.parametrize("br,bc", [(256, 64), (64, 128), (128, 64)])
def test_visited_tiles_match_the_tile_map(n, causal, br, bc):
    # The closed form counts the tiles with at least one visible element,
    # i.e. the nonzero codes of the brute-force map.
    expected = int(np.count_nonzero(oracle.tile_map(n, br, bc, causal)))
    assert bench.visited_tiles(n, br, bc, causal) == expected


def test_work_model_flop_conventions():
    w = workloads.WORKLOADS[4]
    wm = bench.work_model(w)
    heads, n, d = w.B * w.H, w.N, w.d
    half = n * n * d * heads // 2          # causal counts half of N^2 d per head
    assert wm["fwd_flop"] == 4 * half
    assert wm["bwd_flop"] == 10 * half
    assert wm["step_flop"] == 14 * half
    assert wm["bwd_dkdv"]["flop"] + wm["bwd_dq"]["flop"] == wm["bwd_flop"]
    # Bytes: forward reads Q, K, V and writes O (bf16) plus a float LSE per row.
    assert wm["fwd"]["bytes"] == heads * (4 * n * d * 2 + 4 * n)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True,
                       cwd=bench.ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_decode_work_model_is_one_flop_per_cache_byte():
    # Lecture 9 notes §9.8: one query against the cache does 4*S*d FLOPs on
    # 2*S*d*b bytes of cache, 2/b = 1 FLOP per byte in a 16-bit type.
    w = workloads.DECODE_WORKLOAD
    wm = bench.decode_work_model(w)
    assert w.Nq == 1 and w.dtype == "bf16"
    assert wm["flop"] == wm["cache_bytes"]
    assert wm["cache_bytes"] == w.B * w.H * 2 * w.Nk * w.d * 2
    # causal with Nq queries: query i sees Nk - Nq + i + 1 keys
    w3 = workloads.DecodeWorkload("t", "bf16", 1, 1, 3, 10, 4, True, 0)
    assert bench.decode_work_model(w3)["flop"] == 4 * 4 * (8 + 9 + 10)


def test_decode_work_model_counts_the_shared_cache_once():
    w = workloads.DECODE_WORKLOAD_GQA
    wm = bench.decode_work_model(w)
    g = w.H // w.kv_heads
    assert g == 8
    assert wm["cache_bytes"] == w.B * w.kv_heads * 2 * w.Nk * w.d * 2
    assert wm["flop"] == g * wm["cache_bytes"]      # g FLOP per cache byte


def test_fp8_quant_bytes_per_launch():
    # 16-bit rows read, one code byte per value and one fp32 scale per row written:
    # Q of the N=4096 workload (2 * 16 * 4096 rows of 128) is 50.86 MB per launch.
    assert bench.fp8_quant_bytes(1, 64) == 64 * 2 + 64 + 4
    assert bench.fp8_quant_bytes(131072, 128) == 131072 * (256 + 128 + 4) == 50855936


def test_fp8_quant_cpu_baseline_is_a_bounded_oracle_sample():
    q = torch.randn((1, 2, 2500, 64)).to(torch.bfloat16)
    signs = workloads.draw_signs(64, 3).double().numpy()
    r = bench.fp8_quant_cpu_baseline(q, signs, budget_s=0.0)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["sample"].startswith("4096 of 5000 Q rows")    # one block, then the budget stops it


def test_draw_signs_are_seeded_plus_minus_one():
    a, b = workloads.draw_signs(128, 7), workloads.draw_signs(128, 7)
    assert a.dtype == torch.float32 and a.shape == (128,)
    assert torch.equal(a, b) and set(a.tolist()) <= {-1.0, 1.0}
    assert not torch.equal(a, workloads.draw_signs(128, 8))


def test_calculator_reproduces_the_printed_lecture9_arithmetic():
    # Every value the Lecture 9 notes print for attention's FLOPs, bytes,
    # intensities and crossovers (sections 9.2 and 9.6, exercise 1, the
    # key-takeaways table), recomputed by the bench's calculator; a printed value
    # may be rounded or cut off in its last place, so the bound is one unit there.
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "lecture9_arithmetic.json")) as f:
        golden = json.load(f)["items"]
    calc = bench.lecture9_arithmetic()
    assert set(calc) == set(golden)
    for key, item in golden.items():
        unit = 10.0 ** -item["decimals"]
        assert abs(calc[key] - item["value"]) <= unit, (key, calc[key], item["value"])


def test_calculator_matches_the_work_model():
    # The benchmark's forward FLOPs are the calculator's 4 S^2 d per head.
    w = workloads.WORKLOADS[3]
    wm = bench.work_model(w)
    assert wm["fwd_flop"] == w.B * w.H * bench.attention_flop(w.N, w.d)
    assert bench.fused_intensity(w.N, w.d, 2) == w.N / 2
    assert bench.unfused_intensity(w.N, w.d, 2) == w.d / 2


def test_cpu_baseline_names_the_cpu_and_blas_threads():
    info = bench.blas_info()
    assert info.get("threads", 0) >= 1 and "library" in info
    assert bench.cpu_model()


def test_fp8_mixed_peak():
    # Equal halves on pipes of 5.0 and 2.5 PFLOP/s: 2 / (1/5000 + 1/2500).
    assert abs(bench.fp8_mixed_peak(1.0, 1.0) - 10000.0 / 3.0) < 1e-9
    assert bench.fp8_mixed_peak(1.0, 0.0) == bench.PEAK_FP8_TFLOPS
    assert bench.fp8_mixed_peak(0.0, 1.0) == bench.PEAK_TFLOPS["bf16"]
