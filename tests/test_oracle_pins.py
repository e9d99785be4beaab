"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: closed forms,
invariants, an independent pure-Python evaluation on tiny inputs, finite
differences, a library routine (torch's fp64 CPU attention and autograd), the
online-softmax identities the pages state, and the one worked value the pages
print (178.6).  Chosen so that a dropped term, a wrong sign or index, a missing
scale, an off-by-one in the causal mask or a transposed operand fails at least
one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261202)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# --------------------------------------------------------------------------- forward

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_A_sum_to_one(causal):
    q, k = rand(37, 8), rand(37, 8)
    a = oracle.probabilities(q, k, causal, 0.3)
    np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (a >= 0).all()
    if causal:
        assert np.all(np.triu(a, 1) == 0.0)   # masked weights are exactly zero


def test_identical_keys_give_mean_of_values_noncausal():
    n, d = 23, 6
    q, v = rand(n, d), rand(n, d)
    k = np.tile(rand(1, d), (n, 1))
    scale = 0.7
    o, lse = oracle.forward_head(q, k, v, False, scale)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (n, 1)), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, scale * (q @ k[0]) + math.log(n), rtol=0, atol=1e-13)


def test_identical_keys_give_prefix_mean_causal():
    n, d = 19, 5
    q, v = rand(n, d), rand(n, d)
    k = np.tile(rand(1, d), (n, 1))
    scale = 1.3
    o, lse = oracle.forward_head(q, k, v, True, scale)
    prefix = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(o, prefix, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, scale * (q @ k[0]) + np.log(np.arange(1, n + 1)),
                               rtol=0, atol=1e-13)


def test_zero_queries_lse_is_log_count():
    n, d = 11, 4
    q, k, v = np.zeros((n, d)), rand(n, d), rand(n, d)
    _, lse_nc = oracle.forward_head(q, k, v, False, 0.5)
    _, lse_c = oracle.forward_head(q, k, v, True, 0.5)
    np.testing.assert_allclose(lse_nc, math.log(n), atol=1e-14)
    np.testing.assert_allclose(lse_c, np.log(np.arange(1, n + 1)), atol=1e-14)


def test_single_key_and_causal_first_row():
    q, k, v = rand(1, 7), rand(1, 7), rand(1, 7)
    o, lse = oracle.forward_head(q, k, v, False, 0.25)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.25 * (q @ k.T)[0], atol=1e-15)
    q, k, v = rand(9, 7), rand(9, 7), rand(9, 7)
    o, _ = oracle.forward_head(q, k, v, True, 0.25)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)


def test_shift_invariance_of_keys():
    n, d, scale = 17, 6, 0.4
    q, k, v, u = rand(n, d), rand(n, d), rand(n, d), rand(d)
    for causal in (False, True):
        o1, l1 = oracle.forward_head(q, k, v, causal, scale)
        o2, l2 = oracle.forward_head(q, k + u, v, causal, scale)
        np.testing.assert_allclose(o2, o1, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, scale * (q @ u), atol=1e-12)


def test_joint_permutation_of_keys_and_values_noncausal():
    n, d = 21, 5
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    perm = RNG.permutation(n)
    o1, l1 = oracle.forward_head(q, k, v, False, 0.6)
    o2, l2 = oracle.forward_head(q, k[perm], v[perm], False, 0.6)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)


def test_large_scores_do_not_overflow():
    # Two keys with scores 1000 and 1001: weights 1/(1+e) and e/(1+e).
    q = np.array([[1.0]])
    k = np.array([[1000.0], [1001.0]])
    v = np.array([[3.0], [-5.0]])
    o, lse = oracle.forward_head(q, k, v, False, 1.0)
    w1 = math.e / (1 + math.e)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o[0, 0], 3.0 * (1 - w1) - 5.0 * w1, rtol=1e-14)
    np.testing.assert_allclose(lse[0], 1001.0 + math.log1p(math.exp(-1.0)), rtol=1e-15)


def _pure_python_attention(q, k, v, causal, scale):
    n, d = len(q), len(q[0])
    out, lses = [], []
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        sc = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        top = max(sc)
        w = [math.exp(s - top) for s in sc]
        tot = math.fsum(w)
        out.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(keys)) / tot
                    for c in range(d)])
        lses.append(top + math.log(tot))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("n,d,causal", [(1, 3, False), (4, 2, True), (7, 3, False), (9, 4, True)])
def test_matches_independent_pure_python_loops(n, d, causal):
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o_ref, l_ref = _pure_python_attention(q.tolist(), k.tolist(), v.tolist(), causal, 0.9)
    o, lse = oracle.forward_head(q, k, v, causal, 0.9)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, l_ref, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_fp64_sdpa(causal):
    B, H, N, d = 2, 3, 45, 16
    q, k, v = rand(B, H, N, d), rand(B, H, N, d), rand(B, H, N, d)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, causal, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)
    s = scale * torch.einsum("bhnd,bhmd->bhnm", tq, tk)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


def test_chunking_does_not_change_results():
    q, k, v = rand(70, 8), rand(70, 8), rand(70, 8)
    for causal in (False, True):
        o1, l1 = oracle.forward_head(q, k, v, causal, 0.5, chunk=512)
        o2, l2 = oracle.forward_head(q, k, v, causal, 0.5, chunk=7)
        np.testing.assert_allclose(o2, o1, atol=1e-14)
        np.testing.assert_allclose(l2, l1, atol=1e-14)
        rows = np.array([3, 69, 0, 41])
        o3, l3 = oracle.forward_head(q, k, v, causal, 0.5, rows=rows)
        np.testing.assert_allclose(o3, o1[rows], atol=1e-14)
        np.testing.assert_allclose(l3, l1[rows], atol=1e-14)


# ---------------------------------------------- the online-softmax identities of the pages

def _two_block_normalized(q, k, v, split, scale):
    """CMU 11-868 FlashAttention notes, slide page 12: output of block one under its
    own denominator, then corrected by l1/l2 when block two arrives.  Scores are
    exponentiated without a max (fine for the small test values)."""
    a1 = np.exp(scale * q @ k[:split].T)
    a2 = np.exp(scale * q @ k[split:].T)
    l1 = a1.sum(axis=1, keepdims=True)
    o1 = a1 @ v[:split] / l1
    l2 = l1 + a2.sum(axis=1, keepdims=True)
    return (l1 / l2) * o1 + a2 @ v[split:] / l2, np.log(l2[:, 0])


def test_two_block_rescaling_identity_every_split():
    n, d, scale = 24, 6, 0.35
    q, k, v = rand(n, d), rand(n, d), rand(n, d)
    o_ref, lse_ref = oracle.forward_head(q, k, v, False, scale)
    for split in range(1, n):
        o, lse = _two_block_normalized(q, k, v, split, scale)
        np.testing.assert_allclose(o, o_ref, atol=1e-13)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-13)


def _online_unnormalized(q, k, v, bounds, scale, causal):
    """Lecture 9 §9.4: carry a running max m, a running denominator l relative to m
    and an unnormalised output; rescale both by exp(m_old - m_new) when the max
    grows; divide by l once at the end."""
    n = q.shape[0]
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    acc = np.zeros((n, v.shape[1]))
    rows = np.arange(n)
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        x = scale * q @ k[b0:b1].T
        if causal:
            x = np.where(np.arange(b0, b1)[None, :] <= rows[:, None], x, -np.inf)
        m_new = np.maximum(m, x.max(axis=1))
        alpha = np.where(np.isneginf(m_new), 1.0, np.exp(m - m_new))
        p = np.exp(x - np.where(np.isneginf(m_new), 0.0, m_new)[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ v[b0:b1]
        m = m_new
    return acc / l[:, None], m + np.log(l)


@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_k_blocks_reproduce_the_definition(causal):
    n, d, scale = 50, 8, 0.8
    q, k, v = rand(n, d), rand(n, d, scale=3.0), rand(n, d)
    o_ref, lse_ref = oracle.forward_head(q, k, v, causal, scale)
    for nblocks in (1, 2, 3, 7, 50):
        cuts = np.sort(RNG.choice(np.arange(1, n), size=nblocks - 1, replace=False))
        bounds = [0, *cuts.tolist(), n]
        o, lse = _online_unnormalized(q, k, v, bounds, scale, causal)
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_hand_check_178_6_from_lecture9():
    with open(os.path.join(GOLDEN, "online_softmax_hand_check.json")) as f:
        g = json.load(f)
    blocks = g["our_blocks"]
    m, l = -math.inf, 0.0
    for blk in blocks:                      # online update on our two blocks
        m_new = max(m, max(blk))
        l = l * math.exp(m - m_new) + sum(math.exp(x - m_new) for x in blk)
        m = m_new
    assert round(l * math.exp(m), g["printed_decimals"]) == g["printed_value"]
    # The oracle's LSE for one query whose scaled scores are these values.
    scores = [x for blk in blocks for x in blk]
    q = np.array([[1.0]])
    k = np.array([[x] for x in scores])
    v = rand(len(scores), 2)
    _, lse = oracle.forward_head(q, k, v, False, 1.0)
    assert round(math.exp(lse[0]), g["printed_decimals"]) == g["printed_value"]


# --------------------------------------------------------------------------- backward

def _loss(q, k, v, do, causal, scale):
    o, _ = oracle.forward_head(q, k, v, causal, scale)
    return float((o * do).sum())


@pytest.mark.parametrize("n,d,causal", [(1, 1, False), (2, 2, True), (3, 4, False),
                                        (5, 2, True), (8, 4, False), (8, 4, True)])
def test_gradients_match_central_finite_differences(n, d, causal):
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    scale = 0.75
    g = oracle.backward_head(q, k, v, do, causal, scale)
    h = 1e-5
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss(q, k, v, do, causal, scale)
            x[idx] = old - h
            lm = _loss(q, k, v, do, causal, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g[name]).max()
        assert err <= 1e-7 * max(1.0, np.abs(num).max()), (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_fp64_autograd(causal):
    B, H, N, d = 1, 2, 33, 8
    q, k, v, do = (rand(B, H, N, d) for _ in range(4))
    scale = 1 / math.sqrt(d)
    g = oracle.backward(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    n, d, scale = 40, 8, 0.5
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    g = oracle.backward_head(q, k, v, do, causal, scale)
    o, _ = oracle.forward_head(q, k, v, causal, scale)
    # D = rowsum(dO * O): the preprocess identity the backward relies on.
    np.testing.assert_allclose(g["D"], (do * o).sum(axis=1), atol=1e-12)
    # Softmax rows sum to one, so the values' gradient sums to the sum of dO.
    np.testing.assert_allclose(g["dv"].sum(axis=0), do.sum(axis=0), atol=1e-12)
    # Rows of dS sum to zero, hence sum_i dK_i = 0 (shift invariance in K).
    np.testing.assert_allclose(g["dk"].sum(axis=0), 0.0, atol=1e-12)


def test_identical_keys_give_zero_query_gradient():
    n, d = 12, 4
    q, v, do = rand(n, d), rand(n, d), rand(n, d)
    k = np.tile(rand(1, d), (n, 1))
    for causal in (False, True):
        g = oracle.backward_head(q, k, v, do, causal, 0.9)
        np.testing.assert_allclose(g["dq"], 0.0, atol=1e-13)


def test_backward_chunking_does_not_change_results():
    n, d = 30, 4
    q, k, v, do = rand(n, d), rand(n, d), rand(n, d), rand(n, d)
    a = oracle.backward_head(q, k, v, do, True, 0.5, chunk=512)
    b = oracle.backward_head(q, k, v, do, True, 0.5, chunk=4)
    for name in a:
        np.testing.assert_allclose(b[name], a[name], atol=1e-13)


# --------------------------------------------------------------------------- tile map

def test_tile_map_hand_examples():
    # N=4, 2x2 tiles, causal: diagonal tiles are partial, the upper one empty.
    np.testing.assert_array_equal(oracle.tile_map(4, 2, 2, True), [[2, 0], [1, 2]])
    np.testing.assert_array_equal(oracle.tile_map(4, 2, 2, False), [[1, 1], [1, 1]])
    # N=5, 2x2 tiles, non-causal: the last row and column of tiles are ragged.
    np.testing.assert_array_equal(oracle.tile_map(5, 2, 2, False),
                                  [[1, 1, 6], [1, 1, 6], [6, 6, 6]])
    # N=3, 4x2 tiles, causal: one row of tiles reaching past N.
    np.testing.assert_array_equal(oracle.tile_map(3, 4, 2, True), [[6, 6]])


def _closed_form(n, br, bc, causal):
    nq, nk = -(-n // br), -(-n // bc)
    out = np.zeros((nq, nk), np.uint8)
    for i in range(nq):
        last_row = min((i + 1) * br, n) - 1
        for j in range(nk):
            c0 = j * bc
            if causal and c0 > last_row:
                continue
            inside = (i + 1) * br <= n and (j + 1) * bc <= n
            full = inside and (not causal or (j + 1) * bc - 1 <= i * br)
            out[i, j] = 1 if full else (2 | (0 if inside else 4))
    return out


@pytest.mark.parametrize("br,bc", [(128, 64), (64, 64), (32, 64), (64, 128), (32, 128), (16, 16),
                                   (256, 64), (256, 32), (512, 64)])
def test_tile_map_equals_closed_form_rule(br, bc):
    # The kernels' tiles, checked past one and two row tiles: forward (256, 64)
    # and (512, 64) (d = 64 without the causal mask); dQ (256, 32) at d = 128 and
    # (256, 64) at d = 64; dK/dV (query rows, key columns) (64, 128) at d = 128
    # and (32, 128) at d = 64.
    for n in list(range(1, 301, 7)) + [256, 257, 300, 511, 512, 513, 1000, 1100]:
        for causal in (False, True):
            np.testing.assert_array_equal(oracle.tile_map(n, br, bc, causal),
                                          _closed_form(n, br, bc, causal))


def test_tile_map_counts_for_square_multiples():
    # With Br = Bc and N a multiple: nq full tiles strictly below the diagonal band
    # count nq(nq-1)/2, the nq diagonal tiles are partial, the rest empty.
    m = oracle.tile_map(1024, 128, 128, True)
    nq = 8
    assert (m == 2).sum() == nq
    assert (m == 1).sum() == nq * (nq - 1) // 2
    assert (m == 0).sum() == nq * (nq - 1) // 2


# ------------------------------------------------- grouped key/value heads (GQA)

@pytest.mark.parametrize("causal", [False, True])
def test_grouped_forward_backward_match_torch_autograd_enable_gqa(causal):
    # Library cross-check: torch's fp64 SDPA with enable_gqa shares key/value
    # head h among query heads h*g .. h*g+g-1, and autograd sums their gradients.
    B, H, hkv, N, d, scale = 2, 6, 2, 19, 8, 0.4
    q, k, v, do = rand(B, H, N, d), rand(B, hkv, N, d), rand(B, hkv, N, d), rand(B, H, N, d)
    o, _ = oracle.forward(q, k, v, causal, scale)
    g = oracle.backward(q, k, v, do, causal, scale)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                           scale=scale, enable_gqa=True)
    ref.backward(torch.from_numpy(do))
    np.testing.assert_allclose(o, ref.detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(g["dq"], tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dk"], tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dv"], tv.grad.numpy(), atol=1e-12)


def test_grouped_gradients_are_sums_over_the_group():
    B, H, hkv, N, d = 1, 4, 1, 11, 3
    q, k, v, do = rand(B, H, N, d), rand(B, hkv, N, d), rand(B, hkv, N, d), rand(B, H, N, d)
    g = oracle.backward(q, k, v, do, True, 0.7)
    rep = oracle.backward(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), do, True, 0.7)
    np.testing.assert_allclose(g["dk"][:, 0], rep["dk"].sum(axis=1), atol=1e-14)
    np.testing.assert_allclose(g["dv"][:, 0], rep["dv"].sum(axis=1), atol=1e-14)
    np.testing.assert_array_equal(g["dq"], rep["dq"])
