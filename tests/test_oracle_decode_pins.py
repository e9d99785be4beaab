"""Pins of the oracle's decode function (a short block of queries against a long
key/value cache) against what the pages and the mathematics fix.

The decode setting and its split-K combine come from the Lecture 9 notes
(cs2680.com), §9.8, and the CMU 11-868 FlashAttention notes (quidproquo.cc),
slide pages 57-60.  Checked here: an independent pure-Python evaluation, closed
forms for identical keys (with the bottom-right causal alignment), the last
causal row against the unmasked one, torch's fp64 CPU attention with an explicit
mask, and the split-K combine of per-slice partial statistics reproducing the
full result for every slice count.  A mask aligned at the top-left instead of
the bottom-right, a dropped scale or a wrong combine weight fails one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(20261203)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def _pure_python_decode(q, k, v, causal, scale):
    nq, nk, d = len(q), len(k), len(q[0])
    out, lses = [], []
    for i in range(nq):
        last = nk - nq + i if causal else nk - 1
        keys = range(last + 1)
        sc = [scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in keys]
        top = max(sc)
        w = [math.exp(s - top) for s in sc]
        tot = math.fsum(w)
        out.append([math.fsum(w[t] * v[j][c] for t, j in enumerate(keys)) / tot
                    for c in range(d)])
        lses.append(top + math.log(tot))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("nq,nk,d,causal", [(1, 1, 3, False), (1, 9, 4, True), (2, 7, 3, True),
                                            (3, 11, 2, False), (5, 5, 3, True), (4, 13, 5, True)])
def test_decode_matches_independent_pure_python_loops(nq, nk, d, causal):
    q, k, v = rand(nq, d), rand(nk, d), rand(nk, d)
    o_ref, l_ref = _pure_python_decode(q.tolist(), k.tolist(), v.tolist(), causal, 0.7)
    o, lse = oracle.decode_head(q, k, v, causal, 0.7)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, l_ref, atol=1e-13)


def test_decode_with_nq_equal_nk_is_the_forward():
    q, k, v = rand(33, 8), rand(33, 8), rand(33, 8)
    for causal in (False, True):
        o, lse = oracle.decode_head(q, k, v, causal, 0.4)
        o_f, lse_f = oracle.forward_head(q, k, v, causal, 0.4)
        np.testing.assert_array_equal(o, o_f)
        np.testing.assert_array_equal(lse, lse_f)


def test_identical_keys_give_bottom_right_prefix_means():
    nq, nk, d, scale = 6, 40, 5, 0.5
    q, v = rand(nq, d), rand(nk, d)
    key = rand(d)
    k = np.tile(key, (nk, 1))
    o, lse = oracle.decode_head(q, k, v, True, scale)
    for i in range(nq):
        count = nk - nq + i + 1          # query i sits at position nk - nq + i
        np.testing.assert_allclose(o[i], v[:count].mean(axis=0), atol=1e-14)
        np.testing.assert_allclose(lse[i], scale * q[i] @ key + math.log(count), atol=1e-13)
    o_nc, lse_nc = oracle.decode_head(q, k, v, False, scale)
    np.testing.assert_allclose(o_nc, np.tile(v.mean(axis=0), (nq, 1)), atol=1e-14)
    np.testing.assert_allclose(lse_nc, scale * q @ key + math.log(nk), atol=1e-13)


def test_single_query_and_last_causal_row_see_every_key():
    nq, nk, d = 4, 29, 6
    q, k, v = rand(nq, d), rand(nk, d), rand(nk, d)
    o_c, lse_c = oracle.decode_head(q, k, v, True, 0.6)
    o_n, lse_n = oracle.decode_head(q, k, v, False, 0.6)
    np.testing.assert_allclose(o_c[-1], o_n[-1], atol=1e-15)
    np.testing.assert_allclose(lse_c[-1], lse_n[-1], atol=1e-15)
    assert not np.allclose(o_c[0], o_n[0])        # earlier rows do lose keys
    o1, l1 = oracle.decode_head(q[:1], k, v, True, 0.6)
    o1n, l1n = oracle.decode_head(q[:1], k, v, False, 0.6)
    np.testing.assert_array_equal(o1, o1n)
    np.testing.assert_array_equal(l1, l1n)


@pytest.mark.parametrize("causal", [False, True])
def test_decode_matches_torch_fp64_sdpa_with_mask(causal):
    B, H, nq, nk, d, scale = 2, 3, 7, 50, 16, 0.3
    q, k, v = rand(B, H, nq, d), rand(B, H, nk, d), rand(B, H, nk, d)
    o, lse = oracle.decode(q, k, v, causal, scale)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    mask = None
    if causal:
        mask = torch.arange(nk)[None, :] <= (torch.arange(nq) + nk - nq)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-13)
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-13)


def _split_partials(q, k, v, causal, scale, bounds):
    """Per key slice [b0, b1): the unnormalised output, the slice's row max and the
    denominator relative to it (Lecture 9 §9.8: each slice reduces over its own
    part of the cache; a row with no visible key in the slice has m = -inf)."""
    nq, nk = q.shape[0], k.shape[0]
    pos = np.arange(nq) + nk - nq
    parts = []
    for b0, b1 in zip(bounds[:-1], bounds[1:]):
        x = scale * q @ k[b0:b1].T
        if causal:
            x = np.where(np.arange(b0, b1)[None, :] <= pos[:, None], x, -np.inf)
        m = x.max(axis=1)
        safe = np.where(np.isneginf(m), 0.0, m)
        p = np.exp(x - safe[:, None])
        parts.append((p @ v[b0:b1], m, p.sum(axis=1)))
    return parts


def _combine(parts):
    """Merge the slices' statistics with the rescaling of Lecture 9 §9.4: bring every
    slice to the common max M, add, divide once."""
    M = np.max([m for _, m, _ in parts], axis=0)
    acc = sum(np.where(np.isneginf(m), 0.0, np.exp(m - M))[:, None] * o for o, m, _ in parts)
    den = sum(np.where(np.isneginf(m), 0.0, np.exp(m - M)) * l for _, m, l in parts)
    return acc / den[:, None], M + np.log(den)


@pytest.mark.parametrize("causal", [False, True])
def test_split_k_combine_reproduces_the_definition(causal):
    nq, nk, d, scale = 5, 97, 8, 0.9
    q, k, v = rand(nq, d), rand(nk, d, scale=2.0), rand(nk, d)
    o_ref, lse_ref = oracle.decode_head(q, k, v, causal, scale)
    for nsplit in (1, 2, 3, 8, 97):
        cuts = np.sort(RNG.choice(np.arange(1, nk), size=nsplit - 1, replace=False))
        bounds = [0, *cuts.tolist(), nk]
        o, lse = _combine(_split_partials(q, k, v, causal, scale, bounds))
        np.testing.assert_allclose(o, o_ref, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_decode_rejects_more_queries_than_keys():
    with pytest.raises(ValueError):
        oracle.decode_head(rand(4, 2), rand(3, 2), rand(3, 2), False, 1.0)


@pytest.mark.parametrize("hkv", [1, 2, 3, 6])
def test_grouped_kv_heads_equal_repeated_kv_heads(hkv):
    # Sharing a key/value head among g query heads is the same as giving each
    # query head its own copy of it (heads h*g .. h*g+g-1 share head h).
    B, H, nq, nk, d = 2, 6, 3, 40, 5
    q, k, v = rand(B, H, nq, d), rand(B, hkv, nk, d), rand(B, hkv, nk, d)
    g = H // hkv
    o, lse = oracle.decode(q, k, v, True, 0.5)
    o_r, lse_r = oracle.decode(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), True, 0.5)
    np.testing.assert_array_equal(o, o_r)
    np.testing.assert_array_equal(lse, lse_r)
    # head 0 and head g-1 use key/value head 0; head g uses head 1 (when it exists)
    o0, _ = oracle.decode_head(q[1, g - 1], k[1, 0], v[1, 0], True, 0.5)
    np.testing.assert_array_equal(o[1, g - 1], o0)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_decode_matches_torch_sdpa_enable_gqa(causal):
    B, H, hkv, nq, nk, d, scale = 2, 8, 2, 4, 33, 16, 0.25
    q, k, v = rand(B, H, nq, d), rand(B, hkv, nk, d), rand(B, hkv, nk, d)
    o, _ = oracle.decode(q, k, v, causal, scale)
    mask = None
    if causal:
        mask = torch.arange(nk)[None, :] <= (torch.arange(nq) + nk - nq)[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), attn_mask=mask, scale=scale, enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-13)


def test_grouped_decode_rejects_non_dividing_head_counts():
    with pytest.raises(ValueError):
        oracle.decode(rand(1, 6, 1, 2), rand(1, 4, 3, 2), rand(1, 4, 3, 2), False, 1.0)
