"""Float64 CPU oracle for exact attention: the plain definition, written out.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
The product path (the HIP library and its Python binding) never touches it, and
this module imports nothing from the product: it shares no kernels, helpers,
tables or constants with the GPU path.

What it computes.  The pages state that the tiled, IO-aware method returns the
same result as standard attention, with no approximation (quidproquo.cc
FlashAttention tag page, the Hung-yi Lee ML 2026 entry; Lecture 9 notes at
cs2680.com, §9.4, on the exactness of every rescaling update; CMU 11-868
FlashAttention notes at quidproquo.cc, "Tiling: fix the wrong denominator
afterward", slide page 12).  So the oracle is the three-step definition of
attention (CMU 11-868 notes, "The scenario", slide page 5: S = QK^T,
A = softmax(S) row-wise, O = AV), with these readings where the pages are silent:

* the scores carry a caller-given ``scale`` (S = scale * Q K^T; the pages'
  three steps omit it, every workload uses 1/sqrt(d));
* causal masking means key j is visible to query i iff j <= i; masked entries get
  weight exactly zero (exp(-inf) = 0); every causal row holds j = i, so no row is
  empty;
* the saved per-row statistic (Lecture 9 §9.6: the running max and denominator;
  CMU notes slide page 14: one normalisation constant per row) is the natural
  log-sum-exp of the scaled, masked scores, LSE_i = m_i + ln(l_i);
* the backward pass is the chain rule through softmax (not written on the
  pages): dA = dO V^T, D_i = sum_j A_ij dA_ij, dS = A * (dA - D), dQ = scale dS K,
  dK = scale dS^T Q, dV = A^T dO.

Every chunk of query rows sees complete rows of S, so no online rescaling is
used here; the identities that make tiling exact are checked against this
definition in the tests, not built into it.

Parity is pinned for every function here (see tests/test_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

CHUNK_ROWS = 512


def _visible(rows: np.ndarray, n_keys: int, causal: bool) -> np.ndarray | None:
    """Boolean [len(rows), n_keys] visibility; None means every key is visible."""
    if not causal:
        return None
    return np.arange(n_keys)[None, :] <= rows[:, None]


def _row_probs(q_rows, k, rows, causal, scale):
    """Scores of the given query rows against all keys, then the row softmax.

    Returns (A, m, l): the probabilities, the row max of the scaled masked scores
    and the row sum of exp(S - m).  Subtracting the row max is the safe softmax of
    Lecture 9 §9.4 (it keeps exp from overflowing and changes nothing exactly).
    """
    s = scale * (q_rows @ k.T)
    vis = _visible(rows, k.shape[0], causal)
    if vis is not None:
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return p / l, m[:, 0], l[:, 0]


def probabilities(q, k, causal, scale, rows=None):
    """The attention matrix A (rows of it) for one head; q, k are [N, d]."""
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    a, _, _ = _row_probs(q[rows], k, rows, causal, scale)
    return a


def forward_head(q, k, v, causal, scale, rows=None, chunk=CHUNK_ROWS):
    """O and LSE for one head (q, k, v: [N, d] float64), optionally for a subset of
    query rows.  Returns (O[rows], LSE[rows])."""
    n = q.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    o = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.size, dtype=np.float64)
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        a, m, l = _row_probs(q[r], k, r, causal, scale)
        o[c0:c0 + r.size] = a @ v
        lse[c0:c0 + r.size] = m + np.log(l)
    return o, lse


def decode_head(q, k, v, causal, scale, chunk=CHUNK_ROWS):
    """O and LSE of a short block of Nq queries against a cache of Nk >= Nq keys
    (q: [Nq, d]; k, v: [Nk, d] float64).  Returns (O [Nq, d], LSE [Nq]).

    The decode setting of Lecture 9 §9.8 (one or a few new query tokens against
    the whole key/value cache; CMU 11-868 notes, slide pages 57-60): the same
    three-step definition, with a rectangular score matrix.  Reading where the
    pages are silent: the queries are the last Nq positions of the sequence, so
    with ``causal`` query i (position Nk - Nq + i) sees keys j <= Nk - Nq + i.
    For Nq = Nk this is forward_head's mask; for Nq = 1 every key is visible.
    No split of the keys is made here: the split-K combine the pages describe is
    how a GPU reaches this result, not part of its definition.
    """
    nq, nk = q.shape[0], k.shape[0]
    if nq > nk:
        raise ValueError("decode needs Nq <= Nk")
    pos = np.arange(nq) + (nk - nq)
    o = np.empty((nq, v.shape[1]), dtype=np.float64)
    lse = np.empty(nq, dtype=np.float64)
    for c0 in range(0, nq, chunk):
        r = slice(c0, min(nq, c0 + chunk))
        a, m, l = _row_probs(q[r], k, pos[r], causal, scale)
        o[r] = a @ v
        lse[r] = m + np.log(l)
    return o, lse


def decode(q, k, v, causal, scale):
    """Batched decode over q [B, H, Nq, d] and k, v [B, Hkv, Nk, d] float64 arrays
    -> (O [B, H, Nq, d], LSE [B, H, Nq]).

    Hkv divides H.  With Hkv < H the query heads share key/value heads in groups
    of g = H / Hkv adjacent heads: query head h attends to key/value head h // g
    (grouped-query attention, named with the GQA packing of the CMU 11-868 notes'
    decoding slides, pages 57-60).  Hkv = H is ordinary multi-head attention."""
    B, H, nq, _ = q.shape
    hkv = k.shape[1]
    if H % hkv:
        raise ValueError("the key/value head count must divide the query head count")
    g = H // hkv
    o = np.empty_like(q)
    lse = np.empty((B, H, nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = decode_head(q[b, h], k[b, h // g], v[b, h // g], causal, scale)
    return o, lse


def backward_head(q, k, v, do, causal, scale, chunk=CHUNK_ROWS):
    """dQ, dK, dV (and D) of L = <dO, O> for one head, by the chain rule through
    the row softmax.  All inputs are [N, d] float64."""
    n = q.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dvec = np.empty(n, dtype=np.float64)
    for c0 in range(0, n, chunk):
        r = np.arange(c0, min(n, c0 + chunk))
        a, _, _ = _row_probs(q[r], k, r, causal, scale)
        da = do[r] @ v.T                       # dA = dO V^T
        dr = (a * da).sum(axis=1)              # D_i = sum_j A_ij dA_ij
        ds = a * (da - dr[:, None])            # softmax Jacobian applied row-wise
        dq[r] = scale * (ds @ k)
        dk += scale * (ds.T @ q[r])
        dv += a.T @ do[r]
        dvec[r] = dr
    return {"dq": dq, "dk": dk, "dv": dv, "D": dvec}


def _group(H, hkv):
    if H % hkv:
        raise ValueError("the key/value head count must divide the query head count")
    return H // hkv


def forward(q, k, v, causal, scale):
    """Batched forward over q [B, H, N, d] and k, v [B, Hkv, N, d] float64 arrays
    -> (O, LSE[B, H, N]).  Query head h reads key/value head h // (H // Hkv)
    (grouped-query attention; Hkv = H is multi-head attention)."""
    B, H, N, _ = q.shape
    g = _group(H, k.shape[1])
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h // g], v[b, h // g], causal, scale)
    return o, lse


def backward(q, k, v, do, causal, scale):
    """Batched backward over q, do [B, H, N, d] and k, v [B, Hkv, N, d] float64
    arrays -> dict(dq, dk, dv, D).  A key/value head shared by g query heads
    receives the sum of the g heads' gradients (the chain rule for a shared
    input)."""
    B, H, N, _ = q.shape
    g = _group(H, k.shape[1])
    out = {"dq": np.empty_like(q), "dk": np.zeros_like(k), "dv": np.zeros_like(v),
           "D": np.empty((B, H, N), dtype=np.float64)}
    for b in range(B):
        for h in range(H):
            gr = backward_head(q[b, h], k[b, h // g], v[b, h // g], do[b, h], causal, scale)
            out["dq"][b, h] = gr["dq"]
            out["D"][b, h] = gr["D"]
            out["dk"][b, h // g] += gr["dk"]
            out["dv"][b, h // g] += gr["dv"]
    return out


def tile_map(n, br, bc, causal):
    """Brute-force tile classes over the element visibility mask.

    A tile (i, j) covers query rows [i*br, (i+1)*br) and key columns
    [j*bc, (j+1)*bc).  An element is visible iff row < n, col < n and (not
    causal or col <= row).  Code 0: no visible element; 1: every element
    visible; 2: some but not all visible, plus 4 when the tile reaches past n in
    rows or columns.  Returns uint8 [ceil(n/br), ceil(n/bc)].
    """
    nq = -(-n // br)
    nk = -(-n // bc)
    codes = np.zeros((nq, nk), dtype=np.uint8)
    cols = np.arange(nk * bc)
    for i in range(nq):
        rows = np.arange(i * br, (i + 1) * br)
        vis = (rows[:, None] < n) & (cols[None, :] < n)
        if causal:
            vis &= cols[None, :] <= rows[:, None]
        for j in range(nk):
            blk = vis[:, j * bc:(j + 1) * bc]
            if not blk.any():
                code = 0
            elif blk.all():
                code = 1
            else:
                code = 2
                if (i + 1) * br > n or (j + 1) * bc > n:
                    code |= 4
            codes[i, j] = code
    return codes
