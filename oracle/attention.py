"""Float64 reference for softmax attention forward and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The method reaches the exact gradient of softmax attention (up to floating
point rounding order), so this file is that gradient written out from its
definition.  [summary] §1 and §2.1 fix what the backward pass produces (the
gradients, with dQ accumulated over KV tiles); the formulas below are the
textbook chain rule for

    S = scale * Q K^T            (causal: S_ij = -inf for j > i + Sk - Sq)
    P = softmax_rows(S),  LSE_i = log sum_j exp(S_ij)
    O = P V

given dO:

    dV = P^T dO
    dP = dO V^T
    Delta_i = sum_d dO_id O_id           (= sum_j P_ij dP_ij)
    dS = P * (dP - Delta[:, None])
    dQ = scale * dS K,   dK = scale * dS^T Q.

Queries and keys may differ in length (Sq query rows, Sk key rows).  The
causal mask is then aligned at the bottom right: query row i sees keys
0 .. i + Sk - Sq, so the last query row sees every key (the usual convention
for queries that continue a longer key sequence); with Sq = Sk it is the
ordinary lower triangle.

Banded (sliding-window) masks: with window = (left, right), query row i
sees keys j with -left <= j - (i + Sk - Sq) <= right; None on a side means
unbounded, so causal is window (None, 0) and the full mask (None, None).
A window with causal=True keeps its left side and takes right = 0.  Every
query row sees at least the key on its diagonal, so no row is empty when
Sk >= Sq.

Grouped-query attention: query head hq reads key/value head hq // g with
g = Hq / Hkv (contiguous groups); dK/dV of a key/value head sum over its g
query heads.  Layout is BHSD.  Rows are processed in blocks only to bound
memory; every row's softmax is independent, and the block sums of dK/dV are
plain float64 additions.  Parity status: pinned (finite differences, row
identities, closed forms, causal-vs-bias equality; see tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np


def band(causal: bool, window=None):
    """(left, right) extent of the visible keys around the diagonal, None = unbounded."""
    left, right = (None, None) if window is None else window
    if causal:
        right = 0
    return left, right


def visible(i, j, offset: int, causal: bool, window=None):
    """Boolean mask: query row(s) i see key(s) j (broadcasting)."""
    left, right = band(causal, window)
    d = j - (i + offset)  # key position relative to the query's diagonal key
    ok = np.ones(np.broadcast(i, j).shape, dtype=bool)
    if right is not None:
        ok &= d <= right
    if left is not None:
        ok &= d >= -left
    return ok


def _scores(qrows: np.ndarray, k: np.ndarray, scale: float, row0: int, causal: bool,
            bias: np.ndarray | None = None, offset: int = 0, window=None) -> np.ndarray:
    """Scores of query rows row0.. against all keys; ``offset`` = Sk - Sq."""
    s = scale * (qrows @ k.T)
    if bias is not None:
        s = s + bias
    if causal or window is not None:
        i = np.arange(row0, row0 + qrows.shape[0])[:, None]
        j = np.arange(k.shape[0])[None, :]
        s = np.where(visible(i, j, offset, causal, window), s, -np.inf)
    return s


def _softmax_rows(s: np.ndarray):
    m = s.max(axis=1)
    ell = np.exp(s - m[:, None]).sum(axis=1)
    lse = m + np.log(ell)
    p = np.exp(s - lse[:, None])
    return p, lse


def forward(q, k, v, scale: float, causal: bool, row_block: int = 1024, bias=None, window=None):
    """O [B,Hq,S,D] and LSE [B,Hq,S] (natural log) in float64.

    ``bias`` (optional, [S,S]) is an additive score bias used by the tests.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, Hq, S, D = q.shape
    g = Hq // k.shape[1]
    off = k.shape[2] - S
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, S))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // g
            for r0 in range(0, S, row_block):
                r1 = min(S, r0 + row_block)
                s = _scores(q[b, hq, r0:r1], k[b, hk], scale, r0, causal,
                            None if bias is None else bias[r0:r1], off, window)
                p, l_ = _softmax_rows(s)
                o[b, hq, r0:r1] = p @ v[b, hk]
                lse[b, hq, r0:r1] = l_
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool, row_block: int = 1024, bias=None, window=None):
    """Full gradients.  Returns dict with dq, dk, dv, o, lse, delta (float64)."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    off = k.shape[2] - S
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros_like(q)
    lse = np.zeros((B, Hq, S))
    delta = np.zeros((B, Hq, S))
    for b in range(B):
        for hq in range(Hq):
            hk = hq // g
            for r0 in range(0, S, row_block):
                r1 = min(S, r0 + row_block)
                qr, dor = q[b, hq, r0:r1], do[b, hq, r0:r1]
                s = _scores(qr, k[b, hk], scale, r0, causal,
                            None if bias is None else bias[r0:r1], off, window)
                p, l_ = _softmax_rows(s)
                orow = p @ v[b, hk]
                dlt = (dor * orow).sum(axis=1)
                dv[b, hk] += p.T @ dor
                dp = dor @ v[b, hk].T
                ds = p * (dp - dlt[:, None])
                dq[b, hq, r0:r1] = scale * (ds @ k[b, hk])
                dk[b, hk] += scale * (ds.T @ qr)
                o[b, hq, r0:r1] = orow
                lse[b, hq, r0:r1] = l_
                delta[b, hq, r0:r1] = dlt
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "delta": delta}


def head_stats(q, k, v, do, b: int, hq: int, scale: float, causal: bool, row_block: int = 1024, window=None):
    """LSE and Delta of every query row of one (batch, query head), float64.

    Needed to evaluate single rows of dK/dV, which depend on all query rows.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    g = q.shape[1] // k.shape[1]
    hk = hq // g
    S = q.shape[2]
    off = k.shape[2] - S
    lse = np.zeros(S)
    delta = np.zeros(S)
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        s = _scores(q[b, hq, r0:r1], k[b, hk], scale, r0, causal, None, off, window)
        p, l_ = _softmax_rows(s)
        lse[r0:r1] = l_
        delta[r0:r1] = (do[b, hq, r0:r1] * (p @ v[b, hk])).sum(axis=1)
    return lse, delta


def dq_rows(q, k, v, do, b: int, hq: int, rows, scale: float, causal: bool, window=None):
    """dQ[b, hq, rows, :] from the definition, one query row at a time."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    g = q.shape[1] // k.shape[1]
    hk = hq // g
    off = k.shape[2] - q.shape[2]
    out = []
    for i in rows:
        s = _scores(q[b, hq, i:i + 1], k[b, hk], scale, i, causal, None, off, window)
        p, _ = _softmax_rows(s)
        o_i = p @ v[b, hk]
        dp = do[b, hq, i:i + 1] @ v[b, hk].T
        ds = p * (dp - (do[b, hq, i] * o_i[0]).sum())
        out.append(scale * (ds @ k[b, hk])[0])
    return np.array(out)


def dkdv_rows(q, k, v, do, b: int, hk: int, cols, scale: float, causal: bool, stats=None, window=None):
    """dK[b, hk, cols, :] and dV[b, hk, cols, :] from the definition.

    ``stats`` maps each query head of the group to its (LSE, Delta) from
    ``head_stats``; computed here when not given.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    Hq, S = q.shape[1], q.shape[2]
    g = Hq // k.shape[1]
    off = k.shape[2] - S
    dk_out, dv_out = [], []
    heads = list(range(hk * g, hk * g + g))
    if stats is None:
        stats = {hq: head_stats(q, k, v, do, b, hq, scale, causal, window=window) for hq in heads}
    for j in cols:
        dkj = np.zeros(q.shape[3])
        dvj = np.zeros(q.shape[3])
        for hq in heads:
            lse, delta = stats[hq]
            i = np.arange(S)
            s = scale * (q[b, hq] @ k[b, hk, j])
            p = np.exp(s - lse)
            if causal or window is not None:
                p = np.where(visible(i, j, off, causal, window), p, 0.0)
            dp = do[b, hq] @ v[b, hk, j]
            ds = p * (dp - delta)
            dvj += p @ do[b, hq]
            dkj += scale * (ds @ q[b, hq])
        dk_out.append(dkj)
        dv_out.append(dvj)
    return np.array(dk_out), np.array(dv_out)


def head_matrices(q_head, k_head, v_head, do_head, scale: float, causal: bool, window=None):
    """P, dP and dS of one head, float64 ([Sq, Sk] each); used by the row-identity tests."""
    q_head, k_head, v_head, do_head = (np.asarray(x, dtype=np.float64) for x in (q_head, k_head, v_head, do_head))
    s = _scores(q_head, k_head, scale, 0, causal, None, k_head.shape[0] - q_head.shape[0], window)
    p, _ = _softmax_rows(s)
    o = p @ v_head
    dp = do_head @ v_head.T
    ds = p * (dp - (do_head * o).sum(axis=1)[:, None])
    return p, dp, ds
