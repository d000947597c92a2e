"""Plain float64 definition of exact attention, forward and backward.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.

What it computes, and where the pages fix it
--------------------------------------------
* The method is *exact* attention: the tiled, IO-aware algorithm returns the
  same output as the standard softmax(Q K^T) V, with no approximation
  ("[Paper Review] FlashAttention-2 ...", nubint.ai, Abstract and "Proposed
  method"; "Researchers at Stanford University Propose FlashAttention ...",
  the paragraph introducing FlashAttention). So the oracle is that standard
  definition written out: S = (Q K^T) * scale, masked entries -inf, row
  softmax, O = P V.
* The forward keeps one per-row softmax normalisation statistic for the
  backward (Stanford FlashAttention summary, paragraph on the two techniques).
  Reading taken: the natural-log logsumexp of the scaled, masked score row,
  lse_i = m_i + ln(sum_j exp(S_ij - m_i)).
* Causal masking (FlashAttention-2 review, "Proposed method"): one sequence
  length N for queries and keys, key j visible from query i iff j <= i.
* Block-sparse attention (Stanford FlashAttention summary, paragraph on
  block-sparse FlashAttention): a per-head block mask over (query block,
  key block); an element is visible iff its block is kept (and, with causal,
  also j <= i). Block size 128 unless a test says otherwise.
* Backward: the pages print no formula; the oracle uses the textbook
  gradient of O = softmax(S) V with upstream dO:
  dV = P^T dO, dP = dO V^T, D_i = sum_k dO_ik O_ik, dS = P o (dP - D),
  dQ = scale * dS K, dK = scale * dS^T Q. lse is not differentiated.
* A fully masked row has O = 0, lse = -inf and zero gradient (reading: the
  pages are silent; the empty sum has no softmax).

Evaluation in pieces: rows of S are independent, so ``head_forward`` may be
called on any subset of query rows and gives the definition's value for
those rows; ``head_grad_cols`` evaluates whole key columns of the gradient.
Neither reorders any sum.

Every function here is pinned in ``tests/test_oracle.py`` against something
other than itself (brute-force loops, closed forms, invariants, finite
differences).
"""
from __future__ import annotations

import math
import struct

import numpy as np

__all__ = [
    "widen_bf16",
    "keep_matrix",
    "head_forward",
    "head_backward",
    "head_grad_rows",
    "head_grad_cols",
    "attn_fwd_ref",
    "attn_bwd_ref",
    "online_softmax_ref",
    "naive_bruteforce",
    "naive_bruteforce_bits",
]


def widen_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (bf16 is the top half
    of an IEEE binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _scale64(scale) -> float:
    """The score scale as the library receives it (an fp32), widened."""
    return float(np.float64(np.float32(scale)))


def keep_matrix(rows, cols, causal: bool, mask_h=None, mask_block: int = 128) -> np.ndarray:
    """Boolean visibility of (query row, key col) pairs for one head.

    rows, cols: integer index arrays. mask_h: [nb, nb] block mask of this
    head (nonzero = keep) or None.
    """
    r = np.asarray(rows, dtype=np.int64)[:, None]
    c = np.asarray(cols, dtype=np.int64)[None, :]
    keep = np.ones((r.shape[0], c.shape[1]), dtype=bool)
    if causal:
        keep &= c <= r
    if mask_h is not None:
        keep &= np.asarray(mask_h)[r // mask_block, c // mask_block] != 0
    return keep


def head_forward(Q, K, V, causal, scale, mask_h=None, mask_block=128, rows=None):
    """Standard attention for one head, on the query rows ``rows``.

    Q, K, V: float64 [N, d]. Returns (O [R, d], lse [R]) for R selected rows.
    """
    N = K.shape[0]
    s = _scale64(scale)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    S = (Q[rows] @ K.T) * s
    keep = keep_matrix(rows, np.arange(N), causal, mask_h, mask_block)
    S = np.where(keep, S, -np.inf)
    m = S.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    E = np.where(keep, np.exp(S - m_safe[:, None]), 0.0)
    ell = E.sum(axis=1)
    ell_safe = np.where(empty, 1.0, ell)
    P = E / ell_safe[:, None]
    O = P @ V
    lse = np.where(empty, -np.inf, m_safe + np.log(ell_safe))
    return O, lse


def _probs_from_lse(S, keep, lse):
    """P = exp(S - lse) on visible entries, 0 elsewhere (and on empty rows)."""
    lse_safe = np.where(np.isfinite(lse), lse, 0.0)
    P = np.exp(np.where(keep, S, -np.inf) - lse_safe[:, None])
    return np.where(keep & np.isfinite(lse)[:, None], P, 0.0)


def head_backward(Q, K, V, dO, causal, scale, mask_h=None, mask_block=128):
    """Full forward + analytic backward for one head with all N x N entries.

    Returns dict with O, lse, D, dQ, dK, dV (float64). For small N.
    """
    N = Q.shape[0]
    s = _scale64(scale)
    O, lse = head_forward(Q, K, V, causal, scale, mask_h, mask_block)
    keep = keep_matrix(np.arange(N), np.arange(N), causal, mask_h, mask_block)
    S = (Q @ K.T) * s
    P = _probs_from_lse(S, keep, lse)
    D = np.sum(dO * O, axis=1)
    dV = P.T @ dO
    dP = dO @ V.T
    dS = P * (dP - D[:, None])
    dQ = s * (dS @ K)
    dK = s * (dS.T @ Q)
    return {"O": O, "lse": lse, "D": D, "dQ": dQ, "dK": dK, "dV": dV}


def head_grad_rows(Q, K, V, dO, causal, scale, rows, mask_h=None, mask_block=128):
    """dQ (and O, lse, D) for the selected query rows of one head.

    Row i of dQ needs only row i of P and dP, and D_i = dO_i . O_i.
    """
    N = K.shape[0]
    s = _scale64(scale)
    rows = np.asarray(rows, dtype=np.int64)
    O, lse = head_forward(Q, K, V, causal, scale, mask_h, mask_block, rows=rows)
    keep = keep_matrix(rows, np.arange(N), causal, mask_h, mask_block)
    S = (Q[rows] @ K.T) * s
    P = _probs_from_lse(S, keep, lse)
    D = np.sum(dO[rows] * O, axis=1)
    dP = dO[rows] @ V.T
    dS = P * (dP - D[:, None])
    dQ = s * (dS @ K)
    return {"O": O, "lse": lse, "D": D, "dQ": dQ}


def head_grad_cols(Q, K, V, dO, causal, scale, cols, mask_h=None, mask_block=128,
                   row_chunk=1024, lse=None, D=None):
    """dK, dV for the selected key columns of one head.

    Column j of dK/dV sums over every query row, so this needs lse_i and
    D_i for all rows; they are computed row by row (rows independent) unless
    given.
    """
    N = Q.shape[0]
    s = _scale64(scale)
    cols = np.asarray(cols, dtype=np.int64)
    if lse is None or D is None:
        lse = np.empty(N)
        D = np.empty(N)
        for r0 in range(0, N, row_chunk):
            rr = np.arange(r0, min(N, r0 + row_chunk))
            O_r, lse_r = head_forward(Q, K, V, causal, scale, mask_h, mask_block, rows=rr)
            lse[rr] = lse_r
            D[rr] = np.sum(dO[rr] * O_r, axis=1)
    keep = keep_matrix(np.arange(N), cols, causal, mask_h, mask_block)
    S = (Q @ K[cols].T) * s
    P = _probs_from_lse(S, keep, lse)
    dV = P.T @ dO
    dP = dO @ V[cols].T
    dS = P * (dP - D[:, None])
    dK = s * (dS.T @ Q)
    return {"dK": dK, "dV": dV, "lse": lse, "D": D}


def _heads(x):
    return widen_bf16(x)


def attn_fwd_ref(q, k, v, causal, scale, block_mask=None, mask_block=128, row_chunk=1024):
    """Forward over [B, H, N, d] bf16 bits: returns (O, lse) float64."""
    q, k, v = _heads(q), _heads(k), _heads(v)
    B, H, N, d = q.shape
    O = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            mh = None if block_mask is None else block_mask[h]
            for r0 in range(0, N, row_chunk):
                rr = np.arange(r0, min(N, r0 + row_chunk))
                O[b, h, rr], lse[b, h, rr] = head_forward(
                    q[b, h], k[b, h], v[b, h], causal, scale, mh, mask_block, rows=rr)
    return O, lse


def attn_bwd_ref(q, k, v, do, causal, scale, block_mask=None, mask_block=128):
    """Full backward over [B, H, N, d] bf16 bits (small N): dict of float64."""
    q, k, v, do = _heads(q), _heads(k), _heads(v), _heads(do)
    B, H, N, d = q.shape
    out = {name: np.empty((B, H, N, d)) for name in ("O", "dQ", "dK", "dV")}
    out["lse"] = np.empty((B, H, N))
    out["D"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            mh = None if block_mask is None else block_mask[h]
            r = head_backward(q[b, h], k[b, h], v[b, h], do[b, h], causal, scale, mh, mask_block)
            for name in out:
                out[name][b, h] = r[name]
    return out


def online_softmax_ref(Q, K, V, causal, scale, kv_block, mask_h=None, mask_block=128):
    """The method's incremental softmax over key blocks, one head, float64.

    Follows the pages' description of the forward (FlashAttention-2 review,
    "Proposed method": block-wise softmax with correct final outputs;
    Stanford FlashAttention summary: the softmax reduction done
    incrementally over blocks of the input). Per query row keep a running
    max m, running sum l and unnormalised accumulator acc; for each key
    block: m' = max(m, block max), l = l*exp(m-m') + sum exp(S-m'),
    acc = acc*exp(m-m') + exp(S-m') V_block; at the end O = acc / l and
    lse = m + ln l. ``kv_block`` need not divide N.
    """
    N, d = Q.shape
    s = _scale64(scale)
    m = np.full(N, -np.inf)
    ell = np.zeros(N)
    acc = np.zeros((N, d))
    for c0 in range(0, K.shape[0], kv_block):
        cols = np.arange(c0, min(K.shape[0], c0 + kv_block))
        keep = keep_matrix(np.arange(N), cols, causal, mask_h, mask_block)
        S = np.where(keep, (Q @ K[cols].T) * s, -np.inf)
        m_new = np.maximum(m, S.max(axis=1))
        fin = np.isfinite(m_new)
        m_ref = np.where(fin, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - m_ref), 0.0)
        E = np.where(keep, np.exp(S - m_ref[:, None]), 0.0)
        ell = ell * alpha + E.sum(axis=1)
        acc = acc * alpha[:, None] + E @ V[cols]
        m = m_new
    empty = ell == 0.0
    O = np.where(empty[:, None], 0.0, acc / np.where(empty, 1.0, ell)[:, None])
    lse = np.where(empty, -np.inf, np.where(np.isfinite(m), m, 0.0) + np.log(np.where(empty, 1.0, ell)))
    return O, lse


def naive_bruteforce(Q, K, V, causal, scale, visible=None):
    """Scalar-loop attention for tiny inputs: lists of floats in, lists out.

    ``visible(i, j)`` -> bool adds a mask on top of causal. Uses math.exp and
    sums in plain Python; no numpy, so it shares nothing with head_forward.
    """
    N = len(Q)
    d = len(Q[0])
    s = float(np.float64(np.float32(scale)))
    O, lse = [], []
    for i in range(N):
        scores = []
        for j in range(len(K)):
            ok = (not causal or j <= i) and (visible is None or visible(i, j))
            if ok:
                dot = 0.0
                for t in range(d):
                    dot += Q[i][t] * K[j][t]
                scores.append((j, dot * s))
        if not scores:
            O.append([0.0] * len(V[0]))
            lse.append(-math.inf)
            continue
        mx = max(val for _, val in scores)
        w = [(j, math.exp(val - mx)) for j, val in scores]
        tot = sum(x for _, x in w)
        row = [0.0] * len(V[0])
        for j, x in w:
            for t in range(len(V[0])):
                row[t] += x / tot * V[j][t]
        O.append(row)
        lse.append(mx + math.log(tot))
    return O, lse


def naive_bruteforce_bits(qb, kb, vb, causal, scale, visible=None):
    """naive_bruteforce on bf16 bit patterns, widened with ``struct`` (a
    second, independent widening)."""
    def w(bits):
        return [[struct.unpack(">f", struct.pack(">I", int(x) << 16))[0] for x in row] for row in bits]
    return naive_bruteforce(w(qb), w(kb), w(vb), causal, scale, visible)
