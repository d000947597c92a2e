"""Attention dropout in float64: a counter-based keep mask and the dropout
forward and backward -- TEST INFRASTRUCTURE, with the same import rules as
the rest of ``oracle/`` (only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may use it).

The pages name dropout among attention's O(N^2) elementwise operations and
give it no semantics ("PagedAttention" page, paragraph on bandwidth-bound
operations). Readings taken here, used identically by the GPU library:

* Dropout acts on the normalised probabilities before they multiply V:
  O = (P o Z) V / (1 - p), with Z_ij in {0, 1}. The saved statistic lse is
  that of the undropped row (the softmax is unchanged).
* Z is drawn with Philox4x32-10, the counter-based generator of Salmon,
  Moraes, Dror and Shaw ("Parallel random numbers: as easy as 1, 2, 3",
  SC 2011), because a fused kernel must be able to regenerate any element
  without storing the mask. One call covers four consecutive keys of one
  query row: counter (j // 4, i, b*H + h, offset), key (seed mod 2^32,
  seed div 2^32); output word j % 4 decides key j. Key j of row i is dropped
  iff that word is < T = floor(p * 2^32), with p the fp32 the library
  receives (T capped at 2^32 - 1).
* Backward: the gradient of O = (P o Z) V / (1 - p) with Z held fixed:
  dV = (P o Z)^T dO / (1 - p), dP = (dO V^T) o Z / (1 - p),
  D_i = sum_k dO_ik O_ik (which still equals sum_j P_ij dP_ij),
  dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
"""
import math

import numpy as np

from .attention import _probs_from_lse, _scale64, head_forward, keep_matrix, widen_bf16

# Philox4x32 constants (Salmon et al. 2011): the two round multipliers and
# the two Weyl increments of the key schedule.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on uint32 values held in uint64 arrays.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as full 64-bit
    products; the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).
    The key gains the Weyl increments (W0, W1) between rounds. Returns the
    four output words.
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    for rnd in range(10):
        p0 = np.uint64(PHILOX_M0) * c0  # < 2^64: both factors < 2^32
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if rnd < 9:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return c0, c1, c2, c3


def philox4x32_10_scalar(ctr, key):
    """The same generator on Python integers, one call (for pinning the
    vectorised version)."""
    c = [int(x) & 0xFFFFFFFF for x in ctr]
    k = [int(x) & 0xFFFFFFFF for x in key]
    for rnd in range(10):
        p0 = PHILOX_M0 * c[0]
        p1 = PHILOX_M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & 0xFFFFFFFF, (p0 >> 32) ^ c[3] ^ k[1], p0 & 0xFFFFFFFF]
        if rnd < 9:
            k = [(k[0] + PHILOX_W0) & 0xFFFFFFFF, (k[1] + PHILOX_W1) & 0xFFFFFFFF]
    return c


def dropout_threshold(p) -> int:
    """T = floor(p * 2^32) for the fp32 value of p, capped at 2^32 - 1."""
    p64 = float(np.float64(np.float32(p)))
    if not (0.0 <= p64 < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(math.floor(p64 * 4294967296.0)), 0xFFFFFFFF)


def dropout_keep_head(bh, rows, cols, p, seed, offset) -> np.ndarray:
    """Keep mask Z (bool) of head index bh = b*H + h for query rows x key
    cols."""
    rows = np.asarray(rows, dtype=np.uint64)[:, None]
    cols = np.asarray(cols, dtype=np.uint64)[None, :]
    seed = int(seed)
    words = philox4x32_10(cols >> np.uint64(2), rows, np.uint64(bh), np.uint64(int(offset) & 0xFFFFFFFF),
                          np.uint64(seed & 0xFFFFFFFF), np.uint64((seed >> 32) & 0xFFFFFFFF))
    sel = (cols & np.uint64(3)) + np.zeros_like(rows)
    w = np.choose(sel.astype(np.int64), [np.broadcast_to(x, sel.shape) for x in words])
    return w >= np.uint64(dropout_threshold(p))


def dropout_keep(B, H, N, p, seed, offset) -> np.ndarray:
    """Keep mask [B, H, N, N] (bool)."""
    out = np.empty((B, H, N, N), dtype=bool)
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            out[b, h] = dropout_keep_head(b * H + h, idx, idx, p, seed, offset)
    return out


def head_forward_dropout(Q, K, V, causal, scale, Z, p, mask_h=None, mask_block=128, rows=None):
    """(O, lse) of one head with dropout mask Z (rows x N, bool) on the
    probabilities; lse is the undropped one."""
    N = K.shape[0]
    s = _scale64(scale)
    rows = np.arange(Q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    _, lse = head_forward(Q, K, V, causal, scale, mask_h, mask_block, rows=rows)
    keep = keep_matrix(rows, np.arange(N), causal, mask_h, mask_block)
    P = _probs_from_lse((Q[rows] @ K.T) * s, keep, lse)
    keep_p = 1.0 - float(np.float64(np.float32(p)))
    O = (np.where(Z, P, 0.0) @ V) / keep_p
    return O, lse


def head_backward_dropout(Q, K, V, dO, causal, scale, Z, p, mask_h=None, mask_block=128):
    """Forward and analytic backward of one head with dropout mask Z (N x N)."""
    N = Q.shape[0]
    s = _scale64(scale)
    keep_p = 1.0 - float(np.float64(np.float32(p)))
    O, lse = head_forward_dropout(Q, K, V, causal, scale, Z, p, mask_h, mask_block)
    keep = keep_matrix(np.arange(N), np.arange(N), causal, mask_h, mask_block)
    P = _probs_from_lse((Q @ K.T) * s, keep, lse)
    Pd = np.where(Z, P, 0.0) / keep_p
    D = np.sum(dO * O, axis=1)
    dV = Pd.T @ dO
    dP = np.where(Z, dO @ V.T, 0.0) / keep_p
    dS = P * (dP - D[:, None])
    return {"O": O, "lse": lse, "D": D, "dQ": s * (dS @ K), "dK": s * (dS.T @ Q), "dV": dV}


def head_grad_rows_dropout(Q, K, V, dO, causal, scale, p, bh, seed, offset, rows, mask_h=None, mask_block=128):
    """O, lse, D and dQ of the selected query rows of head index bh with
    dropout (row i of dQ needs only row i of P, Z and dP)."""
    N = K.shape[0]
    s = _scale64(scale)
    keep_p = 1.0 - float(np.float64(np.float32(p)))
    rows = np.asarray(rows, dtype=np.int64)
    Z = dropout_keep_head(bh, rows, np.arange(N), p, seed, offset)
    O, lse = head_forward_dropout(Q, K, V, causal, scale, Z, p, mask_h, mask_block, rows=rows)
    keep = keep_matrix(rows, np.arange(N), causal, mask_h, mask_block)
    P = _probs_from_lse((Q[rows] @ K.T) * s, keep, lse)
    D = np.sum(dO[rows] * O, axis=1)
    dP = np.where(Z, dO[rows] @ V.T, 0.0) / keep_p
    dS = P * (dP - D[:, None])
    return {"O": O, "lse": lse, "D": D, "dQ": s * (dS @ K)}


def head_grad_cols_dropout(Q, K, V, dO, causal, scale, p, bh, seed, offset, cols, mask_h=None, mask_block=128,
                           row_chunk=1024):
    """dK, dV of the selected key columns of head index bh with dropout;
    lse and D of every row are recomputed row chunk by row chunk."""
    N = Q.shape[0]
    s = _scale64(scale)
    keep_p = 1.0 - float(np.float64(np.float32(p)))
    cols = np.asarray(cols, dtype=np.int64)
    lse = np.empty(N)
    D = np.empty(N)
    for r0 in range(0, N, row_chunk):
        rr = np.arange(r0, min(N, r0 + row_chunk))
        Zr = dropout_keep_head(bh, rr, np.arange(N), p, seed, offset)
        O_r, lse_r = head_forward_dropout(Q, K, V, causal, scale, Zr, p, mask_h, mask_block, rows=rr)
        lse[rr] = lse_r
        D[rr] = np.sum(dO[rr] * O_r, axis=1)
    Z = dropout_keep_head(bh, np.arange(N), cols, p, seed, offset)
    keep = keep_matrix(np.arange(N), cols, causal, mask_h, mask_block)
    P = _probs_from_lse((Q @ K[cols].T) * s, keep, lse)
    dV = (np.where(Z, P, 0.0) / keep_p).T @ dO
    dP = np.where(Z, dO @ V[cols].T, 0.0) / keep_p
    dS = P * (dP - D[:, None])
    return {"dK": s * (dS.T @ Q), "dV": dV, "lse": lse, "D": D}


def attn_fwd_dropout_ref(q, k, v, causal, scale, p, seed, offset, block_mask=None, mask_block=128):
    """Dropout forward over [B, H, N, d] bf16 bits: (O, lse) float64."""
    q, k, v = widen_bf16(q), widen_bf16(k), widen_bf16(v)
    B, H, N, d = q.shape
    O = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            Z = dropout_keep_head(b * H + h, idx, idx, p, seed, offset)
            mh = None if block_mask is None else block_mask[h]
            O[b, h], lse[b, h] = head_forward_dropout(q[b, h], k[b, h], v[b, h], causal, scale, Z, p, mh, mask_block)
    return O, lse


def attn_bwd_dropout_ref(q, k, v, do, causal, scale, p, seed, offset, block_mask=None, mask_block=128):
    """Dropout backward over [B, H, N, d] bf16 bits (small N): dict of float64."""
    q, k, v, do = widen_bf16(q), widen_bf16(k), widen_bf16(v), widen_bf16(do)
    B, H, N, d = q.shape
    out = {name: np.empty((B, H, N, d)) for name in ("O", "dQ", "dK", "dV")}
    out["lse"] = np.empty((B, H, N))
    out["D"] = np.empty((B, H, N))
    idx = np.arange(N)
    for b in range(B):
        for h in range(H):
            Z = dropout_keep_head(b * H + h, idx, idx, p, seed, offset)
            mh = None if block_mask is None else block_mask[h]
            r = head_backward_dropout(q[b, h], k[b, h], v[b, h], do[b, h], causal, scale, Z, p, mh, mask_block)
            for name in out:
                out[name][b, h] = r[name]
    return out
