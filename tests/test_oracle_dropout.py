"""Pins of the dropout oracle (CPU): the generator against its published
known-answer vectors and a scalar re-implementation, the keep mask against
per-element brute force and its expected rate, and the dropout gradients
against finite differences and the identities they must satisfy."""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dropout as od
from synth import make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                v = [int(x, 16) for x in line.split()]
                rows.append((v[:4], v[4:6], v[6:]))
    return rows


@pytest.mark.parametrize("ctr,key,out", _kat())
def test_philox_known_answers(ctr, key, out):
    assert od.philox4x32_10_scalar(ctr, key) == out
    vec = od.philox4x32_10(*[np.uint64(x) for x in ctr], *[np.uint64(x) for x in key])
    assert [int(x) for x in vec] == out


def test_philox_vectorised_matches_scalar():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(4, 64), dtype=np.uint64)
    k = rng.integers(0, 2**32, size=(2,), dtype=np.uint64)
    vec = od.philox4x32_10(c[0], c[1], c[2], c[3], k[0], k[1])
    for n in range(64):
        assert [int(w[n]) for w in vec] == od.philox4x32_10_scalar([c[i, n] for i in range(4)], k)


def test_philox_output_is_uniform():
    """Bytes of 4096 outputs: a chi-square test at a loose level (a wrong
    round, e.g. a dropped xor, leaves visible structure for a zero key)."""
    i = np.arange(4096, dtype=np.uint64)
    words = np.concatenate(od.philox4x32_10(i, 0, 0, 0, 0, 0))
    byts = np.concatenate([(words >> np.uint64(8 * s)) & np.uint64(255) for s in range(4)]).astype(np.int64)
    counts = np.bincount(byts, minlength=256)
    exp = byts.size / 256
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 400  # 255 degrees of freedom: mean 255, sd 22.6


def test_keep_mask_matches_per_element_brute_force():
    B, H, N, p, seed, off = 1, 2, 9, 0.3, 0x1234_5678_9ABC, 7
    Z = od.dropout_keep(B, H, N, p, seed, off)
    T = od.dropout_threshold(p)
    for h in range(H):
        for i in range(N):
            for j in range(N):
                w = od.philox4x32_10_scalar([j // 4, i, h, off], [seed & 0xFFFFFFFF, seed >> 32])[j % 4]
                assert Z[0, h, i, j] == (w >= T)


def test_threshold_definition():
    assert od.dropout_threshold(0.0) == 0
    assert od.dropout_threshold(0.5) == 2**31
    assert od.dropout_threshold(0.25) == 2**30
    assert od.dropout_threshold(np.nextafter(np.float32(1), np.float32(0))) == 2**32 - 2**8
    with pytest.raises(ValueError):
        od.dropout_threshold(1.0)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_keep_rate(p):
    Z = od.dropout_keep(1, 2, 256, p, 42, 0)
    n = Z.size
    assert abs(Z.mean() - (1 - p)) < 5 * math.sqrt(p * (1 - p) / n)


def test_zero_dropout_is_plain_attention():
    inp = make_inputs(3, 1, 2, 37, 8)
    ref = oracle.attn_bwd_ref(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.35)
    got = od.attn_bwd_dropout_ref(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.35, 0.0, 9, 0)
    for name in ("O", "lse", "D", "dQ", "dK", "dV"):
        np.testing.assert_allclose(got[name], ref[name], rtol=1e-13, atol=1e-13)


def test_expectation_over_masks_is_plain_attention():
    """E_Z[O] = O without dropout: pins the 1/(1-p) scale and that dropout
    acts on normalised probabilities (not on exponentials before the sum)."""
    inp = make_inputs(4, 1, 1, 12, 4)
    O_ref, _ = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], False, 0.5)
    acc = np.zeros_like(O_ref)
    n = 3000
    for s in range(n):
        O, lse = od.attn_fwd_dropout_ref(inp["q"], inp["k"], inp["v"], False, 0.5, 0.4, s, 0)
        acc += O
    err = np.abs(acc / n - O_ref).max()
    assert err < 0.05 * np.abs(O_ref).max() + 0.02


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_gradients_match_finite_differences(causal):
    """Central differences of L = <O, dO> with the keep mask held fixed."""
    rng = np.random.default_rng(8)
    N, d, p, scale = 7, 4, 0.35, 0.6
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    Z = od.dropout_keep_head(0, np.arange(N), np.arange(N), p, 11, 3)
    g = od.head_backward_dropout(Q, K, V, dO, causal, scale, Z, p)

    def loss(Q_, K_, V_):
        O, _ = od.head_forward_dropout(Q_, K_, V_, causal, scale, Z, p)
        return float((O * dO).sum())

    h = 1e-6
    for name, X in (("dQ", Q), ("dK", K), ("dV", V)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Xp if X is Y else Y for Y in (Q, K, V)]
            args_m = [Xm if X is Y else Y for Y in (Q, K, V)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - g[name]).max() <= 1e-7 * max(1.0, np.abs(num).max()), name


def test_dropout_backward_identities():
    inp = make_inputs(6, 1, 2, 40, 8)
    r = od.attn_bwd_dropout_ref(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.3, 0.25, 77, 1)
    # sum over keys of dK vanishes (rows of dS sum to zero)
    assert np.abs(r["dK"].sum(axis=2)).max() < 1e-10 * max(1.0, np.abs(r["dK"]).max())
    # D = rowsum(P o dP) with the dropout-aware dP
    q, k, v, do = (oracle.widen_bf16(inp[x]) for x in ("q", "k", "v", "do"))
    for h in range(2):
        N = q.shape[2]
        Z = od.dropout_keep_head(h, np.arange(N), np.arange(N), 0.25, 77, 1)
        keep = oracle.keep_matrix(np.arange(N), np.arange(N), True)
        S = (q[0, h] @ k[0, h].T) * float(np.float32(0.3))
        P = np.where(keep, np.exp(np.where(keep, S, -np.inf) - r["lse"][0, h][:, None]), 0.0)
        dP = np.where(Z, do[0, h] @ v[0, h].T, 0.0) / 0.75
        np.testing.assert_allclose((P * dP).sum(axis=1), r["D"][0, h], rtol=1e-10, atol=1e-12)


def test_planted_missing_scale_is_caught():
    """A mutant that forgets 1/(1-p) on dV fails the finite-difference pin."""
    rng = np.random.default_rng(9)
    N, d, p = 6, 3, 0.5
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    Z = od.dropout_keep_head(0, np.arange(N), np.arange(N), p, 1, 0)
    g = od.head_backward_dropout(Q, K, V, dO, False, 1.0, Z, p)
    mutant_dV = g["dV"] * (1 - p)

    def loss(V_):
        O, _ = od.head_forward_dropout(Q, K, V_, False, 1.0, Z, p)
        return float((O * dO).sum())

    h = 1e-6
    num = np.zeros_like(V)
    for idx in np.ndindex(V.shape):
        Vp, Vm = V.copy(), V.copy()
        Vp[idx] += h
        Vm[idx] -= h
        num[idx] = (loss(Vp) - loss(Vm)) / (2 * h)
    assert np.abs(num - g["dV"]).max() < 1e-7
    assert np.abs(num - mutant_dV).max() > 1e-2


@pytest.mark.parametrize("causal", [False, True])
def test_row_and_column_pieces_match_full_backward(causal):
    """The sampled-row and sampled-column dropout evaluations equal the full
    backward on the same inputs (rows of dQ and columns of dK, dV are
    independent pieces of the same definition)."""
    rng = np.random.default_rng(12)
    N, d, p, scale, seed, off, bh = 70, 8, 0.3, 0.4, 99, 2, 5
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    Z = od.dropout_keep_head(bh, np.arange(N), np.arange(N), p, seed, off)
    full = od.head_backward_dropout(Q, K, V, dO, causal, scale, Z, p)
    rows = np.array([0, 1, 31, 32, 63, 69])
    r = od.head_grad_rows_dropout(Q, K, V, dO, causal, scale, p, bh, seed, off, rows)
    for name in ("O", "lse", "D", "dQ"):
        np.testing.assert_allclose(r[name], full[name][rows], rtol=1e-12, atol=1e-12)
    cols = np.array([0, 3, 4, 64, 69])
    c = od.head_grad_cols_dropout(Q, K, V, dO, causal, scale, p, bh, seed, off, cols, row_chunk=16)
    for name in ("dK", "dV"):
        np.testing.assert_allclose(c[name], full[name][cols], rtol=1e-12, atol=1e-12)
