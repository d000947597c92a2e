"""Pins for the CPU oracle (CPU only).

Each test checks the oracle against something other than itself: scalar
brute force, the incremental-softmax recombination the pages describe,
closed forms, invariants of softmax attention, and central finite
differences for the gradient. A plausible mistake in the oracle (dropped
scale, wrong log base, transposed operand, wrong mask index, sign error in
dS, missing D) fails at least one of them; ``test_planted_mistakes`` checks
exactly that on mutated copies of the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_block_mask, make_inputs, draw_bf16


def _rand_bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


# ---------------------------------------------------------------- bf16 plumbing

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    # include exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 2**31, 1000, dtype=np.int64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x)]
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_widen_matches_torch_and_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x7F7F], dtype=np.uint16)
    w = oracle.widen_bf16(bits)
    assert w[0] == 1.0 and w[1] == -2.0 and w[2] == 0.0 and w[3] == 0.0
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(w, ref)
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), w)


def test_chunked_draw_equals_whole_draw():
    a = draw_bf16(np.random.default_rng(3), (2, 3, 50, 8), chunk_rows=7)
    rng = np.random.default_rng(3)
    b = f32_to_bf16_bits(rng.standard_normal((2, 3, 50, 8)).astype(np.float32))
    assert np.array_equal(a, b)


def test_block_mask_recipe():
    m = make_block_mask(np.random.default_rng(0), 16, 8192)
    assert m.shape == (16, 64, 64) and m.dtype == np.uint8
    assert np.all(m[:, np.arange(64), np.arange(64)] == 1)
    off = m[:, ~np.eye(64, dtype=bool)]
    assert abs(off.mean() - 0.25) < 0.01


# ---------------------------------------------------------------- forward pins

TINY = [(1, 1), (2, 4), (3, 8), (5, 4), (17, 8), (9, 1)]


def _tiny_mask(rng, N, blk, p=0.5, empty_row=False):
    nb = (N + blk - 1) // blk
    m = (rng.random((nb, nb)) < p).astype(np.uint8)
    if empty_row and nb > 1:
        m[nb - 1, :] = 0
    return m


@pytest.mark.parametrize("N,d", TINY)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_forward_equals_bruteforce(N, d, causal, masked):
    rng = np.random.default_rng(100 + N * 10 + d)
    qb, kb, vb = (_rand_bits(rng, (N, d)) for _ in range(3))
    scale = 1.0 / math.sqrt(d) if d > 1 else 0.7
    mask = _tiny_mask(rng, N, 2, empty_row=True) if masked else None
    vis = None if mask is None else (lambda i, j: mask[i // 2, j // 2] != 0)
    O_n, lse_n = oracle.naive_bruteforce_bits(qb, kb, vb, causal, scale, vis)
    Q, K, V = (oracle.widen_bf16(x) for x in (qb, kb, vb))
    O, lse = oracle.head_forward(Q, K, V, causal, scale, mask, 2)
    assert np.allclose(O, np.array(O_n), rtol=0, atol=1e-12)
    fin = np.isfinite(np.array(lse_n))
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.allclose(lse[fin], np.array(lse_n)[fin], rtol=0, atol=1e-12)
    assert not np.any(np.isnan(O))


@pytest.mark.parametrize("N,d", [(17, 8), (33, 4), (64, 16), (5, 4)])
@pytest.mark.parametrize("kv_block", [1, 2, 3, 7, 16, 100])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recombination_is_exact(N, d, kv_block, causal):
    rng = np.random.default_rng(7 * N + kv_block)
    Q, K, V = (oracle.widen_bf16(_rand_bits(rng, (N, d))) * 2.0 for _ in range(3))
    mask = _tiny_mask(rng, N, 4, p=0.6, empty_row=True)
    for mh in (None, mask):
        O, lse = oracle.head_forward(Q, K, V, causal, 0.5, mh, 4)
        O2, lse2 = oracle.online_softmax_ref(Q, K, V, causal, 0.5, kv_block, mh, 4)
        assert np.allclose(O, O2, rtol=0, atol=1e-12)
        assert np.array_equal(np.isfinite(lse), np.isfinite(lse2))
        f = np.isfinite(lse)
        assert np.allclose(lse[f], lse2[f], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    rng = np.random.default_rng(11)
    N, d = 40, 8
    Q, K = (oracle.widen_bf16(_rand_bits(rng, (N, d))) * 3 for _ in range(2))
    mask = _tiny_mask(rng, N, 8, p=0.5, empty_row=True)
    V = np.ones((N, 1))
    O, lse = oracle.head_forward(Q, K, V, causal, 0.3, mask, 8)
    nonempty = np.isfinite(lse)
    assert np.all(np.abs(O[nonempty, 0] - 1.0) < 1e-14)
    assert np.all(O[~nonempty] == 0.0)


def test_single_key_closed_form():
    # N = 1: the only key gets weight 1, so O = V and lse = s * q.k
    rng = np.random.default_rng(5)
    q, k, v = (oracle.widen_bf16(_rand_bits(rng, (1, 64))) for _ in range(3))
    s = 0.125
    O, lse = oracle.head_forward(q, k, v, False, s, None)
    assert np.allclose(O, v, atol=1e-15)
    assert abs(lse[0] - s * float(q[0] @ k[0])) < 1e-12


def test_two_key_closed_form():
    # one query, two keys; exact numbers chosen representable in bf16
    q = np.array([[1.5, -0.5]])
    k = np.array([[1.0, 2.0], [-0.25, 0.75]])
    v = np.array([[3.0, -1.0], [0.5, 4.0]])
    s = 0.5
    a, b = s * (1.5 * 1.0 - 0.5 * 2.0), s * (1.5 * -0.25 - 0.5 * 0.75)
    wa, wb = math.exp(a), math.exp(b)
    want_o = [(wa * 3.0 + wb * 0.5) / (wa + wb), (wa * -1.0 + wb * 4.0) / (wa + wb)]
    want_lse = math.log(wa + wb)
    O, lse = oracle.head_forward(q, k, v, False, s, None)
    assert np.allclose(O[0], want_o, atol=1e-14)
    assert abs(lse[0] - want_lse) < 1e-14
    # causal: query 0 sees only key 0
    O, lse = oracle.head_forward(np.vstack([q, q]), k, v, True, s, None)
    assert np.allclose(O[0], v[0], atol=1e-15) and abs(lse[0] - a) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_mean_of_visible_values(causal):
    rng = np.random.default_rng(6)
    N, d = 23, 16
    Q, V = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(2))
    k = oracle.widen_bf16(_rand_bits(rng, (1, d)))
    K = np.repeat(k, N, axis=0)
    s = 0.25
    O, lse = oracle.head_forward(Q, K, V, causal, s, None)
    for i in range(N):
        nvis = i + 1 if causal else N
        assert np.allclose(O[i], V[:nvis].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - (s * float(Q[i] @ k[0]) + math.log(nvis))) < 1e-12


def test_causal_row_zero():
    rng = np.random.default_rng(8)
    Q, K, V = (oracle.widen_bf16(_rand_bits(rng, (31, 32))) for _ in range(3))
    O, lse = oracle.head_forward(Q, K, V, True, 0.2, None)
    assert np.allclose(O[0], V[0], atol=1e-15)
    assert abs(lse[0] - float(np.float32(0.2)) * float(Q[0] @ K[0])) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    rng = np.random.default_rng(9)
    N, d = 29, 8
    Q, K, V = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(3))
    c = rng.standard_normal(d)
    s = 0.4
    O1, l1 = oracle.head_forward(Q, K, V, causal, s, None)
    O2, l2 = oracle.head_forward(Q, K + c, V, causal, s, None)
    sf = float(np.float32(s))
    assert np.allclose(O1, O2, atol=1e-12)
    assert np.allclose(l2 - l1, sf * (Q @ c), atol=1e-12)


def test_key_permutation_invariance_noncausal():
    rng = np.random.default_rng(10)
    N, d = 37, 8
    Q, K, V = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(3))
    perm = rng.permutation(N)
    O1, l1 = oracle.head_forward(Q, K, V, False, 0.3, None)
    O2, l2 = oracle.head_forward(Q, K[perm], V[perm], False, 0.3, None)
    assert np.allclose(O1, O2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)


def test_mask_special_cases():
    rng = np.random.default_rng(12)
    N, d = 300, 16
    Q, K, V = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(3))
    nb = 3
    ones = np.ones((nb, nb), dtype=np.uint8)
    lower = np.tril(ones)
    Od, ld = oracle.head_forward(Q, K, V, False, 0.25, None)
    Om, lm = oracle.head_forward(Q, K, V, False, 0.25, ones, 128)
    assert np.array_equal(Od, Om) and np.array_equal(ld, lm)
    Oc, lc = oracle.head_forward(Q, K, V, True, 0.25, None)
    Oc2, lc2 = oracle.head_forward(Q, K, V, True, 0.25, lower, 128)
    assert np.array_equal(Oc, Oc2) and np.array_equal(lc, lc2)
    # diagonal-only mask: each row block attends to its own block, which is
    # the dense result restricted to that block
    diag = np.eye(nb, dtype=np.uint8)
    Og, lg = oracle.head_forward(Q, K, V, False, 0.25, diag, 128)
    for bi in range(nb):
        sl = slice(bi * 128, min(N, bi * 128 + 128))
        Ob, lb = oracle.head_forward(Q[sl], K[sl], V[sl], False, 0.25, None)
        assert np.allclose(Og[sl], Ob, atol=1e-13) and np.allclose(lg[sl], lb, atol=1e-13)


def test_fully_masked_rows():
    rng = np.random.default_rng(13)
    N, d = 8, 4
    Q, K, V, dO = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(4))
    mask = np.array([[1, 0], [0, 0]], dtype=np.uint8)  # block size 4: rows 4..7 see nothing
    r = oracle.head_backward(Q, K, V, dO, False, 0.5, mask, 4)
    assert np.all(r["O"][4:] == 0) and np.all(np.isneginf(r["lse"][4:]))
    assert np.all(np.isfinite(r["lse"][:4]))
    for g in ("dQ", "dK", "dV"):
        assert not np.any(np.isnan(r[g]))
    assert np.all(r["dQ"][4:] == 0)
    assert np.all(r["dK"][4:] == 0) and np.all(r["dV"][4:] == 0)


def test_batched_wrapper_matches_heads():
    inp = make_inputs(4, 2, 3, 130, 16, sparse=True)
    mask = inp["mask"]
    O, lse = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], True, 0.25, mask, row_chunk=50)
    for b in range(2):
        for h in range(3):
            Q, K, V = (oracle.widen_bf16(inp[n][b, h]) for n in "qkv")
            O1, l1 = oracle.head_forward(Q, K, V, True, 0.25, mask[h], 128)
            assert np.array_equal(O[b, h], O1) and np.array_equal(lse[b, h], l1)


# ---------------------------------------------------------------- backward pins

def _loss(Q, K, V, dO, causal, s, mask, blk):
    O, _ = oracle.head_forward(Q, K, V, causal, s, mask, blk)
    return float(np.sum(O * dO))


@pytest.mark.parametrize("N,d", [(1, 3), (4, 3), (7, 5), (12, 4)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_gradient_finite_differences(N, d, causal, masked):
    rng = np.random.default_rng(1000 + 13 * N + d)
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    s = 0.6
    mask = _tiny_mask(rng, N, 3, p=0.6) if masked else None
    if mask is not None:
        np.fill_diagonal(mask, 1)
    r = oracle.head_backward(Q, K, V, dO, causal, s, mask, 3)
    h = 1e-6
    for name, X, G in (("Q", Q, r["dQ"]), ("K", K, r["dK"]), ("V", V, r["dV"])):
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"Q": Q, "K": K, "V": V}
            args[name] = Xp
            lp = _loss(args["Q"], args["K"], args["V"], dO, causal, s, mask, 3)
            args[name] = Xm
            lm = _loss(args["Q"], args["K"], args["V"], dO, causal, s, mask, 3)
            num[idx] = (lp - lm) / (2 * h)
        den = max(np.max(np.abs(num)), 1e-3)
        assert np.max(np.abs(num - G)) / den < 1e-7, name


def test_D_identity_and_sum_invariants():
    rng = np.random.default_rng(21)
    N, d = 50, 16
    Q, K, V, dO = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(4))
    s = 0.25
    for causal in (False, True):
        r = oracle.head_backward(Q, K, V, dO, causal, s, None)
        keep = oracle.keep_matrix(np.arange(N), np.arange(N), causal)
        S = np.where(keep, (Q @ K.T) * float(np.float32(s)), -np.inf)
        P = np.exp(S - r["lse"][:, None])
        dP = dO @ V.T
        assert np.allclose(r["D"], np.sum(P * dP, axis=1), atol=1e-12)
        # shift invariance in K => columns of dK sum to zero
        assert np.allclose(r["dK"].sum(axis=0), 0.0, atol=1e-12)
        # rows of P sum to one => sum_j dV_j = sum_i dO_i
        assert np.allclose(r["dV"].sum(axis=0), dO.sum(axis=0), atol=1e-12)


def test_backward_single_key_and_identical_keys():
    rng = np.random.default_rng(22)
    q, k, v, do = (oracle.widen_bf16(_rand_bits(rng, (1, 8))) for _ in range(4))
    r = oracle.head_backward(q, k, v, do, False, 0.3, None)
    assert np.allclose(r["dV"], do, atol=1e-15)
    assert np.all(np.abs(r["dQ"]) < 1e-15) and np.all(np.abs(r["dK"]) < 1e-15)
    N = 19
    Q, V, dO = (oracle.widen_bf16(_rand_bits(rng, (N, 8))) for _ in range(3))
    K = np.repeat(oracle.widen_bf16(_rand_bits(rng, (1, 8))), N, axis=0)
    for causal in (False, True):
        r = oracle.head_backward(Q, K, V, dO, causal, 0.3, None)
        assert np.all(np.abs(r["dQ"]) < 1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("masked", [False, True])
def test_pieces_equal_whole(causal, masked):
    rng = np.random.default_rng(31)
    N, d = 70, 8
    Q, K, V, dO = (oracle.widen_bf16(_rand_bits(rng, (N, d))) for _ in range(4))
    mask = _tiny_mask(rng, N, 16, p=0.5) if masked else None
    if mask is not None:
        np.fill_diagonal(mask, 1)
    r = oracle.head_backward(Q, K, V, dO, causal, 0.3, mask, 16)
    rows = np.array([0, 5, 33, 69])
    rr = oracle.head_grad_rows(Q, K, V, dO, causal, 0.3, rows, mask, 16)
    assert np.allclose(rr["dQ"], r["dQ"][rows], atol=1e-13)
    assert np.allclose(rr["lse"], r["lse"][rows], atol=1e-13)
    cols = np.array([0, 1, 40, 69])
    rc = oracle.head_grad_cols(Q, K, V, dO, causal, 0.3, cols, mask, 16, row_chunk=9)
    assert np.allclose(rc["dK"], r["dK"][cols], atol=1e-13)
    assert np.allclose(rc["dV"], r["dV"][cols], atol=1e-13)


def test_batched_backward_matches_heads():
    inp = make_inputs(5, 1, 2, 40, 8)
    out = oracle.attn_bwd_ref(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.35)
    for h in range(2):
        Q, K, V, dO = (oracle.widen_bf16(inp[n][0, h]) for n in ("q", "k", "v", "do"))
        r = oracle.head_backward(Q, K, V, dO, True, 0.35, None)
        for name in ("dQ", "dK", "dV", "O", "lse"):
            assert np.array_equal(out[name][0, h], r[name])


# ---------------------------------------------------------------- planted mistakes

def _mutants():
    """Wrong variants of head_forward / head_backward a slip could produce."""
    def fwd_no_scale(Q, K, V, causal, scale, mh=None, mb=128, rows=None):
        return A.head_forward(Q, K, V, causal, 1.0, mh, mb, rows)

    def fwd_log2(Q, K, V, causal, scale, mh=None, mb=128, rows=None):
        O, lse = A.head_forward(Q, K, V, causal, scale, mh, mb, rows)
        return O, lse / math.log(2.0)

    def fwd_transposed_mask(Q, K, V, causal, scale, mh=None, mb=128, rows=None):
        return A.head_forward(Q, K, V, causal, scale, None if mh is None else mh.T, mb, rows)

    def fwd_causal_strict(Q, K, V, causal, scale, mh=None, mb=128, rows=None):
        # j < i instead of j <= i
        N = Q.shape[0]
        if not causal:
            return A.head_forward(Q, K, V, causal, scale, mh, mb, rows)
        O = np.zeros_like(Q @ np.zeros((Q.shape[1], V.shape[1])))
        lse = np.full(N, -np.inf)
        for i in range(1, N):
            o, l_ = A.head_forward(Q[i:i + 1], K[:i], V[:i], False, scale)
            O[i], lse[i] = o[0], l_[0]
        return O, lse

    return [fwd_no_scale, fwd_log2, fwd_transposed_mask, fwd_causal_strict]


def test_planted_mistakes_are_caught():
    """Each mutant disagrees with the brute force or the closed forms."""
    rng = np.random.default_rng(77)
    N, d = 6, 4
    qb, kb, vb = (_rand_bits(rng, (N, d)) for _ in range(3))
    mask = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], dtype=np.uint8)
    Q, K, V = (oracle.widen_bf16(x) for x in (qb, kb, vb))
    for mut in _mutants():
        caught = False
        for causal in (False, True):
            for mh in (None, mask):
                vis = None if mh is None else (lambda i, j, m=mh: m[i // 2, j // 2] != 0)
                O_n, lse_n = oracle.naive_bruteforce_bits(qb, kb, vb, causal, 0.5, vis)
                O, lse = mut(Q, K, V, causal, 0.5, mh, 2)
                lse_n = np.array(lse_n)
                if not (np.allclose(O, O_n, atol=1e-9) and np.allclose(lse, lse_n, atol=1e-9)):
                    caught = True
        assert caught, mut.__name__


def test_planted_gradient_mistakes_are_caught():
    rng = np.random.default_rng(78)
    N, d = 5, 3
    Q, K, V, dO = (rng.standard_normal((N, d)) for _ in range(4))
    r = oracle.head_backward(Q, K, V, dO, True, 0.6, None)
    h = 1e-6

    def fd(name):
        X = {"Q": Q, "K": K, "V": V}[name]
        num = np.zeros_like(X)
        for idx in np.ndindex(*X.shape):
            a = {"Q": Q.copy(), "K": K.copy(), "V": V.copy()}
            a[name][idx] += h
            lp = _loss(a["Q"], a["K"], a["V"], dO, True, 0.6, None, 128)
            a[name][idx] -= 2 * h
            lm = _loss(a["Q"], a["K"], a["V"], dO, True, 0.6, None, 128)
            num[idx] = (lp - lm) / (2 * h)
        return num

    nQ, nK, nV = fd("Q"), fd("K"), fd("V")
    assert np.allclose(r["dQ"], nQ, atol=1e-7) and np.allclose(r["dK"], nK, atol=1e-7)
    # mistakes: missing D, sign flip in dS, unscaled dK, dV from P not P^T
    keep = oracle.keep_matrix(np.arange(N), np.arange(N), True)
    S = np.where(keep, (Q @ K.T) * float(np.float32(0.6)), -np.inf)
    P = np.exp(S - r["lse"][:, None])
    dP = dO @ V.T
    s = float(np.float32(0.6))
    bad = {
        "no_D": s * ((P * dP) @ K),
        "sign": s * ((P * (r["D"][:, None] - dP)) @ K),
    }
    for name, g in bad.items():
        assert not np.allclose(g, nQ, atol=1e-5), name
    assert not np.allclose(r["dK"] / s, nK, atol=1e-5)
    assert not np.allclose(P @ dO, nV, atol=1e-5)


# ---------------------------------------------------------------- frozen fixture

def test_oracle_matches_frozen_fixture():
    """Regression guard: tests/golden/oracle_small.json was written by
    tests/golden/make_golden.py from this oracle; a change to the oracle's
    arithmetic must regenerate it (and say why in its commit)."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    with open(path) as f:
        cases = json.load(f)
    for c in cases:
        inp = make_inputs(c["seed"], c["B"], c["H"], c["N"], c["d"])
        for n in ("q", "k", "v", "do"):
            chk = int(np.sum(inp[n].astype(np.int64) * np.arange(1, inp[n].size + 1).reshape(inp[n].shape)))
            assert chk == c["inputs_sha"][n], "seeded input generator changed"
        r = oracle.attn_bwd_ref(inp["q"], inp["k"], inp["v"], inp["do"], c["causal"], c["scale"])
        for n in ("O", "lse", "dQ", "dK", "dV"):
            want = np.array([float.fromhex(x) for x in c[n]])
            got = r[n].ravel()
            assert np.array_equal(np.isfinite(got), np.isfinite(want)), (c["name"], n)
            f = np.isfinite(want)
            assert np.allclose(got[f], want[f], rtol=1e-12, atol=1e-14), (c["name"], n)
