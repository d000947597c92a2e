"""GPU: block-sparse masks with more than 64 blocks per row and column.

The kernels read the block mask 64 blocks at a time (one byte per lane,
packed by a ballot), so a mask with nb > 64 makes every kernel move its
window. The mask built here keeps, in each query block r, the blocks r,
(r + 66) mod nb and (7r + 3 + h) mod nb: rows and columns jump across the
window boundary, in both directions, over long empty stretches. Query block
69 keeps nothing (its rows see no key: O = 0, lse = -inf), and key block 2
is kept by no query block (its dK, dV are 0).

Checked for the forward, dK/dV and dQ kernels, dense-masked and causal, at
d = 64 and 128: the visited (query tile, key tile) pairs bit for bit against
the element-level rule, and O, lse, dQ (sampled rows) and dK, dV (sampled
key rows) against the oracle, with the bars of the other parity tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import check_grad, check_lse, check_o, dev, say
from tests.test_parity_fullsize import run_like_bench, sample_indices
from tests.visitmap import expected_visits

pytestmark = pytest.mark.gpu

B, H, N = 1, 2, 9000  # nb = 71 mask blocks per row
MB = 128


def wide_mask():
    nb = -(-N // MB)
    m = np.zeros((H, nb, nb), dtype=np.uint8)
    for h in range(H):
        for r in range(nb):
            for c in (r, (r + 66) % nb, (7 * r + 3 + h) % nb):
                m[h, r, c] = 1
        m[h, 69, :] = 0
        m[h, :, 2] = 0
    return m


def boundary_rows():
    """Rows at the edges of mask blocks 2, 63, 64, 65, 69, 70 and the end."""
    s = set()
    for blk in (2, 63, 64, 65, 69, 70):
        for off in (-1, 0, 1, MB - 1):
            i = blk * MB + off
            if 0 <= i < N:
                s.add(i)
    s.update((N - 2, N - 1))
    return s


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_wide_mask(d, causal):
    from exact_io_aware_69_amd import attention
    say(f"sparse wide mask d={d} causal={causal}")
    mask = wide_mask()
    inp = make_inputs(7, B, H, N, d, with_do=True)
    inp["mask"] = mask
    scale = 1.0 / math.sqrt(d)

    # Visit maps, bit for bit.
    m = torch.from_numpy(mask).to("cuda:0")
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse, vis = attention.forward_visits(q, k, v, causal, scale, m)
    _, _, _, vkv, vq = attention.backward_visits(q, k, v, o, lse, do, causal, scale, m)
    torch.cuda.synchronize()
    tiles = [attention.tile_config(s, d, causal) for s in range(3)]
    e0 = expected_visits(N, *tiles[0], causal, mask, H)
    e1 = expected_visits(N, *tiles[1], causal, mask, H, key_major=True)
    e2 = expected_visits(N, *tiles[2], causal, mask, H)
    assert np.array_equal(vis.cpu().numpy()[0], e0), "forward visit map"
    assert np.array_equal(vkv.cpu().numpy()[0], e1), "dK/dV visit map"
    assert np.array_equal(vq.cpu().numpy()[0], e2), "dQ visit map"

    # Values, launched as the benchmark launches them.
    got = run_like_bench(inp, B, H, N, d, causal, True, True)
    rng = np.random.default_rng(99)
    for h in range(H):
        Q, K, V, dO = (oracle.widen_bf16(inp[n][0, h]) for n in ("q", "k", "v", "do"))
        rows = np.array(sorted(set(sample_indices(N, rng).tolist()) | boundary_rows()), dtype=np.int64)
        r = oracle.head_grad_rows(Q, K, V, dO, causal, scale, rows, mask[h])
        check_o(got["o"][0, h, rows], r["O"], f"O[{h}]")
        check_lse(got["lse"][0, h, rows], r["lse"], f"lse[{h}]")
        cols = np.array(sorted(set(sample_indices(N, rng).tolist()) | boundary_rows()), dtype=np.int64)
        c = oracle.head_grad_cols(Q, K, V, dO, causal, scale, cols, mask[h])
        floor = 1e-3 * max(np.max(np.abs(r["dQ"])), np.max(np.abs(c["dK"])), np.max(np.abs(c["dV"])))
        check_grad(got["dq"][0, h, rows], r["dQ"], f"dQ[{h}]", floor)
        check_grad(got["dk"][0, h, cols], c["dK"], f"dK[{h}]", floor)
        check_grad(got["dv"][0, h, cols], c["dV"], f"dV[{h}]", floor)
        # The rows of query block 69 see nothing; key block 2 is seen by nobody.
        empty = np.arange(69 * MB, 70 * MB)
        assert np.all(got["lse"][0, h, empty] == -np.inf) and np.all(got["o"][0, h, empty] == 0.0)
        assert np.all(got["dq"][0, h, empty] == 0.0)
        unseen = np.arange(2 * MB, 3 * MB)
        assert np.all(got["dk"][0, h, unseen] == 0.0) and np.all(got["dv"][0, h, unseen] == 0.0)
        say(f"  head {h} ok")
