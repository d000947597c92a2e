"""GPU: a block-sparse mask with more blocks per row than the backward ranks.

The backward's schedule stage ranks the mask blocks of a head by work only up
to 2048 blocks per row; beyond that the dK/dV and dQ launches take their
tiles in plain order. N = 2049 * 128 = 262272 (nb = 2049) checks that path
and the kernels' mask windows at their largest (33 windows of 64 blocks per
row): the order stored in the workspace is the identity, the visited tile
pairs match the mask bit for bit, and sampled outputs match the oracle.

Mask: query block r keeps blocks r and (7r + 5) mod nb; query block 1500
keeps nothing and key block 3 is kept by no query block. At this N the
expected visit map is the block mask expanded to tiles (a tile lies inside
one mask block; under causal a tile pair is visited when its first key is
not after its last query); the element-level construction of the other
visit tests would need an N x N matrix.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import check_grad, check_lse, check_o, dev, say
from tests.test_parity_fullsize import run_like_bench

pytestmark = pytest.mark.gpu

MB = 128
NB = 2049
N = NB * MB
EMPTY_ROW, UNSEEN_COL = 1500, 3


def huge_mask():
    m = np.zeros((1, NB, NB), dtype=np.uint8)
    r = np.arange(NB)
    m[0, r, r] = 1
    m[0, r, (7 * r + 5) % NB] = 1
    m[0, EMPTY_ROW, :] = 0
    m[0, :, UNSEEN_COL] = 0
    return m


def tile_visits(mask_h, causal, bq, bk, key_major=False):
    """[nq, nk] (or [nk, nq]) uint8: the block mask at (bq, bk) tiles."""
    qt = np.arange(-(-N // bq))
    kt = np.arange(-(-N // bk))
    v = mask_h[(qt * bq // MB)[:, None], (kt * bk // MB)[None, :]] != 0
    if causal:
        v &= (kt * bk)[None, :] <= np.minimum(qt * bq + bq, N)[:, None] - 1
    v = v.astype(np.uint8)
    return v.T.copy() if key_major else v


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_sparse_mask_beyond_ranked_size(d, causal):
    from exact_io_aware_69_amd import _lib, attention
    say(f"sparse nb={NB} d={d} causal={causal}")
    mask = huge_mask()
    inp = make_inputs(5, 1, 1, N, d, with_do=True)
    inp["mask"] = mask
    scale = 1.0 / math.sqrt(d)
    m = torch.from_numpy(mask).to("cuda:0")
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))

    # The stored order is the plain one.
    o = torch.zeros_like(q)
    lse = torch.zeros((1, 1, N), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st, ws_bytes = _lib.fa_bwd_workspace_size(1, 1, N, d)
    _lib.check(st, "fa_bwd_workspace_size")
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
    _lib.check(_lib.fa_bwd_stage(0, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), 1, 1, N, d, causal,
                                 scale, m.data_ptr(), ws.data_ptr(), ws_bytes,
                                 torch.cuda.current_stream().cuda_stream), "fa_bwd_stage")
    torch.cuda.synchronize()
    half = (N * 4 + 255) // 256 * 256  # one head, N a multiple of 128
    sched = ws.cpu().numpy()[2 * half:].view(np.int32)
    tpb = MB // attention.tile_config(1, d, causal)[1]
    assert np.array_equal(sched[:NB * tpb], np.arange(NB * tpb)), "key-tile order"
    assert np.array_equal(sched[2 * NB:3 * NB], np.arange(NB)), "query-block order"
    del o, lse, dq, dk, dv, ws

    # Visited tile pairs.
    o, lse, vis = attention.forward_visits(q, k, v, causal, scale, m)
    _, _, _, vkv, vq = attention.backward_visits(q, k, v, o, lse, do, causal, scale, m)
    torch.cuda.synchronize()
    t = [attention.tile_config(s, d, causal) for s in range(3)]
    assert np.array_equal(vis.cpu().numpy()[0, 0], tile_visits(mask[0], causal, *t[0])), "forward visit map"
    assert np.array_equal(vkv.cpu().numpy()[0, 0], tile_visits(mask[0], causal, *t[1], key_major=True)), \
        "dK/dV visit map"
    assert np.array_equal(vq.cpu().numpy()[0, 0], tile_visits(mask[0], causal, *t[2])), "dQ visit map"
    del o, lse, vis, vkv, vq

    # Values, launched as the benchmark launches them.
    got = run_like_bench(inp, 1, 1, N, d, causal, True, True)
    Q, K, V, dO = (oracle.widen_bf16(inp[n][0, 0]) for n in ("q", "k", "v", "do"))
    rows = np.array([0, 1, 127, 128, 64 * MB - 1, 64 * MB, 1024 * MB + 77, 2047 * MB + 5, N - 2, N - 1])
    r = oracle.head_grad_rows(Q, K, V, dO, causal, scale, rows, mask[0])
    check_o(got["o"][0, 0, rows], r["O"], "O")
    check_lse(got["lse"][0, 0, rows], r["lse"], "lse")
    # Key columns in blocks 0, 64, 1024 and 2048; lse and D of the query
    # blocks that see them (all other rows have P = 0 in these columns).
    cols = np.array([0, 5, 127, 64 * MB, 64 * MB + 100, 1024 * MB + 3, 2048 * MB, N - 1])
    cb = np.unique(cols // MB)
    seen_by = np.unique(np.nonzero(mask[0][:, cb].any(axis=1))[0])
    lse_all, D_all = np.zeros(N), np.zeros(N)
    for rb in seen_by:
        rr = np.arange(rb * MB, (rb + 1) * MB)
        O_r, l_r = oracle.head_forward(Q, K, V, causal, scale, mask[0], rows=rr)
        lse_all[rr], D_all[rr] = l_r, np.sum(dO[rr] * O_r, axis=1)
    c = oracle.head_grad_cols(Q, K, V, dO, causal, scale, cols, mask[0], lse=lse_all, D=D_all)
    floor = 1e-3 * max(np.max(np.abs(r["dQ"])), np.max(np.abs(c["dK"])), np.max(np.abs(c["dV"])))
    check_grad(got["dq"][0, 0, rows], r["dQ"], "dQ", floor)
    check_grad(got["dk"][0, 0, cols], c["dK"], "dK", floor)
    check_grad(got["dv"][0, 0, cols], c["dV"], "dV", floor)
    empty = np.arange(EMPTY_ROW * MB, (EMPTY_ROW + 1) * MB)
    assert np.all(got["lse"][0, 0, empty] == -np.inf) and np.all(got["o"][0, 0, empty] == 0.0)
    assert np.all(got["dq"][0, 0, empty] == 0.0)
    unseen = np.arange(UNSEEN_COL * MB, (UNSEEN_COL + 1) * MB)
    assert np.all(got["dk"][0, 0, unseen] == 0.0) and np.all(got["dv"][0, 0, unseen] == 0.0)
    say("  ok")
