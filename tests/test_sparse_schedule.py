"""GPU: the block-sparse backward schedule that the schedule stage writes.

For a block-sparse backward the schedule launch (stage 0) ranks, per head, the
key blocks and the query blocks by the number of mask blocks of their column
(row) that some query sees, falling, ties by index, and stores the order in
the backward workspace after D and lse * log2(e): three int32 per (head,
mask block) -- the key tiles in two slots per block (one key tile per block
when the key tiles span the whole 128-block), then the query blocks. The
dK/dV and dQ kernels dispatch their tiles in that order.

The expected order is computed here in numpy from the mask alone. The
result of the backward does not depend on the order; these tests pin the
schedule itself: a wrong ranking would only cost time, or, if it were not a
permutation, skip tiles, which the parity tests would also catch.
"""
import math

import numpy as np
import pytest
import torch

from synth import make_inputs
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu

MB = 128


def expected_orders(mask_h, causal, tpb):
    nb = mask_h.shape[0]
    keep = mask_h != 0
    if causal:
        keep = keep & np.tril(np.ones((nb, nb), dtype=bool))  # query block r sees key block c iff c <= r
    col = keep.sum(axis=0)  # work of each key block
    row = keep.sum(axis=1)  # work of each query block
    kord = sorted(range(nb), key=lambda i: (-int(col[i]), i))
    qord = sorted(range(nb), key=lambda i: (-int(row[i]), i))
    ktiles = [b * tpb + t for b in kord for t in range(tpb)]
    return np.array(ktiles, dtype=np.int32), np.array(qord, dtype=np.int32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [700, 9000, 40000])  # nb = 6, 71, 313 (above 256: one row per many threads)
def test_schedule_matches_mask_ranking(d, causal, N):
    from exact_io_aware_69_amd import _lib, attention
    B, H = 1, 3
    say(f"schedule d={d} causal={causal} N={N}")
    inp = make_inputs(11, B, H, N, d, with_do=True, sparse=True, p=0.3)
    mask = inp["mask"]
    nb = mask.shape[1]
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))
    o = torch.zeros_like(q)
    lse = torch.zeros((B, H, N), dtype=torch.float32, device="cuda:0")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    m = torch.from_numpy(mask).to("cuda:0")
    st, ws_bytes = _lib.fa_bwd_workspace_size(B, H, N, d)
    _lib.check(st, "fa_bwd_workspace_size")
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda:0")
    st = _lib.fa_bwd_stage(0, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, 1.0 / math.sqrt(d),
                           m.data_ptr(), ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "fa_bwd_stage")
    torch.cuda.synchronize()
    host = ws.cpu().numpy()
    # D and lse * log2(e): two fp32 arrays of B*H*Npad rows, each padded to 256 bytes.
    npad = -(-N // MB) * MB
    half = (B * H * npad * 4 + 255) // 256 * 256
    sched = host[2 * half:].view(np.int32)
    korder = sched[:H * 2 * nb].reshape(H, 2 * nb)
    qorder = sched[H * 2 * nb:H * 3 * nb].reshape(H, nb)
    tpb = MB // attention.tile_config(1, d, causal)[1]  # key tiles per mask block in the dK/dV pass
    for h in range(H):
        ek, eq = expected_orders(mask[h], causal, tpb)
        assert np.array_equal(qorder[h], eq), f"query order, head {h}"
        assert np.array_equal(korder[h, :nb * tpb], ek), f"key order, head {h}"

