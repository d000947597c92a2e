"""GPU: the (query tile, key tile) pairs the kernels process equal, bit for
bit, the pairs that contain a visible element (causal and block-sparse
skipping), for the forward and both backward kernels."""
import math

import numpy as np
import pytest
import torch

from synth import make_block_mask, make_inputs
from tests.gpu_util import dev, say
from tests.visitmap import expected_visits

pytestmark = pytest.mark.gpu


CASES = [
    # (B, H, N, d, causal, sparse)
    (1, 2, 256, 64, False, False),
    (2, 2, 300, 128, True, False),
    (1, 3, 1000, 64, True, False),
    (2, 3, 700, 64, False, True),
    (2, 3, 700, 128, True, True),
    (1, 2, 1, 64, True, False),
    (1, 4, 2048, 128, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_visit_maps(case):
    from exact_io_aware_69_amd import attention
    B, H, N, d, causal, sparse = case
    say(f"visits {case}")
    inp = make_inputs(31, B, H, N, d, sparse=sparse, p=0.3)
    mask = inp.get("mask")
    m = None if mask is None else torch.from_numpy(mask).to("cuda:0")
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse, vis = attention.forward_visits(q, k, v, causal, scale, m)
    _, _, _, vkv, vq = attention.backward_visits(q, k, v, o, lse, do, causal, scale, m)
    torch.cuda.synchronize()
    bm0, bn0 = attention.tile_config(0, d, causal)
    bm1, bn1 = attention.tile_config(1, d, causal)
    bm2, bn2 = attention.tile_config(2, d, causal)
    e0 = expected_visits(N, bm0, bn0, causal, mask, H)
    e1 = expected_visits(N, bm1, bn1, causal, mask, H, key_major=True)
    e2 = expected_visits(N, bm2, bn2, causal, mask, H)
    got0, got1, got2 = vis.cpu().numpy(), vkv.cpu().numpy(), vq.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got0[b], e0), "forward visit map"
        assert np.array_equal(got1[b], e1), "dK/dV visit map"
        assert np.array_equal(got2[b], e2), "dQ visit map"
