"""GPU parity, whole outputs, for launches whose head count B*H is a multiple
of 8 with more than one head per XCD: there the causal and block-sparse
backward launches (and the causal forward) dispatch their tiles interleaved
across a group of G > 1 heads (head_rank_order / head_group in fa_params.h),
so every workgroup's (head, tile) comes from that mapping. Every element of
O, lse, dQ, dK and dV is compared with the oracle, and the visit maps of all
three kernels bit for bit, so a wrong (head, tile) for any head fails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import check_grads, check_lse, check_o, dev, host64, say
from tests.visitmap import expected_visits

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, N, d, causal, sparse)
    (1, 16, 1024, 128, True, False),
    (2, 8, 1000, 64, True, False),
    (1, 16, 700, 64, True, True),
    (1, 16, 700, 64, False, True),
    (1, 16, 700, 128, True, True),
]


def group_size(wgs_per_cu, cus_per_xcd, BH, ntile, cover=2, cap=16):
    """The group rule stated in fa_params.h (head_group), for the assertion
    below that these shapes interleave heads."""
    if BH % 8 or ntile < 1:
        return 1
    hx = BH // 8
    g = 1
    while g < hx and g < cap and (g * ntile < cover * wgs_per_cu * cus_per_xcd or hx % g):
        g += 1
    while hx % g:
        g -= 1
    return g


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_interleaved_whole_outputs(case):
    from exact_io_aware_69_amd import attention
    B, H, N, d, causal, sparse = case
    say(f"interleaved {case}")
    # Every kernel's tile count is at most ceil(N / 32) <= 32 here, far below
    # 2 * 32 CUs * (1..4 workgroups per CU): G = B*H/8 = 2 for every kernel.
    for wgs in (1, 2, 3, 4):
        assert group_size(wgs, 32, B * H, -(-N // 32)) == 2
        assert group_size(wgs, 32, B * H, -(-N // 32), cover=8, cap=8) == 2  # dense causal dK/dV
    inp = make_inputs(41, B, H, N, d, sparse=sparse, p=0.3)
    mask = inp.get("mask")
    m = None if mask is None else torch.from_numpy(mask).to("cuda:0")
    q, k, v, do = (dev(inp[n]) for n in ("q", "k", "v", "do"))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention.forward(q, k, v, causal=causal, scale=scale, block_mask=m)
    dq, dk, dv = attention.backward(q, k, v, o, lse, do, causal=causal, scale=scale, block_mask=m)
    _, _, vis = attention.forward_visits(q, k, v, causal, scale, m)
    _, _, _, vkv, vq = attention.backward_visits(q, k, v, o, lse, do, causal, scale, m)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd_ref(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, mask)
    check_o(host64(o), ref["O"])
    check_lse(host64(lse), ref["lse"])
    check_grads((host64(dq), host64(dk), host64(dv)), ref)
    for p_, got, key_major in ((0, vis, False), (1, vkv, True), (2, vq, False)):
        bm, bn = attention.tile_config(p_, d, causal)
        exp = expected_visits(N, bm, bn, causal, mask, H, key_major=key_major)
        g = got.cpu().numpy()
        for b in range(B):
            assert np.array_equal(g[b], exp), f"visit map of pass {p_}, batch {b}"
