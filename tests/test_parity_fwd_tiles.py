"""GPU forward parity for every tile configuration fa_fwd_tiles offers
(query rows per workgroup x keys per tile), against the fp64 oracle,
element by element, on ragged shapes: dense, causal and block-sparse
(with 256-row tiles a workgroup spans two mask rows)."""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import check_lse, check_o, dev, host64, say

pytestmark = pytest.mark.gpu

CONFIGS = [(128, 32), (128, 64), (128, 128), (256, 64), (256, 128)]


def run_tiles(inp, causal, scale, bm, bn, mask=None):
    from exact_io_aware_69_amd import _lib
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    m = None if mask is None else torch.from_numpy(mask).to("cuda:0")
    st = _lib.fa_fwd_tiles(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                           causal, scale, None if m is None else m.data_ptr(), bm, bn,
                           torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "fa_fwd_tiles")
    torch.cuda.synchronize()
    return host64(o), host64(lse)


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"bm{c[0]}-bn{c[1]}")
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", ["dense", "causal", "sparse", "sparse_causal"])
def test_forward_tiles(cfg, d, mode):
    bm, bn = cfg
    B, H, N = 1, 2, 700
    causal = "causal" in mode
    sparse = "sparse" in mode
    say(f"fwd tiles bm{bm} bn{bn} d{d} {mode}")
    inp = make_inputs(41, B, H, N, d, with_do=False, sparse=sparse, p=0.3)
    mask = inp.get("mask")
    if sparse:
        mask[:, 2, :] = 0  # a query block that sees nothing, next to one that does
    scale = 1.0 / math.sqrt(d)
    o, lse = run_tiles(inp, causal, scale, bm, bn, mask)
    O_ref, lse_ref = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], causal, scale, mask)
    check_o(o, O_ref)
    check_lse(lse, lse_ref)


def test_forward_tiles_rejects_unsupported():
    from exact_io_aware_69_amd import _lib
    for bm, bn in [(64, 64), (256, 32), (128, 256), (512, 64)]:
        assert _lib.fa_fwd_tiles(1 << 12, 1 << 12, 1 << 12, 1 << 12, 1 << 12, 1, 1, 16, 64, 0, 0.125, None, bm, bn,
                                 None) == -2
