"""GPU parity of the FlashAttention-1-style forward (ablation) against the
fp64 oracle, element by element, on ragged shapes: it must compute the same
attention as the IO-aware path, only with the older work partitioning."""
import math

import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import check_lse, check_o, dev, host64, say

pytestmark = pytest.mark.gpu


def run_fa1(inp, causal, scale, groups=1):
    from exact_io_aware_69_amd import _lib
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    st, nbytes = _lib.fa_fa1_workspace_size(B, H, N, d)
    _lib.check(st, "fa_fa1_workspace_size")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    st = _lib.fa_fwd_fa1(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d, causal,
                         scale, groups, ws.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    _lib.check(st, "fa_fwd_fa1")
    torch.cuda.synchronize()
    return host64(o), host64(lse)


@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (1, 1, 1, 128), (2, 2, 300, 128), (1, 3, 700, 64),
                                   (1, 2, 129, 128)], ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_fa1_forward(shape, causal):
    B, H, N, d = shape
    say(f"fa1 {shape} causal={causal}")
    inp = make_inputs(61, B, H, N, d, with_do=False)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_fa1(inp, causal, scale)
    O_ref, lse_ref = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], causal, scale)
    check_o(o, O_ref)
    check_lse(lse, lse_ref)


@pytest.mark.parametrize("causal", [False, True])
def test_fa1_forward_peaky(causal):
    """q drawn 4x larger: the running max moves across K/V tiles, so the
    eager rescaling of the stored output is exercised."""
    inp = make_inputs(62, 1, 2, 600, 128, with_do=False, q_gain=4.0)
    o, lse = run_fa1(inp, causal, 1.0 / math.sqrt(128))
    O_ref, lse_ref = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], causal, 1.0 / math.sqrt(128))
    check_o(o, O_ref)
    check_lse(lse, lse_ref)


@pytest.mark.parametrize("groups", [2, 3, 7, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_fa1_forward_seq_groups(groups, causal):
    """Query tiles dealt round-robin to several workgroups per head (1000 is
    clamped to the 22 query tiles of N = 700)."""
    say(f"fa1 groups={groups} causal={causal}")
    inp = make_inputs(63, 2, 2, 700, 64, with_do=False)
    o, lse = run_fa1(inp, causal, 0.125, groups)
    O_ref, lse_ref = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], causal, 0.125)
    check_o(o, O_ref)
    check_lse(lse, lse_ref)
