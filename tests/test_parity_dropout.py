"""GPU parity of attention dropout (fa_fwd_dropout, fa_bwd_dropout,
fa_dropout_keep) against the fp64 dropout oracle.

The keep decisions are integer results: the generator's mask is compared
bit for bit, and so are the decisions the fused kernels take, extracted
through inputs that expose them (Q = 0 and V = identity make O_ij nonzero
exactly where (i, j) is kept; dO = identity does the same for dV^T).
Values are compared with the usual tolerances."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import dropout as od
from synth import f32_to_bf16_bits, make_block_mask, make_inputs
from tests.gpu_util import check_grads, check_lse, check_o, dev, host64, say

pytestmark = pytest.mark.gpu

SEED = 0x1234_5678_9ABC_DEF0


def _stream():
    return torch.cuda.current_stream().cuda_stream


def run_fwd(inp, causal, scale, p, seed, off, mask=None):
    from exact_io_aware_69_amd import _lib
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    m = None if mask is None else torch.from_numpy(mask).to("cuda:0")
    st = _lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                             causal, scale, None if m is None else m.data_ptr(), p, seed, off, _stream())
    _lib.check(st, "fa_fwd_dropout")
    torch.cuda.synchronize()
    return q, k, v, o, lse, m


def run_fwd_bwd(inp, causal, scale, p, seed, off, mask=None):
    from exact_io_aware_69_amd import _lib
    q, k, v, o, lse, m = run_fwd(inp, causal, scale, p, seed, off, mask)
    B, H, N, d = q.shape
    do = dev(inp["do"])
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    st, nbytes = _lib.fa_bwd_workspace_size(B, H, N, d)
    _lib.check(st, "fa_bwd_workspace_size")
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    st = _lib.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale,
                             None if m is None else m.data_ptr(), p, seed, off, ws.data_ptr(), nbytes, _stream())
    _lib.check(st, "fa_bwd_dropout")
    torch.cuda.synchronize()
    return host64(o), host64(lse), host64(dq), host64(dk), host64(dv)


@pytest.mark.parametrize("B,H,N", [(1, 3, 130), (2, 1, 1), (1, 2, 5), (1, 1, 257)])
@pytest.mark.parametrize("p", [0.0, 0.3, 0.9])
def test_keep_mask_bitexact(B, H, N, p):
    from exact_io_aware_69_amd import _lib
    say(f"keep B{B} H{H} N{N} p{p}")
    keep = torch.full((B, H, N, N), 7, dtype=torch.uint8, device="cuda:0")
    _lib.check(_lib.fa_dropout_keep(B, H, N, p, SEED, 5, keep.data_ptr(), _stream()), "fa_dropout_keep")
    torch.cuda.synchronize()
    got = keep.cpu().numpy()
    ref = od.dropout_keep(B, H, N, p, SEED, 5).astype(np.uint8)
    assert np.array_equal(got, ref)


def _identity_bits(n, d):
    eye = np.zeros((n, d), dtype=np.float32)
    eye[np.arange(min(n, d)), np.arange(min(n, d))] = 1.0
    return f32_to_bf16_bits(eye)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.3, 0.5])
def test_forward_keep_decisions_bitexact(d, causal, p):
    """Q = 0 makes every visible score 0, so P_ij is 1/(#visible keys of
    row i); with V = I (N = d, two or one key tiles) O_ij = P_ij Z_ij/(1-p):
    nonzero exactly where the fused forward kept (i, j)."""
    say(f"fwd keep extraction d{d} causal={causal} p{p}")
    N, B, H = d, 1, 2
    rng = np.random.default_rng(1)
    inp = {"q": np.zeros((B, H, N, d), dtype=np.uint16),
           "k": f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)),
           "v": np.broadcast_to(_identity_bits(N, d), (B, H, N, d)).copy()}
    _, _, _, o, _, _ = run_fwd(inp, causal, 1.0 / math.sqrt(d), p, SEED, 9)
    got = host64(o) != 0
    vis = oracle.keep_matrix(np.arange(N), np.arange(N), causal)
    ref = od.dropout_keep(B, H, N, p, SEED, 9) & vis[None, None]
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_dv_keep_decisions_bitexact(d, causal):
    """dV = (P o Z)^T dO / (1 - p): with dO = I (N = d), dV^T is the dropped
    P, so its nonzero pattern is the keep mask the dK/dV kernel used (the
    cross-lane exchange of generator words included)."""
    say(f"bwd dV keep extraction d{d} causal={causal}")
    N, B, H, p = d, 1, 2, 0.4
    rng = np.random.default_rng(2)
    inp = {"q": np.zeros((B, H, N, d), dtype=np.uint16),
           "k": f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)),
           "v": f32_to_bf16_bits(rng.standard_normal((B, H, N, d)).astype(np.float32)),
           "do": np.broadcast_to(_identity_bits(N, d), (B, H, N, d)).copy()}
    _, _, _, _, dv = run_fwd_bwd(inp, causal, 1.0 / math.sqrt(d), p, SEED, 3)
    got = np.swapaxes(dv, 2, 3) != 0
    vis = oracle.keep_matrix(np.arange(N), np.arange(N), causal)
    ref = od.dropout_keep(B, H, N, p, SEED, 3) & vis[None, None]
    assert np.array_equal(got, ref)


SHAPES = [(1, 2, 32, 64), (1, 2, 48, 128), (2, 1, 100, 64), (1, 2, 129, 128), (1, 1, 300, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.2, 0.5])
def test_dropout_parity(shape, causal, p):
    B, H, N, d = shape
    say(f"dropout parity {shape} causal={causal} p{p}")
    inp = make_inputs(71, B, H, N, d)
    scale = 1.0 / math.sqrt(d)
    o, lse, dq, dk, dv = run_fwd_bwd(inp, causal, scale, p, SEED, 11)
    ref = od.attn_bwd_dropout_ref(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, p, SEED, 11)
    check_o(o, ref["O"])
    check_lse(lse, ref["lse"])
    check_grads((dq, dk, dv), ref)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_parity_peaky_and_blocksparse(causal):
    B, H, N, d = 1, 2, 260, 64
    say(f"dropout parity peaky/sparse causal={causal}")
    inp = make_inputs(72, B, H, N, d, q_gain=4.0)
    mask = make_block_mask(np.random.default_rng(3), H, N, p=0.5)
    scale = 1.0 / math.sqrt(d)
    o, lse, dq, dk, dv = run_fwd_bwd(inp, causal, scale, 0.25, 99, 0, mask)
    ref = od.attn_bwd_dropout_ref(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, 0.25, 99, 0, mask)
    check_o(o, ref["O"])
    check_lse(lse, ref["lse"])
    check_grads((dq, dk, dv), ref)


@pytest.mark.parametrize("d", [64, 128])
def test_zero_dropout_matches_plain_path(d):
    """p = 0 keeps everything: results equal the plain kernels' bit for bit
    in O and lse (the same arithmetic with every keep test passing)."""
    from exact_io_aware_69_amd import attention
    inp = make_inputs(73, 1, 2, 200, d)
    q, k, v, o, lse, _ = run_fwd(inp, True, 0.088, 0.0, 5, 0)
    o2, lse2 = attention.forward(q, k, v, causal=True, scale=0.088)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
