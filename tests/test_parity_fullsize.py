"""GPU parity at the full workload sizes, launched exactly as bench.py does:
fa_fwd / fa_fwd_blocksparse, then fa_bwd_stage 0, 1, 2 on the current stream.

Where the oracle finishes in seconds (N <= 4096: the two B8 H16 N2048 d64
forwards and the B4 H16 N4096 d128 forward and backward), every element of
every output is compared with it. At N = 8192 and 16384 it is evaluated on
sampled outputs (rows are independent in O, lse and dQ; a column of dK/dV
needs lse and D of every row, which the oracle recomputes on its own):
  * O, lse, dQ on sampled query rows of sampled heads,
  * dK, dV on sampled key rows of sampled heads,
with the same bars as the small parity tests. Properties that hold at any
size are checked on the whole outputs: O is a convex combination of visible
V rows (so each column stays within V's range), every output is finite, and
the gradient identities sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i (over rows
that see some key) hold per head to a rounding bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs
from tests.gpu_util import check_grad, check_grads, check_lse, check_o, dev, host64, say

pytestmark = pytest.mark.gpu

WORKLOADS = {
    # name: (B, H, N, d, causal, sparse, bwd)
    "dense_b1_h2_n256_d64_fwd": (1, 2, 256, 64, False, False, False),
    "causal_b8_h16_n2048_d64_fwd": (8, 16, 2048, 64, True, False, False),
    "dense_b8_h16_n2048_d64_fwd": (8, 16, 2048, 64, False, False, False),
    "causal_b4_h16_n4096_d128_fwdbwd": (4, 16, 4096, 128, True, False, True),
    "causal_b1_h16_n16384_d128_fwdbwd": (1, 16, 16384, 128, True, False, True),
    "blocksparse_b2_h16_n8192_d64_fwdbwd": (2, 16, 8192, 64, False, True, True),
}

# Relative bound for the whole-output gradient identities: the residual of
# sum_j dK_j (resp. sum_j dV_j - sum_i dO_i) in any column is compared with
# the L1 mass sum_j |dK_j| of that column. Exact arithmetic gives 0; bf16
# outputs and bf16 P, dS inside the products leave residuals that average
# out over N rows, far below 1e-2 of the mass. A dropped term or a wrong
# sign leaves residuals of the order of the mass itself.
IDENTITY_REL = 2e-2
# Largest N at which every output element is compared with the oracle.
WHOLE_MAX_N = 4096


def sample_indices(N, rng, extra=24):
    """Tile edges (64 and 128 multiples, both sides), both ends, and random."""
    s = {0, 1, N - 1, N - 2}
    for t in (63, 64, 127, 128, 129, 255, 256):
        if t < N:
            s.add(t)
    s.update(int(x) for x in rng.integers(0, N, size=extra))
    return np.array(sorted(i for i in s if 0 <= i < N), dtype=np.int64)


def sample_heads(B, H, rng):
    heads = {(0, 0), (B - 1, H - 1), (int(rng.integers(B)), int(rng.integers(H)))}
    return sorted(heads)


def run_like_bench(inp, B, H, N, d, causal, sparse, bwd):
    from exact_io_aware_69_amd import _lib
    scale = 1.0 / math.sqrt(d)
    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    mask = torch.from_numpy(inp["mask"]).to("cuda:0") if sparse else None
    mptr = mask.data_ptr() if mask is not None else None
    sptr = torch.cuda.current_stream().cuda_stream
    if mptr is None:
        st = _lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, causal, scale, sptr)
    else:
        st = _lib.fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, causal, scale, mptr, sptr)
    _lib.check(st, "fa_fwd")
    out = {"o": o, "lse": lse}
    if bwd:
        do = dev(inp["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        st, ws_bytes = _lib.fa_bwd_workspace_size(B, H, N, d)
        _lib.check(st, "fa_bwd_workspace_size")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
        for stage in range(3):
            st = _lib.fa_bwd_stage(stage, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal,
                                   scale, mptr, ws.data_ptr(), ws_bytes, sptr)
            _lib.check(st, "fa_bwd_stage")
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: host64(t) for n, t in out.items()}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_fullsize_sampled(name):
    B, H, N, d, causal, sparse, bwd = WORKLOADS[name]
    say(f"full-size {name}")
    inp = make_inputs(0, B, H, N, d, with_do=bwd, sparse=sparse)
    got = run_like_bench(inp, B, H, N, d, causal, sparse, bwd)
    scale = 1.0 / math.sqrt(d)
    mask = inp.get("mask")
    rng = np.random.default_rng(1234)

    # Whole-output properties.
    for n, t in got.items():
        if n != "lse":
            assert np.all(np.isfinite(t)), f"{n}: non-finite values"
    assert np.all(np.isfinite(got["lse"])), "lse: every row sees its diagonal key here"
    v64 = oracle.widen_bf16(inp["v"])
    lo, hi = v64.min(axis=2, keepdims=True), v64.max(axis=2, keepdims=True)
    tol = 2e-2
    assert np.all(got["o"] >= lo - tol) and np.all(got["o"] <= hi + tol), "O outside the range of V"

    if N <= WHOLE_MAX_N:
        # Whole outputs against the oracle, every head.
        if not bwd:
            O_ref, lse_ref = oracle.attn_fwd_ref(inp["q"], inp["k"], inp["v"], causal, scale, mask)
            check_o(got["o"], O_ref)
            check_lse(got["lse"], lse_ref)
        else:
            ref = oracle.attn_bwd_ref(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, mask)
            check_o(got["o"], ref["O"])
            check_lse(got["lse"], ref["lse"])
            check_grads((got["dq"], got["dk"], got["dv"]), ref)
        say("  whole outputs ok")
    heads = [] if N <= WHOLE_MAX_N else sample_heads(B, H, rng)

    # Sampled parity with the oracle.
    for (b, h) in heads:
        Q, K, V = (oracle.widen_bf16(inp[n][b, h]) for n in ("q", "k", "v"))
        mh = None if mask is None else mask[h]
        rows = sample_indices(N, rng)
        if not bwd:
            O_ref, lse_ref = oracle.head_forward(Q, K, V, causal, scale, mh, rows=rows)
            check_o(got["o"][b, h, rows], O_ref, f"O[{b},{h}]")
            check_lse(got["lse"][b, h, rows], lse_ref, f"lse[{b},{h}]")
            continue
        dO = oracle.widen_bf16(inp["do"][b, h])
        r = oracle.head_grad_rows(Q, K, V, dO, causal, scale, rows, mh)
        check_o(got["o"][b, h, rows], r["O"], f"O[{b},{h}]")
        check_lse(got["lse"][b, h, rows], r["lse"], f"lse[{b},{h}]")
        cols = sample_indices(N, rng)
        c = oracle.head_grad_cols(Q, K, V, dO, causal, scale, cols, mh)
        floor = 1e-3 * max(np.max(np.abs(r["dQ"])), np.max(np.abs(c["dK"])), np.max(np.abs(c["dV"])))
        check_grad(got["dq"][b, h, rows], r["dQ"], f"dQ[{b},{h}]", floor)
        check_grad(got["dk"][b, h, cols], c["dK"], f"dK[{b},{h}]", floor)
        check_grad(got["dv"][b, h, cols], c["dV"], f"dV[{b},{h}]", floor)
        say(f"  head ({b},{h}) ok")

    if bwd:
        # Gradient identities on every head, whole outputs.
        do64 = oracle.widen_bf16(inp["do"])
        sk = got["dk"].sum(axis=2)
        mk = np.abs(got["dk"]).sum(axis=2)
        sv = got["dv"].sum(axis=2) - do64.sum(axis=2)
        mv = np.abs(got["dv"]).sum(axis=2)
        wk, wv = float(np.max(np.abs(sk) / (mk + 1e-30))), float(np.max(np.abs(sv) / (mv + 1e-30)))
        say(f"  identities: worst |sum dK| / mass {wk:.2e}, worst |sum dV - sum dO| / mass {wv:.2e}")
        assert np.all(np.abs(sk) <= IDENTITY_REL * mk + 1e-6), f"sum_j dK_j != 0: worst {wk:.3e}"
        assert np.all(np.abs(sv) <= IDENTITY_REL * mv + 1e-6), f"sum_j dV_j != sum_i dO_i: worst {wv:.3e}"
