"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module only *draws* data. It holds none of the attention arithmetic:
no scores, no softmax, no masking rule, no gradient. Both sides receive the
same bf16 bit patterns (uint16 arrays) and each widens them on its own.

Recipe (the pages fix only "i.i.d. N(0, 1) from a seed" and a 128x128 block
mask with off-diagonal keep probability 0.25 and every diagonal block kept):

* ``rng = numpy.random.default_rng(seed)``;
* tensors are drawn in the order q, k, v, dO, each with
  ``rng.standard_normal((B, H, N, d))`` in float64 (drawn in row chunks, which
  numpy's generator makes identical to one whole draw);
* float64 -> float32 with numpy's round-to-nearest-even cast, then
  float32 -> bfloat16 with round-to-nearest-even on the bit pattern;
* after the tensors, the block mask: ``u = rng.random((H, nb, nb))`` with
  ``nb = ceil(N / 128)``; a block is kept when ``u < p`` or it is diagonal.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "draw_bf16",
    "make_inputs",
    "make_block_mask",
    "CONFIGS",
]

MASK_BLOCK = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Only finite inputs occur here (normal draws), so no NaN special case.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> float32 (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw_bf16(rng: np.random.Generator, shape, chunk_rows: int = 1 << 16,
              gain: float = 1.0) -> np.ndarray:
    """Draw an N(0,1)*gain tensor of ``shape`` as bf16 bits, in row chunks.

    ``gain`` scales the float64 draw before rounding (used for the "peaky"
    stress input, where q is drawn larger so rows have a dominant key).
    """
    shape = tuple(int(s) for s in shape)
    last = shape[-1]
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    out = np.empty((rows, last), dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, last))
        if gain != 1.0:
            x = x * gain
        out[r0:r1] = f32_to_bf16_bits(x.astype(np.float32))
    return out.reshape(shape)


def make_block_mask(rng: np.random.Generator, H: int, N: int, p: float = 0.25,
                    block: int = MASK_BLOCK) -> np.ndarray:
    """uint8 [H, nb, nb] block mask, 1 = keep; diagonal blocks always kept."""
    nb = (N + block - 1) // block
    u = rng.random((H, nb, nb))
    keep = (u < p) | np.eye(nb, dtype=bool)[None, :, :]
    return keep.astype(np.uint8)


def make_inputs(seed: int, B: int, H: int, N: int, d: int, *, with_do: bool = True,
                sparse: bool = False, p: float = 0.25, q_gain: float = 1.0):
    """Seeded inputs as bf16 bits: dict with q, k, v (and dO, mask)."""
    rng = np.random.default_rng(seed)
    out = {"q": draw_bf16(rng, (B, H, N, d), gain=q_gain),
           "k": draw_bf16(rng, (B, H, N, d)),
           "v": draw_bf16(rng, (B, H, N, d))}
    if with_do or sparse:
        # dO is always drawn before the mask so the mask stream does not
        # depend on whether the caller wants gradients.
        do = draw_bf16(rng, (B, H, N, d))
        if with_do:
            out["do"] = do
    if sparse:
        out["mask"] = make_block_mask(rng, H, N, p=p)
    return out


# The five workloads: name -> shape and flags.
CONFIGS = {
    "cfg1_fwd_small": dict(B=1, H=2, N=256, d=64, causal=False, sparse=False, bwd=False),
    "cfg2_fwd_d64": dict(B=8, H=16, N=2048, d=64, causal=None, sparse=False, bwd=False),
    "cfg3_causal_d128": dict(B=4, H=16, N=4096, d=128, causal=True, sparse=False, bwd=True),
    "cfg4_long_d128": dict(B=1, H=16, N=16384, d=128, causal=True, sparse=False, bwd=True),
    "cfg5_blocksparse_d64": dict(B=2, H=16, N=8192, d=64, causal=False, sparse=True, bwd=True),
}
