"""Expected (query tile, key tile) visit maps, from the element-level rule.

A tile pair must be visited exactly when it contains at least one visible
(query, key) pair with both indices < N; visibility is the attention mask:
causal (key <= query) and, if given, the 128 x 128 block mask of the head.
This is computed element by element (no tile-level shortcut), so it checks
the kernels' skip predicates rather than restating them.
"""
import numpy as np


def element_keep(N, causal, mask_h=None, mask_block=128):
    i = np.arange(N)
    keep = np.ones((N, N), dtype=bool)
    if causal:
        keep &= i[None, :] <= i[:, None]
    if mask_h is not None:
        blk = i // mask_block
        keep &= np.asarray(mask_h)[blk[:, None], blk[None, :]] != 0
    return keep


def tile_any(keep, bm, bn):
    """[N, N] bool -> [ceil(N/bm), ceil(N/bn)] uint8: any element set."""
    N = keep.shape[0]
    nq, nk = -(-N // bm), -(-N // bn)
    pad = np.zeros((nq * bm, nk * bn), dtype=bool)
    pad[:N, :N] = keep
    return pad.reshape(nq, bm, nk, bn).any(axis=(1, 3)).astype(np.uint8)


def expected_visits(N, bm, bn, causal, mask=None, H=1, mask_block=128, key_major=False):
    """uint8 [H, nq, nk] (or [H, nk, nq] with key_major) expected visit map."""
    out = []
    for h in range(H):
        keep = element_keep(N, causal, None if mask is None else mask[h], mask_block)
        t = tile_any(keep, bm, bn)
        if key_major:
            t = tile_any(keep.T, bn, bm)
        out.append(t)
    return np.stack(out)
