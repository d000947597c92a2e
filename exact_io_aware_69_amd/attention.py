"""Torch-facing wrappers over the C ABI: allocate outputs, pass pointers.

PyTorch only provides device memory and the stream here; every step of the
computation runs in the HIP kernels of libfa.so. Inputs are bf16 CUDA
(ROCm) tensors of shape [B, H, N, d], contiguous.
"""
from __future__ import annotations

import math

import torch

from . import _lib


def _check_inputs(*ts):
    for t in ts:
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous() and t.dim() == 4):
            raise ValueError("expected contiguous bf16 device tensors of shape [B, H, N, d]")
    shape = ts[0].shape
    for t in ts[1:]:
        if t.shape != shape:
            raise ValueError("q, k, v (and o, dO) must have the same shape")


def _stream():
    return torch.cuda.current_stream().cuda_stream


def forward(q, k, v, causal: bool = False, scale: float | None = None, block_mask=None, out=None, lse=None):
    """Returns (o, lse). ``block_mask``: uint8 device tensor [H, nb, nb] or None."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    if block_mask is None:
        st = _lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, causal, scale, _stream())
    else:
        st = _lib.fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, causal, scale, block_mask.data_ptr(), _stream())
    _lib.check(st, "fa_fwd")
    return o, lse


def workspace_bytes(B, H, N, d) -> int:
    st, n = _lib.fa_bwd_workspace_size(B, H, N, d)
    _lib.check(st, "fa_bwd_workspace_size")
    return n


def backward(q, k, v, o, lse, dO, causal: bool = False, scale: float | None = None, block_mask=None,
             workspace=None, grads=None):
    """Returns (dq, dk, dv)."""
    _check_inputs(q, k, v, o, dO)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dO.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale)
    if block_mask is None:
        st = _lib.fa_bwd(*args, workspace.data_ptr(), workspace.numel(), _stream())
    else:
        st = _lib.fa_bwd_blocksparse(*args, block_mask.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                     _stream())
    _lib.check(st, "fa_bwd")
    return dq, dk, dv


def tile_config(pass_: int, d: int, causal: bool):
    st, bm, bn = _lib.fa_tile_config(pass_, d, causal)
    _lib.check(st, "fa_tile_config")
    return bm, bn


def forward_visits(q, k, v, causal, scale=None, block_mask=None):
    """Debug forward: returns (o, lse, visited[B, H, nQt, nKt] uint8)."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    bm, bn = tile_config(0, d, causal)
    vis = torch.zeros((B, H, -(-N // bm), -(-N // bn)), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = _lib.fa_fwd_debug_visits(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, N, d, causal, scale,
                                  None if block_mask is None else block_mask.data_ptr(), vis.data_ptr(), _stream())
    _lib.check(st, "fa_fwd_debug_visits")
    return o, lse, vis


def backward_visits(q, k, v, o, lse, dO, causal, scale=None, block_mask=None):
    """Debug backward: returns (dq, dk, dv, visited_kv, visited_q)."""
    _check_inputs(q, k, v, o, dO)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    bm1, bn1 = tile_config(1, d, causal)
    bm2, bn2 = tile_config(2, d, causal)
    vkv = torch.zeros((B, H, -(-N // bn1), -(-N // bm1)), dtype=torch.uint8, device=q.device)
    vq = torch.zeros((B, H, -(-N // bm2), -(-N // bn2)), dtype=torch.uint8, device=q.device)
    nbytes = workspace_bytes(B, H, N, d)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = _lib.fa_bwd_debug_visits(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  dO.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal,
                                  scale, None if block_mask is None else block_mask.data_ptr(), ws.data_ptr(),
                                  nbytes, vkv.data_ptr(), vq.data_ptr(), _stream())
    _lib.check(st, "fa_bwd_debug_visits")
    return dq, dk, dv, vkv, vq
