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
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()
                and t.dim() == 4):
            raise ValueError("expected contiguous bf16 device tensors of shape [B, H, N, d]")
    shape, device = ts[0].shape, ts[0].device
    for t in ts[1:]:
        if t.shape != shape:
            raise ValueError("q, k, v (and o, dO) must have the same shape")
        if t.device != device:
            raise ValueError("q, k, v (and o, dO) must be on the same device")


# The C ABI sees only pointers: every size the kernels read or write through
# is checked here, so a wrongly shaped, typed or placed tensor is an error
# instead of an out-of-bounds access on the device.
def _check_tensor(t, what, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a torch tensor")
    if t.device != device:
        raise ValueError(f"{what}: expected a tensor on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{what}: expected dtype {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous tensor")


def _check_mask(block_mask, H, N, device):
    """block_mask: uint8 [H, nb, nb] on the inputs' device, nb = ceil(N / 128)."""
    if block_mask is not None:
        nb = -(-N // 128)
        _check_tensor(block_mask, "block_mask", (H, nb, nb), torch.uint8, device)


def _check_lse(lse, B, H, N, device):
    _check_tensor(lse, "lse", (B, H, N), torch.float32, device)


def _check_like(t, what, like):
    _check_tensor(t, what, like.shape, like.dtype, like.device)


def _check_workspace(ws, nbytes, device):
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace: expected a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace: {ws.numel() * ws.element_size()} bytes, need {nbytes}")


def _stream():
    return torch.cuda.current_stream().cuda_stream


def forward(q, k, v, causal: bool = False, scale: float | None = None, block_mask=None, out=None, lse=None):
    """Returns (o, lse). ``block_mask``: uint8 device tensor [H, nb, nb] or None."""
    _check_inputs(q, k, v)
    B, H, N, d = q.shape
    _check_mask(block_mask, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is not None:
        _check_like(out, "out", q)
    if lse is not None:
        _check_lse(lse, B, H, N, q.device)
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
    _check_lse(lse, B, H, N, q.device)
    _check_mask(block_mask, H, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _check_workspace(workspace, nbytes, q.device)
    if grads is not None:
        if len(grads) != 3:
            raise ValueError("grads: expected (dq, dk, dv)")
        for g, n in zip(grads, ("dq", "dk", "dv")):
            _check_like(g, n, q)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dO.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal, scale)
    ws_bytes = workspace.numel() * workspace.element_size()
    if block_mask is None:
        st = _lib.fa_bwd(*args, workspace.data_ptr(), ws_bytes, _stream())
    else:
        st = _lib.fa_bwd_blocksparse(*args, block_mask.data_ptr(), workspace.data_ptr(), ws_bytes, _stream())
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
    _check_mask(block_mask, H, N, q.device)
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
    _check_lse(lse, B, H, N, q.device)
    _check_mask(block_mask, H, N, q.device)
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
