"""CPU checks of the torch wrapper's argument validation: every size the
kernels read or write through is checked before a pointer reaches the C
ABI. Tensors on the "meta" device carry shape and dtype without storage, so
the checks run here without a GPU."""
import pytest
import torch

from exact_io_aware_69_amd import attention as A

META = torch.device("meta")


def t(shape, dtype=torch.float32, device=META):
    return torch.empty(shape, dtype=dtype, device=device)


def test_mask_checks():
    H, N = 3, 300  # nb = 3
    A._check_mask(None, H, N, META)
    A._check_mask(t((H, 3, 3), torch.uint8), H, N, META)
    with pytest.raises(ValueError, match="shape"):
        A._check_mask(t((3, 3), torch.uint8), H, N, META)  # [nb, nb] with H > 1
    with pytest.raises(ValueError, match="shape"):
        A._check_mask(t((H, 2, 3), torch.uint8), H, N, META)
    with pytest.raises(ValueError, match="dtype"):
        A._check_mask(t((H, 3, 3), torch.bool), H, N, META)
    with pytest.raises(ValueError, match="expected a tensor on"):
        A._check_mask(t((H, 3, 3), torch.uint8, "cpu"), H, N, META)  # a host mask
    with pytest.raises(ValueError, match="contiguous"):
        A._check_mask(t((H, 3, 3), torch.uint8).transpose(1, 2), H, N, META)
    with pytest.raises(ValueError, match="tensor"):
        A._check_mask([[1]], H, N, META)


def test_lse_checks():
    A._check_lse(t((2, 3, 5)), 2, 3, 5, META)
    with pytest.raises(ValueError, match="dtype"):
        A._check_lse(t((2, 3, 5), torch.float16), 2, 3, 5, META)
    with pytest.raises(ValueError, match="shape"):
        A._check_lse(t((2, 3, 4)), 2, 3, 5, META)
    with pytest.raises(ValueError, match="contiguous"):
        A._check_lse(t((2, 5, 3)).transpose(1, 2), 2, 3, 5, META)
    with pytest.raises(ValueError, match="expected a tensor on"):
        A._check_lse(t((2, 3, 5), device="cpu"), 2, 3, 5, META)


def test_output_and_workspace_checks():
    q = t((1, 2, 8, 64), torch.bfloat16)
    A._check_like(t((1, 2, 8, 64), torch.bfloat16), "out", q)
    with pytest.raises(ValueError, match="shape"):
        A._check_like(t((1, 2, 8, 128), torch.bfloat16), "out", q)
    with pytest.raises(ValueError, match="dtype"):
        A._check_like(t((1, 2, 8, 64), torch.float16), "out", q)
    A._check_workspace(t((100,), torch.uint8), 100, META)
    with pytest.raises(ValueError, match="need"):
        A._check_workspace(t((99,), torch.uint8), 100, META)
    with pytest.raises(ValueError, match="contiguous"):
        A._check_workspace(t((100,), torch.uint8, "cpu"), 100, META)


def test_inputs_must_be_device_bf16():
    with pytest.raises(ValueError):
        A.forward(t((1, 1, 8, 64), torch.bfloat16, "cpu"), t((1, 1, 8, 64), torch.bfloat16, "cpu"),
                  t((1, 1, 8, 64), torch.bfloat16, "cpu"))
