"""Helpers for the GPU parity tests: move seeded bf16 bits to the device and
apply the parity bars.

Bars (stated for bf16 inputs, fp32 accumulation):
  * O and lse: max |gpu - oracle| <= 2e-2 and <= 1e-2 * max |oracle|
    (both must hold); lse -inf entries must match exactly.
  * dQ, dK, dV: max |gpu - oracle| / max |oracle| <= 5e-2 per tensor.
  * visit maps: exact equality.
"""
import numpy as np
import torch

O_ABS, O_REL, G_REL = 2e-2, 1e-2, 5e-2


def dev(bits):
    """uint16 bf16 bits (numpy) -> contiguous bf16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0").contiguous()


def host64(t):
    """bf16/fp32 device tensor -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_o(got, ref, what="O"):
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    bound = min(O_ABS, O_REL * float(np.max(np.abs(ref)))) if ref.size else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"
    return err


def check_lse(got, ref, what="lse"):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: -inf pattern differs"
    assert np.all(got[~fin] == -np.inf), f"{what}: expected -inf for rows with no visible key"
    if fin.any():
        return check_o(got[fin], ref[fin], what)
    return 0.0


def check_grad(got, ref, what, floor=0.0):
    """Normalised error max|got - ref| / max|ref|. ``floor`` is a lower bound
    for the denominator: a gradient whose exact value is (nearly) zero, e.g.
    dQ when every key is identical or N = 1, is judged against the scale of
    the call's other gradients instead of against 0."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    den = max(float(np.max(np.abs(ref))) if ref.size else 0.0, floor)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        assert err == 0.0, f"{what}: expected exact zeros, max {err}"
        return 0.0
    assert err / den <= G_REL, f"{what}: normalised err {err / den:.3e} > {G_REL}"
    return err / den


def check_grads(got, ref):
    """dQ, dK, dV against the oracle dict; the denominator floor is 1e-3 of
    the largest of the three reference gradients."""
    scale = max(float(np.max(np.abs(ref[n]))) for n in ("dQ", "dK", "dV"))
    return [check_grad(g, ref[n], n, 1e-3 * scale) for g, n in zip(got, ("dQ", "dK", "dV"))]


def say(msg):
    print(msg, flush=True)
