"""Helpers for the GPU parity tests: device transfer of bf16 bit patterns and
the tolerance check. No arithmetic of the method lives here."""
import numpy as np
import torch

# bf16 outputs: max |diff| <= 2e-2 and ||diff||_2 / ||ref||_2 <= 1e-2; fp32 outputs: 1e-5 for both.
BF16_ATOL, BF16_REL = 2e-2, 1e-2
F32_ATOL, F32_REL = 1e-5, 1e-5


def dev(x: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> torch.bfloat16 on the GPU; float32 -> float32 on the GPU."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    if x.dtype == np.float32:
        return torch.from_numpy(x).cuda()
    raise TypeError(x.dtype)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a GPU tensor (uint16 for 2-byte, uint32 for 4-byte elements)."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a GPU bf16/fp32 tensor to float64."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.numpy().astype(np.float64)


def check_close(got, ref, bf16=True, name="", mask=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    atol, rel = (BF16_ATOL, BF16_REL) if bf16 else (F32_ATOL, F32_REL)
    d = got - ref
    maxabs = float(np.max(np.abs(d))) if d.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel_l2 = float(np.linalg.norm(d) / nrm) if nrm > 0 else float(np.linalg.norm(d))
    assert maxabs <= atol and rel_l2 <= rel, f"{name}: max|d|={maxabs:.3e} (<= {atol}), rel_l2={rel_l2:.3e} (<= {rel})"
    return maxabs, rel_l2
