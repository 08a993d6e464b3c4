"""Helpers for the GPU parity tests: host arrays <-> device tensors and the
per-row tolerance max_j |gpu - ref| <= 2e-3 * ||ref_row||_2."""
import numpy as np
import torch

REL = 2e-3


def dev(x: np.ndarray) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:   # bf16 bit patterns
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def dev_f16(bits: np.ndarray) -> torch.Tensor:
    """binary16 bit patterns (uint16) -> float16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype in (torch.float16, torch.float32):
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_rows_close(gpu: np.ndarray, ref: np.ndarray, rel: float = REL, what: str = ""):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    norm = np.linalg.norm(ref, axis=1)
    err = np.abs(gpu - ref).max(axis=1) if ref.shape[1] else np.zeros(ref.shape[0])
    zero = norm == 0
    assert np.all(gpu[zero] == 0), f"{what}: rows with zero reference are not zero"
    bad = ~zero & (err > rel * norm)
    if np.any(bad):
        i = int(np.nonzero(bad)[0][0])
        raise AssertionError(f"{what}: {int(bad.sum())} rows exceed tolerance; row {i}: "
                             f"err {err[i]:.3e} > {rel} * {norm[i]:.3e}")
