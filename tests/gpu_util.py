"""Helpers of the GPU parity tests."""
import numpy as np
import pytest
import torch

BF16_TOL = 1e-2   # atol = rtol for bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # atol = rtol for the fp32 path


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def swa():
    """The HIP binding; a missing library is an error, never a skip."""
    import hybrid_sliding_window_swa_amd as m
    m.load_library()
    return m


def assert_close(got, ref, tol, what=""):
    """Elementwise |got - ref| <= tol + tol * |ref| (numpy float64 ref)."""
    got = got.detach().float().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    excess = err - (tol + tol * np.abs(ref))
    if excess.max() > 0:
        idx = np.unravel_index(np.argmax(excess), excess.shape)
        raise AssertionError(f"{what}: max excess {excess.max():.3e} at {idx} "
                             f"(got {got[idx]:.6f}, ref {ref[idx]:.6f}); max abs err {err.max():.3e}")
    return float(err.max())


def rel_l2(got, ref):
    got = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
