"""Helpers for the GPU parity tests: tolerance checks and host copies."""
import numpy as np
import torch

# Tolerances the method is held to: fp32 inputs -> max abs error 1e-4;
# bf16 inputs with fp32 accumulation -> |x - ref| <= 2e-2 + 1e-2 |ref| per
# element (allclose form).
FP32_ATOL = 1e-4
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def assert_fp32_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    g = host64(got)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref).max()
    assert err <= FP32_ATOL, f"{what}: max abs error {err:.3e} > {FP32_ATOL}"
    return err


def assert_bf16_close(got, ref: np.ndarray, what: str = ""):
    g = host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    excess = np.abs(g - ref) - (BF16_ATOL + BF16_RTOL * np.abs(ref))
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, (f"{what}: element {worst} got {g[worst]:.6f} ref {ref[worst]:.6f} "
                               f"(excess {excess.max():.3e})")
    return np.abs(g - ref).max()


def rel_l2(got, ref: np.ndarray, axis) -> np.ndarray:
    """Relative L2 error per slice (reduced over ``axis``)."""
    g = host64(got) if isinstance(got, torch.Tensor) else got
    num = np.sqrt(np.sum((g - ref) ** 2, axis=axis))
    den = np.sqrt(np.sum(ref ** 2, axis=axis))
    return num / np.maximum(den, 1e-30)
