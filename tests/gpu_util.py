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


# Gradients.  The pages state no tolerance for a backward pass.  Per element:
# the forward's bf16 bar, 2e-2 + 1e-2 |ref|, with its absolute part scaled by
# the gradient tensor's RMS where that exceeds 1 (a gradient's size grows
# with T and the group size, the forward's outputs are O(1)) and raised to
# twice the worst error of the pages' module run in bf16 by PyTorch
# (``yard``, tests/bf16_module.py) where that is larger -- what bf16
# arithmetic itself costs on that input -- plus the fp32 bar 1e-4 for exact
# zeros.  Per tensor (or slice): a relative L2 error of at most 1e-2, which
# is what catches a systematic mistake in a tensor of small elements, raised
# to twice the module's where that is larger (the four lambda-vector
# gradients of V1 share one scalar, a sum over every row with cancellation).
GRAD_REL_L2 = 1e-2


def assert_grad_close(got, ref: np.ndarray, what: str = "", yard=None, rel_l2_max: float = GRAD_REL_L2):
    g = host64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    scale = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    atol = BF16_ATOL * max(1.0, scale)
    if yard is not None:
        y = host64(yard) if isinstance(yard, torch.Tensor) else np.asarray(yard, dtype=np.float64)
        y = y.reshape(ref.shape)
        atol = max(atol, 2.0 * float(np.abs(y - ref).max()))
        if scale > 0:
            rel_l2_max = max(rel_l2_max, 2.0 * float(np.sqrt(np.sum((y - ref) ** 2)) / np.sqrt(np.sum(ref * ref))))
    excess = np.abs(g - ref) - (atol + BF16_RTOL * np.abs(ref) + FP32_ATOL)
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    assert excess.max() <= 0, (f"{what}: element {worst} got {g[worst]:.6f} ref {ref[worst]:.6f} "
                               f"(excess {excess.max():.3e}, absolute bar {atol:.3e}, tensor rms {scale:.3e})")
    if scale > 0:
        rl = float(np.sqrt(np.sum((g - ref) ** 2)) / np.sqrt(np.sum(ref * ref)))
        assert rl <= rel_l2_max, f"{what}: relative L2 error {rl:.3e} > {rel_l2_max}"
        return rl
    return 0.0
