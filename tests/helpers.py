"""Shared helpers for the GPU parity tests."""
import numpy as np

# Tolerance for bf16 inputs with fp32 accumulation against the fp64 oracle:
# max-abs 2e-2 and mean-abs 2e-3 on O, LSE, dq, dk and dv.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(got, ref, name, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s has non-finite values" % name
    err = np.abs(got - ref)
    mx, mn = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    assert mx <= max_abs and mn <= mean_abs, "%s: max-abs %.3e (bar %.1e), mean-abs %.3e (bar %.1e)" % (
        name, mx, max_abs, mn, mean_abs)
    return mx, mn


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False
