"""Shared helpers for the GPU parity tests."""
import json
import os

import numpy as np

# Tolerance for bf16 inputs with fp32 accumulation against the fp64 oracle:
# max-abs 2e-2 and mean-abs 2e-3 on O, LSE, dq, dk and dv.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_round(x):
    """Round float64 values to the nearest bf16 value, ties to even, in one
    step (no intermediate fp32 rounding).  Normal range only, which is all
    the attention outputs reach."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # x = m 2^e, 0.5 <= |m| < 1: 8 significant bits below 2^e
    ulp = np.ldexp(1.0, e - 8)
    return np.where(x == 0, 0.0, np.rint(x / ulp) * ulp)


def parity_stats(got, ref, max_abs=MAX_ABS, out_bf16=False):
    """(passing mask, max-abs error, mean-abs error, elements that pass only
    by the bf16 output clause).

    The bar bounds the kernel's error before its output's own final rounding
    (the reading written down with the tolerances): an element passes when
    |got - ref| <= max_abs, or, for a bf16 output, when got is the bf16
    rounding of some value within max_abs of ref, that is
    bf16(ref - max_abs) <= got <= bf16(ref + max_abs).  The second clause
    admits at most half a bf16 unit in the last place of got beyond the
    absolute bar (2^-9 |got| at most); it decides only where the output's
    rounding takes a large share of the bar (|ref| of 2 and more)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    ok = err <= max_abs
    only_rounding = 0
    if out_bf16:
        within = (got >= bf16_round(ref - max_abs)) & (got <= bf16_round(ref + max_abs))
        only_rounding = int(np.count_nonzero(within & ~ok))
        ok = ok | within
    mx = float(err.max()) if err.size else 0.0
    mn = float(err.mean()) if err.size else 0.0
    return ok, mx, mn, only_rounding


def assert_parity(got, ref, name, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """Element-by-element comparison with the oracle.  `got` is a numpy array
    or a torch tensor; a bf16 tensor is judged as a bf16 output (see
    parity_stats).  max_abs is a number or an array of per-element bars
    (broadcast against ref).  The mean-abs bar is taken over |got - ref| as
    it stands."""
    out_bf16 = False
    if hasattr(got, "detach"):
        import torch

        out_bf16 = got.dtype == torch.bfloat16
        got = to64(got)
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s has non-finite values" % name
    ok, mx, mn, only_rounding = parity_stats(got, ref, max_abs, out_bf16)
    log = os.environ.get("PARITY_LOG")
    if log:
        with open(log, "a") as fh:
            fh.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", ""), "name": name, "n": int(ok.size),
                                 "max_abs": mx, "mean_abs": mn, "only_by_rounding": only_rounding}) + "\n")
    bad = int(ok.size - np.count_nonzero(ok))
    bar = "%.1e" % max_abs if np.ndim(max_abs) == 0 else "per element, up to %.2e" % float(np.max(max_abs))
    assert bad == 0 and mn <= mean_abs, (
        "%s: %d elements outside the bar; max-abs %.3e (bar %s%s), mean-abs %.3e (bar %.1e)" % (
            name, bad, mx, bar, " before bf16 output rounding" if out_bf16 else "", mn, mean_abs))
    if only_rounding:
        print("  %s: %d of %d elements within the bar only before their bf16 output rounding (max-abs %.3e)" % (
            name, only_rounding, ok.size, mx), flush=True)
    return mx, mn


def gpu_available():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False
