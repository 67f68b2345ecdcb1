"""Shared helpers of the GPU parity tests: tolerances and error reporting."""
import sys

import numpy as np

# Floating-point bar on the same seeded bf16 inputs, for O and for LSE.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def errs(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    d = np.abs(got - ref)
    return float(d.max()), float(d.mean())


def assert_close(name, got, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    mx, mn = errs(got, ref)
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2))) or 1.0
    log("  %-28s max-abs %.3e  mean-abs %.3e  (rel to rms %.2e)" % (name, mx, mn, mx / rms))
    assert mx <= max_abs, "%s: max-abs %.3e > %.1e" % (name, mx, max_abs)
    assert mn <= mean_abs, "%s: mean-abs %.3e > %.1e" % (name, mn, mean_abs)


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
