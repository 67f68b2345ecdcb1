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


def worst_element(got, ref):
    """Index (a tuple over the array's axes) and values of the largest |got - ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    idx = np.unravel_index(int(np.argmax(d)), d.shape)
    return tuple(int(i) for i in idx), float(got[idx]), float(ref[idx])


def assert_close(name, got, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS, labels=None):
    """Max-abs and mean-abs error of got against ref within the bar; the log line names
    the worst element (its index along the array's axes, or `labels` of that index)."""
    mx, mn = errs(got, ref)
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2))) or 1.0
    idx, g, r = worst_element(got, ref)
    where = labels(idx) if labels is not None else str(idx)
    log("  %-28s max-abs %.3e  mean-abs %.3e  (rel to rms %.2e; %d values; worst at %s: %.6g vs %.6g)"
        % (name, mx, mn, mx / rms, np.asarray(ref).size, where, g, r))
    assert mx <= max_abs, "%s: max-abs %.3e > %.1e at %s" % (name, mx, max_abs, where)
    assert mn <= mean_abs, "%s: mean-abs %.3e > %.1e" % (name, mn, mean_abs)


def to_np(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def rne_bf16(x):
    """float64 -> the nearest bf16 value (ties to even), as float64, for normal values."""
    m, e = np.frexp(np.asarray(x, np.float64))   # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def ulp_bf16(x):
    """Spacing of bf16 values (8 significant bits) at |x|."""
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, e - 8)


def assert_bf16_rounding_of(name, got, ref, f32_err, min_exact=0.99):
    """got is ref computed in f32 (absolute error at most f32_err, per element) and
    rounded once to bf16 to nearest even: every element within half a bf16 ulp of the
    larger of |got|, |ref| plus f32_err, and at least min_exact of them equal to the
    correctly rounded bf16 of ref (the f32 error can only flip the rounding of values
    next to a midpoint; truncation instead of rounding would fail this)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), "non-finite values in the GPU result"
    bound = 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref))) + f32_err
    ratio = np.abs(got - ref) / bound
    idx, g, r = worst_element(ratio, np.zeros_like(ratio))
    exact = float(np.mean(got == rne_bf16(ref)))
    log("  %-28s max %.3f of the bound (at %s: %.6g vs %.6g), %.4f%% correctly rounded (%d values)"
        % (name, float(ratio.max()), idx, got[idx], ref[idx], 100 * exact, got.size))
    assert ratio.max() <= 1.0, "%s: %.3f of the bound at %s" % (name, float(ratio.max()), idx)
    assert exact >= min_exact, "%s: only %.4f correctly rounded" % (name, exact)


def check_bf16_is_rounded_f32(name, o_bf16, o_f32, o_ref):
    """For outputs whose |O| passes 2 (FLUX: max|O_ref| = 4.004), where one bf16 rounding
    alone can cost up to 0.0156 > 1e-2: the f32 output carries the bar (checked by the
    caller); the bf16 output must be exactly its round-to-nearest-even, element for
    element.  Its distance from the oracle is reported."""
    import torch
    rounded = o_f32.to(torch.bfloat16)
    same = o_bf16.view(torch.int16) == rounded.view(torch.int16)
    n_bad = int((~same).sum())
    d = np.abs(to_np(o_bf16) - o_ref)
    log("  %-28s bf16 == RNE(f32 output) for %d of %d values; bf16 vs oracle max-abs %.3e mean-abs %.3e"
        % (name, same.numel() - n_bad, same.numel(), float(d.max()), float(d.mean())))
    assert n_bad == 0, "%s: %d bf16 values differ from the rounded f32 output" % (name, n_bad)


def kernels_run(fn):
    """Names of the GPU kernels fn() launches, as torch's profiler records them, shortened
    to the name and template arguments (for example 'attn_fwd_kernel<128, 4, 1, false,
    false, true>')."""
    import re
    import torch
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    out = set()
    for e in prof.events():
        m = re.search(r"(\w+_kernel(?:<[^()]*>)?)\(", e.name)
        if m:
            out.add(m.group(1))
    return out
