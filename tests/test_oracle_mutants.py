"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case copies oracle.c, plants one plausible slip (a dropped scale, a wrong
stride or index, a transposed operand, a sign, a missing normalisation), builds
the copy with the host compiler into a temporary directory and runs every pin
of tests/test_oracle_pins.py against it.  At least one pin must fail.  The real
oracle.c is never modified.
"""
import inspect
import os

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "dropped_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "k_row_stride_D": ("const double *kj = kbase + (long)j * row_stride;",
                       "const double *kj = kbase + (long)j * D;"),
    "v_replaced_by_k": ("const double *vj = vbase + (long)j * row_stride;",
                        "const double *vj = kbase + (long)j * row_stride;"),
    "no_normalisation": ("orow[d] /= l;", "orow[d] /= 1.0;"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "exp_sign": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "row_max_not_subtracted": ("            m = s[j];", "            m = 0.0;"),
    "head_offset_dropped": ("const double *kb = k + ((long)b * Nkv * H + h) * D;",
                            "const double *kb = k + ((long)b * Nkv * H) * D;"),
    "batch_stride_uses_nq": ("const double *vb = v + ((long)b * Nkv * H + h) * D;\n            double *orow",
                             "const double *vb = v + ((long)b * Nq * H + h) * D;\n            double *orow"),
    "lse_layout_transposed": ("orow, lse + ((long)b * H + h) * Nq + i);",
                              "orow, lse + ((long)b * Nq + i) * H + h);"),
    "merge_weight_unnormalised": ("double w = exp(lse_parts[t * part_l + li] - L);",
                                  "double w = exp(lse_parts[t * part_l + li] - M);"),
    "merge_lse_is_max": ("lse[li] = L;", "lse[li] = M;"),
    "merge_lse_index_o_order": ("long li = (b * H + h) * N + n;", "long li = (b * N + n) * H + h;"),
    "permute_token_from_dest": ("long di = (((j * B + b) * (long)N + (s * Ns + n))",
                                "long di = (((j * B + b) * (long)N + (j * Ns + n))"),
    "permute_heads_from_src": ("long si = (((s * B + b) * Ns + n) * H + (j * Hs + hh))",
                               "long si = (((s * B + b) * Ns + n) * H + (s * Hs + hh))"),
    "h2s_token_from_dest": ("long si = (((j * B + b) * (long)N + (s * Ns + n))",
                            "long si = (((j * B + b) * (long)N + (j * Ns + n))"),
    "h2s_head_group_from_src": ("long di = (((s * B + b) * Ns + n) * H + (j * Hs + hh))",
                                "long di = (((s * B + b) * Ns + n) * H + (s * Hs + hh))"),
    "qkv_output_tensor_major": ("long di = ((((j * 3 + c) * B + b)", "long di = ((((c * p + j) * B + b)"),
    "nr_norm_over_one_head": ("for (long e = 0; e < HD; ++e)\n                    ss += x[e] * x[e];",
                              "for (long e = 0; e < D; ++e)\n                    ss += x[e] * x[e];"),
    "nr_eps_outside_sqrt": ("1.0 / sqrt(ss / (double)HD + eps);", "1.0 / (sqrt(ss / (double)HD) + eps);"),
    "nr_gamma_k_for_q": ("c == 0 ? gamma_q : gamma_k;", "c == 0 ? gamma_k : gamma_k;"),
    "nr_sin_sign": ("y[h * D + 2 * i] = a * co - bb * si;", "y[h * D + 2 * i] = a * co + bb * si;"),
    "nr_position_within_shard": ("long t = s * Ns + n;\n        double *y", "long t = n;\n        double *y"),
    "nr_half_split_pairs": ("double a = y[h * D + 2 * i], bb = y[h * D + 2 * i + 1];",
                            "double a = y[h * D + i], bb = y[h * D + i + D / 2];"),
    "nr_rope_on_v": ("if (c < 2) {", "if (c < 3) {"),
    "qkv_source_always_q": ("* 3 + c) * H + (j * Hs + hh)) * D + d;", "* 3 + 0) * H + (j * Hs + hh)) * D + d;"),
}


def _all_pins():
    """(name, callable taking an Api) for every pin, parametrised cases expanded."""
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not params:
            out.append((name, lambda api, fn=fn: fn(api)))
            continue
        argnames, values = params[0].args[0], params[0].args[1]
        argnames = [a.strip() for a in argnames.split(",")]
        for val in values:
            val = val if len(argnames) > 1 else (val,)
            out.append((name, lambda api, fn=fn, val=val: fn(api, *val)))
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(mpath), out=str(tmp_path / "liboracle_mutant.so"))
    api = oracle.Api(lib)
    failed = []
    for name, run in _all_pins():
        try:
            run(api)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(name)
    assert failed, "no pin caught the planted mistake %s" % mutant


def test_unmutated_copy_passes_every_pin(tmp_path):
    lib = oracle.build(force=True, src=SRC, out=str(tmp_path / "liboracle_copy.so"))
    api = oracle.Api(lib)
    for name, run in _all_pins():
        run(api)
