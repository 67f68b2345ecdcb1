"""Which kernels the library launches for each workload shape (MI355X, 256 CUs).

The results do not depend on these choices (the parity tests force every schedule through
the test variables), but their speed does, and a test variable left unset can silently send
a test down another path than the one it means to cover.  Each case runs one call under
torch's profiler and compares the kernels it launched with the schedule the library's
rules give on 256 CUs:
* attention, head_dim 128: 256-row tiles (8 waves) when the key range has more than 16
  blocks of 64 and the 128-row tiles would be more than one per CU; two key groups per
  8-wave workgroup when the 128-row tiles are at most one per CU; 4-wave workgroups
  otherwise; the split ("stream-K") second launch only for a short last round of long tiles;
* attention, head_dim 64: 4-wave workgroups;
* merge: the row kernel for P in {2, 4, 8} and D in {64, 128}, the LDS kernel otherwise or
  with DTL_MERGE_KERNEL=lds.
"""
import os

import pytest
import torch

from gpu_helpers import kernels_run, log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(autouse=True)
def clean_env():
    names = ("DTL_ATTN_SLOTS", "DTL_ATTN_WAVES", "DTL_ATTN_KEYSPLIT", "DTL_ATTN_SPLIT",
             "DTL_ATTN_MAX_POLLS", "DTL_MERGE_KERNEL")
    saved = {n: os.environ.pop(n, None) for n in names}
    yield os.environ
    for n in names:
        os.environ.pop(n, None)
        if saved[n] is not None:
            os.environ[n] = saved[n]


@pytest.fixture(scope="module", autouse=True)
def cus_256():
    cus = torch.cuda.get_device_properties(DEV).multi_processor_count
    if cus != 256:
        pytest.skip("expected schedules are those of a 256-CU GPU (this one has %d)" % cus)


def _qkv(Nq, Nkv, H, D, B=1):
    g = torch.Generator(device=DEV).manual_seed(Nq + Nkv + H)
    q = torch.randn(B, Nq, H, D, device=DEV, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Nkv, H, D, device=DEV, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Nkv, H, D, device=DEV, generator=g).to(torch.bfloat16)
    return q, k, v


def _check(name, fn, want, prefix="attn_fwd_kernel<"):
    got = {x for x in kernels_run(fn) if x.startswith(prefix)}
    log("%-40s %s" % (name, ", ".join(sorted(got))))
    assert got == set(want), "%s: launched %s, expected %s" % (name, sorted(got), sorted(want))


def K(d, nw, kg, f32, acc, split):
    return "attn_fwd_kernel<%d, %d, %d, %s, %s, %s>" % (
        d, nw, kg, *("true" if x else "false" for x in (f32, acc, split)))


ATTN_CASES = [
    # name, Nq, Nkv, H, D, expected kernels (bf16 output)
    # 432 256-row tiles: 1.69 rounds, remainder too large to split
    ("FLUX 4608 x 4608, 24 heads", 4608, 4608, 24, 128, [K(128, 8, 1, 0, 0, 0)]),
    # 2568 256-row tiles = 10 rounds + 8: the remainder's key blocks split over the GPU
    ("Wan2.2-5B 27280 x 27280, 24 heads", 27280, 27280, 24, 128,
     [K(128, 8, 1, 0, 0, 0), K(128, 8, 1, 0, 0, 1)]),
    # 8 key blocks: 4-wave workgroups
    ("cross-attention 27280 x 512", 27280, 512, 24, 128, [K(128, 4, 1, 0, 0, 0)]),
    # 16 key blocks: still 4-wave
    ("27280 x 1024", 27280, 1024, 24, 128, [K(128, 4, 1, 0, 0, 0)]),
    # 216 128-row tiles, at most one per CU: two key groups
    ("Ring-4 chunk 1152 x 1152, 24 heads", 1152, 1152, 24, 128, [K(128, 8, 2, 0, 0, 0)]),
    ("1152 x 4608, 24 heads", 1152, 4608, 24, 128, [K(128, 8, 2, 0, 0, 0)]),
    # 432 128-row tiles (more than one per CU), 216 256-row ones: 8 waves
    ("2304 x 4608, 24 heads", 2304, 4608, 24, 128, [K(128, 8, 1, 0, 0, 0)]),
    # head_dim 64: 4-wave workgroups
    ("head_dim 64, 4608 x 4608", 4608, 4608, 24, 64, [K(64, 4, 1, 0, 0, 0)]),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: c[0])
def test_attention_schedule(case):
    import diffusion_transformer_long_amd as dtl
    name, Nq, Nkv, H, D, want = case
    q, k, v = _qkv(Nq, Nkv, H, D)
    want = list(want)
    if any(w.endswith("true>") for w in want):
        want.append("advance_launch_count_kernel")
        _check(name, lambda: dtl.attn_fwd_lse(q, k, v), want, prefix="")
    else:
        _check(name, lambda: dtl.attn_fwd_lse(q, k, v), want)


def test_ring4_share_forms_schedule():
    """The FLUX Ring-4 share (1152 queries, 4 chunks of 1152 keys): all chunks in one launch
    take 256-row tiles (480 of them, 18 key blocks each); the per-round calls and the
    accumulated rounds take two key groups; the merge takes the row kernel."""
    import diffusion_transformer_long_amd as dtl
    q, k, v = _qkv(1152, 4608, 24, 128)
    _check("Ring-4 all chunks in one launch", lambda: dtl.attn_fwd_lse_kv_chunks(q, k, v, 4),
           [K(128, 8, 1, 1, 0, 0)])
    _check("Ring-4 default step (one launch + merge)", lambda: dtl.ring_attention(q, k, v, 4),
           [K(128, 8, 1, 1, 0, 0), "merge_rows_kernel<true, false, 4, 16>"], prefix="")
    _check("Ring-4 per-round calls + merge", lambda: dtl.ring_attention(q, k, v, 4, one_launch=False),
           [K(128, 8, 2, 1, 0, 0), "merge_rows_kernel<true, false, 4, 16>"], prefix="")
    _check("Ring-4 accumulated rounds", lambda: dtl.ring_attention(q, k, v, 4, accumulate=True),
           [K(128, 8, 2, 1, 0, 0), K(128, 8, 2, 1, 1, 0), K(128, 8, 2, 0, 1, 0)])


def test_split_variables_reach_the_split():
    """DTL_ATTN_SLOTS alone does not split a grid of at most one 128-row tile per CU: two key
    groups take it first.  With DTL_ATTN_KEYSPLIT=0 as well, 4-wave tiles and the split
    launch run (the setting the split-schedule tests use)."""
    import diffusion_transformer_long_amd as dtl
    q, k, v = _qkv(1152, 4100, 1, 128)
    os.environ["DTL_ATTN_SLOTS"] = "8"
    os.environ["DTL_ATTN_WAVES"] = "4"
    _check("slots 8, 4 waves", lambda: dtl.attn_fwd_lse(q, k, v), [K(128, 8, 2, 0, 0, 0)])
    os.environ["DTL_ATTN_KEYSPLIT"] = "0"
    _check("slots 8, 4 waves, no key groups", lambda: dtl.attn_fwd_lse(q, k, v),
           [K(128, 4, 1, 0, 0, 0), K(128, 4, 1, 0, 0, 1), "advance_launch_count_kernel"], prefix="")


@pytest.mark.parametrize("P,D,want", [
    (4, 128, "merge_rows_kernel<true, false, 4, 16>"),
    (8, 128, "merge_rows_kernel<true, false, 8, 16>"),
    (2, 64, "merge_rows_kernel<true, false, 2, 8>"),
    (3, 128, "merge_kernel<true, false>"),
    (4, 32, "merge_kernel<true, false>"),
])
def test_merge_schedule(P, D, want):
    import diffusion_transformer_long_amd as dtl
    o_p = torch.randn(P, 1, 300, 4, D, device=DEV)
    l_p = torch.randn(P, 1, 4, 300, device=DEV)
    _check("merge P=%d D=%d" % (P, D), lambda: dtl.attn_merge_lse(o_p, l_p), [want], prefix="merge")
    os.environ["DTL_MERGE_KERNEL"] = "lds"
    _check("merge P=%d D=%d, DTL_MERGE_KERNEL=lds" % (P, D), lambda: dtl.attn_merge_lse(o_p, l_p),
           ["merge_kernel<true, false>"], prefix="merge")
