"""GPU parity of the attention kernel's split ("stream-K") schedule.

On the real GPU only large workloads reach it (more tiles than workgroup slots, a small
remainder, at least 64 key blocks per tile: Wan2.2-5B).  DTL_ATTN_SLOTS schedules as if the
GPU held fewer workgroups, which makes small shapes take the same path: whole tiles for
the first rounds, the remainder's 64-key blocks spread over the slots, pieces published
to the workspace and folded in by each tile's finaliser.  With DTL_ATTN_MAX_POLLS=0 every
finaliser gives up on its helpers at once and computes the rest of its tile itself (the
path taken when helpers are not resident in time); those runs must give the same result.
The cases cover a tile split
over 8 workgroups, ranges crossing tile boundaries, the ragged last key block inside a
split tile, B = 2, D = 64 and 128, 4- and 8-wave workgroups (DTL_ATTN_WAVES), bf16 and
f32 outputs, and the accumulate entry point with rows that hold no keys yet.  Every result
is compared with the oracle.  These grids hold at most one 128-row tile per CU, where the
library would run two key groups per workgroup (whole tiles only), so the 4-wave cases also
set DTL_ATTN_KEYSPLIT=0; the main cases check from torch's profiler that the split launch
ran exactly where the schedule splits.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import assert_close, kernels_run, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture
def slots():
    """DTL_ATTN_SLOTS, with DTL_ATTN_KEYSPLIT=0: these grids hold at most one 128-row tile
    per CU, where the library would otherwise run two key groups per workgroup (whole tiles
    only) instead of the 4-wave split schedule under test."""
    names = ("DTL_ATTN_SLOTS", "DTL_ATTN_KEYSPLIT")
    saved = {n: os.environ.get(n) for n in names}

    def set_slots(n):
        os.environ["DTL_ATTN_SLOTS"] = str(n)
        os.environ["DTL_ATTN_KEYSPLIT"] = "0"
    yield set_slots
    for n, val in saved.items():
        if val is None:
            os.environ.pop(n, None)
        else:
            os.environ[n] = val


@pytest.fixture
def polls():
    """DTL_ATTN_MAX_POLLS: how often a tile's finaliser polls its helpers' flags before it
    computes the rest of the tile itself (0: at once)."""
    old = os.environ.get("DTL_ATTN_MAX_POLLS")

    def set_polls(n):
        os.environ["DTL_ATTN_MAX_POLLS"] = str(n)
    yield set_polls
    if old is None:
        os.environ.pop("DTL_ATTN_MAX_POLLS", None)
    else:
        os.environ["DTL_ATTN_MAX_POLLS"] = old


@pytest.fixture
def waves():
    """DTL_ATTN_WAVES: the workgroup size (4 or 8 waves) for head_dim 128."""
    old = os.environ.get("DTL_ATTN_WAVES")

    def set_waves(n):
        os.environ["DTL_ATTN_WAVES"] = str(n)
    yield set_waves
    if old is None:
        os.environ.pop("DTL_ATTN_WAVES", None)
    else:
        os.environ["DTL_ATTN_WAVES"] = old


def _inputs(seed, B, Nq, Nkv, H, D, k_scale):
    g = np.random.Generator(np.random.PCG64(seed))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * np.float32(k_scale))
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    return q, k, v


CASES = [
    # slots, B, Nq, Nkv, H, D, k_scale      tiles / remainder, key blocks
    (8, 1, 1152, 4100, 1, 128, 1.0),       # 9 / 1, 65: one tile over 8 workgroups, ragged block
    (8, 2, 300, 4097, 3, 64, 2.0),         # 18 / 2, 65: ranges cross tiles
    (8, 1, 129, 64 * 66 + 7, 5, 128, 3.0),  # 10 / 2, 67
    (4, 1, 640, 4096, 1, 128, 1.0),        # 5 / 1, 64: 4 workgroups of 16 blocks
    (4, 1, 512, 4096, 1, 64, 1.0),         # 4 / 0: no split (control)
    (8, 1, 1152, 1000, 1, 128, 1.0),       # 9 / 1, 16: too few key blocks to split (control)
]


def _expect_split(n, B, Nq, Nkv, H, rows):
    """Whether the schedule splits: at least one full round of tiles over the n slots, a
    remainder of at most a quarter of them, at least 64 key blocks per tile."""
    tiles = -(-Nq // rows) * H * B
    rem = tiles % n
    return tiles >= n and rem > 0 and rem * 4 <= n and -(-Nkv // 64) >= 64


def _run_checked(fn, D, nw, split):
    """fn() under the profiler: the attention kernels it ran must be the D, nw-wave ones,
    with the split part (SPLIT = true) exactly when the schedule splits."""
    out = {}
    names = kernels_run(lambda: out.setdefault("r", fn()))
    attn = sorted(x for x in names if x.startswith("attn_fwd_kernel<"))
    log("  kernels: %s" % ", ".join(attn))
    assert attn and all(x.startswith("attn_fwd_kernel<%d, %d, 1," % (D, nw)) for x in attn), attn
    assert any(x.endswith("true>") for x in attn) == split, "split expected: %s, ran %s" % (split, attn)
    return out["r"]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "slots%d_B%d_Nq%d_Nkv%d_H%d_D%d" % c[:6])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_split_schedule_matches_oracle(slots, case, o_dtype):
    import diffusion_transformer_long_amd as dtl
    n, B, Nq, Nkv, H, D, ks = case
    log("split schedule slots=%d %s o=%s" % (n, case[1:], o_dtype))
    q, k, v = _inputs(3000 + Nq + Nkv, B, Nq, Nkv, H, D, ks)
    slots(n)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = _run_checked(lambda: dtl.attn_fwd_lse(qd, kd, vd, o_dtype=o_dtype), D, 4,
                          _expect_split(n, B, Nq, Nkv, H, 128))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("O", to_np(o), o_ref)
    assert_close("LSE", to_np(lse), l_ref)


# 8-wave workgroups (256-row tiles): the same paths with half as many tiles
CASES8 = [
    # slots, B, Nq, Nkv, H, D, k_scale      tiles / remainder, key blocks
    (4, 1, 1152, 4100, 1, 128, 1.0),       # 5 / 1, 65: a 128-row last tile over 4 workgroups
    (10, 2, 300, 4097, 3, 128, 2.0),       # 12 / 2, 65: ranges cross tiles
    (4, 1, 129, 64 * 66 + 7, 5, 128, 3.0),  # 5 / 1, 67: 129-row tiles
    (4, 1, 1024, 4096, 1, 128, 1.0),       # 4 / 0: no split (control)
]


@pytest.mark.parametrize("case", CASES8, ids=lambda c: "slots%d_B%d_Nq%d_Nkv%d_H%d_D%d" % c[:6])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_split_schedule_8_waves_matches_oracle(slots, waves, case, o_dtype):
    import diffusion_transformer_long_amd as dtl
    n, B, Nq, Nkv, H, D, ks = case
    log("split schedule, 8 waves, slots=%d %s o=%s" % (n, case[1:], o_dtype))
    q, k, v = _inputs(5000 + Nq + Nkv, B, Nq, Nkv, H, D, ks)
    slots(n)
    waves(8)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = _run_checked(lambda: dtl.attn_fwd_lse(qd, kd, vd, o_dtype=o_dtype), D, 8,
                          _expect_split(n, B, Nq, Nkv, H, 256))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("O", to_np(o), o_ref)
    assert_close("LSE", to_np(lse), l_ref)


@pytest.mark.parametrize("nw", [4, 8])
def test_split_schedule_accumulate(slots, waves, nw):
    """attn_fwd_lse_accumulate through the split schedule, rows without previous keys."""
    import diffusion_transformer_long_amd as dtl
    B, Nq, Np, Nkv, H, D = 1, 1152, 300, 4100, 1, 128
    g = np.random.Generator(np.random.PCG64(77))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    kp = synthetic.to_bf16(g.standard_normal((B, Np, H, D), dtype=np.float32))
    vp = synthetic.to_bf16(g.standard_normal((B, Np, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    o_p, l_p = oracle.attn(q, kp, vp)
    o_p32, l_p32 = o_p.astype(np.float32), l_p.astype(np.float32)
    empty = np.arange(Nq) % 5 == 2
    l_p32[:, :, empty] = -np.inf
    o_p32[:, empty] = np.nan
    o_c, l_c = oracle.attn(q, k, v)
    o_ref, l_ref = oracle.merge(np.stack([np.nan_to_num(o_p32.astype(np.float64)), o_c]),
                                np.stack([l_p32.astype(np.float64), l_c]))
    slots(8 if nw == 4 else 4)   # 9 or 5 tiles: one remainder tile split over the slots
    waves(nw)
    o, lse = dtl.attn_fwd_lse_accumulate(q.to(DEV), k.to(DEV), v.to(DEV),
                                         torch.from_numpy(o_p32).to(DEV), torch.from_numpy(l_p32).to(DEV))
    torch.cuda.synchronize()
    assert_close("O", to_np(o), o_ref)
    assert_close("LSE", to_np(lse), l_ref)


def test_split_schedule_kv_chunks(slots):
    """attn_fwd_lse_kv_chunks through the split schedule: 2 chunks of 4100 keys, 18 tiles
    on 8 slots (a remainder of 2 tiles split), each part against the oracle."""
    import diffusion_transformer_long_amd as dtl
    q, k, v = _inputs(92, 1, 1152, 2 * 4100, 1, 128, 2.0)
    slots(8)
    o_parts, l_parts = dtl.attn_fwd_lse_kv_chunks(q.to(DEV), k.to(DEV), v.to(DEV), 2)
    torch.cuda.synchronize()
    for t in range(2):
        o_ref, l_ref = oracle.attn(q, k[:, t * 4100:(t + 1) * 4100], v[:, t * 4100:(t + 1) * 4100])
        assert_close("part %d O" % t, to_np(o_parts[t]), o_ref)
        assert_close("part %d LSE" % t, to_np(l_parts[t]), l_ref)


def test_split_schedule_repeated_calls_agree(slots):
    """Back-to-back split launches (fresh epochs, reused pool memory) give one result."""
    import diffusion_transformer_long_amd as dtl
    q, k, v = _inputs(91, 1, 1152, 4100, 1, 128, 3.0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    slots(8)
    outs = [dtl.attn_fwd_lse(qd, kd, vd, o_dtype=torch.float32) for _ in range(6)]
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v)
    for o, lse in outs:
        assert_close("O", to_np(o), o_ref)
        assert_close("LSE", to_np(lse), l_ref)


# (waves, slots, B, Nq, Nkv, H, D, k_scale): the split cases of both workgroup sizes
FALLBACK_CASES = [(4,) + c for c in CASES[:4]] + [(8,) + c for c in CASES8[:3]]


@pytest.mark.parametrize("case", FALLBACK_CASES, ids=lambda c: "w%d_slots%d_B%d_Nq%d_Nkv%d_H%d_D%d" % c[:7])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_split_finaliser_fallback_matches_oracle(slots, waves, polls, case, o_dtype):
    """Every finaliser computes the keys its helpers own itself (no wait): same result."""
    import diffusion_transformer_long_amd as dtl
    nw, n, B, Nq, Nkv, H, D, ks = case
    log("split finaliser fallback, %d waves, slots=%d %s o=%s" % (nw, n, case[2:], o_dtype))
    q, k, v = _inputs(7000 + Nq + Nkv, B, Nq, Nkv, H, D, ks)
    slots(n)
    if D == 128:
        waves(nw)
    polls(0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = dtl.attn_fwd_lse(qd, kd, vd, o_dtype=o_dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("O", to_np(o), o_ref)
    assert_close("LSE", to_np(lse), l_ref)
    # the waiting path (helper states folded in) on the same inputs, also against the
    # oracle: the two round their bf16 weights against different running maxima, so they
    # agree with each other only to the parity bar, not bitwise
    os.environ.pop("DTL_ATTN_MAX_POLLS")
    o2, lse2 = dtl.attn_fwd_lse(qd, kd, vd, o_dtype=o_dtype)
    torch.cuda.synchronize()
    assert_close("O, waiting path", to_np(o2), o_ref)
    assert_close("LSE, waiting path", to_np(lse2), l_ref)


@pytest.mark.parametrize("nw", [4, 8])
def test_split_finaliser_fallback_accumulate(slots, waves, polls, nw):
    """attn_fwd_lse_accumulate through the split schedule with every finaliser computing
    its whole tile, rows without previous keys included."""
    import diffusion_transformer_long_amd as dtl
    B, Nq, Np, Nkv, H, D = 1, 1152, 300, 4100, 1, 128
    g = np.random.Generator(np.random.PCG64(78))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    kp = synthetic.to_bf16(g.standard_normal((B, Np, H, D), dtype=np.float32))
    vp = synthetic.to_bf16(g.standard_normal((B, Np, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * np.float32(2.0))
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    o_p, l_p = oracle.attn(q, kp, vp)
    o_p32, l_p32 = o_p.astype(np.float32), l_p.astype(np.float32)
    empty = np.arange(Nq) % 7 == 3
    l_p32[:, :, empty] = -np.inf
    o_p32[:, empty] = np.nan
    o_c, l_c = oracle.attn(q, k, v)
    o_ref, l_ref = oracle.merge(np.stack([np.nan_to_num(o_p32.astype(np.float64)), o_c]),
                                np.stack([l_p32.astype(np.float64), l_c]))
    slots(8 if nw == 4 else 4)
    waves(nw)
    polls(0)
    for o_dtype in (torch.float32, torch.bfloat16):
        o, lse = dtl.attn_fwd_lse_accumulate(q.to(DEV), k.to(DEV), v.to(DEV),
                                             torch.from_numpy(o_p32).to(DEV), torch.from_numpy(l_p32).to(DEV),
                                             o_dtype=o_dtype)
        torch.cuda.synchronize()
        assert_close("O %s" % o_dtype, to_np(o), o_ref)
        assert_close("LSE", to_np(lse), l_ref)


def test_split_calls_on_two_streams_at_once(slots):
    """Split-schedule calls on two streams of equal (default) priority, enqueued
    alternately so that they overlap: each takes its own workspace from the pool and
    carries its own launch counter value, so both match the oracle."""
    import diffusion_transformer_long_amd as dtl
    slots(8)
    ins = [_inputs(95 + i, 1, 1152, 4100, 1, 128, 2.0 + i) for i in range(2)]
    dev_ins = [tuple(t.to(DEV) for t in x) for x in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)]
    outs = [[], []]
    for rep in range(4):
        for i, s in enumerate(streams):
            with torch.cuda.stream(s):
                outs[i].append(dtl.attn_fwd_lse(*dev_ins[i], o_dtype=torch.float32))
    torch.cuda.synchronize()
    for i in range(2):
        o_ref, l_ref = oracle.attn(*ins[i])
        for o, lse in outs[i]:
            assert_close("stream %d O" % i, to_np(o), o_ref)
            assert_close("stream %d LSE" % i, to_np(lse), l_ref)
