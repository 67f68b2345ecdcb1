"""GPU checks of calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A captured call keeps the host arguments of the moment of capture.  The split schedule's
flags therefore carry a value that also changes per replay (a launch count kept in the
workspace and advanced by a kernel enqueued after the split launch), so that a replay
never takes the flags of the previous replay for its own.  Each test replays a graph
several times with eager work in between and compares every replay with the eager result
on the same inputs, bit for bit; the eager results are compared with the oracle.

* attn_fwd_lse_noalloc with a split schedule (DTL_ATTN_SLOTS makes a small shape split:
  one tile's key blocks spread over several workgroups), 4- and 8-wave workgroups, with the
  captured call's inputs switched between two sets before each replay.
* The FLUX Ring-4 share step (Ulysses-4 permute, the four rounds' partials from one
  launch, the merge), a launch-bound sequence of three kernels.
* The same share's four rounds as four launches: accumulated in place into an f32 running
  result, or per-round partials and the merge.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import assert_close, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 3


@pytest.fixture
def env():
    names = ("DTL_ATTN_SLOTS", "DTL_ATTN_WAVES", "DTL_ATTN_KEYSPLIT")
    saved = {n: os.environ.get(n) for n in names}
    yield os.environ
    for n, val in saved.items():
        if val is None:
            os.environ.pop(n, None)
        else:
            os.environ[n] = val


def _inputs(seed, B, Nq, Nkv, H, D, k_scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * np.float32(k_scale))
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    return q, k, v


def _capture(fn):
    """Capture fn() in a graph after a warm-up on a side stream (torch's recipe)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("nw", [4, 8])
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_split_call_replays_in_a_graph(env, nw, o_dtype):
    """The captured call's inputs are rewritten between replays (input sets A, B, A, B):
    a replay that took the previous replay's flags for its own would fold that replay's
    pieces, computed from the other inputs."""
    import diffusion_transformer_long_amd as dtl
    # 1152 queries x 4100 keys, one head: 9 (4-wave) or 5 (8-wave) tiles on 8 or 4 slots,
    # the last tile's 65 key blocks split over every slot
    env["DTL_ATTN_SLOTS"] = "8" if nw == 4 else "4"
    env["DTL_ATTN_WAVES"] = str(nw)
    env["DTL_ATTN_KEYSPLIT"] = "0"   # 9 tiles of 128 rows would otherwise take two key groups
    B, Nq, Nkv, H, D = 1, 1152, 4100, 1, 128
    log("graph replay: noalloc split, %d waves, o %s" % (nw, o_dtype))
    sets = [_inputs(11, B, Nq, Nkv, H, D, k_scale=2.0), _inputs(12, B, Nq, Nkv, H, D, k_scale=2.0)]
    dev_sets = [tuple(t.to(DEV) for t in qkv) for qkv in sets]
    eager = []
    for (qd, kd, vd), (q, k, v) in zip(dev_sets, sets):
        o_e = torch.empty((B, Nq, H, D), dtype=o_dtype, device=DEV)
        l_e = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
        dtl.attn_fwd_lse_noalloc(qd, kd, vd, o_e, l_e)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attn(q, k, v)
        assert_close("eager noalloc O", to_np(o_e), o_ref)
        assert_close("eager noalloc LSE", to_np(l_e), l_ref)
        eager.append((o_e, l_e))

    qg, kg, vg = (t.clone() for t in dev_sets[0])
    o_g = torch.empty_like(eager[0][0])
    l_g = torch.empty_like(eager[0][1])
    g = _capture(lambda: dtl.attn_fwd_lse_noalloc(qg, kg, vg, o_g, l_g))
    for r in range(2 * REPLAYS):
        s = r % 2
        for dst, src in zip((qg, kg, vg), dev_sets[s]):
            dst.copy_(src)
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same_o = torch.equal(o_g, eager[s][0])
        same_l = torch.equal(l_g, eager[s][1])
        log("  replay %d (inputs %s): O %s, LSE %s the eager call" % (
            r, "AB"[s], "equals" if same_o else "DIFFERS FROM", "equals" if same_l else "DIFFERS FROM"))
        assert same_o and same_l, "replay %d differs from the eager call on the same inputs" % r


def test_flux_ring4_share_step_replays_in_a_graph():
    import diffusion_transformer_long_amd as dtl
    w = synthetic.FLUX_RING4
    log("graph replay: %s (permute, one-launch rounds, merge)" % w.name)
    qf, k, v = synthetic.workload_qkv(synthetic.FLUX)
    qd = qf[:, :w.Nq].contiguous().to(DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    shards = qf.reshape(1, 4, w.Nq, w.H, w.D).transpose(0, 1).contiguous().to(DEV)
    perm = torch.empty((4, 1, w.Nkv, w.H // 4, w.D), dtype=torch.bfloat16, device=DEV)
    parts = torch.empty((w.chunks, 1, w.Nq, w.H, w.D), dtype=torch.float32, device=DEV)
    lparts = torch.empty((w.chunks, 1, w.H, w.Nq), dtype=torch.float32, device=DEV)
    o = torch.empty((1, w.Nq, w.H, w.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, w.H, w.Nq), dtype=torch.float32, device=DEV)

    def step():
        dtl.seq_to_head_permute(shards, 4, out=perm)
        dtl.ring_attention(qd, kd, vd, w.chunks, o_parts=parts, lse_parts=lparts, o=o, lse=lse,
                           one_launch=True)

    step()
    torch.cuda.synchronize()
    perm_e, o_e, l_e = perm.clone(), o.clone(), lse.clone()
    g = _capture(step)
    for r in range(REPLAYS):
        # eager work in between that rewrites every buffer the graph uses
        perm.zero_()
        parts.fill_(float("nan"))
        lparts.fill_(float("nan"))
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = torch.equal(perm, perm_e) and torch.equal(o, o_e) and torch.equal(lse, l_e)
        log("  replay %d: %s the eager step" % (r, "equals" if ok else "DIFFERS FROM"))
        assert ok, "replay %d differs from the eager step" % r
    # the permute against the oracle's index map, bit-exact, and the step's rank-0 output
    # against the oracle over all of its rows
    ref = oracle.permute(shards.cpu().view(torch.int16).numpy(), 4)
    assert perm.cpu().view(torch.int16).numpy().tobytes() == ref.tobytes()
    _, l_ref = oracle.attn(qf[:, :w.Nq].contiguous(), k, v)
    assert_close("graph step LSE", to_np(lse), l_ref)


@pytest.mark.parametrize("form", ["accumulate", "per_round"])
def test_flux_ring4_rounds_replay_in_a_graph(form):
    """The FLUX Ring-4 share's four rounds as four launches captured in one graph: folded
    into an f32 running result in place (accumulate), or as per-round partials and the merge.
    Each replay starts from buffers the eager work in between has overwritten."""
    import diffusion_transformer_long_amd as dtl
    w = synthetic.FLUX_RING4
    log("graph replay: %s, rounds %s" % (w.name, form))
    qf, k, v = synthetic.workload_qkv(synthetic.FLUX)
    qd = qf[:, :w.Nq].contiguous().to(DEV)
    kd, vd = k.to(DEV), v.to(DEV)
    acc = torch.empty((1, w.Nq, w.H, w.D), dtype=torch.float32, device=DEV)
    parts = torch.empty((w.chunks, 1, w.Nq, w.H, w.D), dtype=torch.float32, device=DEV)
    lparts = torch.empty((w.chunks, 1, w.H, w.Nq), dtype=torch.float32, device=DEV)
    o = torch.empty((1, w.Nq, w.H, w.D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, w.H, w.Nq), dtype=torch.float32, device=DEV)

    def step():
        if form == "accumulate":
            dtl.ring_attention(qd, kd, vd, w.chunks, accumulate=True, o_acc=acc, o=o, lse=lse)
        else:
            dtl.ring_attention(qd, kd, vd, w.chunks, o_parts=parts, lse_parts=lparts, o=o, lse=lse,
                               one_launch=False)

    step()
    torch.cuda.synchronize()
    o_e, l_e = o.clone(), lse.clone()
    g = _capture(step)
    for r in range(REPLAYS):
        for t in (acc, parts, lparts):
            t.fill_(float("nan"))
        o.zero_()
        lse.fill_(float("-inf"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ok = torch.equal(o, o_e) and torch.equal(lse, l_e)
        log("  replay %d: %s the eager step" % (r, "equals" if ok else "DIFFERS FROM"))
        assert ok, "replay %d differs from the eager step" % r
    _, l_ref = oracle.attn(qf[:, :w.Nq].contiguous(), k, v)
    assert_close("graph rounds LSE", to_np(lse), l_ref)
