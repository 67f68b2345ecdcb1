"""GPU check of attn_fwd_lse_noalloc, the entry point that allocates nothing (named to be
collected last: it must pass after every other test as well as alone): its split
schedule keeps the pieces' states in the library's static device array instead of a
pool workspace.  Two calls in a row (the second on a smaller input, so the array still
holds the first call's states) are compared with attn_fwd_lse on the same inputs and
with the oracle; then the Wan2.2-5B sequence, whose last round the library splits on
the real GPU, is compared with attn_fwd_lse."""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import assert_close, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(seed, B, Nq, Nkv, H, D, k_scale):
    g = np.random.Generator(np.random.PCG64(seed))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * np.float32(k_scale))
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    return q, k, v


@pytest.fixture
def env():
    saved = {n: os.environ.get(n) for n in ("DTL_ATTN_SLOTS", "DTL_ATTN_WAVES", "DTL_ATTN_KEYSPLIT")}
    yield os.environ
    for n, val in saved.items():
        if val is None:
            os.environ.pop(n, None)
        else:
            os.environ[n] = val


def _both(q, k, v, o_dtype):
    import diffusion_transformer_long_amd as dtl
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    B, Nq, H, D = q.shape
    o = torch.empty((B, Nq, H, D), dtype=o_dtype, device=DEV)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    dtl.attn_fwd_lse_noalloc(qd, kd, vd, o, lse)
    o_ref_gpu, l_ref_gpu = dtl.attn_fwd_lse(qd, kd, vd, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return o, lse, o_ref_gpu, l_ref_gpu


@pytest.mark.parametrize("nw", [4, 8])
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_two_calls_match_attn_fwd_lse_and_oracle(env, nw, o_dtype):
    # call 1: 1152 x 4100 keys, one head (9 or 5 tiles; slots 8 or 4 split the last one);
    # call 2: smaller, 640 x 4096 keys (5 or 3 tiles), over what call 1 left in the array
    slots = 8 if nw == 4 else 4
    env["DTL_ATTN_WAVES"] = str(nw)
    env["DTL_ATTN_SLOTS"] = str(slots)
    env["DTL_ATTN_KEYSPLIT"] = "0"   # one 128-row tile per CU would otherwise take two key groups
    for call, (seed, Nq, Nkv, ks) in enumerate(((41, 1152, 4100, 3.0), (42, 640, 4096, 1.0))):
        log("attn_fwd_lse_noalloc call %d: %d waves, slots %d, Nq=%d Nkv=%d o=%s" % (call + 1, nw, slots, Nq, Nkv, o_dtype))
        q, k, v = _inputs(seed, 1, Nq, Nkv, 1, 128, ks)
        o, lse, o2, l2 = _both(q, k, v, o_dtype)
        assert_close("O vs attn_fwd_lse", to_np(o), to_np(o2))
        assert_close("LSE vs attn_fwd_lse", to_np(lse), to_np(l2))
        log("  bitwise equal to attn_fwd_lse: O %s, LSE %s" % (torch.equal(o, o2), torch.equal(lse, l2)))
        o_ref, l_ref = oracle.attn(q, k, v)
        assert_close("O vs oracle", to_np(o), o_ref)
        assert_close("LSE vs oracle", to_np(lse), l_ref)


def test_noalloc_wan22_5b_split_schedule():
    """Wan2.2-5B (N=27280, 24 x 128): the library splits its last round on the real GPU."""
    w = synthetic.WAN5B
    log("attn_fwd_lse_noalloc %s" % w.name)
    q, k, v = synthetic.workload_qkv(w)
    o, lse, o2, l2 = _both(q, k, v, torch.bfloat16)
    assert_close("O vs attn_fwd_lse", to_np(o), to_np(o2))
    assert_close("LSE vs attn_fwd_lse", to_np(lse), to_np(l2))
    log("  bitwise equal to attn_fwd_lse: O %s, LSE %s" % (torch.equal(o, o2), torch.equal(lse, l2)))
