"""GPU checks of the hard-attention limit: one key per (batch, head) whose logit exceeds every
other key's by more than 110 for every query.

exp(-110) is below the smallest positive f32, so every other weight is exactly zero in the
kernels' arithmetic and, up to a relative 1e-47, in exact arithmetic: softmax attention then
returns that key's V row for every query and LSE equals that key's scaled logit.  These are
closed forms of the definition, checked without the oracle: O in bf16 must equal the V row
bit for bit, O in f32 within a few f32 ulps of it, LSE within the usual bar of the logit
computed in float64 from the same bf16 inputs.

The dominant key sits first, at a 64-key tile boundary, inside a tile, and last (in the
ragged tail), so the paths under test include: the running reference jumping by about 360
(old accumulators scaled by exactly zero), tiles and split pieces that hold no dominant key
(merged with weight zero), and the Ring rounds' LSE merge or running accumulation where only
one KV chunk holds it.  Construction: q = N(0,1) with q[..., 0] = 64; k = N(0,1) with
k[..., 0] = 0 except k[b, j*, h, 0] = 64; v = N(0,1); all rounded to bf16.  The logit gap is
then about 4096 / sqrt(D) minus a noise term of a few tens; the test asserts the gap from the
inputs before it runs anything.
"""
import math
import os

import numpy as np
import pytest
import torch

import synthetic
from gpu_helpers import assert_close, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
MIN_GAP = 110.0


def _hard_inputs(seed, B, Nq, Nkv, H, D, jstar):
    """bf16 q, k, v with key jstar[b][h] dominant for (b, h), and the float64 scaled logits'
    gap check; returns q, k, v and the dominant keys' logits [B, H, Nq] in float64."""
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.standard_normal((B, Nq, H, D), dtype=np.float32)
    k = g.standard_normal((B, Nkv, H, D), dtype=np.float32)
    v = g.standard_normal((B, Nkv, H, D), dtype=np.float32)
    q[..., 0] = 64.0
    k[..., 0] = 0.0
    for b in range(B):
        for h in range(H):
            k[b, jstar[b][h], h, 0] = 64.0
    q, k, v = synthetic.to_bf16(q), synthetic.to_bf16(k), synthetic.to_bf16(v)
    qf, kf = q.double().numpy(), k.double().numpy()
    top = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            s = qf[b, :, h] @ kf[b, :, h].T / math.sqrt(D)   # [Nq, Nkv], exact products
            j = jstar[b][h]
            others = np.delete(s, j, axis=1)
            gap = s[:, j] - others.max(axis=1) if others.size else np.full(Nq, np.inf)
            assert gap.min() > MIN_GAP, "input construction: logit gap %.1f" % gap.min()
            top[b, h] = s[:, j]
    return q, k, v, top


def _expected_o(v, jstar, Nq):
    B, _, H, D = v.shape
    rows = torch.stack([torch.stack([v[b, jstar[b][h], h] for h in range(H)]) for b in range(B)])
    return rows[:, None].expand(B, Nq, H, D)   # [B, Nq, H, D]


def _check(o, lse, v, jstar, top, label):
    B, Nq, H, D = o.shape
    want = _expected_o(v, jstar, Nq)
    got = o.cpu()
    if o.dtype == torch.bfloat16:
        diff = int((got.view(torch.int16) != want.contiguous().view(torch.int16)).sum())
        log("  %-28s %d of %d bf16 values differ from the dominant key's V" % (label + " O", diff, got.numel()))
        assert diff == 0, "%s: O is not the dominant key's V bit for bit" % label
    else:
        w = want.double()
        rel = float(((got.double() - w).abs() / w.abs().clamp_min(1e-30)).max())
        log("  %-28s max relative error %.3e against the dominant key's V" % (label + " O", rel))
        assert rel <= 2.0 ** -20, "%s: O off the dominant key's V by %.3e relative" % (label, rel)
    assert_close(label + " LSE", to_np(lse), top)


@pytest.fixture
def env():
    names = ("DTL_ATTN_WAVES", "DTL_ATTN_KEYSPLIT", "DTL_ATTN_SLOTS", "DTL_ATTN_MAX_POLLS")
    saved = {n: os.environ.get(n) for n in names}
    yield os.environ
    for n, val in saved.items():
        if val is None:
            os.environ.pop(n, None)
        else:
            os.environ[n] = val


SCHEDULES = [
    # name, environment, B, Nq, Nkv, H, D
    ("auto_D128", {}, 2, 200, 333, 3, 128),
    ("auto_D64", {}, 2, 200, 333, 3, 64),
    ("8_waves", {"DTL_ATTN_WAVES": "8"}, 2, 300, 333, 3, 128),
    ("key_groups_on", {"DTL_ATTN_KEYSPLIT": "1"}, 2, 200, 333, 3, 128),
    ("key_groups_off", {"DTL_ATTN_KEYSPLIT": "0"}, 2, 200, 333, 3, 128),
]
# per (b, h): first key, last key of the first tile, first key of the second tile, a key
# inside a tile, the last (ragged-tail) key
JSTAR = [[0, 63, 64], [200, 332, 131]]


@pytest.mark.parametrize("sched", SCHEDULES, ids=lambda s: s[0])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_dominant_key_whole_tiles(env, sched, o_dtype):
    import diffusion_transformer_long_amd as dtl
    name, vars_, B, Nq, Nkv, H, D = sched
    for n, val in vars_.items():
        env[n] = val
    log("hard attention %s %s o=%s" % (name, (B, Nq, Nkv, H, D), o_dtype))
    q, k, v, top = _hard_inputs(7100 + D, B, Nq, Nkv, H, D, JSTAR)
    o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), o_dtype=o_dtype)
    torch.cuda.synchronize()
    _check(o, lse, v, JSTAR, top, name)


SPLITS = [
    # name, environment: one head's last 128-row tile (1152 x 4100) split over the slots
    ("split_4_waves", {"DTL_ATTN_SLOTS": "8", "DTL_ATTN_WAVES": "4", "DTL_ATTN_KEYSPLIT": "0"}),
    ("split_8_waves", {"DTL_ATTN_SLOTS": "4", "DTL_ATTN_WAVES": "8"}),
    ("split_no_polls", {"DTL_ATTN_SLOTS": "8", "DTL_ATTN_WAVES": "4", "DTL_ATTN_KEYSPLIT": "0",
                        "DTL_ATTN_MAX_POLLS": "0"}),
]


@pytest.mark.parametrize("split", SPLITS, ids=lambda s: s[0])
@pytest.mark.parametrize("j", [0, 2050, 4099])
def test_dominant_key_split_schedule(env, split, j):
    """Split pieces without the dominant key are folded in with weight zero."""
    import diffusion_transformer_long_amd as dtl
    name, vars_ = split
    for n, val in vars_.items():
        env[n] = val
    B, Nq, Nkv, H, D = 1, 1152, 4100, 1, 128
    log("hard attention %s, dominant key %d" % (name, j))
    q, k, v, top = _hard_inputs(7300 + j, B, Nq, Nkv, H, D, [[j]])
    o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check(o, lse, v, [[j]], top, name)


@pytest.mark.parametrize("mode", ["one_launch", "per_round", "accumulate"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_dominant_key_ring_rounds(mode, out_dtype):
    """Four KV chunks of 256 keys; per head the dominant key lies in chunk 0, 2 or 3, so
    the other chunks' partials (or accumulation steps) carry weight zero."""
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D, chunks = 1, 300, 1024, 3, 128, 4
    jstar = [[0, 600, 1023]]
    log("hard attention, Ring rounds %s, out %s" % (mode, out_dtype))
    q, k, v, top = _hard_inputs(7500, B, Nq, Nkv, H, D, jstar)
    o, lse = dtl.ring_attention(q.to(DEV), k.to(DEV), v.to(DEV), chunks, out_dtype=out_dtype,
                                accumulate=mode == "accumulate", one_launch=mode == "one_launch")
    torch.cuda.synchronize()
    _check(o, lse, v, jstar, top, "ring " + mode)
