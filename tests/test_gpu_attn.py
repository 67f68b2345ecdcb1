"""GPU parity of attn_fwd_lse against the fp64 oracle (small and ragged shapes, full oracle).

Shapes span several 128-row query tiles and 64-key tiles with ragged tails in both,
head_dim 64 and 128, B = 2, one and five heads, bf16 and f32 outputs, each with the
library's choice of workgroup and with the two-key-group workgroup forced off and on.  Closed-form
cases: a single key (O equals V bit for bit), identical keys (mean of V), zero
queries (mean of V, LSE = ln Nkv).  Also: determinism, untouched memory past the
outputs, and the validation errors raised through the binding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import assert_close, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _inputs(seed, B, Nq, Nkv, H, D, k_scale=1.0):
    g = np.random.Generator(np.random.PCG64(seed))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * np.float32(k_scale))
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    return q, k, v


SHAPES = [
    # B, Nq, Nkv, H, D, k_scale
    (1, 1, 1, 1, 128, 1.0),
    (1, 1, 1, 1, 64, 1.0),
    (1, 64, 64, 2, 64, 1.0),
    (2, 63, 65, 3, 128, 1.0),
    (1, 65, 127, 1, 128, 3.0),
    (1, 129, 129, 5, 128, 1.0),
    (1, 127, 1000, 2, 128, 3.0),
    (2, 300, 77, 1, 64, 1.0),
    (1, 257, 513, 4, 64, 2.0),
    (1, 384, 2049, 2, 128, 1.0),
    (2, 130, 200, 6, 128, 2.0),     # short last tiles of 8 of the 12 (batch, head) pairs go first
    (1, 257, 513, 16, 64, 1.0),     # 16 short last tiles first
]


@pytest.fixture
def keysplit_env():
    """Sets DTL_ATTN_KEYSPLIT for one test: "auto" (the library's choice), or two key groups
    per workgroup forced off ("0") or on ("1") where they apply."""
    import os
    old = os.environ.get("DTL_ATTN_KEYSPLIT")

    def set_mode(mode):
        if mode == "auto":
            os.environ.pop("DTL_ATTN_KEYSPLIT", None)
        else:
            os.environ["DTL_ATTN_KEYSPLIT"] = mode
    yield set_mode
    if old is None:
        os.environ.pop("DTL_ATTN_KEYSPLIT", None)
    else:
        os.environ["DTL_ATTN_KEYSPLIT"] = old


# key groups apply to head_dim 128 only: the other shapes run with the library's choice
CASES = [(s, m) for s in SHAPES for m in (("auto", "0", "1") if s[4] == 128 else ("auto",))]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Nq%d_Nkv%d_H%d_D%d_ks%g" % c[0] + "_keysplit-" + c[1])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_attention_matches_oracle(case, o_dtype, keysplit_env):
    import diffusion_transformer_long_amd as dtl
    shape, mode = case
    B, Nq, Nkv, H, D, ks = shape
    keysplit_env(mode)
    log("attn_fwd_lse %s o=%s key groups %s" % (shape, o_dtype, mode))
    q, k, v = _inputs(1000 + Nq + Nkv, B, Nq, Nkv, H, D, ks)
    o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), o_dtype=o_dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("O", to_np(o), o_ref)
    assert_close("LSE", to_np(lse), l_ref)


@pytest.mark.parametrize("shape", [s for s in SHAPES if s[4] == 128], ids=lambda s: "B%d_Nq%d_Nkv%d_H%d_D%d_ks%g" % s)
def test_attention_8_wave_workgroups_match_oracle(shape):
    """The 256-row-tile kernel (chosen on the GPU for long key ranges) on the same shapes."""
    import os
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D, ks = shape
    log("attn_fwd_lse 8 waves %s" % (shape,))
    q, k, v = _inputs(1000 + Nq + Nkv, B, Nq, Nkv, H, D, ks)
    old = os.environ.get("DTL_ATTN_WAVES")
    os.environ["DTL_ATTN_WAVES"] = "8"
    try:
        o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), o_dtype=torch.float32)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("DTL_ATTN_WAVES", None)
        else:
            os.environ["DTL_ATTN_WAVES"] = old
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("O", to_np(o), o_ref)
    assert_close("LSE", to_np(lse), l_ref)


def test_single_key_output_is_v_bitwise():
    import diffusion_transformer_long_amd as dtl
    for D in (64, 128):
        q, k, v = _inputs(77 + D, 2, 200, 1, 3, D, 3.0)
        o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV))
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), v.expand(2, 200, 3, D)), "O != V with one key"
        qf, kf = q.double().numpy(), k.double().numpy()
        l_exact = np.einsum("bihd,bhd->bhi", qf, kf[:, 0]) / math.sqrt(D)
        assert_close("LSE single key", to_np(lse), l_exact)


def test_identical_keys_and_zero_query():
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D = 1, 130, 333, 2, 128
    q, k, v = _inputs(91, B, Nq, Nkv, H, D)
    k_same = k[:, :1].expand(B, Nkv, H, D).contiguous()
    o, lse = dtl.attn_fwd_lse(q.to(DEV), k_same.to(DEV), v.to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    mean_v = v.double().mean(dim=1, keepdim=True).expand(B, Nq, H, D).numpy()
    assert_close("O identical keys", to_np(o), mean_v)
    l_exact = np.einsum("bihd,bhd->bhi", q.double().numpy(), k.double().numpy()[:, 0]) / math.sqrt(D) \
        + math.log(Nkv)
    assert_close("LSE identical keys", to_np(lse), l_exact)
    qz = torch.zeros_like(q)
    o, lse = dtl.attn_fwd_lse(qz.to(DEV), k.to(DEV), v.to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close("O zero query", to_np(o), mean_v)
    assert_close("LSE zero query", to_np(lse), np.full((B, H, Nq), math.log(Nkv)))


def test_explicit_scale():
    import diffusion_transformer_long_amd as dtl
    q, k, v = _inputs(93, 1, 100, 200, 2, 64)
    o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), softmax_scale=0.05)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v, scale=0.05)
    assert_close("O scale 0.05", to_np(o), o_ref)
    assert_close("LSE scale 0.05", to_np(lse), l_ref)


@pytest.mark.parametrize("order", ["ascending", "descending"])
def test_logit_ramp_along_keys(order):
    """Keys scaled by a ramp along the key axis (logit std 0.25 -> 4, or the reverse). Ascending,
    every later tile holds larger logits than all before it, so the running reference moves and
    the accumulators are rescaled again and again; descending, the largest logits come first and
    the reference stays put after the first tiles."""
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D = 1, 130, 700, 3, 128
    q, k, v = _inputs(101 if order == "ascending" else 103, B, Nq, Nkv, H, D)
    ramp = np.linspace(0.25, 4.0, Nkv, dtype=np.float32)
    if order == "descending":
        ramp = ramp[::-1].copy()
    k = synthetic.to_bf16(k.float().numpy() * ramp[None, :, None, None])
    log("attn_fwd_lse logit ramp %s" % order)
    o, lse = dtl.attn_fwd_lse(q.to(DEV), k.to(DEV), v.to(DEV), o_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("O ramp " + order, to_np(o), o_ref)
    assert_close("LSE ramp " + order, to_np(lse), l_ref)


def test_deterministic_and_no_writes_past_outputs():
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D = 1, 333, 517, 3, 128
    q, k, v = _inputs(95, B, Nq, Nkv, H, D, 3.0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    n_o, n_l = B * Nq * H * D, B * H * Nq
    canary_o = torch.full((n_o + 4096,), 12345.0, device=DEV)
    canary_l = torch.full((n_l + 4096,), -777.0, device=DEV)
    o1, l1 = dtl.attn_fwd_lse(qd, kd, vd, o=canary_o[:n_o].view(B, Nq, H, D),
                              lse=canary_l[:n_l].view(B, H, Nq), o_dtype=torch.float32)
    o2, l2 = dtl.attn_fwd_lse(qd, kd, vd, o_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(canary_o[n_o:] == 12345.0) and torch.all(canary_l[n_l:] == -777.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "two runs differ"


def test_binding_errors_on_gpu_tensors():
    import diffusion_transformer_long_amd as dtl
    q = torch.zeros((1, 16, 2, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dtl.DtlError) as e:
        dtl.attn_fwd_lse(q, q, q)
    assert e.value.status == dtl.DTL_ERR_UNSUPPORTED
    q = torch.zeros((1, 16, 2, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dtl.DtlError) as e:
        dtl.attn_fwd_lse(q, q, q, o=q)  # output aliases the inputs
    assert e.value.status == dtl.DTL_ERR_INVALID_ARG
