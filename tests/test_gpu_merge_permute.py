"""GPU parity of attn_merge_lse and seq_to_head_permute.

Merge: Ring equivalence on GPU partials; the merge alone fed oracle partials (rounded
to f32) against the oracle's merge of the same values; P = 1 identity; an empty
(-inf) part; all parts empty; order of parts; bf16 partials.
Permute: bit-exact against the oracle's index map for bf16/f32/1-byte/8-byte
elements, the vector path and the element path, p = 1, and untouched memory past
the output; errors for p not dividing N or H.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import assert_close, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _parts(seed, P, B, N, H, D, lse_scale=3.0):
    g = np.random.Generator(np.random.PCG64(seed))
    o_p = g.standard_normal((P, B, N, H, D)).astype(np.float32)
    l_p = (g.standard_normal((P, B, H, N)) * lse_scale).astype(np.float32)
    return o_p, l_p


@pytest.mark.parametrize("P,B,N,H,D", [(1, 1, 5, 1, 8), (2, 2, 33, 3, 64), (4, 1, 1152, 24, 128),
                                       (8, 1, 301, 5, 128), (3, 1, 7, 2, 16)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_merge_alone_matches_oracle(P, B, N, H, D, out_dtype):
    import diffusion_transformer_long_amd as dtl
    log("attn_merge_lse P=%d B=%d N=%d H=%d D=%d out=%s" % (P, B, N, H, D, out_dtype))
    o_p, l_p = _parts(P * 100 + N, P, B, N, H, D)
    o, lse = dtl.attn_merge_lse(torch.from_numpy(o_p).to(DEV), torch.from_numpy(l_p).to(DEV),
                                out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge(o_p, l_p)
    tol = 1e-5 if out_dtype == torch.float32 else 1e-2
    assert_close("merged O", to_np(o), o_ref, max_abs=tol * 4, mean_abs=tol)
    assert_close("merged LSE", to_np(lse), l_ref, max_abs=1e-5, mean_abs=1e-6)


def test_merge_identity_empty_parts_order():
    import diffusion_transformer_long_amd as dtl
    o_p, l_p = _parts(5, 4, 1, 50, 3, 64)
    od, ld = torch.from_numpy(o_p).to(DEV), torch.from_numpy(l_p).to(DEV)
    # P = 1 is the identity
    o1, l1 = dtl.attn_merge_lse(od[:1], ld[:1], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1.cpu(), od[0].cpu()) and torch.equal(l1.cpu(), ld[0].cpu())
    # an empty part (lse = -inf) adds nothing, whatever its o holds
    ld2 = ld.clone()
    ld2[2] = -float("inf")
    od2 = od.clone()
    od2[2] = float("nan")
    o_a, l_a = dtl.attn_merge_lse(od2, ld2, out_dtype=torch.float32)
    o_b, l_b = dtl.attn_merge_lse(od[[0, 1, 3]].contiguous(), ld[[0, 1, 3]].contiguous(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close("empty part O", to_np(o_a), to_np(o_b), max_abs=1e-6, mean_abs=1e-7)
    assert_close("empty part LSE", to_np(l_a), to_np(l_b), max_abs=1e-6, mean_abs=1e-7)
    # every part empty: o = 0, lse = -inf
    o_e, l_e = dtl.attn_merge_lse(od, torch.full_like(ld, -float("inf")), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(o_e == 0) and torch.all(torch.isneginf(l_e))
    # order of parts
    perm = [3, 1, 0, 2]
    o_c, l_c = dtl.attn_merge_lse(od[perm].contiguous(), ld[perm].contiguous(), out_dtype=torch.float32)
    o_d, l_d = dtl.attn_merge_lse(od, ld, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close("order O", to_np(o_c), to_np(o_d), max_abs=1e-6, mean_abs=1e-7)
    # lse may be skipped
    o_n, l_n = dtl.attn_merge_lse(od, ld, out_dtype=torch.float32, write_lse=False)
    torch.cuda.synchronize()
    assert l_n is None and torch.equal(o_n, o_d)


def test_merge_bf16_parts():
    import diffusion_transformer_long_amd as dtl
    o_p, l_p = _parts(6, 3, 1, 40, 2, 128)
    ob = torch.from_numpy(o_p).to(torch.bfloat16)
    o, lse = dtl.attn_merge_lse(ob.to(DEV), torch.from_numpy(l_p).to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.merge(ob, l_p)
    assert_close("bf16 parts O", to_np(o), o_ref, max_abs=1e-5, mean_abs=1e-6)


def test_ring_equivalence_on_gpu_partials():
    """Ring rounds on one GPU: chunked attn_fwd_lse + merge equals full attention."""
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D = 1, 200, 768, 3, 128
    g = np.random.Generator(np.random.PCG64(8))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * 3)
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    o_ref, l_ref = oracle.attn(q, k, v)
    for chunks in (1, 2, 3, 6, 12):
        o, lse = dtl.ring_attention(q.to(DEV), k.to(DEV), v.to(DEV), chunks)
        torch.cuda.synchronize()
        assert_close("ring %d chunks O" % chunks, to_np(o), o_ref)
        assert_close("ring %d chunks LSE" % chunks, to_np(lse), l_ref)


# ------------------------------------------------------------------ permute

@pytest.mark.parametrize("p,B,N,H,D,dtype", [
    (4, 1, 4608, 24, 128, torch.bfloat16),   # the FLUX Ulysses-4 shape
    (2, 1, 64, 24, 128, torch.bfloat16),
    (1, 2, 10, 3, 64, torch.bfloat16),
    (8, 1, 80, 40, 128, torch.bfloat16),
    (4, 2, 12, 8, 3, torch.bfloat16),        # 3-element runs: element path
    (3, 1, 9, 6, 5, torch.float32),
    (4, 1, 16, 4, 16, torch.uint8),
    (2, 1, 6, 2, 4, torch.float64),
])
def test_permute_bit_exact(p, B, N, H, D, dtype):
    import diffusion_transformer_long_amd as dtl
    log("seq_to_head_permute p=%d B=%d N=%d H=%d D=%d %s" % (p, B, N, H, D, dtype))
    g = np.random.Generator(np.random.PCG64(N + H))
    nbytes = p * B * (N // p) * H * D * torch.tensor([], dtype=dtype).element_size()
    raw = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    x = torch.from_numpy(raw).view(dtype).reshape(p, B, N // p, H, D)
    n_out = x.numel()
    canary = torch.empty((n_out + 64,), dtype=dtype, device=DEV)
    canary.view(torch.uint8).fill_(0xA5)
    out = canary[:n_out].view(p, B, N, H // p, D)
    dtl.seq_to_head_permute(x.to(DEV), p, out=out)
    torch.cuda.synchronize()
    ref = oracle.permute(x.view(torch.uint8).numpy(), p)   # same index map, D*elem bytes per row
    assert out.cpu().view(torch.uint8).numpy().tobytes() == ref.tobytes()
    assert np.all(canary[n_out:].cpu().view(torch.uint8).numpy() == 0xA5)


def test_permute_rejects_bad_divisibility():
    import diffusion_transformer_long_amd as dtl
    x = torch.zeros((4, 1, 3, 6, 8), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        dtl.seq_to_head_permute(x, 4)
    x = torch.zeros((4, 1, 3, 8, 8), dtype=torch.bfloat16, device=DEV)
    st = dtl.lib.seq_to_head_permute(x.data_ptr(), x.data_ptr() + x.numel() * 2 + 4096, 4, 1, 14, 8, 8, 2, None)
    assert st == dtl.DTL_ERR_INVALID_ARG  # p does not divide N: rejected before any launch
