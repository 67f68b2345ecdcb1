"""GPU parity of attn_merge_lse and the three Ulysses permutes.

Merge: Ring equivalence on GPU partials; the merge alone fed f32 partials against the
oracle's merge of the same values (f32 output within the f32 error; bf16 output within
half a bf16 ulp plus that error and >= 99% correctly rounded); P = 1 identity; an empty
(-inf) part; all parts empty; order of parts; bf16 partials.
Permutes (seq->head, head->seq, fused QKV seq->head): bit-exact against the oracle's
index maps for bf16/f32/1-byte/8-byte elements, 16-byte and narrower copy units, p = 1,
and untouched memory past the output; the round trip at the Wan2.1-14B Ulysses-8
shape; errors for p not dividing N or H.  Ulysses-4 on the FLUX sequence end to end
(fused QKV permute, attention per head group, head->seq permute) against the oracle's
attention.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_helpers import assert_bf16_rounding_of, assert_close, log, to_np

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
    # The kernel works in f32: weights exp(lse_t - L) with a few ulps of relative error
    # (arguments up to ~30 in magnitude), then a sum of P weighted parts.  Its absolute
    # error is below 2^-17 times the largest |o_t| of the element (about 8 ulps of f32
    # relative error at P = 8, with margin).
    f32_err = 2.0 ** -17 * np.abs(o_p).max(axis=0).astype(np.float64)
    if out_dtype == torch.float32:
        assert_close("merged O", to_np(o), o_ref, max_abs=float(f32_err.max()), mean_abs=1e-6)
    else:
        assert_bf16_rounding_of("merged O (bf16)", to_np(o), o_ref, f32_err)
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


@pytest.mark.parametrize("P", [3, 4])
def test_merge_bf16_parts(P):
    """bf16 partials: P = 3 takes the LDS kernel, P = 4 the row kernel."""
    import diffusion_transformer_long_amd as dtl
    o_p, l_p = _parts(6 + P, P, 1, 40, 2, 128)
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


KV_CHUNK_CASES = [
    # B, Nq, Nkv, H, D, P, waves (None: the library's choice)
    (2, 63, 4 * 65, 3, 128, 4, None),     # ragged 65-key chunks, B = 2
    (1, 200, 3 * 129, 2, 64, 3, None),
    (1, 130, 2 * 1000, 2, 128, 2, None),
    (2, 300, 5 * 77, 1, 64, 5, None),
    (1, 97, 300, 2, 128, 1, None),         # P = 1 is attn_fwd_lse
    (2, 63, 4 * 65, 3, 128, 4, 8),        # 256-row tiles
    (1, 257, 2 * 4160, 1, 128, 2, 8),
]


def test_kv_chunks_bf16_parts():
    """attn_fwd_lse_kv_chunks with bf16 partials: each part is attn_fwd_lse's bf16 result."""
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D, P = 1, 150, 3 * 100, 4, 128, 3
    g = np.random.Generator(np.random.PCG64(7777))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * 3)
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_parts, l_parts = dtl.attn_fwd_lse_kv_chunks(qd, kd, vd, P, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o_parts.dtype == torch.bfloat16
    C = Nkv // P
    for t in range(P):
        o_ref, l_ref = oracle.attn(q, k[:, t * C:(t + 1) * C], v[:, t * C:(t + 1) * C])
        assert_close("part %d O" % t, to_np(o_parts[t]), o_ref)
        assert_close("part %d LSE" % t, to_np(l_parts[t]), l_ref)


@pytest.mark.parametrize("case", KV_CHUNK_CASES, ids=lambda c: "B%d_Nq%d_Nkv%d_H%d_D%d_P%d_w%s" % c)
def test_kv_chunks_one_launch_match_oracle(case):
    """attn_fwd_lse_kv_chunks: part t is attention over keys [tC, (t+1)C), and the merge of
    the parts is attention over all keys (also through ring_attention(one_launch=True))."""
    import os
    import diffusion_transformer_long_amd as dtl
    B, Nq, Nkv, H, D, P, nw = case
    log("attn_fwd_lse_kv_chunks %s" % (case,))
    g = np.random.Generator(np.random.PCG64(7000 + Nq + Nkv + P))
    q = synthetic.to_bf16(g.standard_normal((B, Nq, H, D), dtype=np.float32))
    k = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32) * 2)
    v = synthetic.to_bf16(g.standard_normal((B, Nkv, H, D), dtype=np.float32))
    old = os.environ.get("DTL_ATTN_WAVES")
    if nw is not None:
        os.environ["DTL_ATTN_WAVES"] = str(nw)
    try:
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        o_parts, l_parts = dtl.attn_fwd_lse_kv_chunks(qd, kd, vd, P)
        o, lse = dtl.ring_attention(qd, kd, vd, P, one_launch=True, out_dtype=torch.float32)
        torch.cuda.synchronize()
    finally:
        if old is None:
            os.environ.pop("DTL_ATTN_WAVES", None)
        else:
            os.environ["DTL_ATTN_WAVES"] = old
    C = Nkv // P
    for t in range(P):
        o_ref, l_ref = oracle.attn(q, k[:, t * C:(t + 1) * C], v[:, t * C:(t + 1) * C])
        assert_close("part %d O" % t, to_np(o_parts[t]), o_ref)
        assert_close("part %d LSE" % t, to_np(l_parts[t]), l_ref)
    o_ref, l_ref = oracle.attn(q, k, v)
    assert_close("merged O", to_np(o), o_ref)
    assert_close("merged LSE", to_np(lse), l_ref)


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


PERMUTE_SHAPES = [
    (4, 1, 4608, 24, 128, torch.bfloat16),   # the FLUX Ulysses-4 shape
    (2, 1, 64, 24, 128, torch.bfloat16),
    (1, 2, 10, 3, 64, torch.bfloat16),
    (8, 1, 80, 40, 128, torch.bfloat16),
    (4, 2, 12, 8, 3, torch.bfloat16),        # 6-byte runs: 2-byte units
    (3, 1, 9, 6, 5, torch.float32),          # 20-byte runs: 4-byte units
    (4, 1, 16, 4, 16, torch.uint8),
    (2, 1, 6, 2, 4, torch.float64),
    (5, 1, 15, 5, 1, torch.uint8),           # 1-byte runs
]


def _random_tensor(seed, shape, dtype):
    g = np.random.Generator(np.random.PCG64(seed))
    nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return torch.from_numpy(g.integers(0, 256, size=nbytes, dtype=np.uint8)).view(dtype).reshape(shape)


def _canaried(shape, dtype):
    n = int(np.prod(shape))
    canary = torch.empty((n + 64,), dtype=dtype, device=DEV)
    canary.view(torch.uint8).fill_(0xA5)
    return canary, canary[:n].view(shape)


def _bytes(t):
    return t.cpu().contiguous().view(torch.uint8).numpy()


@pytest.mark.parametrize("p,B,N,H,D,dtype", PERMUTE_SHAPES)
def test_head_to_seq_bit_exact(p, B, N, H, D, dtype):
    import diffusion_transformer_long_amd as dtl
    log("head_to_seq_permute p=%d B=%d N=%d H=%d D=%d %s" % (p, B, N, H, D, dtype))
    y = _random_tensor(N + 3 * H, (p, B, N, H // p, D), dtype)
    canary, out = _canaried((p, B, N // p, H, D), dtype)
    dtl.head_to_seq_permute(y.to(DEV), p, out=out)
    torch.cuda.synchronize()
    ref = oracle.head_to_seq(y.view(torch.uint8).numpy(), p)   # D*elem bytes per row
    assert _bytes(out).tobytes() == ref.tobytes()
    assert np.all(_bytes(canary[out.numel():]) == 0xA5)


@pytest.mark.parametrize("p,B,N,H,D,dtype", PERMUTE_SHAPES)
def test_qkv_permute_bit_exact(p, B, N, H, D, dtype):
    import diffusion_transformer_long_amd as dtl
    log("qkv_seq_to_head_permute p=%d B=%d N=%d H=%d D=%d %s" % (p, B, N, H, D, dtype))
    x = _random_tensor(N + 5 * H, (p, B, N // p, 3, H, D), dtype)
    canary, out = _canaried((p, 3, B, N, H // p, D), dtype)
    dtl.qkv_seq_to_head_permute(x.to(DEV), p, out=out)
    torch.cuda.synchronize()
    ref = oracle.qkv_permute(x.view(torch.uint8).numpy(), p)
    assert _bytes(out).tobytes() == ref.tobytes()
    assert np.all(_bytes(canary[out.numel():]) == 0xA5)


def test_ulysses8_round_trip_wan14b_shape():
    """seq->head then head->seq returns the input bit for bit at [8,1,9450,40,128]."""
    import diffusion_transformer_long_amd as dtl
    log("round trip [8,1,9450,40,128] bf16")
    x = torch.empty((8, 1, 9450, 40, 128), dtype=torch.bfloat16, device=DEV)
    x.view(torch.int16).random_(-32768, 32767, generator=torch.Generator(DEV).manual_seed(7))
    y = dtl.seq_to_head_permute(x, 8)
    back = dtl.head_to_seq_permute(y, 8)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))
    # every head group's tokens are the concatenation of the sequence shards
    assert torch.equal(y[3, 0, 9450 * 5:9450 * 6].view(torch.int16), x[5, 0, :, 15:20].view(torch.int16))


def test_permutes_reject_bad_divisibility():
    import diffusion_transformer_long_amd as dtl
    y = torch.zeros((4, 1, 6, 2, 8), dtype=torch.bfloat16, device=DEV)   # 6 tokens, p = 4
    with pytest.raises(ValueError):
        dtl.head_to_seq_permute(y, 4)
    x = torch.zeros((4, 1, 3, 3, 6, 8), dtype=torch.bfloat16, device=DEV)  # 6 heads, p = 4
    with pytest.raises(ValueError):
        dtl.qkv_seq_to_head_permute(x, 4)


def test_ulysses4_flux_end_to_end():
    """One Ulysses-4 attention layer on the FLUX sequence, every GPU's share on this one:
    pack the four sequence shards' q, k, v, exchange them with the fused QKV permute,
    attend per head group (6 heads, all 4608 tokens), bring O back with the head->seq
    permute, and compare with attention over the whole sequence."""
    import diffusion_transformer_long_amd as dtl
    w = synthetic.FLUX
    log("ulysses-4 end to end on %s" % w.name)
    q, k, v = synthetic.workload_qkv(w)                                    # [1,4608,24,128]
    packed = torch.stack([q, k, v], dim=2).reshape(1, 4, w.Nq // 4, 3, w.H, w.D)
    packed = packed.transpose(0, 1).contiguous().to(DEV)                  # [4,1,1152,3,24,128]
    qkv = dtl.qkv_seq_to_head_permute(packed, 4)                          # [4,3,1,4608,6,128]
    o_heads = torch.empty((4, 1, w.Nq, w.H // 4, w.D), dtype=torch.bfloat16, device=DEV)
    lse_heads = torch.empty((4, 1, w.H // 4, w.Nq), dtype=torch.float32, device=DEV)
    for j in range(4):
        dtl.attn_fwd_lse(qkv[j, 0], qkv[j, 1], qkv[j, 2], o=o_heads[j], lse=lse_heads[j])
    o_seq = dtl.head_to_seq_permute(o_heads, 4)                           # [4,1,1152,24,128]
    torch.cuda.synchronize()
    o = o_seq.transpose(0, 1).reshape(1, w.Nq, w.H, w.D)
    lse = lse_heads.transpose(0, 1).reshape(1, w.H, w.Nq)                 # head group j = heads 6j..6j+5
    rows = synthetic.sample_rows(w.seed + 400, w.B, w.H, w.Nq, 4096)
    o_ref, l_ref = oracle.attn_rows(q, k, v, rows)
    b, h, i = rows[:, 0], rows[:, 1], rows[:, 2]
    assert_close("ulysses4 O (%d rows)" % len(rows), o.float().cpu().numpy()[b, i, h].astype(np.float64), o_ref)
    assert_close("ulysses4 LSE (%d rows)" % len(rows), lse.cpu().numpy()[b, h, i].astype(np.float64), l_ref)


@pytest.mark.parametrize("P,D", [(2, 64), (4, 128), (8, 128), (4, 64)])
@pytest.mark.parametrize("parts_dtype", [torch.float32, torch.bfloat16], ids=["f32parts", "bf16parts"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_merge_row_kernel_equals_lds_kernel(P, D, parts_dtype, out_dtype):
    """The row kernel (P in {2, 4, 8}, D in {64, 128}) against the LDS kernel
    (DTL_MERGE_KERNEL=lds) on the same inputs, bit for bit: a third of the rows have an
    empty part holding NaN, some rows have every part empty, and the row count is not a
    multiple of either kernel's rows per workgroup."""
    import os
    import diffusion_transformer_long_amd as dtl
    B, N, H = 2, 301, 3
    log("merge row kernel vs LDS kernel P=%d D=%d parts %s out %s" % (P, D, parts_dtype, out_dtype))
    o_p, l_p = _parts(900 + P + D, P, B, N, H, D)
    l_p[1, :, :, ::3] = -np.inf
    o_p[1, :, ::3] = np.nan
    l_p[:, 1, 0, 7:11] = -np.inf
    od = torch.from_numpy(o_p).to(parts_dtype).to(DEV)
    ld = torch.from_numpy(l_p).to(DEV)
    o_r, l_r = dtl.attn_merge_lse(od, ld, out_dtype=out_dtype)
    old = os.environ.get("DTL_MERGE_KERNEL")
    os.environ["DTL_MERGE_KERNEL"] = "lds"
    try:
        o_l, l_l = dtl.attn_merge_lse(od, ld, out_dtype=out_dtype)
    finally:
        if old is None:
            os.environ.pop("DTL_MERGE_KERNEL", None)
        else:
            os.environ["DTL_MERGE_KERNEL"] = old
    torch.cuda.synchronize()
    iv = torch.int16 if out_dtype == torch.bfloat16 else torch.int32
    assert torch.equal(o_r.view(iv), o_l.view(iv)), "O differs between the two merge kernels"
    assert torch.equal(l_r.view(torch.int32), l_l.view(torch.int32)), "LSE differs between the two merge kernels"
    o_ref, l_ref = oracle.merge(od.float().cpu().numpy(), l_p)
    finite = np.isfinite(l_ref)
    assert np.all(to_np(o_r)[~np.broadcast_to(finite.transpose(0, 2, 1)[..., None], o_ref.shape)] == 0)
    assert_close("row kernel LSE (finite rows)", to_np(l_r)[finite], l_ref[finite], max_abs=1e-5, mean_abs=1e-6)
