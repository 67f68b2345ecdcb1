"""GPU parity at tensors of more than 2^31 elements (element and byte offsets past 32 bits).

The C ABI accepts any shape whose row counts (B*N*H) and tile count fit an int, so a
query, output or partials tensor may hold far more than 2^31 elements.  These tests run
such shapes through attn_fwd_lse (bf16 and f32 outputs), attn_fwd_lse_kv_chunks and
attn_merge_lse and compare the oracle's results on sampled rows with the GPU's: the rows
on both sides of the 2^31-element boundary, the ragged last query tile, and a seeded
sample.  A 32-bit wrap of an element or byte offset would read or write rows 2^20 tokens
away (16 heads x 128) and fail here.  The inputs come from torch's seeded GPU generator
(every value distinct); the sampled rows are copied to the host for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_bf16_rounding_of, assert_close, check_bf16_is_rounded_f32, log, to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
# 1 049 000 tokens x 16 heads x 128 = 2 148 532 224 elements > 2^31 = 2 147 483 648; the
# last query tile holds 40 rows
NQ = 1_049_000


def _randn(seed, shape, dtype, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=DEV, dtype=torch.float32 if dtype != torch.bfloat16 else dtype)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def _sample_rows(n_rows, row_elems, seed, n_random=512):
    """Token indices: around the token where the element offset passes 2^31, the last 300
    (the ragged last tile and the tiles before it), the first 8, and a seeded sample."""
    edge = (1 << 31) // row_elems
    fixed = np.concatenate([np.arange(8), np.arange(edge - 100, min(edge + 100, n_rows)),
                            np.arange(n_rows - 300, n_rows)])
    g = np.random.Generator(np.random.PCG64(seed))
    rows = np.unique(np.concatenate([fixed, g.integers(0, n_rows, n_random)]))
    return torch.from_numpy(rows)


def test_attention_past_2_31_elements():
    """f32 and bf16 outputs.  With 130 keys and logit std 2 some rows are peaked and |O|
    passes 2, where one bf16 rounding alone can cost up to 0.0156: the f32 output carries
    the bar and the bf16 output must be exactly its round-to-nearest-even."""
    import diffusion_transformer_long_amd as dtl
    B, Nkv, H, D = 1, 130, 16, 128
    assert B * NQ * H * D > (1 << 31)
    log("attn_fwd_lse B=%d Nq=%d Nkv=%d H=%d D=%d, f32 and bf16 out (%.2e elements per Q/O)"
        % (B, NQ, Nkv, H, D, B * NQ * H * D))
    q = _randn(61, (B, NQ, H, D), torch.bfloat16)
    k = _randn(62, (B, Nkv, H, D), torch.bfloat16, 2.0)
    v = _randn(63, (B, Nkv, H, D), torch.bfloat16)
    o32, lse32 = dtl.attn_fwd_lse(q, k, v, o_dtype=torch.float32)
    o16, lse16 = dtl.attn_fwd_lse(q, k, v, o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = _sample_rows(NQ, H * D, 64).to(DEV)
    q_s = q.index_select(1, rows).cpu()
    o32_s, l32_s = o32.index_select(1, rows), lse32.index_select(2, rows)
    o16_s, l16_s = o16.index_select(1, rows), lse16.index_select(2, rows)
    del q, o32, lse32, o16, lse16
    o_ref, l_ref = oracle.attn(q_s, k.cpu(), v.cpu())
    log("  %d sampled tokens x %d heads" % (rows.numel(), H))
    assert_close("O (f32 out)", to_np(o32_s), o_ref)
    assert_close("LSE", to_np(l32_s), l_ref)
    check_bf16_is_rounded_f32("O (bf16 out)", o16_s, o32_s, o_ref)
    assert torch.equal(l16_s, l32_s)


def test_kv_chunks_past_2_31_elements():
    """Two key chunks of 130 keys: the f32 partials [2, 1, Nq, 8, 128] hold 2.15e9
    elements, chunk 1's past 2^31."""
    import diffusion_transformer_long_amd as dtl
    B, Nkv, H, D, P = 1, 260, 8, 128, 2
    assert P * B * NQ * H * D > (1 << 31)
    log("attn_fwd_lse_kv_chunks P=%d B=%d Nq=%d Nkv=%d H=%d D=%d" % (P, B, NQ, Nkv, H, D))
    q = _randn(71, (B, NQ, H, D), torch.bfloat16)
    k = _randn(72, (B, Nkv, H, D), torch.bfloat16, 2.0)
    v = _randn(73, (B, Nkv, H, D), torch.bfloat16)
    o_p, l_p = dtl.attn_fwd_lse_kv_chunks(q, k, v, P)
    torch.cuda.synchronize()
    rows = _sample_rows(NQ, H * D, 74).to(DEV)
    # chunk 1's element offsets pass 2^31 at token (2^31 - NQ*H*D) / (H*D); sample there too
    edge1 = ((1 << 31) - NQ * H * D) // (H * D)
    rows = torch.unique(torch.cat([rows, torch.arange(edge1 - 100, edge1 + 100, device=DEV)]))
    q_s = q.index_select(1, rows).cpu()
    o_s, l_s = o_p.index_select(2, rows), l_p.index_select(3, rows)
    del q, o_p, l_p
    kc, vc = k.cpu(), v.cpu()
    C = Nkv // P
    for t in range(P):
        o_ref, l_ref = oracle.attn(q_s, kc[:, t * C:(t + 1) * C], vc[:, t * C:(t + 1) * C])
        assert_close("chunk %d O" % t, to_np(o_s[t]), o_ref)
        assert_close("chunk %d LSE" % t, to_np(l_s[t]), l_ref)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_merge_past_2_31_elements(out_dtype):
    """P = 2 f32 parts [2, 1, Nq, 8, 128]: part 1's element offsets pass 2^31."""
    import diffusion_transformer_long_amd as dtl
    P, B, H, D = 2, 1, 8, 128
    assert P * B * NQ * H * D > (1 << 31)
    log("attn_merge_lse P=%d B=%d N=%d H=%d D=%d out=%s" % (P, B, NQ, H, D, out_dtype))
    o_p = _randn(81, (P, B, NQ, H, D), torch.float32)
    l_p = _randn(82, (P, B, H, NQ), torch.float32, 3.0)
    o, lse = dtl.attn_merge_lse(o_p, l_p, out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = _sample_rows(NQ, H * D, 83).to(DEV)
    edge1 = ((1 << 31) - NQ * H * D) // (H * D)
    rows = torch.unique(torch.cat([rows, torch.arange(edge1 - 100, edge1 + 100, device=DEV)]))
    op_s = o_p.index_select(2, rows).cpu().numpy()
    lp_s = l_p.index_select(3, rows).cpu().numpy()
    o_s, l_s = o.index_select(1, rows), lse.index_select(2, rows)
    del o_p, l_p, o, lse
    o_ref, l_ref = oracle.merge(op_s, lp_s)
    # the same f32 error bound as the merge tests at small shapes
    f32_err = 2.0 ** -17 * np.abs(op_s).max(axis=0).astype(np.float64)
    if out_dtype == torch.float32:
        assert_close("merged O", to_np(o_s), o_ref, max_abs=float(f32_err.max()), mean_abs=1e-6)
    else:
        assert_bf16_rounding_of("merged O (bf16)", to_np(o_s), o_ref, f32_err)
    assert_close("merged LSE", to_np(l_s), l_ref, max_abs=1e-5, mean_abs=1e-6)


def test_permutes_past_4_gib():
    """seq->head and head->seq permutes of 1 050 000 tokens x 8 heads x 64 eight-byte
    elements: 4.3 GB each way, byte offsets past 2^32.  The forward permute against the
    oracle's index map over the whole tensor, bit for bit; the inverse brings it back to
    the input (the oracle's head->seq undoes its seq->head exactly, as the CPU pins check)."""
    import diffusion_transformer_long_amd as dtl
    p, B, N, H, D = 4, 1, 1_050_000, 8, 64
    nbytes = B * N * H * D * 8
    assert nbytes > (1 << 32)
    log("seq_to_head_permute / head_to_seq_permute p=%d B=%d N=%d H=%d D=%d int64 (%.2f GB)"
        % (p, B, N, H, D, nbytes / 1e9))
    g = torch.Generator(device=DEV)
    g.manual_seed(91)
    x = torch.randint(-(1 << 62), 1 << 62, (p, B, N // p, H, D), generator=g, device=DEV,
                      dtype=torch.int64)
    y = dtl.seq_to_head_permute(x, p)
    torch.cuda.synchronize()
    x_h = x.cpu().numpy()
    ref = oracle.permute(x_h, p)
    same = np.array_equal(y.cpu().numpy(), ref)
    log("  seq->head equals the oracle's permute: %s" % same)
    assert same, "seq->head permute differs from the oracle past 4 GiB"
    del ref
    z = dtl.head_to_seq_permute(y, p)
    torch.cuda.synchronize()
    back = np.array_equal(z.cpu().numpy(), x_h)
    log("  head->seq gives the input back: %s" % back)
    assert back, "head->seq permute does not invert seq->head past 4 GiB"
