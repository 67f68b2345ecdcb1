"""GPU parity of qkv_norm_rope_permute (QK-RMSNorm + rotary embedding fused with the
fused-QKV seq->head permute) against the oracle.

Bar, derived from the arithmetic: the kernel computes in f32 and rounds once to bf16.
The f32 error of the rotation (y_2i cos - y_2i+1 sin) is a few f32 ulps of the pair's
length |(y_2i, y_2i+1)|, which the rotation preserves, so an output that cancels to near
zero carries that absolute error rather than a relative one.  Hence every q/k element
must lie within one bf16 ulp of the oracle's float64 value plus 2^-18 times its pair's
length, and nearly all of them (>= 99%) must equal the round-to-nearest-even bf16 of the
oracle's value (the f32 error only flips the rounding of values next to a midpoint; a
kernel that truncated instead of rounding would fail this).  v is copied: bit-exact.

Cases: small ragged shapes against the whole oracle (p = 1, several p, D = 64 and 128,
B = 2), and at full size the FLUX Ulysses-4 sequence (a 1 x 72 x 64 grid), Wan2.2-5B at
CP-2 (the 31 x 22 x 40 latent grid) and Wan2.1-14B at Ulysses-8 (21 x 45 x 80, 40 heads),
with 3D rotary tables, on a seeded sample of tokens the oracle computes alone.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import log

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
EPS = 1e-6


def _rne_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> the nearest bf16 value (ties to even), as float64, for normal values."""
    m, e = np.frexp(x)                      # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def _ulp_bf16(x: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, e - 8)             # 8 significant bits


def _check_qk(name, got, ref):
    """got, ref [..., D]: (2i, 2i+1) pairs along the last axis."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    pair = np.repeat(np.hypot(ref[..., 0::2], ref[..., 1::2]), 2, axis=-1)
    bound = _ulp_bf16(ref) + 2.0 ** -18 * pair
    worst = float(np.max(np.abs(got - ref) / bound))
    ulps = float(np.max(np.abs(got - ref) / np.maximum(_ulp_bf16(ref), 2.0 ** -126)))
    exact = np.mean(got == _rne_bf16(ref))
    log("  %-26s max %.3f of the bound (%.2f bf16 ulp), %.4f%% correctly rounded (%d values)"
        % (name, worst, ulps, 100 * exact, got.size))
    assert worst <= 1.0, "%s: %.3f of the error bound" % (name, worst)
    assert exact >= 0.99, "%s: only %.4f correctly rounded" % (name, exact)


def _inputs(seed, p, B, N, H, D, grid=None):
    g = np.random.Generator(np.random.PCG64(seed))
    x = torch.from_numpy(g.standard_normal((p, B, N // p, 3, H, D), dtype=np.float32)).to(torch.bfloat16)
    gq = (0.5 + g.random(H * D)).astype(np.float32)
    gk = (0.5 + g.random(H * D)).astype(np.float32)
    if grid is None:
        ang = g.uniform(-6.0, 6.0, size=(N, D // 2))
    else:
        ang = oracle.rope_3d_angles(*grid, D)
    return x, gq, gk, np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _run(x, gq, gk, cs, sn, p):
    import diffusion_transformer_long_amd as dtl
    t = lambda a: torch.from_numpy(a).to(DEV)
    out = dtl.qkv_norm_rope_permute(x.to(DEV), t(gq), t(gk), t(cs), t(sn), p, eps=EPS)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("p,B,N,H,D", [
    (1, 1, 1, 1, 64), (1, 2, 6, 3, 64), (3, 1, 9, 6, 128), (2, 1, 10, 2, 64), (4, 2, 8, 8, 128),
    (1, 1, 5, 64, 128),   # H*D = 8192, the largest row
])
def test_norm_rope_small_full_oracle(p, B, N, H, D):
    log("qkv_norm_rope_permute p=%d B=%d N=%d H=%d D=%d" % (p, B, N, H, D))
    x, gq, gk, cs, sn = _inputs(N * 7 + H, p, B, N, H, D)
    out = _run(x, gq, gk, cs, sn, p)
    ref = oracle.qkv_norm_rope(x, gq, gk, cs, sn, p, eps=EPS)
    o = out.double().cpu().numpy()
    _check_qk("q", o[:, 0], ref[:, 0])
    _check_qk("k", o[:, 1], ref[:, 1])
    assert np.array_equal(o[:, 2], ref[:, 2])


@pytest.mark.parametrize("name,p,H,grid,seed", [
    ("flux_u4", 4, 24, (1, 72, 64), 21),
    ("wan22_5b_cp2", 2, 24, (31, 22, 40), 22),
    ("wan21_14b_u8", 8, 40, (21, 45, 80), 23),
])
def test_norm_rope_full_size_sampled(name, p, H, grid, seed):
    D, B = 128, 1
    N = grid[0] * grid[1] * grid[2]
    log("qkv_norm_rope_permute %s N=%d H=%d p=%d" % (name, N, H, p))
    x, gq, gk, cs, sn = _inputs(seed, p, B, N, H, D, grid)
    out = _run(x, gq, gk, cs, sn, p)
    g = np.random.Generator(np.random.PCG64(5))
    toks = np.unique(np.concatenate([[0, N - 1, N // p - 1, N // p], g.choice(N, 2000, replace=False)]))
    # the oracle on the sampled tokens alone: every token is normalised and rotated by itself
    xs = x.reshape(N, 3, H, D)[torch.from_numpy(toks)].reshape(1, 1, len(toks), 3, H, D)
    ref = oracle.qkv_norm_rope(xs, gq, gk, cs[toks], sn[toks], 1, eps=EPS)[0, :, 0]   # [3, n, H, D]
    o = out[:, :, 0, torch.from_numpy(toks).to(DEV)]                                    # [p, 3, n, H/p, D]
    o = o.permute(1, 2, 0, 3, 4).reshape(3, len(toks), H, D).double().cpu().numpy()
    _check_qk("q", o[0], ref[0])
    _check_qk("k", o[1], ref[1])
    assert np.array_equal(o[2], ref[2])


def test_norm_rope_rejects_bad_arguments():
    import diffusion_transformer_long_amd as dtl
    x = torch.zeros((2, 1, 4, 3, 4, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(4 * 64, device=DEV)
    t = torch.ones((8, 32), device=DEV)
    with pytest.raises(ValueError):
        dtl.qkv_norm_rope_permute(x, g[:-1], g, t, t, 2)           # gamma too short
    with pytest.raises(ValueError):
        dtl.qkv_norm_rope_permute(x, g, g, t[:-1], t, 2)           # table too short
    with pytest.raises(dtl.DtlError):
        dtl.qkv_norm_rope_permute(x, g, g, t, t, 2, eps=-1.0)
    y = torch.zeros((1, 1, 4, 3, 4, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(dtl.DtlError):                              # D = 96: unsupported
        dtl.qkv_norm_rope_permute(y, torch.ones(384, device=DEV), torch.ones(384, device=DEV),
                                  torch.ones((4, 48), device=DEV), torch.ones((4, 48), device=DEV), 1)
