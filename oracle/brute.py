"""50-digit decimal brute force for tiny shapes (TEST INFRASTRUCTURE ONLY).

Written from the definitions directly and independently of oracle.c: no row-max
subtraction (decimal's exponent range makes exp(s) safe), exact products and
sums at 50 significant digits.

  attention (MindIE SD "多卡并行", Ring Sequence Parallel usage example):
      s_j = (q . k_j) / sqrt(D);  w_j = exp(s_j);  o = sum_j w_j v_j / sum_j w_j;
      lse = ln sum_j w_j.
  merge (arganzheng.life, multi-GPU diffusion parallelism, section 4.2, the
  online-softmax accumulation across Ring rounds):
      W_t = exp(lse_t);  o = sum_t W_t o_t / sum_t W_t;  lse = ln sum_t W_t.
  QK-RMSNorm + rotary embedding of one token's hidden vector ("AIGC 分布式推理：从 Wan2.2
  理解 DP/TP/CP/SP/PP", TP section: the norm spans all heads; RoPE acts by position):
      y = x * gamma / sqrt(sum(x^2) / len(x) + eps); each head's pair (y_2i, y_2i+1)
      multiplied, as a complex number y_2i + i y_2i+1, by cos_i + i sin_i.
"""
from __future__ import annotations

from decimal import Decimal, localcontext
from typing import List, Sequence, Tuple

PREC = 50


def _d(x) -> Decimal:
    return Decimal(float(x)) if not isinstance(x, Decimal) else x


def attn_row(q: Sequence, keys: Sequence[Sequence], vals: Sequence[Sequence],
             scale=None) -> Tuple[List[Decimal], Decimal]:
    """One query row against Nkv keys.  Inputs are floats (converted exactly)."""
    with localcontext() as ctx:
        ctx.prec = PREC
        D = len(q)
        sc = (Decimal(1) / Decimal(D).sqrt()) if scale is None else _d(scale)
        qd = [_d(x) for x in q]
        w = []
        for kj in keys:
            s = sum((qd[d] * _d(kj[d]) for d in range(D)), Decimal(0)) * sc
            w.append(s.exp())
        total = sum(w, Decimal(0))
        Dv = len(vals[0])
        o = []
        for d in range(Dv):
            o.append(sum((w[j] * _d(vals[j][d]) for j in range(len(w))), Decimal(0)) / total)
        return o, total.ln()


def attn(q, k, v, scale=None):
    """Nested-list attention: q [B][Nq][H][D], k/v [B][Nkv][H][D] -> (o, lse) as nested
    lists of Decimal with o [B][Nq][H][D] and lse [B][H][Nq]."""
    B, Nq, H = len(q), len(q[0]), len(q[0][0])
    Nkv = len(k[0])
    o = [[[None] * H for _ in range(Nq)] for _ in range(B)]
    lse = [[[None] * Nq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            keys = [k[b][j][h] for j in range(Nkv)]
            vals = [v[b][j][h] for j in range(Nkv)]
            for i in range(Nq):
                orow, l = attn_row(q[b][i][h], keys, vals, scale)
                o[b][i][h] = orow
                lse[b][h][i] = l
    return o, lse


def merge_row(o_parts: Sequence[Sequence], lse_parts: Sequence) -> Tuple[List[Decimal], Decimal]:
    """Merge one row from P parts (floats, lse may be -inf)."""
    with localcontext() as ctx:
        ctx.prec = PREC
        W = [(_d(l).exp() if l != float("-inf") else Decimal(0)) for l in lse_parts]
        total = sum(W, Decimal(0))
        D = len(o_parts[0])
        if total == 0:
            return [Decimal(0)] * D, None
        o = [sum((W[t] * _d(o_parts[t][d]) for t in range(len(W))), Decimal(0)) / total
             for d in range(D)]
        return o, total.ln()


def norm_rope_token(x: Sequence, gamma: Sequence, cos: Sequence, sin: Sequence, D: int,
                    eps) -> List[Decimal]:
    """One token's q (or k): x and gamma have H*D values, cos/sin the D/2 values of the
    token's position.  Returns H*D decimals."""
    with localcontext() as ctx:
        ctx.prec = PREC
        xd = [_d(a) for a in x]
        n = len(xd)
        ms = sum((a * a for a in xd), Decimal(0)) / Decimal(n)
        inv = Decimal(1) / (ms + _d(eps)).sqrt()
        y = [xd[e] * inv * _d(gamma[e]) for e in range(n)]
        out = []
        for h in range(n // D):
            for i in range(D // 2):
                re, im = y[h * D + 2 * i], y[h * D + 2 * i + 1]
                c, s_ = _d(cos[i]), _d(sin[i])
                out.append(re * c - im * s_)
                out.append(re * s_ + im * c)
        return out
