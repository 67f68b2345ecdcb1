"""Seeded synthetic inputs shared by the HIP path's tests/bench and the CPU oracle.

This module only draws random numbers and lays them out; it holds none of the
attention, merge or permute arithmetic.  Both sides consume the same bf16 bits.

Recipe (one generator per workload):
  * ``numpy.random.Generator(PCG64(seed))``, ``standard_normal(shape, float32)``
    drawn in the order Q, K, V;
  * K is multiplied by ``k_scale`` in float32 *before* the bf16 cast (3.0 for
    the FLUX-shaped workloads, giving attention logits of standard deviation
    about 3; 1.0 elsewhere);
  * the cast to bf16 is round-to-nearest-even (torch's ``.to(torch.bfloat16)``).

Shapes follow the pages' workloads: the FLUX.1 1024^2 sequence of 4096 image
plus 512 text tokens with 24 heads of 128 (arganzheng.life, multi-GPU diffusion
parallelism, section 1 communication table: N = 4608, d = 3072); the Wan2.2
TI2V-5B video sequence of 27280 tokens with 24 heads of 128 ("AIGC 分布式推理：
从 Wan2.2 理解 DP/TP/CP/SP/PP", model parameters); one Ulysses-8 share of
Wan2.1-14B 720p (N = 75600, 40 heads of 128, 5 heads per GPU; arganzheng.life,
section 1 table and section 4.1); Wan2.2's cross-attention, whose 27280 video queries
attend to 512 text keys and values that every GPU holds whole ("AIGC 分布式推理", CP
section; Q comes from the video tokens, K and V from the text).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Nq: int          # query rows handled by this GPU
    Nkv: int         # keys/values this GPU attends to
    H: int
    D: int
    seed: int
    k_scale: float = 1.0
    chunks: int = 1  # KV split into this many equal chunks (Ring rounds), merged by LSE
    q_row0: int = 0  # first query row of the full draw used as this share's Q block
    permute_p: int = 0  # Ulysses degree of the seq->head permute check (0: none)

    @property
    def flops(self) -> float:
        """4 * Nq * Nkv * H * D per batch element: two contractions of 2*Nq*Nkv*D each."""
        return 4.0 * self.B * self.Nq * self.Nkv * self.H * self.D

    @property
    def chunk_len(self) -> int:
        assert self.Nkv % self.chunks == 0
        return self.Nkv // self.chunks


# The workloads.  The seed of each is fixed here once, not chosen after the fact.
TINY_RING = Workload("tiny_ring_N256_H4_D64_kv4x64", 1, 256, 256, 4, 64, seed=1, chunks=4)
FLUX = Workload("flux_1024_N4608_H24_D128", 1, 4608, 4608, 24, 128, seed=2, k_scale=3.0)
FLUX_RING4 = Workload("flux_ring4_share_Nq1152_Nkv4608_H24_D128_kv4x1152", 1, 1152, 4608, 24, 128,
                      seed=2, k_scale=3.0, chunks=4, q_row0=0, permute_p=4)
WAN5B = Workload("wan22_ti2v5b_N27280_H24_D128", 1, 27280, 27280, 24, 128, seed=4)
WAN14B_U8 = Workload("wan21_14b_720p_u8_share_N75600_H5_D128_kv8x9450", 1, 75600, 75600, 5, 128,
                     seed=5, chunks=8)
# Cross-attention: Q draws 27280 rows, then K and V 512 each.
WAN5B_CROSS = Workload("wan22_ti2v5b_cross_Nq27280_Nkv512_H24_D128", 1, 27280, 512, 24, 128, seed=6)

ALL = (TINY_RING, FLUX, FLUX_RING4, WAN5B, WAN14B_U8, WAN5B_CROSS)
BY_NAME = {w.name: w for w in ALL}


def draw_f32(seed: int, B: int, N: int, H: int, D: int, k_scale: float = 1.0,
             n_kv: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q as float32 [B, N, H, D], then K and V as [B, n_kv (default N), H, D], in draw
    order Q, K, V; K scaled before rounding."""
    g = np.random.Generator(np.random.PCG64(seed))
    n_kv = N if n_kv is None else n_kv
    q = g.standard_normal((B, N, H, D), dtype=np.float32)
    k = g.standard_normal((B, n_kv, H, D), dtype=np.float32)
    v = g.standard_normal((B, n_kv, H, D), dtype=np.float32)
    if k_scale != 1.0:
        k *= np.float32(k_scale)
    return q, k, v


def to_bf16(x: np.ndarray):
    """float32 numpy -> bf16 torch CPU tensor (round to nearest even)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def workload_qkv(w: Workload):
    """bf16 CPU tensors (q, k, v) of one workload: q is [B, Nq, H, D] (its Q block),
    k and v are [B, Nkv, H, D]."""
    n_q = max(w.Nkv, w.q_row0 + w.Nq)   # a Q block is cut from the full sequence's draw
    q, k, v = draw_f32(w.seed, w.B, n_q, w.H, w.D, w.k_scale, n_kv=w.Nkv)
    q = q[:, w.q_row0:w.q_row0 + w.Nq]
    return to_bf16(q), to_bf16(k), to_bf16(v)


def random_bf16(seed: int, shape, scale: float = 1.0):
    """Generic seeded bf16 CPU tensor ~ scale * N(0, 1)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return to_bf16(x)


def sample_rows(seed: int, B: int, H: int, Nq: int, n: int) -> np.ndarray:
    """A seeded sample of n distinct (b, h, i) query rows as an int64 array [n, 3].

    The first and last rows of every head are always included (they exercise the
    first tile and the ragged tail); the rest are uniform without replacement."""
    g = np.random.Generator(np.random.PCG64(seed))
    fixed = []
    for b in range(B):
        for h in range(H):
            fixed.append((b, h, 0))
            fixed.append((b, h, Nq - 1))
    fixed = sorted(set(fixed))
    total = B * H * Nq
    n_rand = max(0, min(n - len(fixed), total - len(fixed)))
    picks = set(fixed)
    out = list(fixed)
    while len(out) < len(fixed) + n_rand:
        cand = g.integers(0, total, size=2 * n_rand + 16)
        for c in cand:
            c = int(c)
            t = (c // (H * Nq), (c // Nq) % H, c % Nq)
            if t not in picks:
                picks.add(t)
                out.append(t)
                if len(out) >= len(fixed) + n_rand:
                    break
    return np.asarray(out, dtype=np.int64).reshape(-1, 3)
