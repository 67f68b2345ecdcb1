"""CPU oracle for the DiT long-sequence attention path (TEST INFRASTRUCTURE ONLY).

Only tests/, the smoke check and the bench's cpu_baseline leg may import this
package.  The library's product path never touches it; the two share no code.

The arithmetic lives in ``oracle.c`` (float64, plain loops, OpenMP over rows),
built with the host C compiler into ``liboracle.so`` beside it.  This module
marshals numpy float64 arrays in and out.  ``brute`` holds an independent
50-digit ``decimal`` implementation for tiny shapes.

Parity status of each function (what pins it, in tests/test_oracle_pins.py):
  attn, attn_rows : brute force (decimal), closed forms (single key, identical
                    keys, zero query), a worked two-key example, invariants.
  merge           : Ring equivalence against attn, decimal brute force, invariants.
  permute         : numpy reshape/transpose, an emulation of the split / exchange
                    / concatenate sequence, round trip, the pages' byte counts.
  head_to_seq     : an emulation of the split-by-tokens / exchange / concatenate-
                    along-heads sequence, numpy reshape/transpose, round trips with
                    permute in both orders.
  qkv_permute     : the exchange emulation on a packed [.., 3, H, D] tensor, and
                    per-tensor agreement with permute on the q, k, v slices.
  qkv_norm_rope   : closed forms (constant rows, gamma, zero angles, quarter turns),
                    invariances (scale of x, norm of each rotated pair), RoPE's
                    relative-position property on the 3D tables, a decimal brute force,
                    agreement with qkv_permute on v.
  rope_3d_angles  : positions of a (frames, rows, cols) grid, each axis owning a slice
                    of the head's pairs; pinned through the relative-position property.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")



class Api:
    """The oracle's functions bound to one compiled copy of oracle.c."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_attn.argtypes = [dp, dp, dp, i, i, i, i, i, ctypes.c_double, dp, dp]
        lib.oracle_attn.restype = i
        lib.oracle_attn_rows.argtypes = [dp, dp, dp, i, i, i, i, i, ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_int64), ctypes.c_long, dp, dp]
        lib.oracle_attn_rows.restype = i
        lib.oracle_merge.argtypes = [dp, dp, i, i, i, i, i, dp, dp]
        lib.oracle_merge.restype = i
        lib.oracle_permute.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i, i, i, i, i, i]
        lib.oracle_permute.restype = i
        lib.oracle_head_to_seq.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i, i, i, i, i, i]
        lib.oracle_head_to_seq.restype = i
        lib.oracle_qkv_seq_to_head.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i, i, i, i, i, i]
        lib.oracle_qkv_seq_to_head.restype = i
        lib.oracle_qkv_norm_rope.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i, i, ctypes.c_double]
        lib.oracle_qkv_norm_rope.restype = i
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = i
        self.lib = lib

    def threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def attn(self, q, k, v, scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
        """softmax(q k^T * scale) v per head.  q [B,Nq,H,D], k/v [B,Nkv,H,D] ->
        (o [B,Nq,H,D] float64, lse [B,H,Nq] float64); scale defaults to 1/sqrt(D)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Nq, H, D = q.shape
        Nkv = k.shape[1]
        assert k.shape == (B, Nkv, H, D) and v.shape == (B, Nkv, H, D)
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        o = np.empty((B, Nq, H, D), np.float64)
        lse = np.empty((B, H, Nq), np.float64)
        rc = self.lib.oracle_attn(_dp(q), _dp(k), _dp(v), B, Nq, Nkv, H, D, float(scale),
                                  _dp(o), _dp(lse))
        if rc != 0:
            raise ValueError("oracle_attn: bad sizes")
        return o, lse

    def attn_rows(self, q, k, v, rows, scale: float | None = None) -> Tuple[np.ndarray, np.ndarray]:
        """Attention for selected rows only: rows is int64 [n,3] of (b, h, i).
        Returns (o_rows [n,D], lse_rows [n])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Nq, H, D = q.shape
        Nkv = k.shape[1]
        rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
        if scale is None:
            scale = 1.0 / math.sqrt(D)
        n = rows.shape[0]
        o = np.empty((n, D), np.float64)
        lse = np.empty((n,), np.float64)
        rc = self.lib.oracle_attn_rows(_dp(q), _dp(k), _dp(v), B, Nq, Nkv, H, D, float(scale),
                                       rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), n,
                                       _dp(o), _dp(lse))
        if rc != 0:
            raise ValueError("oracle_attn_rows: bad sizes or rows")
        return o, lse

    def merge(self, o_parts, lse_parts) -> Tuple[np.ndarray, np.ndarray]:
        """LSE merge: o_parts [P,B,N,H,D], lse_parts [P,B,H,N] -> (o [B,N,H,D], lse [B,H,N])."""
        o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
        P, B, N, H, D = o_parts.shape
        assert lse_parts.shape == (P, B, H, N)
        o = np.empty((B, N, H, D), np.float64)
        lse = np.empty((B, H, N), np.float64)
        rc = self.lib.oracle_merge(_dp(o_parts), _dp(lse_parts), P, B, N, H, D, _dp(o), _dp(lse))
        if rc != 0:
            raise ValueError("oracle_merge: bad sizes")
        return o, lse

    def permute(self, x: np.ndarray, p: int) -> np.ndarray:
        """Ulysses seq->head permute of stacked shards: [p,B,N/p,H,D] -> [p,B,N,H/p,D].
        Any dtype; a byte-exact copy."""
        x = np.ascontiguousarray(x)
        P_, B, Ns, H, D = x.shape
        assert P_ == p
        N = Ns * p
        if H % p != 0:
            raise ValueError("p must divide H")
        out = np.empty((p, B, N, H // p, D), dtype=x.dtype)
        rc = self.lib.oracle_permute(x.ctypes.data, out.ctypes.data, p, B, N, H, D,
                                     x.dtype.itemsize)
        if rc != 0:
            raise ValueError("oracle_permute: bad sizes")
        return out

    def head_to_seq(self, x: np.ndarray, p: int) -> np.ndarray:
        """Ulysses head->seq permute of stacked head shards: [p,B,N,H/p,D] ->
        [p,B,N/p,H,D].  Any dtype; a byte-exact copy."""
        x = np.ascontiguousarray(x)
        P_, B, N, Hs, D = x.shape
        assert P_ == p
        if N % p != 0:
            raise ValueError("p must divide N")
        out = np.empty((p, B, N // p, Hs * p, D), dtype=x.dtype)
        rc = self.lib.oracle_head_to_seq(x.ctypes.data, out.ctypes.data, p, B, N, Hs * p, D,
                                         x.dtype.itemsize)
        if rc != 0:
            raise ValueError("oracle_head_to_seq: bad sizes")
        return out

    def qkv_permute(self, x: np.ndarray, p: int) -> np.ndarray:
        """Fused QKV seq->head permute: [p,B,N/p,3,H,D] -> [p,3,B,N,H/p,D].  Any dtype;
        a byte-exact copy."""
        x = np.ascontiguousarray(x)
        P_, B, Ns, three, H, D = x.shape
        assert P_ == p and three == 3
        N = Ns * p
        if H % p != 0:
            raise ValueError("p must divide H")
        out = np.empty((p, 3, B, N, H // p, D), dtype=x.dtype)
        rc = self.lib.oracle_qkv_seq_to_head(x.ctypes.data, out.ctypes.data, p, B, N, H, D,
                                             x.dtype.itemsize)
        if rc != 0:
            raise ValueError("oracle_qkv_seq_to_head: bad sizes")
        return out

    def qkv_norm_rope(self, x, gamma_q, gamma_k, cos, sin, p: int, eps: float = 1e-6) -> np.ndarray:
        """QK-RMSNorm over each token's H*D values, rotary embedding of each head's
        (2i, 2i+1) pairs by cos/sin[token, i], v unchanged, written in the fused QKV
        seq->head layout: x [p,B,N/p,3,H,D] -> [p,3,B,N,H/p,D] float64."""
        x = _f64(x)
        P_, B, Ns, three, H, D = x.shape
        assert P_ == p and three == 3
        N = Ns * p
        gq, gk = _f64(gamma_q).reshape(-1), _f64(gamma_k).reshape(-1)
        cs, sn = _f64(cos), _f64(sin)
        assert gq.size == H * D and gk.size == H * D
        assert cs.shape == (N, D // 2) and sn.shape == (N, D // 2)
        out = np.empty((p, 3, B, N, H // p, D), np.float64)
        rc = self.lib.oracle_qkv_norm_rope(_dp(x), _dp(gq), _dp(gk), _dp(cs), _dp(sn), _dp(out),
                                           p, B, N, H, D, float(eps))
        if rc != 0:
            raise ValueError("oracle_qkv_norm_rope: bad sizes")
        return out


def rope_3d_angles(frames: int, rows: int, cols: int, D: int, split=None,
                   base: float = 10000.0) -> np.ndarray:
    """Rotary angles [F*R*C, D/2] (float64) of a (frame, row, col) token grid, tokens in
    row-major grid order (the flattening of a latent video grid into tokens).  The head's
    D/2 rotation pairs are divided among the three axes, `split` pairs each (default: as
    evenly as possible, the remainder to frames), and pair i of an axis that owns d_a
    pairs turns by pos_a * base^(-i / d_a), the one-axis rotary frequencies."""
    half = D // 2
    if split is None:
        hw = half // 3
        split = (half - 2 * hw, hw, hw)
    assert sum(split) == half
    f, r, c = np.meshgrid(np.arange(frames), np.arange(rows), np.arange(cols), indexing="ij")
    pos = [f.reshape(-1).astype(np.float64), r.reshape(-1).astype(np.float64),
           c.reshape(-1).astype(np.float64)]
    cols_out = []
    for a, d_a in enumerate(split):
        inv = base ** (-np.arange(d_a, dtype=np.float64) / d_a)
        cols_out.append(np.outer(pos[a], inv))
    return np.concatenate(cols_out, axis=1)


def _f64(x) -> np.ndarray:
    """Accept numpy arrays or torch tensors (any float dtype); exact upcast to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16/fp32 -> fp64 is exact
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


_default = None


def api() -> Api:
    """The oracle bound to liboracle.so (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        _default = Api(_LIB_PATH)
    return _default


def build(force: bool = True, src: str = None, out: str = None) -> str:
    """Compile oracle.c (or another copy of it) with the host compiler (gcc, -O2, OpenMP)."""
    src = src or _SRC
    out = out or _LIB_PATH
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
               src, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, out)
    return out


def threads() -> int:
    return api().threads()


def attn(q, k, v, scale: float | None = None):
    return api().attn(q, k, v, scale)


def attn_rows(q, k, v, rows, scale: float | None = None):
    return api().attn_rows(q, k, v, rows, scale)


def merge(o_parts, lse_parts):
    return api().merge(o_parts, lse_parts)


def permute(x, p: int):
    return api().permute(x, p)


def head_to_seq(x, p: int):
    return api().head_to_seq(x, p)


def qkv_permute(x, p: int):
    return api().qkv_permute(x, p)


def qkv_norm_rope(x, gamma_q, gamma_k, cos, sin, p: int, eps: float = 1e-6):
    return api().qkv_norm_rope(x, gamma_q, gamma_k, cos, sin, p, eps)
