"""Python binding of libdtl.so: DiT long-sequence attention on one MI355X (gfx950).

Argument marshalling only.  Every function here checks tensor devices, dtypes and
shapes, allocates outputs with torch when none are given, and calls the C ABI of
``include/dtl.h`` with raw device pointers and torch's current HIP stream.  All
arithmetic runs in the HIP kernels.  Importing this package fails when the
library has not been built; there is no fallback.

Entry points (same names as the C ABI):
  attn_fwd_lse(q, k, v, ...)            -> (o, lse)
  attn_fwd_lse_noalloc(q, k, v, o, lse)  -> (o, lse)  nothing allocated, outputs given
  attn_fwd_lse_accumulate(q, k, v, o_prev, lse_prev, ...) -> (o, lse)
  attn_merge_lse(o_parts, lse_parts, ...) -> (o, lse)
  seq_to_head_permute(x, p, ...)        -> out
  head_to_seq_permute(y, p, ...)        -> out
  qkv_seq_to_head_permute(x, p, ...)    -> out
  qkv_norm_rope_permute(x, gamma_q, gamma_k, cos, sin, p, ...) -> out
  attn_fwd_lse_kv_chunks(q, k, v, chunks) -> (o_parts, lse_parts)  all KV chunks, one launch
and a driver that only sequences those calls:
  ring_attention(q, k, v, chunks)          -> (o, lse)              the rounds' partials (one
                                                                    launch or one per round),
                                                                    then the merge; or rounds
                                                                    accumulated
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdtl.so")

DTL_OK, DTL_ERR_INVALID_ARG, DTL_ERR_UNSUPPORTED, DTL_ERR_HIP, DTL_ERR_WORKSPACE = 0, 1, 2, 3, 4
DTL_BF16, DTL_F32 = 0, 1

EXPORTS = ("attn_fwd_lse", "attn_fwd_lse_noalloc", "attn_fwd_lse_accumulate", "attn_fwd_lse_kv_chunks", "attn_merge_lse",
           "seq_to_head_permute", "head_to_seq_permute", "qkv_seq_to_head_permute",
           "qkv_norm_rope_permute", "dtl_status_string")


class DtlError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libdtl.so is not built (%s). Build it with `python __graft_entry__.py` or "
            "`python -m diffusion_transformer_long_amd.build`." % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd_lse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_lse.restype = i
    lib.attn_fwd_lse_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_lse_noalloc.restype = i
    lib.attn_fwd_lse_accumulate.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_lse_accumulate.restype = i
    lib.attn_fwd_lse_kv_chunks.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.attn_fwd_lse_kv_chunks.restype = i
    lib.attn_merge_lse.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.attn_merge_lse.restype = i
    for name in ("seq_to_head_permute", "head_to_seq_permute", "qkv_seq_to_head_permute"):
        getattr(lib, name).argtypes = [vp, vp, i, i, i, i, i, i, vp]
        getattr(lib, name).restype = i
    lib.qkv_norm_rope_permute.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    lib.qkv_norm_rope_permute.restype = i
    lib.dtl_status_string.argtypes = [i]
    lib.dtl_status_string.restype = ctypes.c_char_p
    return lib


lib = _load_library()


def status_string(status: int) -> str:
    return lib.dtl_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != DTL_OK:
        raise DtlError(status, status_string(status))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return DTL_BF16
    if dt == torch.float32:
        return DTL_F32
    raise TypeError("unsupported dtype %s (bf16 or f32)" % dt)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))


def attn_fwd_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                 o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 softmax_scale: Optional[float] = None, o_dtype: torch.dtype = torch.bfloat16,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """o = softmax(q k^T * scale) v and lse = ln sum exp(scale q.k) per (b, h, row).
    q [B,Nq,H,D], k/v [B,Nkv,H,D] bf16 -> o [B,Nq,H,D] (o_dtype), lse [B,H,Nq] f32."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, torch.bfloat16, 4)
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, D) or tuple(v.shape) != (B, Nkv, H, D):
        raise ValueError("k and v must be [B, Nkv, H, D] matching q %s" % (tuple(q.shape),))
    if o is None:
        o = torch.empty((B, Nq, H, D), dtype=o_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _dev(o, "o", None, 4)
    _dev(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Nq, H, D) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o must be [B,Nq,H,D] and lse [B,H,Nq]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, Nq, Nkv, H, D, scale, _dtype_code(o.dtype), _stream(q, stream)))
    return o, lse


def attn_fwd_lse_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                         lse: torch.Tensor, softmax_scale: Optional[float] = None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_fwd_lse for callers that cannot allocate: the caller passes o (bf16 or f32)
    and lse; the library's split workspace is a static device array shared by every call
    on the device (calls that overlap in time on one device race)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, torch.bfloat16, 4)
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, D) or tuple(v.shape) != (B, Nkv, H, D):
        raise ValueError("k and v must be [B, Nkv, H, D] matching q %s" % (tuple(q.shape),))
    _dev(o, "o", None, 4)
    _dev(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Nq, H, D) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o must be [B,Nq,H,D] and lse [B,H,Nq]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_lse_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, Nq, Nkv, H, D, scale, _dtype_code(o.dtype),
                                    _stream(q, stream)))
    return o, lse


def attn_fwd_lse_accumulate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            o_prev: torch.Tensor, lse_prev: torch.Tensor,
                            o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                            softmax_scale: Optional[float] = None,
                            o_dtype: torch.dtype = torch.float32,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One Ring round: attention of q over these k/v folded into the previous result
    (o_prev [B,Nq,H,D] f32, lse_prev [B,H,Nq] f32; lse_prev = -inf rows hold no keys yet).
    By default the result overwrites o_prev and lse_prev (f32); pass o_dtype=bf16 (and
    no o) for the last round's final output."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, torch.bfloat16, 4)
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, D) or tuple(v.shape) != (B, Nkv, H, D):
        raise ValueError("k and v must be [B, Nkv, H, D] matching q %s" % (tuple(q.shape),))
    _dev(o_prev, "o_prev", torch.float32, 4)
    _dev(lse_prev, "lse_prev", torch.float32, 3)
    if tuple(o_prev.shape) != (B, Nq, H, D) or tuple(lse_prev.shape) != (B, H, Nq):
        raise ValueError("o_prev must be [B,Nq,H,D] and lse_prev [B,H,Nq]")
    if o is None:
        o = o_prev if o_dtype == torch.float32 else torch.empty((B, Nq, H, D), dtype=o_dtype,
                                                                 device=q.device)
    if lse is None:
        lse = lse_prev
    _dev(o, "o", None, 4)
    _dev(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Nq, H, D) or tuple(lse.shape) != (B, H, Nq):
        raise ValueError("o must be [B,Nq,H,D] and lse [B,H,Nq]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_lse_accumulate(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_prev.data_ptr(),
                                       lse_prev.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       B, Nq, Nkv, H, D, scale, _dtype_code(o.dtype),
                                       _stream(q, stream)))
    return o, lse


def attn_merge_lse(o_parts: torch.Tensor, lse_parts: torch.Tensor,
                   o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.bfloat16, write_lse: bool = True,
                   stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Exact merge of partials over disjoint key sets: o_parts [P,B,N,H,D] (f32 or bf16),
    lse_parts [P,B,H,N] f32 -> o [B,N,H,D] (out_dtype), lse [B,H,N] f32 (or None)."""
    _dev(o_parts, "o_parts", None, 5)
    _dev(lse_parts, "lse_parts", torch.float32, 4)
    P, B, N, H, D = o_parts.shape
    if tuple(lse_parts.shape) != (P, B, H, N):
        raise ValueError("lse_parts must be [P,B,H,N] = %s" % ((P, B, H, N),))
    if o is None:
        o = torch.empty((B, N, H, D), dtype=out_dtype, device=o_parts.device)
    _dev(o, "o", None, 4)
    if tuple(o.shape) != (B, N, H, D):
        raise ValueError("o must be [B,N,H,D]")
    if write_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    if lse is not None:
        _dev(lse, "lse", torch.float32, 3)
        if tuple(lse.shape) != (B, H, N):
            raise ValueError("lse must be [B,H,N]")
    _check(lib.attn_merge_lse(o_parts.data_ptr(), lse_parts.data_ptr(), o.data_ptr(),
                              lse.data_ptr() if lse is not None else None,
                              P, B, N, H, D, _dtype_code(o_parts.dtype), _dtype_code(o.dtype),
                              _stream(o_parts, stream)))
    return o, lse


def seq_to_head_permute(x: torch.Tensor, p: int, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Ulysses seq->head permute: x [p,B,N/p,H,D] (p sequence shards) ->
    out [p,B,N,H/p,D] (p head shards).  Any 1/2/4/8-byte dtype; bit-exact."""
    _dev(x, "x", None, 5)
    p_, B, Ns, H, D = x.shape
    if p_ != p:
        raise ValueError("x.shape[0] must equal p")
    if H % p != 0:
        raise ValueError("p must divide the head count")
    N = Ns * p
    if out is None:
        out = torch.empty((p, B, N, H // p, D), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype, 5)
    if tuple(out.shape) != (p, B, N, H // p, D):
        raise ValueError("out must be [p,B,N,H/p,D]")
    _check(lib.seq_to_head_permute(x.data_ptr(), out.data_ptr(), p, B, N, H, D,
                                   x.element_size(), _stream(x, stream)))
    return out


def head_to_seq_permute(y: torch.Tensor, p: int, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Ulysses head->seq permute (after attention): y [p,B,N,H/p,D] (p head shards) ->
    out [p,B,N/p,H,D] (p sequence shards).  Any 1/2/4/8-byte dtype; bit-exact."""
    _dev(y, "y", None, 5)
    p_, B, N, Hs, D = y.shape
    if p_ != p:
        raise ValueError("y.shape[0] must equal p")
    if N % p != 0:
        raise ValueError("p must divide the token count")
    H = Hs * p
    if out is None:
        out = torch.empty((p, B, N // p, H, D), dtype=y.dtype, device=y.device)
    _dev(out, "out", y.dtype, 5)
    if tuple(out.shape) != (p, B, N // p, H, D):
        raise ValueError("out must be [p,B,N/p,H,D]")
    _check(lib.head_to_seq_permute(y.data_ptr(), out.data_ptr(), p, B, N, H, D,
                                   y.element_size(), _stream(y, stream)))
    return out


def qkv_seq_to_head_permute(x: torch.Tensor, p: int, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Fused QKV seq->head permute: x [p,B,N/p,3,H,D] (p sequence shards of packed q, k,
    v) -> out [p,3,B,N,H/p,D]; out[j, 0], out[j, 1], out[j, 2] are head group j's q, k, v.
    Any 1/2/4/8-byte dtype; bit-exact."""
    _dev(x, "x", None, 6)
    p_, B, Ns, three, H, D = x.shape
    if p_ != p or three != 3:
        raise ValueError("x must be [p,B,N/p,3,H,D]")
    if H % p != 0:
        raise ValueError("p must divide the head count")
    N = Ns * p
    if out is None:
        out = torch.empty((p, 3, B, N, H // p, D), dtype=x.dtype, device=x.device)
    _dev(out, "out", x.dtype, 6)
    if tuple(out.shape) != (p, 3, B, N, H // p, D):
        raise ValueError("out must be [p,3,B,N,H/p,D]")
    _check(lib.qkv_seq_to_head_permute(x.data_ptr(), out.data_ptr(), p, B, N, H, D,
                                       x.element_size(), _stream(x, stream)))
    return out


def qkv_norm_rope_permute(x: torch.Tensor, gamma_q: torch.Tensor, gamma_k: torch.Tensor,
                          cos: torch.Tensor, sin: torch.Tensor, p: int, eps: float = 1e-6,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """QK-RMSNorm (over each token's H*D values) and rotary embedding of each head's
    (2i, 2i+1) pairs by cos/sin[token, i], fused with the fused-QKV seq->head permute:
    x bf16 [p,B,N/p,3,H,D] -> out bf16 [p,3,B,N,H/p,D]; gamma_q/gamma_k f32 [H*D];
    cos/sin f32 [N, D/2] over the whole sequence's positions."""
    _dev(x, "x", torch.bfloat16, 6)
    p_, B, Ns, three, H, D = x.shape
    if p_ != p or three != 3:
        raise ValueError("x must be [p,B,N/p,3,H,D]")
    if H % p != 0:
        raise ValueError("p must divide the head count")
    N = Ns * p
    for t, n in ((gamma_q, "gamma_q"), (gamma_k, "gamma_k")):
        _dev(t, n, torch.float32, None)
        if t.numel() != H * D:
            raise ValueError("%s must hold H*D = %d values" % (n, H * D))
    for t, n in ((cos, "cos"), (sin, "sin")):
        _dev(t, n, torch.float32, 2)
        if tuple(t.shape) != (N, D // 2):
            raise ValueError("%s must be [N, D/2] = %s" % (n, (N, D // 2)))
    if out is None:
        out = torch.empty((p, 3, B, N, H // p, D), dtype=torch.bfloat16, device=x.device)
    _dev(out, "out", torch.bfloat16, 6)
    if tuple(out.shape) != (p, 3, B, N, H // p, D):
        raise ValueError("out must be [p,3,B,N,H/p,D]")
    _check(lib.qkv_norm_rope_permute(x.data_ptr(), gamma_q.data_ptr(), gamma_k.data_ptr(),
                                     cos.data_ptr(), sin.data_ptr(), out.data_ptr(), p, B, N, H, D,
                                     float(eps), _stream(x, stream)))
    return out


def attn_fwd_lse_kv_chunks(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, chunks: int,
                           o_parts: Optional[torch.Tensor] = None,
                           lse_parts: Optional[torch.Tensor] = None,
                           softmax_scale: Optional[float] = None,
                           o_dtype: torch.dtype = torch.float32,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_fwd_lse of q against each contiguous KV chunk [t*C, (t+1)*C), C = Nkv/chunks,
    in one launch: o_parts [P,B,Nq,H,D] (o_dtype, f32 by default), lse_parts [P,B,H,Nq],
    the layout attn_merge_lse takes."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, torch.bfloat16, 4)
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    if tuple(k.shape) != (B, Nkv, H, D) or tuple(v.shape) != (B, Nkv, H, D):
        raise ValueError("k and v must be [B, Nkv, H, D] matching q %s" % (tuple(q.shape),))
    if chunks <= 0 or Nkv % chunks != 0:
        raise ValueError("chunks must be positive and divide Nkv")
    P = chunks
    if o_parts is None:
        o_parts = torch.empty((P, B, Nq, H, D), dtype=o_dtype, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((P, B, H, Nq), dtype=torch.float32, device=q.device)
    _dev(o_parts, "o_parts", None, 5)
    _dev(lse_parts, "lse_parts", torch.float32, 4)
    if tuple(o_parts.shape) != (P, B, Nq, H, D) or tuple(lse_parts.shape) != (P, B, H, Nq):
        raise ValueError("o_parts must be [P,B,Nq,H,D] and lse_parts [P,B,H,Nq]")
    scale = 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)
    _check(lib.attn_fwd_lse_kv_chunks(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_parts.data_ptr(),
                                      lse_parts.data_ptr(), B, Nq, Nkv, H, D, P, scale,
                                      _dtype_code(o_parts.dtype), _stream(q, stream)))
    return o_parts, lse_parts


def _round_fills_gpu(q: torch.Tensor) -> bool:
    """Whether one round's launch (the 128-row query tiles of q, two per compute unit)
    occupies every workgroup slot of the GPU."""
    B, Nq, H, _ = q.shape
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    return B * H * ((Nq + 127) // 128) >= 2 * cus


def ring_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, chunks: int,
                   out_dtype: torch.dtype = torch.bfloat16, softmax_scale: Optional[float] = None,
                   o_parts: Optional[torch.Tensor] = None, lse_parts: Optional[torch.Tensor] = None,
                   o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   accumulate: bool = False, o_acc: Optional[torch.Tensor] = None,
                   one_launch: Optional[bool] = None,
                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention over all keys computed as Ring attention's rounds on one GPU, over
    contiguous KV chunks [t*C, (t+1)*C) (B must be 1 for the per-round forms, whose
    chunks are views of k and v).

    accumulate=False: f32 partials of every round (o_parts, lse_parts), then the LSE
    merge.  The partials come from one attn_fwd_lse call per round (one_launch=False),
    or from one attn_fwd_lse_kv_chunks call for all rounds (one_launch=True, any B);
    by default the one launch is taken when a single round's tiles would leave workgroup
    slots idle (short Q blocks such as the FLUX Ring-4 share), one call per round otherwise.
    accumulate=True: the first round writes an f32 running result (o_acc, and lse), each
    later round folds its chunk into it with attn_fwd_lse_accumulate, and the last round
    writes the final o in out_dtype; no partials are stored."""
    B, Nq, H, D = q.shape
    Nkv = k.shape[1]
    if chunks <= 0 or Nkv % chunks != 0:
        raise ValueError("chunks must be positive and divide Nkv")
    if one_launch is None:
        one_launch = chunks > 1 and not _round_fills_gpu(q)
    if not accumulate and one_launch:
        o_parts, lse_parts = attn_fwd_lse_kv_chunks(q, k, v, chunks, o_parts, lse_parts,
                                                    softmax_scale, stream=stream)
        return attn_merge_lse(o_parts, lse_parts, o=o, lse=lse, out_dtype=out_dtype,
                              stream=stream)
    if B != 1:
        raise ValueError("KV chunking by views needs B == 1")
    C = Nkv // chunks
    if not accumulate:
        if o_parts is None:
            o_parts = torch.empty((chunks, B, Nq, H, D), dtype=torch.float32, device=q.device)
        if lse_parts is None:
            lse_parts = torch.empty((chunks, B, H, Nq), dtype=torch.float32, device=q.device)
        for t in range(chunks):
            attn_fwd_lse(q, k[:, t * C:(t + 1) * C], v[:, t * C:(t + 1) * C], o=o_parts[t],
                         lse=lse_parts[t], softmax_scale=softmax_scale, stream=stream)
        return attn_merge_lse(o_parts, lse_parts, o=o, lse=lse, out_dtype=out_dtype,
                              stream=stream)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if chunks == 1:
        return attn_fwd_lse(q, k, v, o=o, lse=lse, softmax_scale=softmax_scale,
                            o_dtype=out_dtype if o is None else o.dtype, stream=stream)
    if o_acc is None:
        o_acc = torch.empty((B, Nq, H, D), dtype=torch.float32, device=q.device)
    attn_fwd_lse(q, k[:, :C], v[:, :C], o=o_acc, lse=lse, softmax_scale=softmax_scale,
                 stream=stream)
    for t in range(1, chunks - 1):
        attn_fwd_lse_accumulate(q, k[:, t * C:(t + 1) * C], v[:, t * C:(t + 1) * C], o_acc, lse,
                                softmax_scale=softmax_scale, stream=stream)
    if o is None:
        o = o_acc if out_dtype == torch.float32 else torch.empty((B, Nq, H, D), dtype=out_dtype,
                                                                 device=q.device)
    t = chunks - 1
    return attn_fwd_lse_accumulate(q, k[:, t * C:], v[:, t * C:], o_acc, lse, o=o,
                                   softmax_scale=softmax_scale, stream=stream)
