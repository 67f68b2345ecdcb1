"""CPU-only checks of the C ABI library and the host logic (no GPU work is done).

* libdtl.so loads and exports every function include/dtl.h declares.
* Invalid arguments are rejected on the host with the documented status codes,
  before anything is launched (the pointers here are never dereferenced).
* The kernels' index helpers (multiply-high division, XCD-contiguous workgroup
  remapping) are checked on the host.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dtl.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    import diffusion_transformer_long_amd as dtl
    names = _declared_functions()
    assert set(names) == set(dtl.EXPORTS), names
    lib = ctypes.CDLL(dtl.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", dtl.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(r" T %s$" % n, out, flags=re.M), n


def test_status_strings():
    import diffusion_transformer_long_amd as dtl
    for code, word in ((0, "OK"), (1, "INVALID"), (2, "UNSUPPORTED"), (3, "HIP")):
        assert word in dtl.status_string(code)
    assert "UNKNOWN" in dtl.status_string(99)


# Fake, 16-byte aligned, disjoint "device" addresses.  Every call below fails validation,
# so they are never handed to a kernel.
A, Bp, C, Dp, E = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def _attn(lib, q=A, k=Bp, v=C, o=Dp, lse=E, B=1, Nq=128, Nkv=128, H=2, D=128, scale=0.088, dt=0):
    return lib.attn_fwd_lse(q, k, v, o, lse, B, Nq, Nkv, H, D, scale, dt, None)


def test_attn_fwd_lse_validation():
    import diffusion_transformer_long_amd as dtl
    lib = dtl.lib
    INV, UNS = dtl.DTL_ERR_INVALID_ARG, dtl.DTL_ERR_UNSUPPORTED
    assert _attn(lib, q=None) == INV
    assert _attn(lib, lse=None) == INV
    for kw in ({"B": 0}, {"Nq": 0}, {"Nkv": 0}, {"H": -1}, {"D": 0}):
        assert _attn(lib, **kw) == INV, kw
    for sc in (0.0, -1.0, float("inf"), float("nan")):
        assert _attn(lib, scale=sc) == INV, sc
    assert _attn(lib, q=A + 8) == INV          # misaligned
    assert _attn(lib, o=A + 64) == INV         # output overlaps q
    assert _attn(lib, lse=Dp + 16) == INV      # lse overlaps o
    assert _attn(lib, D=96) == UNS
    assert _attn(lib, D=256) == UNS
    assert _attn(lib, dt=7) == UNS
    # size limits, with the buffers 2^44 bytes apart so that no overlap decides: Nq or Nkv
    # past 2^31 - 257 (query rows and key indices are ints in the kernel), B*Nkv*H rows past
    # 2^31 - 1, H*D past 2^24
    far = dict(q=1 << 44, k=2 << 44, v=3 << 44, o=4 << 44, lse=5 << 44)
    imax = 2 ** 31 - 1
    for kw in ({"Nq": imax - 255, "H": 1}, {"Nkv": imax - 255, "H": 1},
               {"Nkv": 2 ** 30, "H": 2}, {"H": 2 ** 17 + 1, "Nq": 1, "Nkv": 1}):
        assert _attn(lib, **far, **kw) == INV, kw


def test_attn_fwd_lse_kv_chunks_validation():
    import diffusion_transformer_long_amd as dtl
    lib = dtl.lib
    INV, UNS = dtl.DTL_ERR_INVALID_ARG, dtl.DTL_ERR_UNSUPPORTED

    def call(q=A, k=Bp, v=C, o=Dp, lse=E, B=1, Nq=128, Nkv=256, H=2, D=128, P=2, scale=0.088, dt=1):
        return lib.attn_fwd_lse_kv_chunks(q, k, v, o, lse, B, Nq, Nkv, H, D, P, scale, dt, None)
    for P in (0, -1, 3):                      # P must be positive and divide Nkv
        assert call(P=P) == INV, P
    assert call(o=None) == INV
    assert call(Nkv=0) == INV
    assert call(o=A + 64) == INV              # parts overlap q
    assert call(lse=Dp + 128 * 2 * 128 * 4) == INV   # lse inside the second part of o
    assert call(D=96) == UNS


def test_attn_fwd_lse_accumulate_validation():
    import diffusion_transformer_long_amd as dtl
    lib = dtl.lib
    INV, UNS = dtl.DTL_ERR_INVALID_ARG, dtl.DTL_ERR_UNSUPPORTED
    F = 0x60000000  # o_prev
    G = 0x70000000  # lse_prev

    def acc(q=A, k=Bp, v=C, op=F, lp=G, o=Dp, lse=E, B=1, Nq=128, Nkv=128, H=2, D=128, sc=0.088, dt=1):
        return lib.attn_fwd_lse_accumulate(q, k, v, op, lp, o, lse, B, Nq, Nkv, H, D, sc, dt, None)
    assert acc(op=None) == INV and acc(lp=None) == INV and acc(o=None) == INV
    assert acc(op=F + 4) == INV and acc(lp=G + 8) == INV          # misaligned
    assert acc(o=F + 1024) == INV                                  # overlaps o_prev, not in place
    assert acc(o=F, dt=0) == INV                                   # bf16 output over the f32 o_prev
    assert acc(lse=G + 16) == INV                                  # overlaps lse_prev, not in place
    assert acc(lse=F + 64) == INV                                  # lse inside o_prev
    assert acc(o=G) == INV                                         # o over lse_prev
    assert acc(Nq=0) == INV and acc(sc=0.0) == INV
    assert acc(D=96) == UNS and acc(dt=3) == UNS


def test_qkv_norm_rope_permute_validation():
    import diffusion_transformer_long_amd as dtl
    lib = dtl.lib
    INV, UNS = dtl.DTL_ERR_INVALID_ARG, dtl.DTL_ERR_UNSUPPORTED
    G1, G2, CS, SN = 0x60000000, 0x61000000, 0x62000000, 0x63000000

    def nr(x=A, gq=G1, gk=G2, cs=CS, sn=SN, o=Bp, p=4, B=1, N=64, H=8, D=128, eps=1e-6):
        return lib.qkv_norm_rope_permute(x, gq, gk, cs, sn, o, p, B, N, H, D, eps, None)
    for kw in ({"x": None}, {"gq": None}, {"gk": None}, {"cs": None}, {"sn": None}, {"o": None}):
        assert nr(**kw) == INV, kw
    assert nr(N=66) == INV and nr(H=6) == INV and nr(p=0) == INV
    assert nr(eps=-1.0) == INV and nr(eps=float("inf")) == INV and nr(eps=float("nan")) == INV
    assert nr(gq=G1 + 4) == INV and nr(o=Bp + 2) == INV
    assert nr(o=A + 1024) == INV                 # out overlaps qkv
    assert nr(o=CS - 1024) == INV                # out runs into the cos table
    assert nr(D=96) == UNS and nr(H=72, p=8) == UNS   # H*D = 9216 > 8192


def test_attn_merge_lse_validation():
    import diffusion_transformer_long_amd as dtl
    lib = dtl.lib
    INV, UNS = dtl.DTL_ERR_INVALID_ARG, dtl.DTL_ERR_UNSUPPORTED

    def m(op=A, lp=Bp, o=C, lse=Dp, P=4, B=1, N=64, H=2, D=128, pd=1, od=0):
        return lib.attn_merge_lse(op, lp, o, lse, P, B, N, H, D, pd, od, None)
    assert m(op=None) == INV and m(lp=None) == INV and m(o=None) == INV
    assert m(P=0) == INV and m(N=0) == INV
    assert m(o=A + 32) == INV                   # o overlaps the parts
    assert m(lse=C + 16) == INV                 # lse overlaps o
    assert m(op=A + 4) == INV
    assert m(D=12) == UNS and m(pd=5) == UNS and m(od=9) == UNS and m(P=257) == UNS


@pytest.mark.parametrize("name", ["seq_to_head_permute", "head_to_seq_permute",
                                  "qkv_seq_to_head_permute"])
def test_permute_validation(name):
    import diffusion_transformer_long_amd as dtl
    lib = dtl.lib
    INV, UNS = dtl.DTL_ERR_INVALID_ARG, dtl.DTL_ERR_UNSUPPORTED
    fn = getattr(lib, name)

    def pm(i=A, o=Bp, p=4, B=1, N=64, H=8, D=128, eb=2):
        return fn(i, o, p, B, N, H, D, eb, None)
    assert pm(i=None) == INV and pm(o=None) == INV
    assert pm(N=66) == INV                      # p does not divide N
    assert pm(H=6) == INV                       # p does not divide H
    assert pm(p=0) == INV
    assert pm(o=A + 1024) == INV                # overlap
    assert pm(i=A + 2) == INV                   # misaligned
    assert pm(eb=3) == UNS and pm(eb=16) == UNS
    # more than 2^31 - 256 copy units: 1-byte runs (p = H = D = 1, 1-byte elements), 2^31 of them
    assert pm(p=1, B=2, N=1 << 30, H=1, D=1, eb=1, o=A + (1 << 33)) == INV
    if name == "qkv_seq_to_head_permute":
        assert pm(o=A + 3 * 64 * 8 * 128 * 2 - 16) == INV   # overlaps the 3x larger input


def test_binding_rejects_cpu_tensors_and_bad_shapes():
    import torch
    import diffusion_transformer_long_amd as dtl
    x = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dtl.attn_fwd_lse(x, x, x)
    with pytest.raises(ValueError):
        dtl.attn_fwd_lse_kv_chunks(x, x, x, 2)
    with pytest.raises(ValueError):
        dtl.ring_attention(x, x, x, 3)   # 3 does not divide the 8 keys
    with pytest.raises(ValueError):
        dtl.seq_to_head_permute(torch.zeros((2, 1, 4, 2, 8)), 2)
    with pytest.raises(ValueError):
        dtl.head_to_seq_permute(torch.zeros((2, 1, 4, 2, 8)), 2)
    with pytest.raises(ValueError):
        dtl.qkv_seq_to_head_permute(torch.zeros((2, 1, 4, 3, 2, 8)), 2)
    with pytest.raises(ValueError):
        z = torch.zeros(16)
        dtl.qkv_norm_rope_permute(torch.zeros((2, 1, 4, 3, 2, 8), dtype=torch.bfloat16), z, z, z, z, 2)


def test_host_index_helpers(tmp_path):
    src = os.path.join(ROOT, "tests", "host", "host_logic_check.cpp")
    exe = str(tmp_path / "host_logic_check")
    csrc = os.path.join(ROOT, "diffusion_transformer_long_amd", "csrc")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-I", csrc, "-I", os.path.join(ROOT, "include"),
                        "--offload-arch=gfx950", "-x", "hip", src, "-o", exe],
                       capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("host check build failed:\n" + r.stderr[-3000:])
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout
    assert out.stdout.strip().startswith("OK")
