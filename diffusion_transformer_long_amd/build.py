"""Build step of libdtl.so: hipcc for gfx950, every HIP source, in-tree."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdtl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["capi.hip", "attn_fwd.hip", "merge.hip", "permute.hip", "norm_rope.hip"]

# Packed-f32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


# The attention kernel's row max runs over logits that are finite or -inf (masked keys), so
# it needs no NaN quieting of operands.  A row's first weights, taken against a -inf reference,
# can be +inf or NaN; the kernel tests their sum as a bit pattern, which this flag cannot fold.
EXTRA = {"attn_fwd.hip": ["-fno-honor-nans"]}


def _obj(src: str) -> str:
    return os.path.join(CSRC, os.path.splitext(src)[0] + ".o")


def _compile(src: str) -> str:
    obj = _obj(src)
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libdtl.so (always rebuilds)."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
