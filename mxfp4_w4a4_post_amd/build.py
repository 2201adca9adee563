"""Build ``libmacaq.so`` (the HIP library behind ``include/macaq.h``) for gfx950.

Runs hipcc directly, in-tree, so the built library sits next to its binding.
Device code is compiled without floating-point contraction (the transform's
multiply and butterflies must round one operation at a time) and without
packed-fp32 instructions.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmacaq.so")
# digest of the sources and flags the library was built from, written after it
DIGEST = LIB + ".digest"
SOURCES = ["abi.hip", "quant.hip", "gemm.hip", "moe.hip", "refine.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def source_digest() -> str:
    """sha256 (16 hex digits) of every file in csrc/, the public header and
    the compiler flags."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)) + [os.path.join(INCLUDE, "macaq.h")]
    for path in files:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    h.update(" ".join(HIPCC_FLAGS).encode())
    return h.hexdigest()[:16]


def is_current() -> bool:
    """True when libmacaq.so exists and was built from the current sources."""
    if not (os.path.exists(LIB) and os.path.exists(DIGEST)):
        return False
    with open(DIGEST) as f:
        return f.read().strip() == source_digest()


def build(verbose: bool = False) -> str:
    """Compile every source into libmacaq.so (always recompiles) and record
    the sources' digest beside it."""
    digest = source_digest()
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
    noise = ("packed-fp32-ops",)
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, err))
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    with open(DIGEST + ".tmp", "w") as f:
        f.write(digest + "\n")
    os.replace(DIGEST + ".tmp", DIGEST)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
