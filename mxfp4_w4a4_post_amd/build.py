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
SOURCES = ["abi.hip", "quant.hip", "gemm.hip", "moe.hip", "refine.hip", "probe.hip"]

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


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (each flag
# applies to the host pass only; device code is built as usual).
SANITIZE_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g",
]


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime, to preload into a
    process that loads the sanitized library."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found (%r)" % path)
    return path


def build_sanitized(out: str, jobs: int = 5) -> str:
    """The same sources as libmacaq.so, host code sanitized, linked to `out`
    (the objects go beside it). For the CPU tests of the host code: nothing
    in it is launched."""
    from concurrent.futures import ThreadPoolExecutor
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + SANITIZE_FLAGS + ["-I", INCLUDE, "-I", CSRC]

    def compile_one(src):
        obj = os.path.join(os.path.dirname(out), os.path.splitext(src)[0] + ".san.o")
        res = subprocess.run([hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                             capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed on %s (%d):\n%s" % (src, res.returncode, res.stderr))
        return obj

    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    res = subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + SANITIZE_FLAGS + ["-o", out] + objs,
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed (%d):\n%s" % (res.returncode, res.stderr))
    return out
