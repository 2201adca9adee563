"""The library's host code and the CPU oracle under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

  - The oracle is compiled with gcc and the sanitizers together with
    tests/oracle_sanitize_main.c, which drives every oracle entry point on
    small inputs, non-finite and overflowing rows and rejected arguments
    included; any invalid access, leak or undefined operation fails the run.
    A planted out-of-bounds read (the E2M1 rounding loop left unbounded on a
    NaN) shows that the build catches one.
  - The HIP library is built with its host code sanitized and the host-side
    ABI tests (argument checks, host multipliers, the device-check hook) run
    against it in a child process, with the sanitizer runtime preloaded.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "macaq_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")
GCC_SAN = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
           "-fno-sanitize-recover=all", "-ffp-contract=off", "-fno-fast-math", "-pthread"]


def _gcc():
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    return gcc


def _build_driver(tmp_path, oracle_src):
    exe = str(tmp_path / "oracle_san")
    res = subprocess.run([_gcc()] + GCC_SAN + [DRIVER_C, oracle_src, "-o", exe, "-lm"], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return exe


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=timeout,
                          env=dict(os.environ, **(env or {})))


def test_oracle_under_sanitizers(tmp_path):
    exe = _build_driver(tmp_path, ORACLE_C)
    res = _run([exe], {"ASAN_OPTIONS": "detect_leaks=1"})
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "oracle checks passed" in res.stdout
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]


def test_sanitizer_build_catches_a_planted_fault(tmp_path):
    """A copy of the oracle with the rounding loop's bound and NaN guard taken
    out (the form that once read past the E2M1 table on a NaN): the
    sanitized run must stop on it."""
    src = open(ORACLE_C).read()
    guard = "  if (!(u >= 0.0)) return 0;"
    bounded = "while (c < 6 && !(u < kE2M1[c + 1])) ++c;"
    assert guard in src and bounded in src, "the planted fault no longer matches the oracle's source"
    lines = [l for l in src.splitlines() if not l.startswith(guard)]
    planted = "\n".join(lines).replace(bounded, "while (!(u < kE2M1[c + 1])) ++c;")
    path = tmp_path / "oracle_planted.c"
    path.write_text(planted)
    exe = _build_driver(tmp_path, str(path))
    res = _run([exe], {"ASAN_OPTIONS": "detect_leaks=1"})
    assert res.returncode != 0
    assert "out of bounds" in res.stderr or "AddressSanitizer" in res.stderr, res.stderr[-2000:]


@pytest.mark.timeout(900)
def test_host_abi_under_sanitizers(tmp_path):
    from mxfp4_w4a4_post_amd import build
    if shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()):
        pytest.skip("hipcc not found")
    lib = build.build_sanitized(str(tmp_path / "libmacaq_san.so"))
    env = {
        "LD_PRELOAD": build.asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0",  # the interpreter's own allocations outlive it
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "MACAQ_LIBRARY": lib,
    }
    res = _run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                "-p", "no:cacheprovider", "-m", "not gpu"], env)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
