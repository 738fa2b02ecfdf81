"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two child processes, each with the sanitizer runtime preloaded and any finding fatal:
  * the oracle's pins (tests/test_oracle_pins.py, tests/test_oracle_ext_pins.py) against the
    oracle built with gcc -fsanitize=address,undefined;
  * the C ABI's host-side checks (tests/test_abi_cpu.py: every invalid call refused before a
    launch, the workspace and scratch size queries, the exported symbols) against libhalo built
    with the sanitizers on its host code (clang, -Xarch_host; the device code is built as usual
    and never launched here).
The sanitized libraries are built under _build/sanitize/ when missing or older than their
sources (the library's takes a few minutes: its device code is compiled too).
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "hadamard_rotated_precision_halo_amd", "csrc")


def _stale(lib, sources):
    return not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib)
                                          for s in sources)


def _run_child(code, preload):
    env = dict(os.environ, LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_sanitizers():
    from oracle import build as ob
    lib = os.path.join(OUT, "libhalo_oracle_san.so")
    if _stale(lib, [ob.SRC]):
        os.makedirs(OUT, exist_ok=True)
        ob.build_sanitized(lib)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    code = ("import sys, pytest\n"
            "import oracle.build as ob\n"
            f"ob.LIB = {lib!r}\n"
            "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', "
            "'tests/test_oracle_pins.py', 'tests/test_oracle_ext_pins.py']))\n")
    out = _run_child(code, asan)
    assert " passed" in out


def test_abi_checks_under_sanitizers():
    from hadamard_rotated_precision_halo_amd import build as hb
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    lib = os.path.join(OUT, "libhalo_san.so")
    sources = [os.path.join(CSRC, f) for f in hb.SOURCES + hb.HEADERS]
    sources.append(os.path.join(ROOT, "include", "halo.h"))
    if _stale(lib, sources):
        os.makedirs(OUT, exist_ok=True)
        hb.build_host_sanitized(lib)
    code = ("import sys, pytest\n"
            "import hadamard_rotated_precision_halo_amd as H\n"
            f"H.LIB_PATH = {lib!r}\n"
            "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', "
            "'tests/test_abi_cpu.py']))\n")
    out = _run_child(code, rt[-1])
    assert " passed" in out
