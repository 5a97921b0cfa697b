"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each run once:
  * the C oracle, linked into tests/sanitize/oracle_driver.c, which calls every
    oracle function on small seeded inputs (ragged contexts, empty and short
    rows, window stores, non-unit scales);
  * libcsa2 with its host code instrumented (device code is unchanged),
    linked into tests/sanitize/abi_driver.c, which drives every entry point's
    argument validation, the workspace-size function over a grid of shapes and
    the status strings -- all paths that return before any kernel launch.
A sanitizer report, an unexpected status or a non-zero exit fails the test.
"""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd[0], r.returncode, r.stdout[-2000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_driver"
    _run(["gcc", "-std=c11", *SAN_FLAGS, "-ffp-contract=off", "-fopenmp", "-o", str(exe),
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "csa2_oracle.c"),
          "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")
    r = _run([str(exe)], env=env, timeout=600)
    assert r.stdout.startswith("oracle driver ok")
    assert "runtime error" not in r.stderr


def test_library_host_code_under_asan_and_ubsan(tmp_path):
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    from fp4_kv_cache_decode_amd import build
    lib = tmp_path / "libcsa2.so"
    # host-side instrumentation only: every sanitizer flag is preceded by -Xarch_host
    host_flags = []
    for f in SAN_FLAGS:
        host_flags += ["-Xarch_host", f]
    _run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", *host_flags,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-o", str(lib), *build.sources()], timeout=900)
    exe = tmp_path / "abi_driver"
    _run([clang, "-std=c11", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
          "-I", os.path.join(ROOT, "include"), os.path.join(SAN, "abi_driver.c"), "-o", str(exe),
          f"-L{tmp_path}", "-l:libcsa2.so", f"-Wl,-rpath,{tmp_path}",
          f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64"])
    # the HIP runtime's own allocations outlive main: leak checking stays off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([str(exe)], env=env, timeout=300)
    assert r.stdout.startswith("abi driver ok")
    assert "runtime error" not in r.stderr
