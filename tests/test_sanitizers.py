"""Host-side AddressSanitizer builds of both shared libraries (CPU only).

Each test compiles an instrumented copy into a temporary folder and re-runs the CPU tests
that load that library in a child process with the sanitizer runtime preloaded: the
oracle with gcc's AddressSanitizer and UndefinedBehaviorSanitizer over its pins, and the
HIP library's host code (argument checks, buffer sizing, status strings, profiling
counters; device code is not instrumented) with clang's AddressSanitizer over the C-ABI
tests.  A sanitizer report fails the child's run and so the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _child_pytest(env_extra, files):
    env = dict(os.environ)
    env.update(env_extra)
    # the interpreter itself is not instrumented and keeps memory until exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " passed" in r.stdout, out[-3000:]


def test_oracle_under_asan_and_ubsan(tmp_path):
    from oracle import build as oracle_build
    libasan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    if not os.path.isabs(libasan):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    lib = oracle_build.build(out=str(tmp_path / "liboracle_asan.so"),
                             extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                                    "-fno-omit-frame-pointer", "-g"))
    _child_pytest({"LD_PRELOAD": libasan, "SFFN_ORACLE_LIB": lib}, ["tests/test_oracle.py"])


def test_hip_library_host_code_under_asan(tmp_path):
    from activation_sparse_transformer_amd import build as hip_build
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    # -Xarch_host: instrument the host compilation only (the device code is left as is)
    lib = hip_build.build(out=str(tmp_path / "libsparse_ffn_asan.so"),
                          extra=("-Xarch_host", "-fsanitize=address",
                                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"))
    _child_pytest({"LD_PRELOAD": rt[-1], "SFFN_LIB": lib}, ["tests/test_abi.py"])
