"""Host sanitizer runs (CPU only, no GPU call):

  * the oracle's C recurrence (oracle/recurrence.c), driven by
    tests/sanitize/oracle_driver.c with exactly-sized arrays, under
    AddressSanitizer + UndefinedBehaviorSanitizer and under ThreadSanitizer
    (its chains run on several threads);
  * the library's host code -- argument validation, workspace sizing and the
    entry points' error paths -- built with AddressSanitizer +
    UndefinedBehaviorSanitizer on the host side only, and exercised by the
    whole of tests/test_abi_cpu.py in a child process (DR_LIBRARY selects the
    sanitized build; the sanitizer runtime is preloaded).

Any sanitizer report fails the run (halt_on_error / no recovery)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
LLVM = "/opt/rocm/lib/llvm/bin"


def _run(cmd, env=None, timeout=600):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


def _gcc_driver(flags, name):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, name)
    cmd = ["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", *flags,
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "recurrence.c"),
           "-lm", "-lpthread", "-o", exe]
    r = _run(cmd)
    assert r.returncode == 0, r.stderr
    return exe


def test_oracle_recurrence_asan_ubsan():
    exe = _gcc_driver(["-fsanitize=address,undefined", "-fno-sanitize-recover=all"], "oracle_asan")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe], env=env)
    assert r.returncode == 0 and "runtime error" not in r.stderr, r.stdout + r.stderr
    assert "0 failure(s)" in r.stdout


def test_oracle_recurrence_tsan():
    exe = _gcc_driver(["-fsanitize=thread"], "oracle_tsan")
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = _run([exe], env=env)
    if r.returncode != 0 and "unexpected memory mapping" in r.stderr:
        pytest.skip("ThreadSanitizer cannot map its shadow memory on this kernel")
    assert r.returncode == 0 and "WARNING: ThreadSanitizer" not in r.stderr, r.stdout + r.stderr


def _sanitized_library():
    """libdeltarule with the host side of deltarule.hip (validation, sizing,
    dispatch) instrumented, linked with the ordinary kernel objects."""
    from delta_rule_rnn_amd import build as B
    hipcc = B.HIPCC
    if not os.path.exists(hipcc) or not os.path.exists(os.path.join(LLVM, "clang++")):
        pytest.skip("ROCm toolchain not available")
    objs = [os.path.join(B.OBJDIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "deltarule.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build_library(incremental=True)
    os.makedirs(OUT, exist_ok=True)
    obj = os.path.join(OUT, "deltarule_host_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    r = _run([hipcc, *B.FLAGS[:1], "-O1", "-g", "-std=c++17", "-fPIC", "--offload-host-only", *san,
              "-c", "-o", obj, os.path.join(B.CSRC, "deltarule.hip")])
    assert r.returncode == 0, r.stderr
    lib = os.path.join(OUT, "libdeltarule_san.so")
    r = _run([os.path.join(LLVM, "clang++"), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan",
              "-o", lib, obj, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    assert r.returncode == 0, r.stderr
    return lib


def test_abi_host_code_asan_ubsan():
    lib = _sanitized_library()
    rt = _run([os.path.join(LLVM, "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    if not os.path.exists(rt):
        pytest.skip("AddressSanitizer runtime not found")
    env = dict(os.environ, DR_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-k", "not requires_library"], env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in r.stdout
