"""The CPU-side code under AddressSanitizer and UndefinedBehaviorSanitizer
(runs without a GPU).

* The oracle (oracle/sla2_oracle.c) is built with gcc and both sanitizers and
  loaded, in a child Python process with the sanitizer runtimes preloaded,
  in place of the plain build; the child calls every oracle entry point on
  small problems (tests/sanitize/oracle_calls.py).
* The host code of the C ABI (csrc/sla2_api.cpp: problem checks, block and
  top-k counts, workspace layouts, argument validation) is built with the
  sanitizers on its host half only, linked with the library's other objects
  into a separate copy of the library, and driven by a small program
  (tests/sanitize/abi_calls.cpp) through every size query and every
  argument check; none of those calls reaches a GPU.
A sanitizer report aborts the child (halt_on_error, no recovery), which
fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_linear_attention_amd import build as B  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libsla2_oracle_san.so")
    rc, out = _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-std=c11", "-fPIC",
                    "-shared", "-pthread", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-o", lib,
                    os.path.join(ROOT, "oracle", "sla2_oracle.c"), "-lm"])
    assert rc == 0, out
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (os.path.exists(asan) and os.path.exists(ubsan)):
        pytest.skip("gcc sanitizer runtimes not installed")
    env = dict(os.environ, **SAN_ENV, SLA2_ORACLE_LIB=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               OMP_NUM_THREADS="4")
    rc, out = _run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "oracle_calls.py")],
                   env=env)
    assert rc == 0 and out.strip().endswith("ok"), out[-4000:]


def test_abi_host_code_under_asan_ubsan(tmp_path):
    # the library's device objects as the normal build makes them (reused
    # when newer than their source), the API object with sanitized host code
    objs = []
    os.makedirs(B.BUILD, exist_ok=True)
    for src in B.SOURCES:
        if src == "sla2_api.cpp":
            continue
        obj = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".o")
        deps = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)
                if f.endswith((".h", ".hip", ".cpp"))]
        if not os.path.exists(obj) or os.path.getmtime(obj) < max(map(os.path.getmtime, deps)):
            B._compile(src)
        objs.append(obj)
    api = str(tmp_path / "sla2_api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
           "-fno-omit-frame-pointer", "-g"]
    rc, out = _run([B.HIPCC, *B.FLAGS, *san, "-x", "hip", "-c",
                    os.path.join(B.CSRC, "sla2_api.cpp"), "-o", api])
    assert rc == 0, out
    lib = str(tmp_path / "libsla2san.so")
    rc, out = _run([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-o", lib, api,
                    *objs])
    assert rc == 0, out
    exe = str(tmp_path / "abi_calls")
    clang = "/opt/rocm/llvm/bin/clang++"
    rc, out = _run([clang, "-std=c++17", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_calls.cpp"), "-o", exe,
                    f"-L{tmp_path}", "-lsla2san", f"-Wl,-rpath,{tmp_path}"])
    assert rc == 0, out
    rc, out = _run([exe], env=dict(os.environ, **SAN_ENV))
    assert rc == 0 and out.strip().endswith("ok"), out[-4000:]
