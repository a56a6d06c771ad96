"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with its host code instrumented (device code is not: GPU
sanitizers are not part of this build) into a temporary directory, links
tests/host_abi_check.c against it with the same sanitizers and runs it on the
CPU: argument validation, workspace sizing and bookkeeping must run clean.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from hstu_pointwise_attention_amd import build as B  # noqa: E402

CLANG = "/opt/rocm/llvm/bin/clang"
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.slow
def test_host_abi_under_asan_ubsan(tmp_path):
    if not os.path.exists(CLANG) or shutil.which(B.hipcc()) is None and not os.path.exists(B.hipcc()):
        pytest.skip("ROCm clang / hipcc not available")
    objs = []
    procs = []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [B.hipcc(), *B.CFLAGS, *SAN_HOST, "-c", os.path.join(B.CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for src, pr in procs:
        out, err = pr.communicate()
        assert pr.returncode == 0, f"{src}: {err[-3000:]}"
    lib = str(tmp_path / "libhstu_attn_san.so")
    r = subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", *objs, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "host_abi_check")
    r = subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "host_abi_check.c"),
                        lib, f"-Wl,-rpath,{tmp_path}", "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"stdout:\n{r.stdout}\nstderr:\n{r.stderr[-6000:]}"
    assert "host ABI checks passed" in r.stdout
