"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

capi.cpp (argument checks, workspace sizing and carve-up, error strings, timing records)
is compiled with g++ -fsanitize=address,undefined into a small executable together with
tests/sanitize/capi_checks.cpp, which drives every validation path of every entry point.
The executable's instrumented idx_* definitions take precedence over libidx.so's (symbol
interposition); the kernel launchers and the no-allocation entry come from the in-tree,
uninstrumented libidx.so.  No call reaches a device: each returns during validation or
from the HIP runtime's own no-device error.  Any sanitizer report or failed check fails
the test.
"""
import os
import shutil
import subprocess

import pytest

import sparse_attention_indexer_score_amd as sai

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CAPI = os.path.join(ROOT, "sparse_attention_indexer_score_amd", "csrc", "capi.cpp")
CHECKS = os.path.join(ROOT, "tests", "sanitize", "capi_checks.cpp")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = [
    pytest.mark.skipif(not os.path.exists(sai.LIB_PATH), reason="libidx.so not built"),
    pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found"),
]

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
FLAGS = ["-std=c++17", "-O1", "-g", *SAN, "-I" + os.path.join(ROOT, "include")]


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nrc={r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_capi_host_paths_under_asan_and_ubsan(tmp_path):
    capi_o, checks_o, exe = (str(tmp_path / n) for n in ("capi.o", "checks.o", "capi_checks"))
    run(["g++", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"), "-c", CAPI, "-o", capi_o])
    run(["g++", *FLAGS, "-c", CHECKS, "-o", checks_o])
    libdir = os.path.dirname(sai.LIB_PATH)
    run(["g++", *SAN, "-o", exe, checks_o, capi_o, "-L" + libdir, "-l:libidx.so", "-Wl,-rpath," + libdir,
         "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    syms = run(["nm", exe]).stdout
    assert " T idx_fused_topk\n" in syms and " T idx_score\n" in syms, "instrumented entry points not linked"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "OK: 0 failed checks" in r.stdout, out[-4000:]
