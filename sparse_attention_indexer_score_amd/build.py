"""Build libidx.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m sparse_attention_indexer_score_amd.build

Every source is compiled for gfx950 only, with packed-fp32 instructions disabled and
floating-point contraction off (the scoring core spells out its fused multiply-adds, so
every kernel rounds identically).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libidx.so")

SOURCES = ["capi.cpp", "fused.hip", "select.hip", "slots.hip", "attn.hip", "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-I" + os.path.join(ROOT, "include"),
]
DEVICE = [
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the head reduce reads them directly (no v_accvgpr_read)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        if verbose and err.strip():
            print(err, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
