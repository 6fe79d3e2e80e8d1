"""Build libcsa2.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Every source is compiled on each call (objects in parallel), then linked
in-tree next to this file, so the built library travels with the source
tree.  Usage: ``python fp4_kv_cache_quant_amd/build.py`` (a plain script:
importing the package needs the library it builds).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libcsa2.so")
SOURCES = ["quant.hip", "keys.hip", "index_score.hip", "topk.hip", "sparse_attn.hip", "attn_many.hip", "capi.cpp",
           "sched.cpp", "prefill.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are switched off (the compiler would form them from
# scalar float code); no fast-math: the quantiser's comparisons and the
# indexer's rounding order are exact by construction and must stay so.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "--offload-arch=gfx950", f"-I{INCLUDE}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# MFMA results go to ordinary VGPRs (-amdgpu-mfma-vgpr-form): the scoring
# kernels read every accumulator with VALU code right away, and results left
# in AGPRs would cost one v_accvgpr_read per value first (the same values
# either way).  An LLVM option: used when this hipcc accepts it.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _accepts(flags) -> bool:
    probe = os.path.join(BUILD_DIR, "probe.hip")
    with open(probe, "w") as fh:
        fh.write("#include <hip/hip_runtime.h>\n__global__ void k(float* p) { p[0] = 1.f; }\n")
    r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-c", probe, "-o", probe + ".o", *flags],
                       capture_output=True, text=True)
    return r.returncode == 0


def _compile(src: str, extra=()) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = MFMA_VGPR if _accepts(MFMA_VGPR) else []
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, extra), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
