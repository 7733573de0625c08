"""Build libqt.so (the int3-g64 HIP library) in-tree for gfx950.

    python -m dequant_matmul_int3_amd.build [-v]

Every HIP source is compiled by hipcc for gfx950 only, without floating-point
contraction (the scale search must round every f32 operation separately; the
multiply kernels use explicit fused multiply-adds where they want them) and
without packed-FP32 instructions.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
SO = os.path.join(PKG, "libqt.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quantize.hip", "gemv.hip", "grouped.hip", "gemm.hip", "hessian.hip",
           "syrk.hip", "factor.hip", "gptq.hip", "moe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]
# The grouped matrix-core kernels scale every MFMA result on the vector ALUs:
# ask the backend to keep MFMA results in VGPRs rather than AGPRs (saves one
# copy per result).  The f64 tile products of the GPTQ factor fit two waves
# per SIMD only in that form.
EXTRA = {"grouped.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "moe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "factor.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD, src + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out and verbose:
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", SO + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
