"""Build libk2moe.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m sparse_moe_transformer_sigmoid_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  The shared library
lands in sparse_moe_transformer_sigmoid_amd/lib/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "lib")
LIBNAME = "libk2moe.so"
SOURCES = ["abi.hip", "norm_router.hip", "permute.hip", "gemm_fp8.hip", "gemm_fp8_wide.hip",
           "gemm_f32.hip", "combine_pack.hip", "mla.hip", "mla_mha.hip", "mla_abi.hip", "balance.hip",
           "train.hip"]
# per-source extra flags: the wide gate/up GEMM is scheduled to minimise registers,
# which lets it keep two token tiles in flight at 2 waves/SIMD without spilling
EXTRA_FLAGS = {"gemm_fp8_wide.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            # keep packed-fp32 instructions out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA results in VGPRs: the fp32 block-scale FMAs read them directly
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def lib_path() -> str:
    return os.path.join(LIBDIR, LIBNAME)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)

    def one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
               "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = lib_path() + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path())
    return lib_path()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
