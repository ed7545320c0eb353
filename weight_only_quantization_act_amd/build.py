"""Build libawq_act.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m weight_only_quantization_act_amd.build

Compiles every .hip file under csrc/ with hipcc for gfx950 and the host-only C ABI
(api.cpp), then links one shared library next to this file.  Always recompiles.
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
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libawq_act.so"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

# Numerics flags are part of the contract: no FMA contraction, IEEE division and sqrt,
# fp32 denormals kept (the gfx9 default), no fast-math.  Packed fp32 vector ops are
# disabled for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# Per-source additions.  The clip-search kernels keep their small MFMA accumulators in
# VGPRs (no accumulator-register moves in the epilogue); the large-tile GEMMs need AGPRs.
HIP_FILE_FLAGS = {
    "clip_search.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM}/include"]


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    return out


def lib_path() -> str:
    return os.path.join(PKG, LIB_NAME)


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "bin", "amdclang++")
    os.makedirs(BUILD, exist_ok=True)
    incs = [f"-I{INCLUDE}", f"-I{CSRC}"]
    jobs_list = []
    for f in sorted(os.listdir(CSRC)):
        src = os.path.join(CSRC, f)
        obj = os.path.join(BUILD, f + ".o")
        if f.endswith(".hip"):
            jobs_list.append([hipcc, *HIP_FLAGS, *HIP_FILE_FLAGS.get(f, []), *incs, "-c", src,
                              "-o", obj])
        elif f.endswith(".cpp"):
            jobs_list.append([clangxx, *HOST_FLAGS, *incs, "-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        outs = list(ex.map(_run, jobs_list))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [cmd[-1] for cmd in jobs_list]
    tmp = lib_path() + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
          f"-L{ROCM}/lib", "-lamdhip64"])
    os.replace(tmp, lib_path())
    if verbose:
        print("built", lib_path())
    return lib_path()


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
