"""Build libhna.so (gfx950 only) from csrc/ with hipcc, in the package directory."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libhna.so")
BUILD_DIR = os.path.join(PKG_DIR, "_build")

SOURCES = ["hna_api.hip", "k_affinity.hip", "k_gram.hip", "k_gemm.hip", "k_mm.hip",
           "k_small.hip", "k_objective.hip", "k_layout.hip", "k_loo.hip", "k_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled on purpose: only scalar fp32 VALU code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]
# Per-source additions.  The affinity kernel's epilogue reads the MFMA results
# with ordinary vector instructions; the VGPR form of MFMA keeps accumulators
# in VGPRs, so no accumulation-register reads are needed (its weight
# fragments still go to accumulation registers, as MFMA operands).
EXTRA = {"k_affinity.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         # the layout search compares fp64 values bit for bit with plain arithmetic
         "k_layout.hip": ["-ffp-contract=off"]}


# every GEMM runs on the library's own kernels: no BLAS library is linked
LIBS: list = []


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in (r.stderr or "").splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + err)
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libhna.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp, *LIBS])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
