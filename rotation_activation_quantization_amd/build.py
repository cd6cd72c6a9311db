"""Build libsignrot.so in-tree with hipcc for gfx950.

Usage: python -m rotation_activation_quantization_amd.build [-v]
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsignrot.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = [
    "api.hip",
    "rq_generic.hip",
    "rq_fast.hip",
    "rq_halves.hip",
    "rq_outer.hip",
    "rq_outer_t1.hip",
    "rq_outer_t2.hip",
    "rq_outer_t4.hip",
    "rq_outer_t8.hip",
    "rq_outer_t16.hip",
    "calib_dequant.hip",
    "ceiling.hip",
    "linear.hip",
    "hadamard28.cpp",
    "outer.cpp",
]

ARCH = "gfx950"

# -packed-fp32-ops: never emit packed binary32 VALU ops (v_pk_add_f32 and
# friends); the compiler otherwise forms them from ordinary float code.
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs (the VALU reads them right away)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out and verbose:
        print(out)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libsignrot.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
