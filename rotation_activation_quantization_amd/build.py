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


def resource_report(sources=None) -> dict:
    """Compile sources (all .hip by default) with the compiler's
    kernel-resource-usage remarks and return {mangled kernel name:
    {"vgprs", "agprs", "scratch", "occupancy"}} (scratch in bytes per lane;
    nonzero means the kernel spills registers)."""
    import re
    import tempfile

    srcs = sources or [s for s in SOURCES if s.endswith(".hip")]
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy"}

    def one(src):
        with tempfile.TemporaryDirectory() as td:
            cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", os.path.join(td, "x.o"),
                   "-Rpass-analysis=kernel-resource-usage"]
            r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-2000:]}")
        out, cur = {}, None
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+(.+?): (\S+) \[-Rpass-analysis", line)
            if not m:
                continue
            k, v = m.group(1).strip(), m.group(2)
            if k == "Function Name":
                cur = out.setdefault(v, {})
            elif cur is not None and k in keys:
                cur[keys[k]] = int(v)
        return out

    res = {}
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for part in ex.map(one, srcs):
            res.update(part)
    return res


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
    if "--resources" in sys.argv:
        # registers and spills per kernel instance, spilling ones first
        rep = resource_report()
        for name, r in sorted(rep.items(), key=lambda kv: (-kv[1].get("scratch", 0), kv[0])):
            print(f"{r.get('vgprs', 0):4d} VGPR {r.get('agprs', 0):4d} AGPR {r.get('scratch', 0):4d} B/lane scratch "
                  f"{r.get('occupancy', 0):2d} waves/SIMD  {name}")
    else:
        print(build(verbose="-v" in sys.argv))
