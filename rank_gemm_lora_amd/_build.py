"""Build liblora_mi355x.so in place with hipcc for gfx950.

    python rank_gemm_lora_amd/_build.py [-v]

Every kernel is compiled for gfx950 only. Files whose arithmetic must follow
an exact rounding sequence (the exact tier, the dense patch) are compiled with
floating-point contraction off. All HIP code is built without packed-fp32
instructions (the compiler then never emits v_pk_{add,mul,fma}_f32).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "liblora_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall", "-Wno-unused-function"]
# file -> extra flags
SOURCES = {
    "gemm.hip": [],
    "merge.hip": [],
    "backward.hip": [],
    "exact.hip": ["-ffp-contract=off"],
    "patch.hip": ["-ffp-contract=off"],
    "probe.hip": [],
    "noalloc.hip": [],
    "api.cpp": [],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build the HIP library)")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="lora_build_") as tmp:
        objs = []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [cc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
            if verbose and r.stderr.strip():
                print(r.stderr, file=sys.stderr)
            objs.append(obj)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        shutil.copyfile(tmp_lib, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
