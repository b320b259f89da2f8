"""Build libmvk.so (the C-ABI HIP library) in-tree for gfx950.

    python -m paged_kv_cache_206_amd.build          # or build() from Python

Every .hip file under csrc/ is compiled with hipcc for gfx950 only, every
.cpp file (host-only code) with g++, and all are linked into
paged_kv_cache_206_amd/libmvk.so. Packed-fp32 instructions are disabled
(-packed-fp32-ops) for all device code.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmvk.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]

# Per-file additions. The prefill kernel has no NaN-dependent logic (its
# logits are MFMA results or -inf), and without NaN semantics the compiler
# drops the quieting instruction it otherwise puts in front of every fmaxf
# operand: 8 of about 37 VALU instructions per 32-token step of a tile.
FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans"]}


def build(verbose: bool = False, defines=()) -> str:
    """Compile every source and link libmvk.so; returns its path. `defines`
    adds -D flags (MVK_TUNING builds a variant whose planner honours the
    MVK_TUNE_P / MVK_TUNE_W environment variables, for tuning sweeps)."""
    cc = hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    host_sources = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))  # host-only C++
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    with tempfile.TemporaryDirectory(prefix="mvk_build_") as tmp:
        objs = []
        for src in sources:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
                   *("-D" + d for d in defines), "-I", os.path.join(ROOT, "include"),
                   "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
            objs.append(obj)
        for src in host_sources:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [shutil.which("g++") or "g++", "-O2", "-std=c++17", "-fPIC", "-Wall",
                   *("-D" + d for d in defines), "-I", os.path.join(ROOT, "include"), "-c", src,
                   "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True, stderr=None if verbose else subprocess.PIPE)
            objs.append(obj)
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    try:
        defs = [a.split("=", 1)[1] for a in sys.argv[1:] if a.startswith("--define=")]
        path = build(verbose="-v" in sys.argv, defines=defs)
    except subprocess.CalledProcessError as e:
        if e.stderr:
            sys.stderr.write(e.stderr.decode(errors="replace"))
        raise SystemExit(1)
    print(path)
