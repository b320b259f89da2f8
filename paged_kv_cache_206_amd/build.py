"""Build libmvk.so (the C-ABI HIP library) in-tree for gfx950.

    python -m paged_kv_cache_206_amd.build          # or build() from Python

Every .hip file under csrc/ is compiled with hipcc for gfx950 only, every
.cpp file (host-only code) with g++ (one compiler process per file, in
parallel), and all are linked into
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
from concurrent.futures import ThreadPoolExecutor

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


def _jobs() -> int:
    """Parallel compiler processes: MAX_JOBS if set, else the CPUs this process
    may use (at most 16)."""
    env = os.environ.get("MAX_JOBS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def build(verbose: bool = False, defines=()) -> str:
    """Compile every source (in parallel, one compiler process per file) and
    link libmvk.so; returns its path. `defines` adds -D flags."""
    cc = hipcc()
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    host_sources = sorted(glob.glob(os.path.join(CSRC, "*.cpp")))  # host-only C++
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    with tempfile.TemporaryDirectory(prefix="mvk_build_") as tmp:
        cmds, objs = [], []
        for src in sources:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmds.append([cc, *COMMON_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
                         *("-D" + d for d in defines), "-I", os.path.join(ROOT, "include"),
                         "-c", src, "-o", obj])
            objs.append(obj)
        for src in host_sources:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmds.append([shutil.which("g++") or "g++", "-O2", "-std=c++17", "-fPIC", "-Wall",
                         *("-D" + d for d in defines), "-I", os.path.join(ROOT, "include"),
                         "-c", src, "-o", obj])
            objs.append(obj)

        def compile_one(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, stderr=None if verbose else subprocess.PIPE)

        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            results = list(pool.map(compile_one, cmds))
        for cmd, r in zip(cmds, results):
            if r.returncode != 0:
                raise subprocess.CalledProcessError(r.returncode, cmd, stderr=r.stderr)
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
