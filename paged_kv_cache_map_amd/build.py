"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_map_amd.build [--verbose]

Every call recompiles (objects go to ``_build/`` at the repository root, the
library to ``paged_kv_cache_map_amd/libpkv.so``).  No GPU is needed to build.
"""

import os
import pathlib
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
OUT = PKG / "libpkv.so"
BUILD = ROOT / "_build"
ROCM = pathlib.Path(os.environ.get("ROCM_PATH", "/opt/rocm"))

# attention.hip includes paged_decode.hip and varlen_prefill.hip (one unit: the
# mixed-step kernel runs the bodies of both)
HIP_SOURCES = ["kv_write.hip", "attention.hip", "block_copy.hip", "decode_scratch.hip"]
HOST_SOURCES = ["pkv_api.cpp", "pkv_plan.cpp", "pkv_blocks.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed fp32 ops stay off: only scalar fp32 VALU instructions are emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep small per-thread staging arrays in registers, never in LDS
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wall",
    "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
              f"-I{ROCM / 'include'}"]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or str(ROCM / "bin" / "hipcc")
    return exe


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ... ({res.returncode})")
    if verbose and (res.stdout or res.stderr):
        sys.stderr.write(res.stdout + res.stderr)


def build(verbose: bool = False) -> pathlib.Path:
    BUILD.mkdir(exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = BUILD / (src + ".o")
        jobs.append([hipcc, *HIPCC_FLAGS, "-c", str(CSRC / src), "-o", str(obj)])
        objs.append(obj)
    cxx = shutil.which("g++") or "c++"
    for src in HOST_SOURCES:
        obj = BUILD / (src + ".o")
        jobs.append([cxx, *HOST_FLAGS, "-c", str(CSRC / src), "-o", str(obj)])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as pool:
        list(pool.map(lambda c: _run(c, verbose), jobs))
    tmp = OUT.with_suffix(".so.tmp")
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *map(str, objs),
          f"-L{ROCM / 'lib'}", "-lamdhip64", f"-Wl,-rpath,{ROCM / 'lib'}"], verbose)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
