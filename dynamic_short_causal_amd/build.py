"""Build ``libdsc.so`` (the gfx950 kernels and the C ABI) in-tree with hipcc.

Every source is compiled for gfx950 only.  Packed-fp32 instruction selection
is switched off for all device code.  Objects go to ``_build/`` at the
repository root; the library lands next to this file.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["dsc_abi.cpp", "headwise.hip", "lowrank.hip", "lowrank_fwd_bf16.hip",
           "lowrank_bwd_bf16.hip", "lowrank_fwd_f32.hip", "lowrank_bwd_f32.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src):
    path = os.path.join(CSRC, src)
    out = os.path.join(OBJ, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *lang, "-c", path, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return out, err


def build(jobs=None):
    """Compile every source and link ``libdsc.so``; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        if err.strip():
            print(err, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
