"""Build ``libdsc.so`` (the gfx950 kernels and the C ABI) in-tree with hipcc.

Every source is compiled for gfx950 only.  Packed-fp32 instruction selection
is switched off for all device code.  Objects go to ``_build/`` at the
repository root; the library lands next to this file.  The compiler's
per-kernel resource report is kept in ``_build/kernel_resources.txt`` and the
build fails if any kernel spills registers to scratch memory.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsc.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# (source, extra defines): the low-rank instantiation units are compiled once
# per block count of 16 ranks (R <= 16, 32, 64)
LR_UNITS = ["lowrank_fwd_bf16.hip", "lowrank_bwd_bf16.hip", "lowrank_fwd_f32.hip",
            "lowrank_bwd_f32.hip", "lowrank_fwd_bf16_vl.hip", "lowrank_bwd_bf16_vl.hip",
            "lowrank_fwd_f32_vl.hip", "lowrank_bwd_f32_vl.hip"]
SOURCES = ([(s, ()) for s in ["dsc_abi.cpp", "headwise.hip", "decode.hip", "static.hip",
                              "gen.hip", "lowrank.hip"]]
           + [(s, (f"-DDSC_LR_RB={rb}",)) for rb in (4, 2, 1) for s in LR_UNITS])

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
         "-Rpass-analysis=kernel-resource-usage"]


def _compile(unit):
    src, defs = unit
    path = os.path.join(CSRC, src)
    out = os.path.join(OBJ, src + "".join(d.replace("-D", ".").replace("=", "") for d in defs)
                       + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC, *FLAGS, *defs, *lang, "-c", path, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in r.stderr.splitlines() if noise not in l]
    remarks = [l for l in lines if "kernel-resource-usage" in l]
    # drop the remarks and their source-context lines ("  37 |  ...", "     | ^")
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l
                    and not re.match(r"^\s*\d*\s*\|", l)
                    and not l.startswith("In file included from"))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return out, err, remarks


def _resources(remarks):
    """(kernel, vgprs, agprs, scratch bytes per lane, waves per SIMD) rows."""
    rows, cur = [], None
    for l in remarks:
        m = re.search(r"remark:\s+(.*?):\s*(\S+)\s+\[-Rpass", l)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = {"name": val}
            rows.append(cur)
        elif cur is not None:
            cur[key] = val
    return rows


def build(jobs=None):
    """Compile every source and link ``libdsc.so``; returns the library path."""
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err, _ in results:
        if err.strip():
            print(err, file=sys.stderr)
    rows = [r for _, _, rem in results for r in _resources(rem)]
    with open(os.path.join(OBJ, "kernel_resources.txt"), "w") as f:
        for r in rows:
            f.write(f"{r['name']} vgpr={r.get('VGPRs')} agpr={r.get('AGPRs')} "
                    f"scratch={r.get('ScratchSize [bytes/lane]')} "
                    f"waves_per_simd={r.get('Occupancy [waves/SIMD]')}\n")
    # The generic low-rank backward for 33..64 ranks (RB = 4, the last template
    # argument) keeps the filter fragments of all four rank blocks resident; its
    # widest instance (bf16, H = 1, W = 8, packed rows) needs a little scratch.
    # That path is correct and untuned; every other kernel must not spill.
    may_spill = re.compile(r"lr_bwd_kernelI.*ELi4EEEv")
    spills = [r["name"] for r in rows if r.get("ScratchSize [bytes/lane]", "0") != "0"
              and not may_spill.search(r["name"])]
    if spills:
        raise RuntimeError(f"{len(spills)} kernels spill to scratch, e.g. {spills[:3]}")
    objs = [o for o, _, _ in results]
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    build_c_consumer()
    build_stream_ceiling()
    build_yardstick()
    build_lds_probe()
    return LIB


STREAM_SRC = os.path.join(CSRC, "stream_ceiling.hip")
STREAM_LIB = os.path.join(PKG, "libdsc_stream.so")


def build_stream_ceiling():
    """libdsc_stream.so: the streaming kernel the benchmark's ceiling mode
    measures read/write mixes with (not part of libdsc.so)."""
    tmp = STREAM_LIB + ".tmp"
    cmd = [HIPCC, *[f for f in FLAGS if not f.startswith("-Rpass")], "-shared", STREAM_SRC,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for stream_ceiling.hip:\n{r.stderr}")
    os.replace(tmp, STREAM_LIB)
    return STREAM_LIB


YARD_SRC = os.path.join(CSRC, "yardstick.hip")
YARD_LIB = os.path.join(PKG, "libdsc_yard.so")


def build_yardstick():
    """libdsc_yard.so: the other side of two kernel choices for filters tied
    over 8 channels (the matrix-core forward, the vector-ALU backward), which
    the benchmark's --tied8-forward and --tied8-backward modes time beside
    the kernels libdsc.so uses there (not part of libdsc.so)."""
    tmp = YARD_LIB + ".tmp"
    cmd = [HIPCC, *[f for f in FLAGS if not f.startswith("-Rpass")], "-shared", "-I", CSRC,
           YARD_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for yardstick.hip:\n{r.stderr}")
    os.replace(tmp, YARD_LIB)
    return YARD_LIB


LDSPROBE_SRC = os.path.join(CSRC, "lds_probe.hip")
LDSPROBE_LIB = os.path.join(PKG, "libdsc_ldsprobe.so")


def build_lds_probe():
    """libdsc_ldsprobe.so: the LDS access probe the benchmark's --lds-banks
    mode runs (not part of libdsc.so)."""
    tmp = LDSPROBE_LIB + ".tmp"
    cmd = [HIPCC, *[f for f in FLAGS if not f.startswith("-Rpass")], "-shared", LDSPROBE_SRC,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for lds_probe.hip:\n{r.stderr}")
    os.replace(tmp, LDSPROBE_LIB)
    return LDSPROBE_LIB


CONSUMER_SRC = os.path.join(PKG, "examples", "c_consumer.c")
CONSUMER = os.path.join(PKG, "examples", "c_consumer")


def build_c_consumer():
    """The plain C example program, built with gcc against include/dsc.h and
    libdsc.so (found next to it at run time through its rpath)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", CONSUMER_SRC,
           "-L", PKG, "-ldsc", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath,/opt/rocm/lib", "-o", CONSUMER]
    subprocess.run(cmd, check=True)
    return CONSUMER


if __name__ == "__main__":
    print(build())
