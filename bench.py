"""Benchmark of the dynamic short causal convolution hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch
(B=8, T=2048, D=6144, W=4, bf16, inputs resident in HBM):
  head-wise  (H=16, 384 filter groups, residual): forward + backward
  low-rank   (R=16, H=1, filters generated on chip, residual): forward +
             backward (+ the fixed-order reduction of its partial sums)
value = tokens of the batch per second of step time (B*T / t_step).
Each op reads its own copy of its inputs, so no op is served from the
last-level cache by data the op before it read.

Also reported: achieved algorithmic HBM bandwidth of the step, a roofline
entry for the dominant kernel (timed with HIP events on the stream the
kernels run on), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --profile-ops K   (K untimed passes of every op plus a
                                          512 MiB device copy, for rocprofv3)
       python bench.py --summarize-profiles DIR --profile-ops K
                                         (rocprofv3 outputs -> profiles/)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD specification
WORKLOAD = dict(B=8, T=2048, D=6144, W=4, H_headwise=16, R=16, H_lowrank=1)


def algorithmic_bytes(B, T, D, W, Hh, R, Hl, es=2):
    """Each input read once, each output written once (bytes per launch)."""
    N = B * T
    Gh, Gl = D // Hh, D // Hl
    return {
        "headwise_fwd": es * (N * D + N * Gh * W + N * D),
        "headwise_bwd": es * (3 * N * D + 2 * N * Gh * W),
        "lowrank_fwd": es * (2 * N * D + N * R + R * Gl * W),
        "lowrank_bwd": es * (3 * N * D + 2 * N * R + 2 * R * Gl * W),
    }


def src_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# kernel -> the sources whose change invalidates its committed counter data
KERNEL_SOURCES = {
    "headwise_fwd": ["dynamic_short_causal_amd/csrc/headwise.hip",
                     "dynamic_short_causal_amd/csrc/dsc_device.hpp"],
    "headwise_bwd": ["dynamic_short_causal_amd/csrc/headwise.hip",
                     "dynamic_short_causal_amd/csrc/dsc_device.hpp"],
    "lowrank_fwd": ["dynamic_short_causal_amd/csrc/lowrank_fwd_cl.hpp",
                    "dynamic_short_causal_amd/csrc/lowrank_bwd_cl.hpp",
                    "dynamic_short_causal_amd/csrc/lowrank_impl.hpp",
                    "dynamic_short_causal_amd/csrc/lowrank_launch.hpp",
                    "dynamic_short_causal_amd/csrc/dsc_device.hpp"],
    "lowrank_bwd": ["dynamic_short_causal_amd/csrc/lowrank_impl.hpp",
                    "dynamic_short_causal_amd/csrc/lowrank_bwd_cl.hpp",
                    "dynamic_short_causal_amd/csrc/lowrank_launch.hpp",
                    "dynamic_short_causal_amd/csrc/dsc_launch.hpp",
                    "dynamic_short_causal_amd/csrc/dsc_device.hpp"],
}


def traffic_from_profiles(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary, or None when absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_qkv_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("src_digest") != src_digest(KERNEL_SOURCES[kernel]):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(target_s=12.0):
    """The fp64 oracle on a bounded sample of the benchmark workload: whole
    sequences of T=2048 tokens (head-wise and low-rank forward + backward, the
    same ops as one step), taken one after another until about target_s of
    CPU time has passed or every sequence of the batch is done."""
    import torch
    import dsc_inputs as di
    import oracle
    orc = oracle.default()
    B, T, D, W = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"]
    Hh, R = WORKLOAD["H_headwise"], WORKLOAD["R"]

    def seq(b):
        g = lambda shape, std, k: di.randn(shape, std, 90000 + 10 * b + k, "bf16").to(
            torch.float64).numpy()
        return (g((1, T, D), 1.0, 0), g((1, T, D), 1.0, 4), g((1, T, D // Hh, W), 0.5, 1),
                g((1, T, R), 1.0, 2), g((R, D * W), (1.0 / (R * W)) ** 0.5, 3))

    done, el = 0, 0.0
    while done < B and (done == 0 or el < target_s):
        x, dy, w, z, U = seq(done)
        t0 = time.perf_counter()
        orc.headwise_fwd(x, w, Hh, residual=True)
        orc.headwise_bwd(x, w, dy, Hh, residual=True)
        orc.lowrank_fwd(x, z, U, W, 1, residual=True)
        orc.lowrank_bwd(x, z, U, dy, W, 1, residual=True)
        el += time.perf_counter() - t0
        done += 1
    cores = orc.num_threads()
    # the same oracle on one thread, over the first sequence
    orc.set_num_threads(1)
    try:
        x, dy, w, z, U = seq(0)
        t0 = time.perf_counter()
        orc.headwise_fwd(x, w, Hh, residual=True)
        orc.headwise_bwd(x, w, dy, Hh, residual=True)
        orc.lowrank_fwd(x, z, U, W, 1, residual=True)
        orc.lowrank_bwd(x, z, U, dy, W, 1, residual=True)
        el1 = time.perf_counter() - t0
    finally:
        orc.set_num_threads(cores)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    per_token = sum(algorithmic_bytes(B, T, D, W, Hh, R, WORKLOAD["H_lowrank"]).values()) / (B * T)
    return {"value": round(done * T / el, 1), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "gbps": round(per_token * done * T / el / 1e9, 3),
            "cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{done} of the {B} sequences (T={T}, D={D}, W={W}; head-wise H={Hh} and "
                      f"low-rank R={R} H=1, residual, fwd+bwd), fp64 C oracle with OpenMP; "
                      f"{el:.1f} s",
            "one_thread": {"value": round(T / el1, 1), "unit": "tokens/s", "cores": 1,
                           "sample": f"the first sequence on one thread; {el1:.1f} s"}}


OP_KERNELS = {  # op -> kernel names (rocprofv3) that one call launches
    "headwise_fwd": ["hw_fwd_kernel"],
    "headwise_bwd": ["hw_bwd_kernel"],
    "lowrank_fwd": ["lr_fwd_cl_kernel", "lr_fwd_kernel"],
    "lowrank_bwd": ["lr_bwd_cl_kernel", "lr_bwd_kernel", "lr_reduce4_kernel", "lr_reduce_kernel"],
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"  # the 512 MiB device copy of --profile-ops
COPY_KIB = 524288
SUM_KERNEL = "native::reduce_kernel"     # torch's read-only sum of the same 512 MiB


def op_spans(trace_csv, kernels, calls):
    """Mean span of one call of an op launching `kernels` in order, from the
    per-dispatch timestamps of a --kernel-trace run: first kernel's start to
    the last kernel's end, over the last `calls` - 1 calls (in us).  The first
    call is left out: the first launch of a kernel loads its code object,
    which can hold the next kernel of the op back by milliseconds."""
    import csv
    rows = [r for r in csv.DictReader(open(trace_csv))
            if any(k in r["Kernel_Name"] for k in kernels)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    first = [i for i, r in enumerate(rows) if kernels[0] in r["Kernel_Name"]]
    spans = []
    for a, i in enumerate(first):
        j = first[a + 1] if a + 1 < len(first) else len(rows)
        spans.append((int(rows[j - 1]["End_Timestamp"]) - int(rows[i]["Start_Timestamp"])) / 1e3)
    spans = spans[1:][-max(calls - 1, 1):]
    return sum(spans) / len(spans) if spans else float("nan")


def summarize_profiles(d, calls):
    """Turn the rocprofv3 outputs of the three profiling runs under `d`
    (trace/: --kernel-trace --stats; fetch/: --pmc FETCH_SIZE; write/: --pmc
    WRITE_SIZE, each of `python3 bench.py --profile-ops <calls>`) into
    profiles/qkv_kernels.md and one profiles/<op>_qkv_traffic.json per op."""
    import csv
    import collections

    def kname(n):
        for k in sorted({k for ks in OP_KERNELS.values() for k in ks} | {COPY_KERNEL, SUM_KERNEL},
                        key=len, reverse=True):
            if k in n:
                return k
        return None

    stats = {}
    for row in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))):
        k = kname(row["Name"])
        if k:
            stats[k] = (int(row["Calls"]), float(row["AverageNs"]) / 1e3)

    def counter(sub, name):
        per = collections.defaultdict(dict)
        for row in csv.DictReader(open(os.path.join(d, sub, "run_counter_collection.csv"))):
            k = kname(row["Kernel_Name"])
            if k and row["Counter_Name"] == name:
                di_ = int(row["Dispatch_Id"])
                per[k][di_] = per[k].get(di_, 0.0) + float(row["Counter_Value"])
        # the device copy kernel also serves the input copies made before the
        # passes: calibrate on its last `calls` dispatches, the 512 MiB copies
        for ck in (COPY_KERNEL, SUM_KERNEL):
            if ck in per:
                last = sorted(per[ck])[-calls:]
                per[ck] = {i: per[ck][i] for i in last}
        return {k: sum(v.values()) / len(v) for k, v in per.items()}

    fetch, write = counter("fetch", "FETCH_SIZE"), counter("write", "WRITE_SIZE")
    ff, wf = COPY_KIB / fetch[COPY_KERNEL], COPY_KIB / write[COPY_KERNEL]
    ff_sum = COPY_KIB / fetch[SUM_KERNEL] if fetch.get(SUM_KERNEL) else float("nan")
    B, T, D, W = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"]
    alg = algorithmic_bytes(B, T, D, W, WORKLOAD["H_headwise"], WORKLOAD["R"],
                            WORKLOAD["H_lowrank"])
    cmd = ("rocprofv3 {opt} --output-format csv -d <out>/{sub} -o run -- "
           f"python3 bench.py --profile-ops {calls}")
    lines = ["# Kernels of one benchmark step, B=8 T=2048 D=6144 W=4 bf16 (residual)", "",
             "Commands (repository root, MI355X, TMPDIR=/tmp), then the summary:", ""]
    for opt, sub in (("--kernel-trace --stats", "trace"), ("--pmc FETCH_SIZE", "fetch"),
                     ("--pmc WRITE_SIZE", "write")):
        lines.append("    " + cmd.format(opt=opt, sub=sub))
    lines += [f"    python3 bench.py --summarize-profiles <out> --profile-ops {calls}", "",
              f"Calibration: the {COPY_KIB // 1024} MiB device copy ({COPY_KERNEL}) reads "
              f"FETCH_SIZE {fetch[COPY_KERNEL]:.0f} KiB and writes WRITE_SIZE "
              f"{write[COPY_KERNEL]:.0f} KiB per call, so HBM bytes = {ff:.3f} x FETCH_SIZE "
              f"+ {wf:.3f} x WRITE_SIZE (KiB).  Cross-check: a read-only sum of the same "
              f"{COPY_KIB // 1024} MiB ({SUM_KERNEL}) reads FETCH_SIZE "
              f"{fetch.get(SUM_KERNEL, float('nan')):.0f} KiB, a factor of {ff_sum:.3f}.", "",
              "Op span: one call's first kernel start to last kernel end, from the per-dispatch "
              "timestamps of the trace run (it includes the gap between the kernels of a "
              "two-kernel op), averaged over all calls but the first, whose launches load the "
              "code objects; the benchmark's event times measure this span.", "",
              "| op | kernel | calls | avg us | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB |",
              "|---|---|---|---|---|---|---|"]
    for op, ks in OP_KERNELS.items():
        ks = [k for k in ks if k in stats]  # the kernels this workload launched
        tot = 0.0
        for k in ks:
            n, us = stats.get(k, (0, float("nan")))
            hb = (ff * fetch.get(k, 0.0) + wf * write.get(k, 0.0)) * 1024
            tot += hb
            lines.append(f"| {op} | {k} | {n} | {us:.1f} | {fetch.get(k, 0):.0f} | "
                         f"{write.get(k, 0):.0f} | {hb / 1e6:.1f} |")
        op_us = sum(stats.get(k, (0, 0.0))[1] for k in ks)
        span = op_spans(os.path.join(d, "trace", "run_kernel_trace.csv"), ks, calls)
        lines.append(f"| {op} | (sum of kernels) | | {op_us:.1f} | | | {tot / 1e6:.1f} "
                     f"(algorithmic {alg[op] / 1e6:.1f}) |")
        lines.append(f"| {op} | (op span) | | {span:.1f} | | | algorithmic "
                     f"{alg[op] / (span * 1e-6) / 1e9:.0f} GB/s = "
                     f"{alg[op] / (span * 1e-6) / 1e9 / HBM_PEAK_GBPS:.3f} of peak |")
        with open(os.path.join(ROOT, "profiles", f"{op}_qkv_traffic.json"), "w") as f:
            json.dump({"op": op, "kernels": ks, "hbm_bytes_per_launch": round(tot),
                       "algorithmic_bytes": alg[op], "avg_us": round(op_us, 2),
                       "span_us": round(span, 2),
                       "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
                       "src_digest": src_digest(KERNEL_SOURCES[op])}, f, indent=1)
            f.write("\n")
    with open(os.path.join(ROOT, "profiles", "qkv_kernels.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(d, name, title, command):
    """profiles/<name>.md: every kernel of a `rocprofv3 --kernel-trace --stats`
    run (its run_kernel_stats.csv under `d`) with calls and average time."""
    import csv
    rows = list(csv.DictReader(open(os.path.join(d, "run_kernel_stats.csv"))))
    lines = [f"# {title}", "", "Command (repository root, MI355X, TMPDIR=/tmp), then the summary:",
             "", f"    rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
             f"{command}", f"    python3 bench.py --summarize-trace <out> {name}", "",
             "| kernel | calls | avg us | total us |", "|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        nm = r["Name"]
        nm = nm[len("void "):] if nm.startswith("void ") else nm
        nm = nm.split("(")[0]
        lines.append(f"| `{nm}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} |")
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# SQ counter passes (at most 8 SQ counters per pass) and the runs they profile
SQ_PASSES = [
    "SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_LDS SQ_WAIT_INST_LDS",
    "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_ACTIVE_INST_VALU SQ_WAIT_ANY",
]
COUNTER_RUNS = {
    # name: (title, command profiled)
    "qkv_counters": ("SQ counters of the step's kernels, B=8 T=2048 D=6144 W=4 bf16 (head-wise "
                     "H=16, low-rank R=16 H=1, residual)", "python3 bench.py --profile-ops 2"),
    "mlp_rnn_counters": ("SQ counters of the MLP (head-wise H=64, B=4 T=4096 D=8192, W in "
                         "2,3,4,8) and linear-RNN (low-rank R=16 H=8 SiLU, B=16 T=4096 D=4608) "
                         "configurations", "python3 bench.py --other-configs"),
    "tied8_forward_counters": ("SQ counters of the linear-RNN forward (low-rank R=16 H=8 SiLU, "
                               "B=16 T=4096 D=4608 W=4) on the vector-ALU kernel "
                               "(lr_fwd_valu_kernel) and the matrix-core kernel (lr_fwd_kernel, "
                               "libdsc_yard.so)",
                               "python3 bench.py --tied8-forward --profile-ops 3"),
    "tied8_backward_counters": ("SQ counters of the linear-RNN backward (low-rank R=16 H=8 "
                                "SiLU, B=16 T=4096 D=4608 W=4) on the matrix-core kernel "
                                "(lr_bwd_kernel) and the vector-ALU kernel (lr_bwd_valu_kernel, "
                                "libdsc_yard.so), each with its reduction",
                                "python3 bench.py --tied8-backward --profile-ops 3"),
}


def summarize_counters(name, dirs):
    """profiles/<name>.md from the rocprofv3 --pmc runs in `dirs` (one per
    pass of SQ_PASSES, each with run_counter_collection.csv): per kernel
    instance, the mean of each counter per dispatch and unit-free ratios."""
    import csv
    import collections
    title, command = COUNTER_RUNS[name]
    per = collections.defaultdict(lambda: collections.defaultdict(dict))
    regs = {}
    for d in dirs:
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            nm = r["Kernel_Name"]
            if "dsc::" not in nm:
                continue
            nm = nm[len("void "):] if nm.startswith("void ") else nm
            nm = nm.split("(")[0].replace("dsc::", "").replace("unsigned short", "bf16")
            di_ = int(r["Dispatch_Id"])
            per[nm][r["Counter_Name"]][di_] = (per[nm][r["Counter_Name"]].get(di_, 0.0)
                                               + float(r["Counter_Value"]))
            regs[nm] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"])
    cols = [c for p_ in SQ_PASSES for c in p_.split()]
    lines = [f"# {title}", "", "Commands (repository root, MI355X, TMPDIR=/tmp), then the summary:",
             ""]
    for i, p_ in enumerate(SQ_PASSES):
        lines.append(f"    rocprofv3 --pmc {p_} --output-format csv -d <out>/pmc{i} -o run -- "
                     f"{command}")
    lines += [f"    python3 bench.py --summarize-counters {name} "
              + " ".join(f"<out>/pmc{i}" for i in range(len(SQ_PASSES))), "",
              "Means per dispatch, summed over the device as rocprofv3 reports them.  Ratios: "
              "VALU/wave and LDS/wave are instructions per wave (VALU includes MFMA); "
              "lds_wait = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES and any_wait = SQ_WAIT_ANY / "
              "SQ_WAVE_CYCLES (share of wave time waiting); conflict = SQ_LDS_BANK_CONFLICT / "
              "SQ_ACTIVE_INST_LDS.", ""]
    lines.append("| kernel | " + " | ".join(cols) + " |")
    lines.append("|---|" + "---|" * len(cols))
    mean = lambda d_: sum(d_.values()) / len(d_) if d_ else float("nan")
    for nm in sorted(per):
        m = {c: mean(per[nm].get(c, {})) for c in cols}
        lines.append(f"| `{nm}` | " + " | ".join(f"{m[c]:.4g}" for c in cols) + " |")
    lines += ["", "| kernel | VGPR, AGPR, LDS bytes (from the trace) | VALU/wave | MFMA/wave | "
                  "LDS/wave | lds_wait | any_wait | conflict |", "|---|---|---|---|---|---|---|---|"]
    for nm in sorted(per):
        m = {c: mean(per[nm].get(c, {})) for c in cols}
        w = m["SQ_WAVES"] or float("nan")
        wc = m["SQ_WAVE_CYCLES"] or float("nan")
        al = m["SQ_ACTIVE_INST_LDS"] or float("nan")
        lines.append(f"| `{nm}` | {', '.join(regs[nm])} | {m['SQ_INSTS_VALU'] / w:.0f} | "
                     f"{m['SQ_INSTS_MFMA'] / w:.0f} | {m['SQ_INSTS_LDS'] / w:.0f} | "
                     f"{m['SQ_WAIT_INST_LDS'] / wc:.3f} | {m['SQ_WAIT_ANY'] / wc:.3f} | "
                     f"{m['SQ_LDS_BANK_CONFLICT'] / al:.3f} |")
    with open(os.path.join(ROOT, "profiles", f"{name}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


TRACES = {
    # name: (title, command traced)
    "bench_all_kernels": ("Every kernel of one default benchmark run (step ops, decode steps, "
                          "static-filter comparator, packed rows)",
                          "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline"),
    "mlp_rnn_kernels": ("Kernels of the MLP (head-wise H=64, B=4 T=4096 D=8192, W in 2,3,4,8) "
                        "and linear-RNN (low-rank R=16 H=8 SiLU, B=16 T=4096 D=4608) "
                        "configurations", "python3 bench.py --other-configs"),
    "tied8_forward_kernels": ("Kernels of the linear-RNN forward comparison (low-rank R=16 H=8 "
                              "SiLU, B=16 T=4096 D=4608 W=4): vector-ALU and matrix-core kernels",
                              "python3 bench.py --tied8-forward"),
    "tied8_backward_kernels": ("Kernels of the linear-RNN backward comparison (low-rank R=16 "
                               "H=8 SiLU, B=16 T=4096 D=4608 W=4): matrix-core and vector-ALU "
                               "kernels, each with its reduction",
                               "python3 bench.py --tied8-backward"),
    "generated_filter_kernels": ("Kernels of the generated-filter comparison, B=8 T=2048 "
                                 "D=6144 Dh=2048 W=4 H=16 bf16 residual: the fused kernel, "
                                 "then the library GEMM writing w and the head-wise forward",
                                 "python3 bench.py --generated-filters --steps 5"),
}


def other_configs(dsc, di, torch, reps=10):
    """fwd + bwd of the MLP and linear-RNN configurations (parity cases, not
    the step): each op on its own input copy, median of `reps` event-timed
    launches.  x of these shapes exceeds the last-level cache."""
    stream = torch.cuda.current_stream()

    def med(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2] * 1e3

    out = {}
    for W in (2, 3, 4, 8):
        wl = di.WORKLOADS["mlp_headwise"].with_(W=W)
        inp = di.make(wl)
        x1, w1 = inp["x"].cuda(), inp["w"].cuda()
        x2, w2, dy2 = inp["x"].cuda(), inp["w"].cuda(), inp["dy"].cuda()
        del inp
        y, dx, dw = torch.empty_like(x1), torch.empty_like(x1), torch.empty_like(w1)
        tf = med(lambda: dsc.dsc_headwise_fwd(x1, w1, y, wl.H, True, False, stream))
        tb = med(lambda: dsc.dsc_headwise_bwd(x2, w2, dy2, dx, dw, wl.H, True, False, stream))
        N, D, G = wl.B * wl.T, wl.D, wl.D // wl.H
        nb = 2 * (2 * N * D + N * G * W) + 2 * (3 * N * D + 2 * N * G * W)
        out[f"mlp_headwise_W{W}"] = {"fwd_us": round(tf, 1), "bwd_us": round(tb, 1),
                                     "tokens_per_s": round(N / ((tf + tb) * 1e-6), 1),
                                     "gbps": round(nb / ((tf + tb) * 1e-6) / 1e9, 1)}
        del x1, w1, x2, w2, dy2, y, dx, dw
        torch.cuda.empty_cache()
    wl = di.WORKLOADS["rnn_lowrank_silu"]
    inp = di.make(wl)
    x1, z1, U1 = inp["x"].cuda(), inp["z"].cuda(), inp["U"].cuda()
    x2, z2, U2, dy2 = inp["x"].cuda(), inp["z"].cuda(), inp["U"].cuda(), inp["dy"].cuda()
    del inp
    y, dx, dz, dU = (torch.empty_like(x1), torch.empty_like(x1), torch.empty_like(z1),
                     torch.empty_like(U1))
    ws = dsc.lowrank_workspace(x2, z2, wl.W, wl.H)
    tf = med(lambda: dsc.dsc_lowrank_fwd(x1, z1, U1, y, wl.W, wl.H, wl.residual, wl.act,
                                         stream))
    tb = med(lambda: dsc.dsc_lowrank_bwd(x2, z2, U2, dy2, dx, dz, dU, ws, wl.W, wl.H,
                                         wl.residual, wl.act, stream))
    N, D, R, GW = wl.B * wl.T, wl.D, wl.R, (wl.D // wl.H) * wl.W
    nb = 2 * (2 * N * D + N * R + R * GW) + 2 * (3 * N * D + 2 * N * R + 2 * R * GW)
    out["rnn_lowrank_silu"] = {"fwd_us": round(tf, 1), "bwd_us": round(tb, 1),
                               "tokens_per_s": round(N / ((tf + tb) * 1e-6), 1),
                               "gbps": round(nb / ((tf + tb) * 1e-6) / 1e9, 1)}
    for v in out.values():
        v["frac_of_peak"] = round(v["gbps"] / HBM_PEAK_GBPS, 4)
    return out


def tied8_forward(dsc, di, torch, reps=10, rounds=5, profile_calls=0):
    """The linear-RNN forward (low-rank R=16 tied over H=8 channels, W=4,
    SiLU, bf16, B=16 T=4096 D=4608) on both kernels that can serve it:
    libdsc.so's vector-ALU kernel and the matrix-core kernel kept in
    libdsc_yard.so.  Both read the same two alternating input sets (x is
    604 MB, beyond the last-level cache) in `rounds` interleaved rounds of
    `reps` event-timed launches; the median launch of each.  With
    profile_calls, only that many untimed launches of each (counter runs)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc_yard.so"))
    lib.dsc_yard_lowrank_fwd_mfma.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3
                                              + [ctypes.c_int] * 3 + [ctypes.c_void_p])
    wl = di.WORKLOADS["rnn_lowrank_silu"]
    inp = di.make(wl, need_dy=False)
    sets = [(inp["x"].cuda(), inp["z"].cuda()) for _ in range(2)]
    U = inp["U"].cuda()
    del inp
    ya, yb = torch.empty_like(sets[0][0]), torch.empty_like(sets[0][0])
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def valu(i):
        x, z = sets[i % 2]
        dsc.dsc_lowrank_fwd(x, z, U, ya, wl.W, wl.H, wl.residual, wl.act, stream)

    def mfma(i):
        x, z = sets[i % 2]
        r = lib.dsc_yard_lowrank_fwd_mfma(P(x), P(z), P(U), P(yb), wl.B, wl.T, wl.D, wl.R,
                                          int(wl.residual), int(wl.act), sp)
        assert r == 0, r

    if profile_calls:
        for i in range(profile_calls):
            valu(i)
            mfma(i)
        torch.cuda.synchronize()
        return None
    valu(0)
    mfma(0)
    torch.cuda.synchronize()
    diff = float((ya.float() - yb.float()).abs().max() / yb.float().abs().max())
    times = {"valu": [], "mfma": []}
    for r in range(rounds):
        for name, fn in (("valu", valu), ("mfma", mfma)):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for i, (a, b) in enumerate(ev):
                a.record(stream)
                fn(i + r)
                b.record(stream)
            torch.cuda.synchronize()
            times[name] += [a.elapsed_time(b) * 1e3 for a, b in ev]
    med = {k: sorted(v)[len(v) // 2] for k, v in times.items()}
    N = wl.B * wl.T
    nb = 2 * (2 * N * wl.D + N * wl.R) + 2 * wl.R * (wl.D // wl.H) * wl.W
    return {"workload": "rnn_lowrank_silu forward (B=16 T=4096 D=4608 W=4 R=16 H=8, SiLU)",
            "vector_alu_us": round(med["valu"], 1), "matrix_core_us": round(med["mfma"], 1),
            "vector_alu_over_matrix_core": round(med["valu"] / med["mfma"], 4),
            "vector_alu_frac_of_peak": round(nb / (med["valu"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "matrix_core_frac_of_peak": round(nb / (med["mfma"] * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                              4),
            "max_rel_diff": diff}


def tied8_backward(dsc, di, torch, reps=10, rounds=5, profile_calls=0):
    """The linear-RNN backward (low-rank R=16 tied over H=8 channels, W=4,
    SiLU, bf16, B=16 T=4096 D=4608) on both kernels that can serve it:
    libdsc.so's matrix-core backward and the vector-ALU backward kept in
    libdsc_yard.so, each with its partial-sum reduction.  Two alternating
    input sets (x and dy are 604 MB each), `rounds` interleaved rounds of
    `reps` event-timed calls, the median call of each.  With profile_calls,
    only that many untimed calls of each (counter runs)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc_yard.so"))
    lib.dsc_yard_lowrank_bwd_valu.argtypes = ([ctypes.c_void_p] * 8 + [ctypes.c_int64] * 3
                                              + [ctypes.c_int] * 3 + [ctypes.c_void_p])
    lib.dsc_yard_lowrank_bwd_valu_workspace.restype = ctypes.c_size_t
    lib.dsc_yard_lowrank_bwd_valu_workspace.argtypes = [ctypes.c_int64] * 3
    wl = di.WORKLOADS["rnn_lowrank_silu"]
    inp = di.make(wl)
    sets = [(inp["x"].cuda(), inp["z"].cuda(), inp["dy"].cuda()) for _ in range(2)]
    U = inp["U"].cuda()
    del inp
    x0, z0 = sets[0][0], sets[0][1]
    outs = {k: (torch.empty_like(x0), torch.empty_like(z0), torch.empty_like(U))
            for k in ("mfma", "valu")}
    ws_m = dsc.lowrank_workspace(x0, z0, wl.W, wl.H)
    ws_v = torch.empty(lib.dsc_yard_lowrank_bwd_valu_workspace(wl.B, wl.T, wl.D),
                       dtype=torch.uint8, device=x0.device)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def mfma(i):
        x, z, dy = sets[i % 2]
        dx, dz, dU = outs["mfma"]
        dsc.dsc_lowrank_bwd(x, z, U, dy, dx, dz, dU, ws_m, wl.W, wl.H, wl.residual, wl.act,
                            stream)

    def valu(i):
        x, z, dy = sets[i % 2]
        dx, dz, dU = outs["valu"]
        r = lib.dsc_yard_lowrank_bwd_valu(P(x), P(z), P(U), P(dy), P(dx), P(dz), P(dU), P(ws_v),
                                          wl.B, wl.T, wl.D, wl.R, int(wl.residual), int(wl.act),
                                          sp)
        assert r == 0, r

    if profile_calls:
        for i in range(profile_calls):
            mfma(i)
            valu(i)
        torch.cuda.synchronize()
        return None
    mfma(0)
    valu(0)
    torch.cuda.synchronize()
    diff = {n: float((a.float() - b.float()).abs().max() / a.float().abs().max())
            for n, a, b in zip(("dx", "dz", "dU"), outs["mfma"], outs["valu"])}
    times = {"mfma": [], "valu": []}
    for r in range(rounds):
        for name, fn in (("mfma", mfma), ("valu", valu)):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for i, (a, b) in enumerate(ev):
                a.record(stream)
                fn(i + r)
                b.record(stream)
            torch.cuda.synchronize()
            times[name] += [a.elapsed_time(b) * 1e3 for a, b in ev]
    med = {k: sorted(v)[len(v) // 2] for k, v in times.items()}
    N = wl.B * wl.T
    nb = 2 * (3 * N * wl.D + 2 * N * wl.R) + 2 * 2 * wl.R * (wl.D // wl.H) * wl.W
    return {"workload": "rnn_lowrank_silu backward (B=16 T=4096 D=4608 W=4 R=16 H=8, SiLU)",
            "matrix_core_us": round(med["mfma"], 1), "vector_alu_us": round(med["valu"], 1),
            "vector_alu_over_matrix_core": round(med["valu"] / med["mfma"], 4),
            "matrix_core_frac_of_peak": round(nb / (med["mfma"] * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                              4),
            "vector_alu_frac_of_peak": round(nb / (med["valu"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "max_rel_diff": diff}


def static_bench(dsc, di, torch, dev, steps, per_kernel_ms):
    """The static-filter comparator at the step's shape: per-channel filters
    (H=1, the depthwise form), bf16, residual, forward and backward, each op on
    its own copy of the inputs, mean of `steps` event-timed launches.  Set
    beside the dynamic ops it answers how much the per-token filters cost over
    a fixed filter.  Not part of the step."""
    B, T, D, W = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"]
    N, es = B * T, 2
    stream = torch.cuda.current_stream()
    x = di.randn((B, T, D), 1.0, 95, "bf16").to(dev)
    w = di.randn((D, W), 0.5, 96, "bf16").to(dev)
    dy = di.randn((B, T, D), 1.0, 97, "bf16").to(dev)
    xb = x.clone()
    y, dx, dw = torch.empty_like(x), torch.empty_like(x), torch.empty_like(w)
    ws = dsc.static_workspace(x, W, 1)
    ops = {"static_fwd": (lambda: dsc.dsc_static_fwd(x, w, y, 1, True, False, stream),
                          es * (2 * N * D + D * W)),
           "static_bwd": (lambda: dsc.dsc_static_bwd(xb, w, dy, dx, dw, ws, 1, True, False,
                                                     stream),
                          es * (3 * N * D + 2 * D * W))}
    out = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps
        out[name] = {"ms": round(ms, 4), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "algorithmic_bytes": nbytes}
    t_static = out["static_fwd"]["ms"] + out["static_bwd"]["ms"]
    out["tokens_per_s"] = round(N / (t_static * 1e-3), 1)
    for v in ("headwise", "lowrank"):
        t_dyn = per_kernel_ms[f"{v}_fwd"] + per_kernel_ms[f"{v}_bwd"]
        out[f"{v}_time_over_static"] = round(t_dyn / t_static, 3)
    return out


def varlen_bench(dsc, di, torch, dev, steps, per_kernel_ms):
    """The step's four ops on packed rows: every row of the batch holds
    documents of 1..512 tokens (mean about 256), positions in pos (B, T).
    Each op reads its own input copies; mean of `steps` event-timed launches.
    Reported beside the plain ops' times (the masking overhead).  Not part of
    the step."""
    import numpy as np
    B, T, D, W = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"]
    Hh, R, Hl = WORKLOAD["H_headwise"], WORKLOAD["R"], WORKLOAD["H_lowrank"]
    rng = np.random.default_rng(98)
    pos = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        t = 0
        while t < T:
            n = int(rng.integers(1, 513))
            pos[b, t:t + n] = np.arange(min(n, T - t))
            t += n
    pd = torch.from_numpy(pos).to(dev)
    stream = torch.cuda.current_stream()
    mk = lambda shape, std, seed: di.randn(shape, std, seed, "bf16").to(dev)
    G = D // Hh
    xa, wa = mk((B, T, D), 1.0, 80), mk((B, T, G, W), 0.5, 81)
    xb, wb, dyb = mk((B, T, D), 1.0, 82), mk((B, T, G, W), 0.5, 83), mk((B, T, D), 1.0, 84)
    xc, zc = mk((B, T, D), 1.0, 85), mk((B, T, R), 1.0, 86)
    Uc = mk((R, (D // Hl) * W), (1.0 / (R * W)) ** 0.5, 87)
    xd, zd, dyd = mk((B, T, D), 1.0, 88), mk((B, T, R), 1.0, 89), mk((B, T, D), 1.0, 90)
    y1, dx1, dw1 = torch.empty_like(xa), torch.empty_like(xa), torch.empty_like(wa)
    y2, dx2, dz2, dU2 = (torch.empty_like(xa), torch.empty_like(xa), torch.empty_like(zc),
                         torch.empty_like(Uc))
    ws = dsc.lowrank_workspace(xd, zd, W, Hl)
    ops = {
        "headwise_fwd": lambda: dsc.dsc_headwise_fwd_varlen(xa, wa, pd, y1, Hh, True, False,
                                                            stream),
        "headwise_bwd": lambda: dsc.dsc_headwise_bwd_varlen(xb, wb, pd, dyb, dx1, dw1, Hh, True,
                                                            False, stream),
        "lowrank_fwd": lambda: dsc.dsc_lowrank_fwd_varlen(xc, zc, Uc, pd, y2, W, Hl, True, False,
                                                          stream),
        "lowrank_bwd": lambda: dsc.dsc_lowrank_bwd_varlen(xd, zd, Uc, pd, dyd, dx2, dz2, dU2, ws,
                                                          W, Hl, True, False, stream),
    }
    out = {"documents": int((pos == 0).sum())}
    for name, fn in ops.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sum(e0.elapsed_time(e1) for e0, e1 in ev) / steps
        out[name] = {"ms": round(ms, 4),
                     "over_plain": round(ms / per_kernel_ms[name], 3)}
    return out


def gen_setup(dsc, di, torch, dev, Dh=2048):
    """Inputs and launchers of the generated-filter comparison: filters from a
    hidden state xh (B, T, Dh) of a 2048-wide model at the step's head-wise
    shape (H=16, W=4, bf16, residual), forward only.  `fused` is the kernel
    that forms w = xh M on chip (M passed as Mt (G*W, Dh)); the unfused pair
    is a library GEMM writing w (torch.matmul on hipBLASLt, with M as (Dh, G*W)
    or as the transposed view of Mt) then the head-wise forward reading it.
    Each launcher takes a set index: two input sets of x and xh alternate
    (536 MB, more than the last-level cache holds), so no call finds its
    inputs cached by the call before."""
    B, T, D, W, Hh = (WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"],
                      WORKLOAD["H_headwise"])
    G, N = D // Hh, B * T
    stream = torch.cuda.current_stream()
    mk = lambda shape, std, seed: di.randn(shape, std, seed, "bf16").to(dev)
    sets = [(mk((B, T, D), 1.0, 70 + 2 * i), mk((B, T, Dh), 1.0, 71 + 2 * i)) for i in range(2)]
    M = mk((Dh, G * W), (0.25 / Dh) ** 0.5, 74)
    Mt = M.t().contiguous()
    ys = [torch.empty_like(sets[0][0]) for _ in range(2)]
    w2 = torch.empty((B, T, G, W), dtype=torch.bfloat16, device=dev)

    def fused(i):
        x, xh = sets[i % 2]
        dsc.dsc_headwise_gen_fwd(x, xh, Mt, ys[i % 2], W, Hh, True, False, stream)

    def unfused_nn(i):
        x, xh = sets[i % 2]
        torch.matmul(xh.view(N, Dh), M, out=w2.view(N, G * W))
        dsc.dsc_headwise_fwd(x, w2, ys[i % 2], Hh, True, False, stream)

    def unfused_nt(i):
        x, xh = sets[i % 2]
        torch.matmul(xh.view(N, Dh), Mt.t(), out=w2.view(N, G * W))
        dsc.dsc_headwise_fwd(x, w2, ys[i % 2], Hh, True, False, stream)

    def gemm_only(i):
        torch.matmul(sets[i % 2][1].view(N, Dh), M, out=w2.view(N, G * W))

    meta = {"B": B, "T": T, "D": D, "Dh": Dh, "W": W, "H": Hh, "G": G, "N": N}
    return {"fused": fused, "unfused_M": unfused_nn, "unfused_Mt": unfused_nt,
            "library_gemm_alone": gemm_only}, meta


def gen_bench(dsc, di, torch, dev, steps, rounds=5):
    """Event-timed comparison of the fused generated-filter forward with the
    unfused pair (see gen_setup), not part of the step: `rounds` rounds, each
    timing `steps` calls of every path in turn; per path the median call."""
    fns, m = gen_setup(dsc, di, torch, dev)
    stream = torch.cuda.current_stream()
    times = {name: [] for name in fns}
    for name, fn in fns.items():
        for i in range(4):
            fn(i)
    torch.cuda.synchronize()
    for _ in range(rounds):
        for name, fn in fns.items():
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)]
            for i, (a, b) in enumerate(ev):
                a.record(stream)
                fn(i)
                b.record(stream)
            torch.cuda.synchronize()
            times[name] += [a.elapsed_time(b) * 1e3 for a, b in ev]
    out = {}
    for name, t in times.items():
        t = sorted(t)
        out[f"{name}_us"] = round(t[len(t) // 2], 1)
    out["unfused_us"] = min(out["unfused_M_us"], out["unfused_Mt_us"])
    flops = 2.0 * m["N"] * m["Dh"] * m["G"] * m["W"]
    out["gemm_tflops_fused"] = round(flops / (out["fused_us"] * 1e-6) / 1e12, 1)
    out["hbm_bytes_fused"] = 2 * (m["N"] * m["Dh"] + m["Dh"] * m["G"] * m["W"]
                                  + 2 * m["N"] * m["D"])
    out["fused_over_unfused"] = round(out["fused_us"] / out["unfused_us"], 3)
    out["timing"] = f"median of {rounds} x {steps} calls per path, rounds interleaved"
    out["config"] = f"B={m['B']} T={m['T']} D={m['D']} Dh={m['Dh']} W={m['W']} H={m['H']}"
    return out


def gen_profile(dsc, di, torch, dev, calls):
    """Counter passes of the generated-filter comparison: `calls` launches of
    the fused kernel and of the unfused pair (M transposed), each followed by
    the 512 MiB device copy that calibrates the counters.  No timing."""
    fns, _ = gen_setup(dsc, di, torch, dev)
    src = torch.empty(1 << 28, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for i in range(calls):
        fns["fused"](i)
        fns["unfused_Mt"](i)
        dst.copy_(src)
    torch.cuda.synchronize()


GEN_KERNELS = {"fused (w formed on chip)": "gen_fwd_kernel",
               "library GEMM writing w": "Cijk_",
               "head-wise forward reading w": "hw_fwd_kernel"}


def summarize_gen_profiles(d, calls):
    """profiles/generated_filter_traffic.md from the three rocprofv3 runs of
    `python3 bench.py --generated-filters --profile-ops <calls>` under `d`
    (trace/, fetch/, write/ as for --summarize-profiles)."""
    import csv
    import collections

    def kname(n):
        for k in list(GEN_KERNELS.values()) + [COPY_KERNEL]:
            if k in n:
                return k
        return None

    stats = {}
    for row in csv.DictReader(open(os.path.join(d, "trace", "run_kernel_stats.csv"))):
        k = kname(row["Name"])
        if k:
            stats[k] = (int(row["Calls"]), float(row["AverageNs"]) / 1e3)

    def counter(sub, name):
        per = collections.defaultdict(dict)
        for row in csv.DictReader(open(os.path.join(d, sub, "run_counter_collection.csv"))):
            k = kname(row["Kernel_Name"])
            if k and row["Counter_Name"] == name:
                di_ = int(row["Dispatch_Id"])
                per[k][di_] = per[k].get(di_, 0.0) + float(row["Counter_Value"])
        last = sorted(per[COPY_KERNEL])[-calls:]  # the 512 MiB copies, not the input copies
        per[COPY_KERNEL] = {i: per[COPY_KERNEL][i] for i in last}
        return {k: sum(v.values()) / len(v) for k, v in per.items()}

    fetch, write = counter("fetch", "FETCH_SIZE"), counter("write", "WRITE_SIZE")
    ff, wf = COPY_KIB / fetch[COPY_KERNEL], COPY_KIB / write[COPY_KERNEL]
    cmd = ("rocprofv3 {opt} --output-format csv -d <out>/{sub} -o run -- "
           f"python3 bench.py --generated-filters --profile-ops {calls}")
    lines = ["# HBM traffic of the generated-filter comparison, B=8 T=2048 D=6144 Dh=2048 W=4 "
             "H=16 bf16 (residual)", "",
             "Commands (repository root, MI355X, TMPDIR=/tmp), then the summary:", ""]
    for opt, sub in (("--kernel-trace --stats", "trace"), ("--pmc FETCH_SIZE", "fetch"),
                     ("--pmc WRITE_SIZE", "write")):
        lines.append("    " + cmd.format(opt=opt, sub=sub))
    lines += [f"    python3 bench.py --summarize-gen-profiles <out> --profile-ops {calls}", "",
              f"Calibration: the {COPY_KIB // 1024} MiB device copy reads FETCH_SIZE "
              f"{fetch[COPY_KERNEL]:.0f} KiB and writes WRITE_SIZE {write[COPY_KERNEL]:.0f} KiB "
              f"per call, so HBM bytes = {ff:.3f} x FETCH_SIZE + {wf:.3f} x WRITE_SIZE (KiB).",
              "", "| path | kernel | calls | avg us | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB |",
              "|---|---|---|---|---|---|---|"]
    for what, k in GEN_KERNELS.items():
        n, us = stats.get(k, (0, float("nan")))
        hb = (ff * fetch.get(k, 0.0) + wf * write.get(k, 0.0)) * 1024
        lines.append(f"| {what} | `{k}` | {n} | {us:.1f} | {fetch.get(k, 0):.0f} | "
                     f"{write.get(k, 0):.0f} | {hb / 1e6:.1f} |")
    with open(os.path.join(ROOT, "profiles", "generated_filter_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Read/write mixes of the step's ops, as (input shifts, output shifts): a
# tensor of shift s has 1/2^s the vectors of x (the head-wise filters w and dw
# are a quarter of x at H=16, W=4).
CEILING_MIXES = {
    "read_only": ([0], []),
    "copy (low-rank fwd)": ([0], [0]),
    "head-wise fwd (x, w -> y)": ([0, 2], [0]),
    "2 reads, 1 write (low-rank bwd)": ([0, 0], [0]),
    "head-wise bwd (x, w, dy -> dx, dw)": ([0, 2, 0], [0, 2]),
}


def lds_banks():
    """How the LDS serves one wave's access for the address patterns behind
    the kernels' LDS layouts (libdsc_ldsprobe.so, see csrc/lds_probe.hip):
    clock units per instruction, and the ratio to the op's conflict-free
    linear pattern.  Prints a markdown table (profiles/lds_banks.md)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc_ldsprobe.so"))
    lib.dsc_lds_probe.argtypes = [ctypes.POINTER(ctypes.c_uint), ctypes.c_int,
                                  ctypes.POINTER(ctypes.c_double)]
    ops = ["16-byte read", "8-byte read", "8-byte transposing read", "16-byte write",
           "8-byte write", "2-byte write"]
    size = [16, 8, 8, 16, 8, 2]
    j_, q_ = (lambda i: i & 15), (lambda i: i >> 4)
    paired = lambda vi: (2 * (vi >> 2) + ((vi & 3) >> 1)) * 32 + (vi & 1) * 256
    gen_swz = lambda j: (0x78 >> (2 * ((j >> 2) & 3))) & 3
    pats = [
        (0, "linear (lane i at 16 i)", lambda i: 16 * i),
        (0, "stride 32", lambda i: 32 * i),
        (0, "stride 64", lambda i: 64 * i),
        (0, "stride 256", lambda i: 256 * i),
        (0, "16 lanes per 256-byte row, rows 256 apart", lambda i: (i % 16) * 16 + (i // 16) * 256),
        (0, "16 lanes per 256-byte row, rows 272 apart", lambda i: (i % 16) * 16 + (i // 16) * 272),
        (0, "16 lanes per 256-byte row, rows 288 apart", lambda i: (i % 16) * 16 + (i // 16) * 288),
        (0, "16 lanes per 256-byte row, rows 512 apart", lambda i: (i % 16) * 16 + (i // 16) * 512),
        (0, "8 lanes per 128-byte row, rows 256 apart", lambda i: (i % 8) * 16 + (i // 8) * 256),
        (0, "8 lanes per 128-byte row, rows 384 apart", lambda i: (i % 8) * 16 + (i // 8) * 384),
        (0, "GEMM fragment, granule q ^ (j >> 2) (before)",
         lambda i: j_(i) * 64 + 16 * (q_(i) ^ (j_(i) >> 2))),
        (0, "GEMM fragment, granule q ^ perm(j >> 2) (kept)",
         lambda i: j_(i) * 64 + 16 * (q_(i) ^ gen_swz(j_(i)))),
        (0, "low-rank ring read, plain vector order (before)", lambda i: j_(i) * 528 + q_(i) * 32),
        (0, "low-rank ring read, quarters paired 256 B apart (kept)",
         lambda i: j_(i) * 528 + paired(q_(i))),
        (1, "linear (lane i at 8 i)", lambda i: 8 * i),
        (1, "stride 16", lambda i: 16 * i),
        (1, "stride 32", lambda i: 32 * i),
        (2, "linear (lane i at 8 i)", lambda i: 8 * i),
        (2, "stride 32", lambda i: 32 * i),
        (2, "low-rank backward ring read: row 4q + j/4 (pitch 288), quad j % 4",
         lambda i: (4 * q_(i) + (j_(i) >> 2)) * 288 + 8 * (j_(i) & 3)),
        (3, "linear (lane i at 16 i)", lambda i: 16 * i),
        (3, "low-rank ring write, plain vector order (16 lanes per row, 528 apart)",
         lambda i: (i // 16) * 528 + (i % 16) * 32),
        (3, "low-rank ring write, paired order, first half of odd vectors swapped (kept)",
         lambda i: (i // 16) * 528 + paired(i % 16) + 16 * ((i % 16) & 1)),
        (4, "linear (lane i at 8 i)", lambda i: 8 * i),
        (4, "stride 32", lambda i: 32 * i),
        (5, "linear (lane i at 2 i)", lambda i: 2 * i),
        (5, "stride 64", lambda i: 64 * i),
    ]
    base = {}
    rows = ["| access | lane address pattern | clock units per instruction | x linear |",
            "|---|---|---|---|"]
    for op, name, f in pats:
        offs = (ctypes.c_uint * 64)(*[f(i) for i in range(64)])
        out = ctypes.c_double(0.0)
        rc = lib.dsc_lds_probe(offs, op, ctypes.byref(out))
        if rc != 0:
            raise RuntimeError(f"dsc_lds_probe failed ({rc}) for {ops[op]} {name}")
        base.setdefault(op, out.value)
        rows.append(f"| {ops[op]} | {name} | {out.value:.2f} | {out.value / base[op]:.2f} |")
    return "\n".join(rows)


def stream_ceilings(torch, dev, reps=8):
    """Best HBM rate of a plain streaming kernel (libdsc_stream.so) for each
    read/write mix of the step's ops, at the step's tensor sizes (x: B*T*D
    bf16), over a sweep of grid and block sizes; two tensor sets alternate
    (more than the last-level cache), median of `reps` launches per shape."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc_stream.so"))
    lib.dsc_stream_mix.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_void_p, ctypes.c_uint, ctypes.c_void_p]
    sink = torch.zeros(16, dtype=torch.uint8, device=dev)
    B, T, D = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"]
    n = B * T * D * 2 // 16
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    out = {}
    for name, (ish, osh) in CEILING_MIXES.items():
        sets = []
        for _ in range(2):
            ins = [torch.empty((n >> s) * 16, dtype=torch.uint8, device=dev) for s in ish]
            outs = [torch.empty((n >> s) * 16, dtype=torch.uint8, device=dev) for s in osh]
            for t in ins:
                t.fill_(1)  # xor of the loads: 0x01010101 or 0, never the sink key
            ip = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in ins])
            op = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in outs])
            sets.append((ins, outs, ip, op))
        ish_c = (ctypes.c_int * 3)(*ish)
        osh_c = (ctypes.c_int * 2)(*osh)
        nbytes = sum(16 * (n >> s) for s in ish + osh)
        best = (0.0, None)
        for block in (256, 512, 1024):
            for grid in (256, 512, 1024, 2048, 4096, 8192):
                def call(i):
                    _, _, ip, op = sets[i % 2]
                    r = lib.dsc_stream_mix(ip, ish_c, len(ish), op, osh_c, len(osh), n, grid,
                                           block, ctypes.c_void_p(sink.data_ptr()), 0xA5A5A5A5,
                                           sp)
                    assert r == 0, r
                for i in range(2):
                    call(i)
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(reps)]
                for i, (a, b) in enumerate(ev):
                    a.record(stream)
                    call(i)
                    b.record(stream)
                torch.cuda.synchronize()
                ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
                gbps = nbytes / (ms * 1e-3) / 1e9
                if gbps > best[0]:
                    best = (gbps, (grid, block))
        out[name] = {"gbps": round(best[0], 1), "frac_of_peak": round(best[0] / HBM_PEAK_GBPS, 4),
                     "bytes": nbytes, "grid": best[1][0], "block": best[1][1]}
        del sets
        torch.cuda.empty_cache()
    return out


def access_order(torch, dev, reps=10):
    """The head-wise forward's bytes (x and a quarter-size filter tensor read,
    y written) moved by the plain probe of libdsc_stream.so in three
    geometries: long per-lane strips (workgroups resident all at once),
    short per-wave chunks swept in address order, and whole rows per
    workgroup.  Two tensor sets alternate; median of `reps` launches."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "dynamic_short_causal_amd", "libdsc_stream.so"))
    lib.dsc_stream_order.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    B, T, D = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"]
    ncol = D * 2 // 16
    n = B * T * ncol
    sets = [(torch.ones(n * 16, dtype=torch.uint8, device=dev),
             torch.ones(n * 4, dtype=torch.uint8, device=dev),
             torch.empty(n * 16, dtype=torch.uint8, device=dev)) for _ in range(2)]
    nbytes = n * 16 * 2 + n * 4
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    cases = [("long strips, 64 tokens per lane", 0, 64, 1),
             ("short chunks, 4 tokens x 8 waves", 1, 4, 8),
             ("whole rows, 1 per workgroup", 2, 1, 1),
             ("whole rows, 4 per workgroup", 2, 4, 1),
             ("whole rows, 16 per workgroup", 2, 16, 1),
             ("whole rows, 64 per workgroup", 2, 64, 1)]
    out = {}
    for name, mode, ln, nw in cases:
        def call(i):
            x, w, y = sets[i % 2]
            r = lib.dsc_stream_order(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                                     ctypes.c_void_p(y.data_ptr()), B, T, ncol, mode, ln, nw, sp)
            assert r == 0, r
        for i in range(2):
            call(i)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for i, (a, b) in enumerate(ev):
            a.record(stream)
            call(i)
            b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
        out[name] = {"us": round(ms * 1e3, 1), "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return {"bytes": nbytes, "config": f"B={B} T={T} D={D} bf16, filter tensor D/4 per token",
            "timing": f"median of {reps} launches, two tensor sets alternating", "cases": out}


def decode_bench(dsc, di, torch, dev, iters=200):
    """One-token steps at serving batches, for head-wise H=16 and low-rank R=16
    H=1 at D=6144, W=4, bf16, residual.  Two timings of `iters` steps in a row:
    "eager" launches each step from Python (binding and launch cost included),
    "graph" replays them from one captured HIP graph (device time per step).
    The state stays the same buffer, as in a serving loop.  Not part of the
    training step."""
    D, W, R = WORKLOAD["D"], WORKLOAD["W"], WORKLOAD["R"]
    Hh, Hl = WORKLOAD["H_headwise"], WORKLOAD["H_lowrank"]
    cur = torch.cuda.current_stream()

    def per_step_us(run):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        run()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    out = {}
    for B in (64, 512):
        x = di.randn((B, D), 1.0, 90, "bf16").to(dev)
        st = di.randn((B, W - 1, D), 1.0, 91, "bf16").to(dev)
        w = di.randn((B, D // Hh, W), 0.5, 92, "bf16").to(dev)
        z = di.randn((B, R), 1.0, 93, "bf16").to(dev)
        U = di.randn((R, (D // Hl) * W), 0.125, 94, "bf16").to(dev)
        y = torch.empty_like(x)
        act_bytes = 2 * B * D * (2 + 2 * (W - 1))
        hw = lambda s: dsc.dsc_headwise_decode(x, w, st, y, Hh, True, False, s)
        lr = lambda s: dsc.dsc_lowrank_decode(x, z, U, st, y, W, Hl, True, False, s)
        cases = {"headwise": (hw, act_bytes + 2 * B * (D // Hh) * W),
                 "lowrank": (lr, act_bytes + 2 * (B * R + R * (D // Hl) * W))}
        for name, (fn, nbytes) in cases.items():
            for _ in range(10):
                fn(cur)
            torch.cuda.synchronize()
            eager = per_step_us(lambda: [fn(cur) for _ in range(iters)])
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cap = torch.cuda.current_stream()
                for _ in range(iters):
                    fn(cap)
            g.replay()
            torch.cuda.synchronize()
            graph = per_step_us(g.replay)
            del g
            out[f"{name}_B{B}"] = {"eager_us_per_step": round(eager, 2),
                                   "graph_us_per_step": round(graph, 2),
                                   "tokens_per_s": round(B / (graph * 1e-6), 1),
                                   "gbps": round(nbytes / (graph * 1e-6) / 1e9, 1),
                                   "algorithmic_bytes": nbytes}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 timed steps (about 0.1 s of device time) after 50 warmup steps: the
    # first few steps after the inputs are made run slower (clocks and caches
    # settling), which 20 steps after 5 did not average away
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lds-banks", action="store_true",
                    help="print the LDS access-pattern costs behind the kernels' LDS layouts")
    ap.add_argument("--profile-ops", type=int, default=0,
                    help="run each op this many times (and a copy of known size), no timing")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="summarise the rocprofv3 runs under DIR into profiles/ (no GPU)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "NAME"),
                    help="kernel table of one --kernel-trace --stats run into profiles/NAME.md; "
                         "NAME is one of " + ", ".join(TRACES))
    ap.add_argument("--other-configs", action="store_true",
                    help="time the MLP and linear-RNN configurations instead of the step")
    ap.add_argument("--generated-filters", action="store_true",
                    help="time only the generated-filter comparison (fused against unfused); "
                         "with --profile-ops, run its counter passes instead")
    ap.add_argument("--summarize-counters", nargs="+", metavar=("NAME", "DIR"),
                    help="SQ counter passes under DIR... into profiles/NAME.md; NAME is one of "
                         + ", ".join(COUNTER_RUNS))
    ap.add_argument("--tied8-forward", action="store_true",
                    help="time the linear-RNN forward on the vector-ALU kernel and on the "
                         "matrix-core kernel of libdsc_yard.so; with --profile-ops, run each "
                         "that many times untimed (counter runs)")
    ap.add_argument("--tied8-backward", action="store_true",
                    help="time the linear-RNN backward on the matrix-core kernel and on the "
                         "vector-ALU kernel of libdsc_yard.so; with --profile-ops, run each "
                         "that many times untimed (counter runs)")
    ap.add_argument("--access-order", action="store_true",
                    help="time the head-wise forward's bytes in three access orders and exit")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the streaming ceilings of the step's read/write mixes")
    ap.add_argument("--summarize-gen-profiles", metavar="DIR",
                    help="summarise the generated-filter counter runs under DIR into profiles/ "
                         "(no GPU)")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.profile_ops)
        return
    if args.summarize_gen_profiles:
        summarize_gen_profiles(args.summarize_gen_profiles, args.profile_ops)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1:])
        return
    if args.summarize_trace:
        d, name = args.summarize_trace
        title, command = TRACES[name]
        summarize_trace(d, name, title, command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the op would shard by batch or by channel blocks, with no exchange in the "
              "forward, so one GPU's share at its real shape is what this measures)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import dsc_inputs as di
    import dynamic_short_causal_amd as dsc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.lds_banks:
        print(lds_banks(), flush=True)
        return
    if args.other_configs:
        print(json.dumps({"other_configs": other_configs(dsc, di, torch)}), flush=True)
        return
    if args.ceilings:
        print(json.dumps({"stream_ceilings": stream_ceilings(torch, dev)}), flush=True)
        return
    if args.access_order:
        print(json.dumps({"access_order": access_order(torch, dev)}), flush=True)
        return
    if args.tied8_backward:
        r = tied8_backward(dsc, di, torch, profile_calls=args.profile_ops)
        if r is None:
            print("bench: profile passes done", file=sys.stderr, flush=True)
        else:
            print(json.dumps({"tied8_backward": r}), flush=True)
        return
    if args.tied8_forward:
        r = tied8_forward(dsc, di, torch, profile_calls=args.profile_ops)
        if r is None:
            print("bench: profile passes done", file=sys.stderr, flush=True)
        else:
            print(json.dumps({"tied8_forward": r}), flush=True)
        return
    if args.generated_filters:
        if args.profile_ops:
            gen_profile(dsc, di, torch, dev, args.profile_ops)
            print("bench: profile passes done", file=sys.stderr, flush=True)
            return
        print(json.dumps({"generated_filters": gen_bench(dsc, di, torch, dev, args.steps)}),
              flush=True)
        return
    B, T, D, W = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"]
    Hh, R, Hl = WORKLOAD["H_headwise"], WORKLOAD["R"], WORKLOAD["H_lowrank"]
    wh, wl = di.WORKLOADS["qkv_headwise"], di.WORKLOADS["qkv_lowrank"]
    assert (wh.B, wh.T, wh.D, wh.W, wh.H) == (B, T, D, W, Hh)
    assert (wl.B, wl.T, wl.D, wl.W, wl.H, wl.R) == (B, T, D, W, Hl, R)
    print("bench: generating inputs", file=sys.stderr, flush=True)
    hin = di.make(wh)
    lin = di.make(wl, need_dy=False)
    # Each op reads its own copy of its inputs: x alone is 201 MB and the
    # MI355X last-level cache holds 256 MB, so ops sharing one x would find
    # much of it cached by the op before and report cache, not HBM, traffic.
    hx, hdy, hw = hin["x"].to(dev), hin["dy"].to(dev), hin["w"].to(dev)
    lz, lU = lin["z"].to(dev), lin["U"].to(dev)
    del hin, lin
    cp = lambda t: t.clone()
    xa, wa = cp(hx), cp(hw)                      # head-wise forward
    xb, wb, dyb = cp(hx), cp(hw), cp(hdy)        # head-wise backward
    xc, zc, Uc = cp(hx), cp(lz), cp(lU)          # low-rank forward
    xd, zd, Ud, dyd = hx, lz, lU, hdy            # low-rank backward
    y_h, dx_h, dw_h = torch.empty_like(hx), torch.empty_like(hx), torch.empty_like(hw)
    y_l, dx_l = torch.empty_like(hx), torch.empty_like(hx)
    dz, dU = torch.empty_like(lz), torch.empty_like(lU)
    ws = dsc.lowrank_workspace(hx, lz, W, Hl)
    stream = torch.cuda.current_stream()

    ops = {
        "headwise_fwd": lambda: dsc.dsc_headwise_fwd(xa, wa, y_h, Hh, True, False, stream),
        "headwise_bwd": lambda: dsc.dsc_headwise_bwd(xb, wb, dyb, dx_h, dw_h, Hh, True, False,
                                                     stream),
        "lowrank_fwd": lambda: dsc.dsc_lowrank_fwd(xc, zc, Uc, y_l, W, Hl, True, False, stream),
        "lowrank_bwd": lambda: dsc.dsc_lowrank_bwd(xd, zd, Ud, dyd, dx_l, dz, dU, ws, W, Hl,
                                                   True, False, stream),
    }
    names = list(ops)

    def step(events=None):
        for i, n in enumerate(names):
            if events is not None:
                events[i][0].record(stream)
            ops[n]()
            if events is not None:
                events[i][1].record(stream)

    if args.profile_ops:
        # counter runs: the 512 MiB copy (read and write of known size) calibrates
        # FETCH_SIZE / WRITE_SIZE against the bytes actually moved
        # and a read-only sum of the same 512 MiB cross-checks FETCH_SIZE
        src = torch.ones(1 << 28, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        tot = torch.empty((), dtype=torch.float32, device=dev)
        for _ in range(args.profile_ops):
            step()
            dst.copy_(src)
            torch.sum(src, dim=0, dtype=torch.float32, out=tot)
        torch.cuda.synchronize()
        print("bench: profile passes done", file=sys.stderr, flush=True)
        return

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides.  The steps
    # carry no event records: 8 timing events per step (one pair per op) added
    # about 12 % to the step (0.52-0.54 against 0.47 ms), so the per-op event
    # times come from a second, instrumented pass of K steps below.
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    print(f"bench: {args.steps} steps with per-op events", file=sys.stderr, flush=True)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in names] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    ms_per_step_events = (time.perf_counter() - t1) / args.steps * 1e3
    per_kernel_ms = {n: sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
                     / args.steps for i, n in enumerate(names)}

    def pct(vals):
        v = sorted(vals)
        at = lambda f: v[min(len(v) - 1, int(f * (len(v) - 1) + 0.5))]
        return {"p10": round(at(0.1), 4), "p50": round(at(0.5), 4), "p90": round(at(0.9), 4)}
    # spread over the K timed steps: each op's event time, and their sum per step
    spread = {n: pct([ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps)])
              for i, n in enumerate(names)}
    spread["step_sum_of_ops"] = pct([sum(ev[k][i][0].elapsed_time(ev[k][i][1])
                                         for i in range(len(names))) for k in range(args.steps)])

    # Each op alone: blocks of 10 back-to-back calls between two events, the
    # calls alternating between two complete sets of the op's tensors (inputs,
    # outputs and workspace: more than the last-level cache holds, so neither
    # set is cached when its turn comes), median of 5 blocks.  This spreads
    # the cost of the event packets over the block, so the figure is the one a
    # kernel trace gives (the roofline entry uses it).
    print("bench: timing each op in blocks", file=sys.stderr, flush=True)
    xa2, wa2, y_h2 = cp(xa), cp(wa), torch.empty_like(y_h)
    xb2, wb2, dyb2 = cp(xb), cp(wb), cp(dyb)
    dx_h2, dw_h2 = torch.empty_like(dx_h), torch.empty_like(dw_h)
    xc2, zc2, y_l2 = cp(xc), cp(zc), torch.empty_like(y_l)
    xd2, zd2, dyd2 = cp(xd), cp(zd), cp(dyd)
    dx_l2, dz2, dU2, ws2 = (torch.empty_like(dx_l), torch.empty_like(dz), torch.empty_like(dU),
                            torch.empty_like(ws))
    alt = {
        "headwise_fwd": lambda: dsc.dsc_headwise_fwd(xa2, wa2, y_h2, Hh, True, False, stream),
        "headwise_bwd": lambda: dsc.dsc_headwise_bwd(xb2, wb2, dyb2, dx_h2, dw_h2, Hh, True, False,
                                                     stream),
        "lowrank_fwd": lambda: dsc.dsc_lowrank_fwd(xc2, zc2, Uc, y_l2, W, Hl, True, False, stream),
        "lowrank_bwd": lambda: dsc.dsc_lowrank_bwd(xd2, zd2, Ud, dyd2, dx_l2, dz2, dU2, ws2, W, Hl,
                                                   True, False, stream),
    }
    block_ms = {}
    for n in names:
        per = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(10):
                (ops if i % 2 == 0 else alt)[n]()
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / 10)
        block_ms[n] = sorted(per)[2]
    del xa2, wa2, y_h2, xb2, wb2, dyb2, dx_h2, dw_h2, xc2, zc2, y_l2, xd2, zd2, dyd2
    del dx_l2, dz2, dU2, ws2

    # a plain device copy of 1 GiB for the achievable-bandwidth context
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 2 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    print("bench: timing decode steps", file=sys.stderr, flush=True)
    decode = decode_bench(dsc, di, torch, dev)
    print("bench: timing the static-filter comparator", file=sys.stderr, flush=True)
    static = static_bench(dsc, di, torch, dev, args.steps, per_kernel_ms)
    print("bench: timing packed rows", file=sys.stderr, flush=True)
    varlen = varlen_bench(dsc, di, torch, dev, args.steps, per_kernel_ms)
    print("bench: timing generated filters", file=sys.stderr, flush=True)
    gen = gen_bench(dsc, di, torch, dev, args.steps)
    print("bench: streaming ceilings", file=sys.stderr, flush=True)
    ceilings = stream_ceilings(torch, dev)
    print("bench: timing the MLP and linear-RNN configurations", file=sys.stderr, flush=True)
    others = other_configs(dsc, di, torch)
    torch.cuda.empty_cache()
    print("bench: timing the linear-RNN forward on both kernels", file=sys.stderr, flush=True)
    tied8 = tied8_forward(dsc, di, torch)
    torch.cuda.empty_cache()
    print("bench: timing the linear-RNN backward on both kernels", file=sys.stderr, flush=True)
    tied8b = tied8_backward(dsc, di, torch)
    torch.cuda.empty_cache()

    nbytes = algorithmic_bytes(B, T, D, W, Hh, R, Hl)
    ms_per_step = elapsed / args.steps * 1e3
    tokens = B * T
    step_bytes = sum(nbytes.values())
    dom = max(names, key=lambda n: per_kernel_ms[n])
    achieved = nbytes[dom] / (block_ms[dom] * 1e-3) / 1e9
    kernels = {n: {"ms": round(per_kernel_ms[n], 4),
                   "gbps": round(nbytes[n] / (per_kernel_ms[n] * 1e-3) / 1e9, 1),
                   "frac_of_peak": round(nbytes[n] / (per_kernel_ms[n] * 1e-3) / 1e9
                                         / HBM_PEAK_GBPS, 4),
                   "ms_block": round(block_ms[n], 4),
                   "frac_of_peak_block": round(nbytes[n] / (block_ms[n] * 1e-3) / 1e9
                                               / HBM_PEAK_GBPS, 4),
                   "algorithmic_bytes": nbytes[n]} for n in names}
    # per variant, as the metric is defined for each (tokens / (t_fwd + t_bwd))
    variants = {}
    for v, (f, bwd) in {"headwise": ("headwise_fwd", "headwise_bwd"),
                        "lowrank": ("lowrank_fwd", "lowrank_bwd")}.items():
        t = (per_kernel_ms[f] + per_kernel_ms[bwd]) * 1e-3
        gbps = (nbytes[f] + nbytes[bwd]) / t / 1e9
        variants[v] = {"tokens_per_s": round(tokens / t, 1), "gbps": round(gbps, 1),
                       "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    out = {
        "metric": "fwd+bwd tokens/s + achieved HBM GB/s (% of peak), D=6144 T=2048 W=4",
        "value": round(tokens / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "one batch B=8 T=2048 D=6144 W=4 (bf16, residual) through "
                               "head-wise H=16 fwd+bwd and low-rank R=16 H=1 fwd+bwd",
                   "B": B, "T": T, "D": D, "W": W, "headwise_H": Hh, "lowrank_R": R,
                   "lowrank_H": Hl, "global_batch": B, "seq_len": T, "parallelism": "none"},
        "hbm_gbps": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "pct_of_peak": round(100 * step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "copy_gbps": round(copy_gbps, 1),
        "kernels": kernels,
        "variants": variants,
        "decode": decode,
        "static_comparator": static,
        "packed_rows": varlen,
        "generated_filters": gen,
        "stream_ceilings": ceilings,
        "spread_ms": spread,
        "ms_per_step_with_op_events": round(ms_per_step_events, 4),
        "other_configs": others,
        "tied8_forward": tied8,
        "tied8_backward": tied8b,
        "roofline": {"bound": "hbm", "kernel": dom, "timing": "blocks of 10 back-to-back calls",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles(dom)},
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
