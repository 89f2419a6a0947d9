"""Benchmark of the dynamic short causal convolution hot path on one MI355X.

One step = one pass of the whole hot path over one synthetic batch
(B=8, T=2048, D=6144, W=4, bf16, inputs resident in HBM):
  head-wise  (H=16, 384 filter groups, residual): forward + backward
  low-rank   (R=16, H=1, filters generated on chip, residual): forward +
             backward (+ the fixed-order reduction of its partial sums)
value = tokens of the batch per second of step time (B*T / t_step).

Also reported: achieved algorithmic HBM bandwidth of the step, a roofline
entry for the dominant kernel (timed with HIP events on the stream the
kernels run on), and the fp64 CPU oracle timed on a bounded sample of the same
workload on this host (cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --profile-ops K   (K untimed passes of every op plus a
                                          512 MiB device copy, for rocprofv3)
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
    "lowrank_fwd": ["dynamic_short_causal_amd/csrc/lowrank_impl.hpp",
                    "dynamic_short_causal_amd/csrc/lowrank_launch.hpp",
                    "dynamic_short_causal_amd/csrc/dsc_device.hpp"],
    "lowrank_bwd": ["dynamic_short_causal_amd/csrc/lowrank_impl.hpp",
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


def cpu_baseline(target_s=15.0):
    """The fp64 oracle on a bounded sample: one sequence of the benchmark
    workload, head-wise and low-rank forward + backward."""
    import numpy as np
    import torch
    import dsc_inputs as di
    import oracle
    orc = oracle.default()
    D, W, Hh, R = WORKLOAD["D"], WORKLOAD["W"], WORKLOAD["H_headwise"], WORKLOAD["R"]

    def run(T):
        g = lambda shape, std, seed: di.randn(shape, std, seed, "bf16").to(torch.float64).numpy()
        x = g((1, T, D), 1.0, 90000)
        dy = g((1, T, D), 1.0, 90004)
        w = g((1, T, D // Hh, W), 0.5, 90001)
        z = g((1, T, R), 1.0, 90002)
        U = g((R, D * W), (1.0 / (R * W)) ** 0.5, 90003)
        t0 = time.perf_counter()
        orc.headwise_fwd(x, w, Hh, residual=True)
        orc.headwise_bwd(x, w, dy, Hh, residual=True)
        orc.lowrank_fwd(x, z, U, W, 1, residual=True)
        orc.lowrank_bwd(x, z, U, dy, W, 1, residual=True)
        return time.perf_counter() - t0

    t_small = run(32)
    T = int(max(32, min(2048, 32 * target_s / max(t_small, 1e-3))))
    T = max(32, (T // 32) * 32)
    el = run(T)
    return {"value": T / el, "unit": "tokens/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": f"1 sequence x {T} tokens of the D=6144 W=4 batch (head-wise H=16 and "
                      f"low-rank R=16 H=1, residual, fwd+bwd), fp64 C oracle with OpenMP; "
                      f"{el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-ops", type=int, default=0,
                    help="run each op this many times (and a copy of known size), no timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by batch or channel blocks with no exchange in the "
              "forward; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dsc_inputs as di
    import dynamic_short_causal_amd as dsc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, T, D, W = WORKLOAD["B"], WORKLOAD["T"], WORKLOAD["D"], WORKLOAD["W"]
    Hh, R, Hl = WORKLOAD["H_headwise"], WORKLOAD["R"], WORKLOAD["H_lowrank"]
    wh, wl = di.WORKLOADS["qkv_headwise"], di.WORKLOADS["qkv_lowrank"]
    assert (wh.B, wh.T, wh.D, wh.W, wh.H) == (B, T, D, W, Hh)
    assert (wl.B, wl.T, wl.D, wl.W, wl.H, wl.R) == (B, T, D, W, Hl, R)
    print("bench: generating inputs", file=sys.stderr, flush=True)
    hin = di.make(wh)
    lin = di.make(wl, need_dy=False)
    x = hin["x"].to(dev)        # one batch of activations for both variants
    dy = hin["dy"].to(dev)
    w = hin["w"].to(dev)
    z = lin["z"].to(dev)
    U = lin["U"].to(dev)
    del hin, lin
    y_h, dx_h, dw_h = torch.empty_like(x), torch.empty_like(x), torch.empty_like(w)
    y_l, dx_l = torch.empty_like(x), torch.empty_like(x)
    dz, dU = torch.empty_like(z), torch.empty_like(U)
    ws = dsc.lowrank_workspace(x, z, W, Hl)
    stream = torch.cuda.current_stream()

    ops = {
        "headwise_fwd": lambda: dsc.dsc_headwise_fwd(x, w, y_h, Hh, True, False, stream),
        "headwise_bwd": lambda: dsc.dsc_headwise_bwd(x, w, dy, dx_h, dw_h, Hh, True, False,
                                                     stream),
        "lowrank_fwd": lambda: dsc.dsc_lowrank_fwd(x, z, U, y_l, W, Hl, True, False, stream),
        "lowrank_bwd": lambda: dsc.dsc_lowrank_bwd(x, z, U, dy, dx_l, dz, dU, ws, W, Hl, True,
                                                   False, stream),
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
        src = torch.empty(1 << 28, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.profile_ops):
            step()
            dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: profile passes done", file=sys.stderr, flush=True)
        return

    print("bench: warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in names] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    per_kernel_ms = {n: sum(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
                     / args.steps for i, n in enumerate(names)}

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

    nbytes = algorithmic_bytes(B, T, D, W, Hh, R, Hl)
    ms_per_step = elapsed / args.steps * 1e3
    tokens = B * T
    step_bytes = sum(nbytes.values())
    dom = max(names, key=lambda n: per_kernel_ms[n])
    achieved = nbytes[dom] / (per_kernel_ms[dom] * 1e-3) / 1e9
    kernels = {n: {"ms": round(per_kernel_ms[n], 4),
                   "gbps": round(nbytes[n] / (per_kernel_ms[n] * 1e-3) / 1e9, 1),
                   "frac_of_peak": round(nbytes[n] / (per_kernel_ms[n] * 1e-3) / 1e9
                                         / HBM_PEAK_GBPS, 4),
                   "algorithmic_bytes": nbytes[n]} for n in names}
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
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
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
