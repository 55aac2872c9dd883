"""Benchmark of the any4 dequantize-GEMM on one MI355X.

Workload: the MLP up/gate-shaped any4 layer N=14336, K=4096, g=128 (synthetic,
seeded; idx uniform 0..15, per-row sorted N(0,1) bf16 table, alpha ~ U[0.005,
0.02], beta ~ N(0, 0.002), x ~ N(0,1) bf16), at decode batches M=1 and M=16.

A step is one any4_gemm at M=1 followed by one at M=16.  Every launch reads a
different copy of the weights (rotating sets whose total exceeds twice the
256 MB last-level cache), so the weights come from HBM.  Inputs are resident
in HBM before the timed region starts.

value = algorithmic bytes of all timed launches / timed wall time (TB/s),
where the algorithmic bytes of one launch are
    N*K/2 (indices) + 4*N*K/g (alpha, beta) + 32*N (tables) + 2*M*K (x) + 2*M*N (y).
Per-launch durations come from HIP events recorded between the launches on
the stream the kernels run on.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("any4_gemm µs + achieved HBM TB/s (% of peak), M=1 and M=16, "
          "N×K=14336×4096")
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
CACHE_BYTES = 256 * 1024 ** 2   # MI355X last-level cache (MALL)
N_, K_, G_ = 14336, 4096, 128
MS = (1, 16)
KERNEL_SRC = os.path.join(ROOT, "gemm_any4_amd", "csrc", "any4.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_config2.json")


def algorithmic_bytes(M: int, N: int, K: int, g: int) -> int:
    """Bytes the method must move for one y = x * W^T launch."""
    return N * K // 2 + 4 * N * (K // g) + 32 * N + 2 * M * K + 2 * M * N


def weight_bytes(N: int, K: int, g: int) -> int:
    return N * K // 2 + 4 * N * (K // g) + 32 * N


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(M: int):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    if none exist for the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    v = t.get("per_m", {}).get(str(M))
    return None if v is None else float(v["hbm_bytes_per_launch"])


def cpu_baseline(seconds: float) -> dict:
    """The CPU oracle (dequant + fp64 GEMM) on the same workload, repeated for
    about `seconds` of wall time on this host's cores."""
    import numpy as np  # noqa: F401

    import oracle
    import workloads

    inp = workloads.generate(2)
    threads = oracle.default_threads()
    packed = oracle.pack(inp.idx)
    steps = 0
    t0 = time.perf_counter()
    while True:
        w = oracle.dequant(packed, inp.lut, inp.alpha, inp.beta, G_)
        for M in MS:
            oracle.gemm(inp.x[:M], w, nthreads=threads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    step_bytes = sum(algorithmic_bytes(M, N_, K_, G_) for M in MS)
    return {
        "value": step_bytes * steps / el / 1e12,
        "unit": "TB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{steps} full steps of the same workload (oracle dequant of the "
                   f"{N_}x{K_} layer, then fp64 GEMM at M=1 and M=16), {el:.1f} s; "
                   "dequant single-threaded, GEMM split over rows"),
        "ms_per_step": 1e3 * el / steps,
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=0, help="rotating weight sets (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the any4 GEMM runs on a single MI355X; "
              "multi-GPU runs are not part of this build (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gemm_any4_amd as any4
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    any4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = workloads.generate(2)
    wb = weight_bytes(N_, K_, G_)
    R = args.sets or max(2, math.ceil(2 * CACHE_BYTES / wb) + 1)

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)

    idx_d = torch.from_numpy(inp.idx).to(dev)
    packed0 = any4.pack(idx_d)
    del idx_d
    sets = []
    for r in range(R):
        sets.append((packed0.clone(), b16(inp.lut), b16(inp.alpha), b16(inp.beta)))
    x = b16(inp.x)
    ys = {M: torch.empty((M, N_), dtype=torch.bfloat16, device=dev) for M in MS}
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def launch(step: int, M: int):
        p, l, a, b = sets[step % R]
        any4.gemm(x[:M], p, l, a, b, G_, out=ys[M])

    for s in range(args.warmup):
        for M in MS:
            launch(s, M)
    torch.cuda.synchronize()

    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(MS) * K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    i = 1
    for s in range(K):
        for M in MS:
            launch(args.warmup + s, M)
            ev[i].record(stream)
            i += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev[0].elapsed_time(ev[-1])
    per = {M: [] for M in MS}
    i = 1
    for s in range(K):
        for M in MS:
            per[M].append(ev[i - 1].elapsed_time(ev[i]))
            i += 1

    step_bytes = sum(algorithmic_bytes(M, N_, K_, G_) for M in MS)
    value = step_bytes * K / (total_ms * 1e-3) / 1e12
    per_m = {}
    for M in MS:
        d = np.array(per[M]) * 1e3            # us
        bts = algorithmic_bytes(M, N_, K_, G_)
        per_m[str(M)] = {
            "us_mean": float(d.mean()), "us_median": float(np.median(d)),
            "us_p10": float(np.percentile(d, 10)), "us_p90": float(np.percentile(d, 90)),
            "bytes": bts,
            "tbps": bts / (d.mean() * 1e-6) / 1e12,
            "weight_gbps": wb / (d.mean() * 1e-6) / 1e9,
            "pct_hbm_peak": 100.0 * bts / (d.mean() * 1e-6) / (HBM_PEAK_GBS * 1e9),
        }
    dom = max(MS, key=lambda M: per_m[str(M)]["us_mean"])
    dm = per_m[str(dom)]
    achieved = dm["bytes"] / (dm["us_mean"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": _traffic(dom),
                "kernel": f"k_gemm<{dom}> (any4_gemm, M={dom})",
                "bytes_per_launch": dm["bytes"], "launch_us_mean": dm["us_mean"]}

    out = {
        "metric": METRIC, "value": value, "unit": "TB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": total_ms / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"any4 MLP up/gate layer N={N_} K={K_} g={G_}, "
                               f"one any4_gemm at M=1 and one at M=16 per step",
                   "N": N_, "K": K_, "g": G_, "M": list(MS), "rotating_weight_sets": R,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "per_m": per_m,
        "host_wall_s": wall,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
