"""Benchmark of the any4 dequantize-GEMM on one MI355X.

Workload: the MLP up/gate-shaped any4 layer N=14336, K=4096, g=128 (synthetic,
seeded; idx uniform 0..15, per-row sorted N(0,1) bf16 table, alpha ~ U[0.005,
0.02], beta ~ N(0, 0.002), x ~ N(0,1) bf16), at decode batches M=1 and M=16.

A step is one any4_gemm at M=1 followed by one at M=16.  Every launch reads a
different copy of the weights (rotating sets whose total exceeds twice the
256 MB last-level cache), so the weights come from HBM.  Inputs are resident
in HBM before the timed region starts.  The launches of the timed steps are
recorded once in a HIP graph and replayed, so that the host's launch cost
does not set the pace; HIP events on the replay stream bracket the timed
region.

value = algorithmic bytes of all timed launches / timed wall time (TB/s),
where the algorithmic bytes of one launch are
    N*K/2 (indices) + 4*N*K/g (alpha, beta) + 32*N (tables) + 2*M*K (x) + 2*M*N (y).
Per-M launch durations come from graphs of that M alone (same events); the
per-launch distribution (p10 / p50 / p90) from 100 eager launches, each
bracketed by HIP events; and `read_probe` is any4_read_probe (one read of
the same packed weights with the GEMM's loads) timed like the GEMM: the
streaming-read ceiling each per-M figure is also given as a percentage of.

The same graph timing is also reported, outside `value`, for the other
layer shape, the MLP down projection N=4096, K=14336, g=1024, at M=1 and
M=16, under "other_layers"; and for both layers with plain int4 weights
(any4_gemm_int4 on the same codes, scales and offsets, no table), under
"int4_no_table", which puts a number on what the table lookup costs; and
at M = 24, 32, 48 on the up/gate layer (one launch against 16-row slices),
under "wide_batch"; at prefill batches M = 64, 256, 1024 on the up/gate layer
(TFLOP/s against the bf16 matrix peak), under "prefill"; both layers with the codes taken to
2 bits through any2_gemm and to 3 bits through any3_gemm, under "any2" and
"any3"; the 70B decoder-layer shapes and their
layer total, under "decoder_layer_70b"; and the GPU quantiser on a 4096x4096
layer at 4, 3 and 2 bits, under "quantize".

Prints one JSON line.  --traffic-probe instead runs a few launches of each M
plus a device copy of known size, for hardware-counter collection.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
CACHE_BYTES = 256 * 1024 ** 2   # MI355X last-level cache (MALL)
N_, K_, G_ = 14336, 4096, 128
MS = (1, 16)
KERNEL_SRC = os.path.join(ROOT, "gemm_any4_amd", "csrc", "any4.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_any4_gemm_14336x4096.json")   # config 2
COPY_BYTES = 256 * 1024 ** 2    # the calibration copy of --traffic-probe


def algorithmic_bytes(M: int, N: int, K: int, g: int) -> int:
    """Bytes the method must move for one y = x * W^T launch."""
    return N * K // 2 + 4 * N * (K // g) + 32 * N + 2 * M * K + 2 * M * N


def weight_bytes(N: int, K: int, g: int) -> int:
    return N * K // 2 + 4 * N * (K // g) + 32 * N


def rotating_sets(wbytes: int) -> int:
    """Weight sets to rotate over: R - 1 consecutive launches read more than
    twice the 256 MB last-level cache, so each launch's weights come from HBM."""
    return max(2, math.ceil(2 * CACHE_BYTES / wbytes) + 2)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(M: int):
    """HBM bytes per launch from the committed counter summary, or None if it
    was taken on another version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    v = t.get("per_m", {}).get(str(M))
    return None if v is None else float(v["hbm_bytes_per_launch"])


def cpu_baseline() -> dict:
    """The CPU oracle on the two MLP layers the targets are stated for (the
    14336x4096 g128 and 4096x14336 g1024 layers), at M = 1 and M = 16, each
    timed single-threaded and split over rows on every host core: one oracle
    dequant of the layer (single-threaded, as the oracle has it) plus one fp64
    GEMM.  µs and effective GB/s use the GPU's algorithmic bytes.  `value`
    is the all-core rate of the benchmark's step (config 2, M = 1 then 16)."""
    import oracle
    import workloads

    threads = oracle.default_threads()
    cases = []
    t0 = time.perf_counter()
    for cfg in (2, 3):
        inp = workloads.generate(cfg)
        packed = oracle.pack(inp.idx)
        c = workloads.CONFIGS[cfg]
        td = time.perf_counter()
        w = oracle.dequant(packed, inp.lut, inp.alpha, inp.beta, c.g)
        t_dq = time.perf_counter() - td
        for M in MS:
            for nt in (1, threads):
                tg = time.perf_counter()
                oracle.gemm(inp.x[:M], w, nthreads=nt)
                t_g = time.perf_counter() - tg
                t = t_dq + t_g
                bts = algorithmic_bytes(M, c.N, c.K, c.g)
                cases.append({"config": cfg, "N": c.N, "K": c.K, "g": c.g, "M": M,
                              "threads": nt, "us": t * 1e6, "dequant_us": t_dq * 1e6,
                              "gemm_us": t_g * 1e6, "gbps": bts / t / 1e9})
        del w, packed, inp
    el = time.perf_counter() - t0
    step = [x for x in cases if x["config"] == 2 and x["threads"] == threads]
    step_us = sum(x["us"] for x in step)
    step_bytes = sum(algorithmic_bytes(M, N_, K_, G_) for M in MS)
    return {
        "value": step_bytes / (step_us * 1e-6) / 1e12,
        "unit": "TB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"one oracle dequant + fp64 GEMM per case: the {N_}x{K_} g{G_} and "
                   "4096x14336 g1024 layers at M=1 and M=16, single-threaded and on "
                   f"{threads} threads (GEMM split over rows); value = config-2 step "
                   f"(M=1 then M=16) on {threads} threads; {el:.1f} s in total"),
        "cases": cases,
    }


def _setup(torch, any4, workloads, sets_arg: int, cfg: int = 2):
    import numpy as np

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workloads.generate(cfg)
    N_, K_, G_ = inp.N, inp.K, inp.g
    wb = weight_bytes(N_, K_, G_)
    R = sets_arg or rotating_sets(wb)

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)

    idx_d = torch.from_numpy(inp.idx).to(dev)
    packed0 = any4.pack(idx_d)
    del idx_d
    sets = [(packed0.clone(), b16(inp.lut), b16(inp.alpha), b16(inp.beta)) for _ in range(R)]
    x = b16(inp.x)
    ys = {M: torch.empty((M, N_), dtype=torch.bfloat16, device=dev) for M in MS}
    return dev, R, sets, x, ys


def other_layer(torch, any4, workloads, cfg: int, steps: int, int4: bool = False) -> dict:
    """Per-launch µs of any4_gemm (or, with int4, of any4_gemm_int4 on the same
    codes, scales and offsets) on config `cfg`'s layer at each M in MS (graph
    replays over rotating weight sets, as for the main workload)."""
    import numpy as np

    c = workloads.CONFIGS[cfg]
    dev, R, sets, x, ys = _setup(torch, any4, workloads, 0, cfg)

    def launch(i: int, M: int):
        p, l, a, b = sets[i % R]
        if int4:
            any4.gemm_int4(x[:M], p, a, b, c.g, out=ys[M])
        else:
            any4.gemm(x[:M], p, l, a, b, c.g, out=ys[M])

    out = {"N": c.N, "K": c.K, "g": c.g, "rotating_weight_sets": R}
    for M in MS:
        for i in range(5):
            launch(i, M)
        g = _graph(torch, launch, steps, (M,))
        _time_graph(torch, g)
        us = float(np.median([_time_graph(torch, g) * 1e3 / steps for _ in range(3)]))
        bts = algorithmic_bytes(M, c.N, c.K, c.g)
        out[str(M)] = {"us_per_launch": us, "bytes": bts,
                       "tbps": bts / (us * 1e-6) / 1e12,
                       "pct_hbm_peak": 100.0 * bts / (us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
        del g
    del sets
    torch.cuda.empty_cache()
    return out


def lowbit_layer(torch, any4, workloads, cfg: int, steps: int, bits: int = 2) -> dict:
    """Per-launch µs of any2_gemm (bits = 2) or any3_gemm (bits = 3) on config
    `cfg`'s layer with the codes taken to that many bits (idx & 3 or idx & 7,
    in that format's tiles), rotating weight sets, graph replays; bytes are the
    format's algorithmic bytes (N*K*bits/8 for the codes)."""
    import numpy as np

    c = workloads.CONFIGS[cfg]
    dev = torch.device("cuda:0")
    inp = workloads.generate(cfg)
    wb = c.N * c.K * bits // 8 + 4 * c.N * (c.K // c.g) + 32 * c.N
    R = rotating_sets(wb)

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)

    codes = torch.from_numpy(inp.idx & ((1 << bits) - 1)).to(dev)
    pack, gemm = (any4.any2_pack, any4.any2_gemm) if bits == 2 else (any4.any3_pack,
                                                                     any4.any3_gemm)
    p0 = pack(codes)
    del codes
    sets = [(p0.clone(), b16(inp.lut), b16(inp.alpha), b16(inp.beta)) for _ in range(R)]
    x = b16(inp.x)
    ys = {M: torch.empty((M, c.N), dtype=torch.bfloat16, device=dev) for M in MS}

    def launch(i: int, M: int):
        p, l, a, b = sets[i % R]
        gemm(x[:M], p, l, a, b, c.g, out=ys[M])

    out = {"N": c.N, "K": c.K, "g": c.g, "rotating_weight_sets": R}
    for M in MS:
        for i in range(5):
            launch(i, M)
        g = _graph(torch, launch, steps, (M,))
        _time_graph(torch, g)
        us = float(np.median([_time_graph(torch, g) * 1e3 / steps for _ in range(3)]))
        bts = wb + 2 * M * c.K + 2 * M * c.N
        out[str(M)] = {"us_per_launch": us, "bytes": bts, "tbps": bts / (us * 1e-6) / 1e12,
                       "pct_hbm_peak": 100.0 * bts / (us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
        del g
    del sets
    torch.cuda.empty_cache()
    return out


def gemv_dot_layer(torch, any4, workloads, cfg: int, steps: int) -> dict:
    """Per-launch µs at M = 1 of the vector-ALU product (any4_gemv_dot: the
    same decode, v_dot2_f32_bf16 instead of the matrix cores) beside any4_gemm
    on config `cfg`'s layer, graph replays over rotating weight sets."""
    import numpy as np

    c = workloads.CONFIGS[cfg]
    dev, R, sets, x, ys = _setup(torch, any4, workloads, 0, cfg)
    out = {"N": c.N, "K": c.K, "g": c.g, "M": 1, "rotating_weight_sets": R}
    for name, fn in (("mfma_us", any4.gemm), ("vdot2_us", any4.gemv_dot)):
        def launch(i: int, M: int, fn=fn):
            p, l, a, b = sets[i % R]
            fn(x[:1], p, l, a, b, c.g, out=ys[1])

        for i in range(5):
            launch(i, 1)
        g = _graph(torch, launch, steps, (1,))
        _time_graph(torch, g)
        out[name] = float(np.median([_time_graph(torch, g) * 1e3 / steps for _ in range(3)]))
        del g
    del sets
    torch.cuda.empty_cache()
    return out


def decoder_layer(torch, any4, workloads, steps: int) -> dict:
    """The 70B decoder-layer shapes (q/k/v/o 8192x8192, up/gate 28672x8192,
    down 8192x28672, g = 128) at M = 1, 4, 16, graph-timed over rotating
    weight sets, and the layer total 4*t(qkvo) + 2*t(up/gate) + t(down).
    Speed does not depend on the values, so the weights here are seeded
    random codes and tables drawn on the device (the parity tests use the
    quantiser's weights for these shapes)."""
    import numpy as np

    dev = torch.device("cuda:0")
    gen = torch.Generator(device="cpu").manual_seed(4)
    g = workloads.CONFIG4_G
    Ms = workloads.CONFIG4_MS
    out = {"g": g, "M": list(Ms)}
    for name, spec in workloads.CONFIG4_LAYERS.items():
        N, K = spec["N"], spec["K"]
        wb = weight_bytes(N, K, g)
        R = rotating_sets(wb)
        idx = torch.randint(0, 16, (N, K), generator=gen, dtype=torch.uint8).to(dev)
        p0 = any4.pack(idx)
        del idx
        lut = torch.randn(N, 16, generator=gen).to(torch.bfloat16).to(dev)
        al = (torch.rand(N, K // g, generator=gen) * 0.015 + 0.005).to(torch.bfloat16).to(dev)
        be = (torch.randn(N, K // g, generator=gen) * 0.002).to(torch.bfloat16).to(dev)
        # every set has its own copy of all four weight tensors
        sets = [(p0.clone(), lut.clone(), al.clone(), be.clone()) for _ in range(R)]
        del lut, al, be
        del p0
        x = torch.randn(max(Ms), K, generator=gen).to(torch.bfloat16).to(dev)
        ys = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in Ms}

        def launch(i: int, M: int):
            p, l, a, b = sets[i % R]
            any4.gemm(x[:M], p, l, a, b, g, out=ys[M])

        res = {"N": N, "K": K, "rotating_weight_sets": R}
        for M in Ms:
            for i in range(3):
                launch(i, M)
            gr = _graph(torch, launch, steps, (M,))
            _time_graph(torch, gr)
            us = float(np.median([_time_graph(torch, gr) * 1e3 / steps for _ in range(3)]))
            bts = algorithmic_bytes(M, N, K, g)
            res[str(M)] = {"us_per_launch": us, "tbps": bts / (us * 1e-6) / 1e12,
                           "pct_hbm_peak": 100.0 * bts / (us * 1e-6) / (HBM_PEAK_GBS * 1e9)}
            del gr
        out[name] = res
        del sets, x, ys
        torch.cuda.empty_cache()
    out["layer_total_us"] = {
        str(M): 4 * out["qkvo"][str(M)]["us_per_launch"] + 2 * out["up_gate"][str(M)]["us_per_launch"]
        + out["down"][str(M)]["us_per_launch"] for M in Ms}
    return out


def prefill(torch, any4, workloads, Ms) -> dict:
    """µs and TFLOP/s of any4_gemm at prefill batches M > 16 on the up/gate
    layer (the tiled MFMA kernel below 128 rows; from 128 on the layer
    dequantised into the workspace, then one library bf16 GEMM), graph-timed
    over rotating weight sets."""
    import numpy as np

    c = workloads.CONFIGS[2]
    dev, R, sets, x, ys = _setup(torch, any4, workloads, 0, 2)
    out = {"N": c.N, "K": c.K, "g": c.g, "peak_tflops_bf16": MFMA_BF16_PEAK_TFLOPS}
    gen = torch.Generator(device="cpu").manual_seed(7)
    for M in Ms:
        xb = torch.randn(M, c.K, generator=gen).to(torch.bfloat16).to(dev)
        yb = torch.empty(M, c.N, device=dev, dtype=torch.bfloat16)

        def launch(i: int, M: int):
            p, l, a, b = sets[i % R]
            any4.gemm(xb, p, l, a, b, c.g, out=yb)

        for i in range(3):
            launch(i, M)
        steps = 20
        g = _graph(torch, launch, steps, (M,))
        _time_graph(torch, g)
        us = float(np.median([_time_graph(torch, g) * 1e3 / steps for _ in range(3)]))
        tf = 2.0 * M * c.N * c.K / (us * 1e-6) / 1e12
        out[str(M)] = {"us_per_launch": us, "tflops": tf,
                       "pct_mfma_peak": 100.0 * tf / MFMA_BF16_PEAK_TFLOPS}
        del g
    del sets
    torch.cuda.empty_cache()
    return out


def wide_batch(torch, any4, workloads, Ms) -> dict:
    """µs and TB/s of any4_gemm at M = 17..48 on the up/gate layer, where one
    launch runs the streaming kernel with two or three 16-row slices of x
    against each decoded weight tile, beside the same product as 16-row slices
    (one launch per slice, each re-reading the weights); graph-timed over
    rotating weight sets."""
    import numpy as np

    c = workloads.CONFIGS[2]
    dev, R, sets, x, ys = _setup(torch, any4, workloads, 0, 2)
    out = {"N": c.N, "K": c.K, "g": c.g}
    gen = torch.Generator(device="cpu").manual_seed(8)
    for M in Ms:
        xb = torch.randn(M, c.K, generator=gen).to(torch.bfloat16).to(dev)
        yb = torch.empty(M, c.N, device=dev, dtype=torch.bfloat16)

        def one_pass(i: int, M: int):
            p, l, a, b = sets[i % R]
            any4.gemm(xb, p, l, a, b, c.g, out=yb)

        def slices(i: int, M: int):
            p, l, a, b = sets[i % R]
            for m0 in range(0, M, 16):
                any4.gemm(xb[m0:m0 + 16], p, l, a, b, c.g, out=yb[m0:m0 + 16])

        res = {}
        for name, fn in (("one_pass", one_pass), ("slices", slices)):
            for i in range(3):
                fn(i, M)
            steps = 20
            g = _graph(torch, fn, steps, (M,))
            _time_graph(torch, g)
            us = float(np.median([_time_graph(torch, g) * 1e3 / steps for _ in range(3)]))
            res[name + "_us"] = us
            del g
        byt = algorithmic_bytes(M, c.N, c.K, c.g)
        res["bytes"] = byt
        res["tbps"] = byt / (res["one_pass_us"] * 1e-6) / 1e12
        res["pct_hbm_peak"] = 100.0 * res["tbps"] * 1e3 / HBM_PEAK_GBS
        out[str(M)] = res
    del sets
    torch.cuda.empty_cache()
    return out


def quantize_timing(torch, any4, N: int, K: int, g: int, iters: int = 10) -> dict:
    """ms of any4_quantize (group scale + 10 rounds of weighted k-means, one
    GPU wave per row) on an N x K layer, for 4, 3 and 2 bits."""
    gen = torch.Generator(device="cpu").manual_seed(11)
    dev = torch.device("cuda:0")
    W = (torch.randn(N, K, generator=gen) * 0.02).to(dev)
    ex = torch.rand(K, generator=gen).add_(0.5).to(dev)
    out = {"N": N, "K": K, "g": g, "iters": iters}
    for bits in (4, 3, 2):
        any4.quantize(W, ex, g, iters, bits=bits)   # warm
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        e0.record(st)
        any4.quantize(W, ex, g, iters, bits=bits)
        e1.record(st)
        torch.cuda.synchronize()
        out[f"any{bits}_ms"] = e0.elapsed_time(e1)
    return out


def launch_numbers(steps: int, Ms) -> list:
    """(launch number, M) of every launch a graph of `steps` steps records, in
    order: the number counts launches, so with weight set number % R no set
    is read twice within R consecutive launches (every launch of a step, every
    M included, reads weights the previous R - 1 launches did not touch)."""
    return [(i * len(Ms) + j, M) for i in range(steps) for j, M in enumerate(Ms)]


def _graph(torch, launch, steps: int, Ms):
    """Record `steps` steps of launches (one per M in Ms) in a HIP graph;
    launch(n, M) gets the running launch number n."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for n, M in launch_numbers(steps, Ms):
                launch(n, M)
    torch.cuda.synchronize()
    return g


def _time_graph(torch, g, reps: int = 1) -> float:
    """ms for `reps` replays of g; the HIP events go on the stream the replay
    runs on (the current stream)."""
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for _ in range(reps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def traffic_file(cfg: int) -> str:
    if cfg == 2:
        return TRAFFIC_FILE
    return os.path.join(ROOT, "profiles", "traffic_any4_gemm_4096x14336.json")


def traffic_probe(torch, any4, workloads, sets_arg: int, cfg: int = 2) -> int:
    """A few launches of each M on config `cfg`'s layer (each on its own
    weight set) and one COPY_BYTES device copy (the scale for the FETCH_SIZE
    / WRITE_SIZE counters)."""
    c = workloads.CONFIGS[cfg]
    dev, R, sets, x, ys = _setup(torch, any4, workloads, sets_arg, cfg)
    for n, M in launch_numbers(6, MS):
        p, l, a, b = sets[n % R]
        any4.gemm(x[:M], p, l, a, b, c.g, out=ys[M])
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": True, "layer": f"N={c.N} K={c.K} g={c.g}",
                      "copy_bytes": COPY_BYTES, "launches_per_m": 6}), flush=True)
    return 0


def _counter_per_dispatch(path: str, counter: str) -> list:
    """[kernel name, value] per dispatch of one rocprofv3 counter CSV, in
    dispatch order (values of one dispatch over several rows are summed)."""
    import csv
    per = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            e = per.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])
            e[1] += float(r["Counter_Value"])
    return [per[d] for d in sorted(per)]


def traffic_summary(fetch_csv: str, write_csv: str, cfg: int = 2) -> int:
    """Write the committed traffic summary of config `cfg`'s layer from the
    counter files of two `--traffic-probe` runs (rocprofv3 --pmc FETCH_SIZE,
    then WRITE_SIZE): HBM bytes per launch of each M, each counter scaled by
    what it reads for the COPY_BYTES device copy that ends the probe.  A
    launch that splits K is its GEMM kernel plus the k_split_sum after it;
    the partial sums' bytes are given apart (they are not algorithmic)."""
    import re
    import workloads
    c = workloads.CONFIGS[cfg]
    fetch = _counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _counter_per_dispatch(write_csv, "WRITE_SIZE")
    for rows in (fetch, write):
        if not rows or "copyBuffer" not in rows[-1][0]:
            raise SystemExit("the last dispatch of a traffic probe is the calibration copy")
    fscale = COPY_BYTES / (fetch[-1][1] * 1024)
    wscale = COPY_BYTES / (write[-1][1] * 1024)
    pat = re.compile(r"(k_gemm_(?:km|kb|st)<(\d+),[^>]*>)")

    def by_m(rows):
        out = {}
        last = None
        for name, v in rows:
            m = pat.search(name)
            if m:
                last = int(m.group(2))
                out.setdefault(last, {"kernel": m.group(1), "gemm": [], "split": []})["gemm"].append(v)
            elif "k_split_sum" in name and last is not None:
                out[last]["split"].append(v)
        return out

    f_m, w_m = by_m(fetch), by_m(write)
    per_m = {}
    for M in MS:
        fe, wr = f_m[M], w_m[M]
        n = len(fe["gemm"])
        fk, wk = sum(fe["gemm"]) / n, sum(wr["gemm"]) / n
        hbm = fk * 1024 * fscale + wk * 1024 * wscale
        alg = algorithmic_bytes(M, c.N, c.K, c.g)
        e = {"kernel": fe["kernel"], "dispatches": n, "fetch_kib_raw": round(fk, 2),
             "write_kib": round(wk, 2), "hbm_bytes_per_launch": round(hbm),
             "algorithmic_bytes": alg, "ratio": hbm / alg}
        if fe["split"]:
            sf = sum(fe["split"]) / len(fe["split"]) * 1024 * fscale
            sw = sum(wr["split"]) / len(wr["split"]) * 1024 * wscale
            e["k_split_sum_hbm_bytes"] = round(sf + sw)
        per_m[str(M)] = e
    t = {"kernel_source_sha256_16": kernel_source_hash(),
         "workload": f"N={c.N} K={c.K} g={c.g}", "copy_bytes": COPY_BYTES,
         "fetch_scale": fscale, "write_scale": wscale, "per_m": per_m}
    with open(traffic_file(cfg), "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print(json.dumps(t))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=0, help="rotating weight sets (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-layers", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two --traffic-probe counter files")
    ap.add_argument("--layer", type=int, default=2, choices=(2, 3),
                    help="layer of --traffic-probe / --traffic-summary: config 2 (14336x4096) "
                         "or 3 (4096x14336 g1024)")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary, cfg=args.layer)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the any4 GEMM runs on a single MI355X; "
              "multi-GPU runs are not supported (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import gemm_any4_amd as any4
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    any4.lib()
    if args.traffic_probe:
        return traffic_probe(torch, any4, workloads, args.sets, args.layer)

    dev, R, sets, x, ys = _setup(torch, any4, workloads, args.sets)
    wb = weight_bytes(N_, K_, G_)

    def launch(i: int, M: int):
        p, l, a, b = sets[i % R]
        any4.gemm(x[:M], p, l, a, b, G_, out=ys[M])

    # warmup (eager), then the graphs: the timed K steps, and K launches of each M
    for n, M in launch_numbers(args.warmup, MS):
        launch(n, M)
    torch.cuda.synchronize()
    K = args.steps
    g_all = _graph(torch, launch, K, MS)
    g_m = {M: _graph(torch, launch, K, (M,)) for M in MS}
    for gg in [g_all] + list(g_m.values()):
        _time_graph(torch, gg)              # one untimed replay of each graph

    t0 = time.perf_counter()
    total_ms = _time_graph(torch, g_all)
    wall = time.perf_counter() - t0

    per_m = {}
    reps = 3
    for M in MS:
        runs = [_time_graph(torch, g_m[M]) * 1e3 / K for _ in range(reps)]   # us per launch
        us = float(np.median(runs))
        bts = algorithmic_bytes(M, N_, K_, G_)
        per_m[str(M)] = {
            "us_per_launch": us,
            "us_per_launch_runs": runs,
            "bytes": bts,
            "tbps": bts / (us * 1e-6) / 1e12,
            "weight_gbps": wb / (us * 1e-6) / 1e9,
            "pct_hbm_peak": 100.0 * bts / (us * 1e-6) / (HBM_PEAK_GBS * 1e9),
        }

    # per-launch distribution: eager launches, each bracketed by HIP events
    st = torch.cuda.current_stream()
    for M in MS:
        ts = []
        for i in range(100):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            launch(i, M)
            e1.record(st)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in ts])
        per_m[str(M)]["per_launch_events_us"] = {
            "p10": float(np.percentile(us, 10)), "p50": float(np.percentile(us, 50)),
            "p90": float(np.percentile(us, 90)), "launches": len(us)}

    # streaming-read ceiling: the read probe over the same rotating packed
    # buffers, graph-timed like the GEMM
    pbytes = sets[0][0].numel()
    flag = torch.zeros(1, dtype=torch.int32, device=dev)

    def probe(i: int, M: int):
        any4.check(any4.read_probe_raw(sets[i % R][0].data_ptr(), pbytes, flag.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream))

    gp = _graph(torch, probe, K, (1,))
    _time_graph(torch, gp)
    probe_us = float(np.median([_time_graph(torch, gp) * 1e3 / K for _ in range(3)]))
    del gp
    probe_tbps = pbytes / (probe_us * 1e-6) / 1e12
    for M in MS:
        per_m[str(M)]["pct_of_read_probe"] = 100.0 * per_m[str(M)]["tbps"] / probe_tbps

    step_bytes = sum(algorithmic_bytes(M, N_, K_, G_) for M in MS)
    value = step_bytes * K / (total_ms * 1e-3) / 1e12
    dom = max(MS, key=lambda M: per_m[str(M)]["us_per_launch"])
    dm = per_m[str(dom)]
    achieved = dm["bytes"] / (dm["us_per_launch"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": _traffic(dom),
                "kernel": f"k_gemm_st (any4_gemm, M={dom})",
                "bytes_per_launch": dm["bytes"], "launch_us": dm["us_per_launch"]}

    out = {
        "metric": METRIC, "value": value, "unit": "TB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": total_ms / K, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"any4 MLP up/gate layer N={N_} K={K_} g={G_}, "
                               f"one any4_gemm at M=1 and one at M=16 per step",
                   "N": N_, "K": K_, "g": G_, "M": list(MS), "rotating_weight_sets": R,
                   "parallelism": "single GPU", "timing": "HIP graph replay, HIP events"},
        "roofline": roofline,
        "per_m": per_m,
        "read_probe": {"bytes": pbytes, "us_per_launch": probe_us, "tbps": probe_tbps,
                       "pct_hbm_peak": 100.0 * probe_tbps * 1e3 / HBM_PEAK_GBS,
                       "what": "any4_read_probe over the packed weights of the same "
                               "rotating sets: the streaming-read ceiling of one launch"},
        "host_wall_s": wall,
    }
    def progress(what):
        print(f"[bench] {what} done", file=sys.stderr, flush=True)

    progress("headline layer")
    if not args.no_other_layers:
        del g_all, g_m, sets
        torch.cuda.empty_cache()
        out["other_layers"] = {"config3": other_layer(torch, any4, workloads, 3, min(K, 100))}
        progress("other layer")
        # the same layers as plain int4 (no table lookup): the cost of the table
        out["int4_no_table"] = {f"config{c}": other_layer(torch, any4, workloads, c,
                                                          min(K, 100), int4=True)
                                for c in (2, 3)}
        progress("int4")
    if not args.no_other_layers:
        out["any2"] = {f"config{c}": lowbit_layer(torch, any4, workloads, c, min(K, 100), 2)
                       for c in (2, 3)}
        progress("any2")
        out["any3"] = {f"config{c}": lowbit_layer(torch, any4, workloads, c, min(K, 100), 3)
                       for c in (2, 3)}
        progress("any3")
        out["gemv_vdot2_vs_mfma"] = {f"config{c}": gemv_dot_layer(torch, any4, workloads, c,
                                                                 min(K, 100)) for c in (2, 3)}
        progress("gemv")
        out["wide_batch"] = wide_batch(torch, any4, workloads, (24, 32, 48))
        progress("wide batch")
        out["prefill"] = prefill(torch, any4, workloads, (64, 128, 256, 512, 1024))
        progress("prefill")
        out["decoder_layer_70b"] = decoder_layer(torch, any4, workloads, min(K, 50))
        progress("70B decoder layer")
        out["quantize"] = quantize_timing(torch, any4, 4096, 4096, 128)
        progress("quantiser")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
