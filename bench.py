"""Benchmark of the quantized-linear hot path on one MI355X.

Workload: the four Llama-3-8B-shaped W8A8 fp8 linears (N,K) = (6144,4096),
(4096,4096), (28672,4096), (4096,14336) -- the layer shapes of the vLLM PR
#4118 micro-benchmark -- with bf16 activations N(0,1) carrying 1% outlier
channels x20, weights N(0,0.02) quantized per tensor to E4M3 once (offline,
not timed), dynamic per-tensor activation quantization every call, exact
fp32 accumulation and a bf16 output.

One step = the whole hot path over one batch: for each of the four linears,
the activation amax, the scale, the E4M3 cast and the fp8 GEMM with its
scale epilogue (bql_fp8_linear, accum exact).  The headline value is the
step's TFLOP/s at M = 1024 tokens; the M = 1 decode pass (the streaming
small-M kernel with its split-K reduce) is timed the same way and reported
in HBM GB/s of algorithmic bytes.  Weights rotate over enough copies that
each pass touches more than twice the 256 MB Infinity Cache.

Prints one JSON line.  --gpus above 1 is refused: the library runs on one GPU.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as wl  # noqa: E402

METRIC = "fp8 linear TFLOP/s at M=1024 + HBM GB/s at M=1, Llama-shaped N×K"
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_F16_TFLOPS = 2500.0
PEAK_I8_TOPS = 5000.0
SHAPES = wl.CFG3_SHAPES
ROTATE_BYTES = 640 * 2 ** 20  # > 2 x 256 MiB Infinity Cache
# steps per captured graph for the microsecond-scale small-M steps (a graph
# launch costs several microseconds)
SMALL_STEPS_PER_GRAPH = 4
# warm-up before each timed leg, in seconds of device time at least (the
# headline steps; the other legs and the per-configuration rows)
WARM_S = 0.5
ROW_WARM_S = 0.2


CALIBRATION_COPY_BYTES = 256 * 2 ** 20
CUS_MI355X = 256
XCDS_MI355X = 8
# sources the tiled GEMM kernels are built from; a traffic summary is only
# used while they are unchanged
KERNEL_SOURCES = ["bit_quantized_linear_amd/csrc/linear.hip",
                  "bit_quantized_linear_amd/csrc/gemm_exact.hip",
                  "bit_quantized_linear_amd/csrc/linear_common.h",
                  "bit_quantized_linear_amd/csrc/device.h",
                  "bit_quantized_linear_amd/csrc/kernels.h"]
EXACT_SIG = "gemm_exact_kernel<"   # the exact fp8 tile kernel at this shape
FAST_SIG = "gemm_kernel<0,"        # the fp8-MFMA tile kernel
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_m1024_n28672_k4096_hbm_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(key):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            fields = dict(line.split(":", 1) for line in fh if ":" in line and not line.startswith(" "))
    except OSError:
        return None
    if fields.get("source_sha256", "").strip() != kernel_source_hash():
        return None
    v = fields.get(key)
    return int(v.strip()) if v else None


def summarize_traffic(fetch_dir, write_dir):
    """Turn two rocprofv3 --pmc runs of `bench.py --roofline-only` (FETCH_SIZE,
    then WRITE_SIZE) into HBM bytes per launch of the two dominant GEMMs.
    Each counter is scaled by what it reads for the run's last plain device
    copy (CALIBRATION_COPY_BYTES read and written)."""
    def per_dispatch(d, counter):
        rows = []
        for root, _, files in os.walk(d):
            for f in files:
                if f.endswith("counter_collection.csv"):
                    with open(os.path.join(root, f)) as fh:
                        rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        acc = {}
        for r in rows:
            k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
        return sorted(acc.items())
    out = {}
    lines = []
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = per_dispatch(d, counter)
        copies = [v for (i, name), v in disp if "copyBuffer" in name]
        if not copies:
            raise SystemExit(f"no calibration copy among the {counter} dispatches in {d}")
        factor = copies[-1] / CALIBRATION_COPY_BYTES
        lines.append(f"  {counter}: calibration copy of {CALIBRATION_COPY_BYTES} B reads {copies[-1]:.1f}"
                     f" counter units -> {1.0 / factor:.2f} B per unit")
        for tag, sig in (("exact", EXACT_SIG), ("fast", FAST_SIG)):
            vals = [v for (i, name), v in disp if sig in name.replace(" ", "")]
            if not vals:
                raise SystemExit(f"no {sig} dispatches in {d}")
            b = sum(vals) / len(vals) / factor
            out.setdefault(tag, 0.0)
            out[tag] += b
            lines.append(f"  {tag} GEMM {counter}: {len(vals)} dispatches, {b / 1e6:.1f} MB per launch")
    alg = algorithmic_bytes_gemm(1024, 28672, 4096)
    text = ["# HBM traffic of the dominant GEMM launches, M=1024 N=28672 K=4096",
            "# (exact = gemm_exact_kernel, f16 MFMA on losslessly decoded fp8; fast = gemm_kernel<0,...>,"
            " fp8 MFMA; pre-quantized A)",
            "commands (repo root; cd /tmp && export TMPDIR=/tmp first, then back):",
            f"  rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o run -- python3 bench.py --roofline-only",
            f"  rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o run -- python3 bench.py --roofline-only",
            f"  python3 bench.py --summarize-traffic {fetch_dir} {write_dir}",
            f"source_sha256: {kernel_source_hash()}",
            "details:"] + lines + [
            f"  algorithmic bytes per launch (Aq + Wq + bf16 Y + scales): {alg}",
            f"exact_hbm_bytes_per_launch: {int(round(out['exact']))}",
            f"fast_hbm_bytes_per_launch: {int(round(out['fast']))}"]
    with open(TRAFFIC_SUMMARY, "w") as fh:
        fh.write("\n".join(text) + "\n")
    print("\n".join(text))


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "gemm_m1024_n28672_k4096_mfma_counters.txt")
MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"]


def summarize_mfma(pmc_dir):
    """Matrix-core counters of the two dominant GEMMs from one rocprofv3
    --pmc run of `bench.py --roofline-only`: MFMA ops per launch (the MOPS
    counters count 512 ops per unit) against the algorithmic 2*M*N*K, and the
    matrix cores' busy cycles per CU against the GPU's active cycles."""
    rows = []
    for root, _, files in os.walk(pmc_dir):
        for f in files:
            if f.endswith("counter_collection.csv"):
                with open(os.path.join(root, f)) as fh:
                    rows += list(csv.DictReader(fh))
    per = {}
    for r in rows:
        k = (int(r["Dispatch_Id"]), r["Kernel_Name"].replace(" ", ""))
        per.setdefault(k, {}).setdefault(r["Counter_Name"], 0.0)
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
    flops = 2 * 1024 * 28672 * 4096
    lines = ["# Matrix-core counters of the dominant GEMM launches, M=1024 N=28672 K=4096",
             "# (pre-quantized A; exact = gemm_exact_kernel, f16 MFMA on losslessly decoded fp8;"
             " fast = gemm_kernel<0,...>, fp8 MFMA)",
             "commands (repo root; cd /tmp && export TMPDIR=/tmp first, then back):",
             "  rocprofv3 --pmc " + " ".join(MFMA_COUNTERS)
             + f" -f csv -d {pmc_dir} -o run -- python3 bench.py --roofline-only",
             f"  python3 bench.py --summarize-mfma {pmc_dir}",
             f"source_sha256: {kernel_source_hash()}",
             f"algorithmic flops per launch (2*M*N*K): {flops}"]
    for tag, sig, mops in (("exact", EXACT_SIG, "SQ_INSTS_VALU_MFMA_MOPS_F16"),
                           ("fast", FAST_SIG, "SQ_INSTS_VALU_MFMA_MOPS_F8")):
        ds = [v for (i, name), v in per.items() if sig in name]
        if not ds:
            raise SystemExit(f"no {sig} dispatches in {pmc_dir}")
        n = len(ds)
        avg = {c: sum(d.get(c, 0.0) for d in ds) / n for c in MFMA_COUNTERS}
        ops = avg[mops] * 512
        # GRBM_GUI_ACTIVE is summed over the 8 XCDs (each reads about clock x
        # duration); MFMA busy cycles are summed over the 4 SIMDs of every CU
        active = avg["GRBM_GUI_ACTIVE"] / XCDS_MI355X
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * CUS_MI355X * 4) if active else float("nan")
        lines += [f"{tag}: {n} dispatches",
                  f"  {mops} x 512 = {ops:.4g} ops per launch ({ops / flops:.4f} of 2*M*N*K)",
                  f"  SQ_VALU_MFMA_BUSY_CYCLES = {avg['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}, "
                  f"SQ_BUSY_CU_CYCLES = {avg['SQ_BUSY_CU_CYCLES']:.4g}, "
                  f"GRBM_GUI_ACTIVE = {avg['GRBM_GUI_ACTIVE']:.4g}",
                  f"  matrix cores busy: MFMA_BUSY / (GUI_ACTIVE / {XCDS_MI355X} XCDs * {CUS_MI355X} CUs"
                  f" * 4 SIMDs) = {busy:.4f}  (the counters slow the kernel; a fraction of its"
                  f" own active cycles)"]
    with open(MFMA_SUMMARY, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def algorithmic_bytes_gemm(M, N, K):
    """The GEMM alone: fp8 A and W, bf16 Y, two scales."""
    return M * K + N * K + 2 * M * N + 8


def algorithmic_bytes(M, N, K):
    """Wq (1 B/elem) + A bf16 + Y bf16 + the two scales."""
    return N * K + 2 * M * K + 2 * M * N + 8


def build_weights(bql, dev):
    """Seeded host weights -> device, packed per tensor, rotated copies."""
    host, packed = [], []
    for idx, (N, K) in enumerate(SHAPES):
        bits = wl.weight(wl.rng(3, idx, 1), N, K, "bf16")
        host.append(bits)
        w = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        pw = bql.prepack_weight(w, "fp8_tensor")
        del w
        packed.append(pw)
    total = sum(N * K for N, K in SHAPES)
    copies = max(1, -(-ROTATE_BYTES // total))
    rot = [packed]
    for _ in range(copies - 1):
        rot.append([bql.PackedWeight(p.packed.clone(), p.scales.clone(), p.N, p.K, p.fmt)
                    for p in packed])
    return host, rot


def build_activations(M, dev, rotate=False):
    """Seeded bf16 activations of the four linears; with rotate, device
    copies of the set enough that a pass over them moves more than
    ROTATE_BYTES (so that the quantizer passes read HBM, not the Infinity
    Cache).  Returns the host bits and, per copy, the four device tensors."""
    bits, first = [], []
    for idx, (N, K) in enumerate(SHAPES):
        b = wl.activation(wl.rng(3, idx, M, 3), M, K, "bf16", "channels")
        bits.append(b)
        first.append(torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16))
    copies = 1
    if rotate:
        copies = max(1, -(-ROTATE_BYTES // sum(2 * M * K for N, K in SHAPES)))
    sets = [first] + [[t.clone() for t in first] for _ in range(copies - 1)]
    return bits, sets


def time_steps(step, steps, warmup, min_warm_s=0.0):
    """Seconds per step over `steps` timed steps, after at least `warmup`
    untimed steps and at least `min_warm_s` seconds of them (so that the
    clocks and caches settle whatever the step count; the host syncs every
    few steps so the warm-up time is device time)."""
    i = 0
    t_end = time.perf_counter() + min_warm_s
    while i < warmup or time.perf_counter() < t_end:
        step(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(steps):
        step(i + j)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / max(steps, 1)


def capture_graphs(step, n, per_graph=1):
    """HIP graphs over the weight-rotation slots: graph g holds steps
    g*per_graph .. g*per_graph + per_graph - 1 back to back (the kernels
    replay without host launch overhead, as a serving loop under graph
    capture runs a whole decode step of many layers; per_graph > 1 keeps
    the launch of one graph from dominating steps of a few microseconds)."""
    ngraphs = max(1, -(-n // per_graph))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(ngraphs * per_graph):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for gi in range(ngraphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in range(per_graph):
                step(gi * per_graph + t)
        graphs.append(g)
    return graphs


def graph_step_time(step, n, steps, warmup, per_graph=1, min_warm_s=WARM_S):
    """Seconds per step from replaying the graphs of capture_graphs: at
    least `steps` steps are timed (a whole number of graphs), after a
    warm-up of at least `warmup` steps and `min_warm_s` seconds."""
    graphs = capture_graphs(step, n, per_graph)
    reps = max(1, -(-steps // per_graph))
    sec = time_steps(lambda i: graphs[i % len(graphs)].replay(), reps, max(1, -(-warmup // per_graph)),
                     min_warm_s)
    return sec / per_graph


def event_avg_us(launch, n, min_warm_s=WARM_S):
    """Average duration of `launch` over n back-to-back launches, HIP events
    on torch's current stream (the stream the library launches on), after
    at least min_warm_s seconds of the same launches."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    time_steps(launch, 0, 1, min_warm_s)
    e0.record(s)
    for i in range(n):
        launch(i)
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def cpu_baseline(host_w, act_bits, M, rows_per_shape):
    """The CPU oracle on a bounded sample of the same M = 1024 step: every
    activation tensor quantized in full, `rows_per_shape` output rows of each
    linear computed; time scaled to all M rows (the quantization is counted
    once, the dot products M / rows times)."""
    import oracle
    t_quant = t_dot = 0.0
    flops = 0
    rows = np.linspace(0, M - 1, rows_per_shape).astype(np.int64)
    for (N, K), wbits, abits in zip(SHAPES, host_w, act_bits):
        wq, sw = oracle.quant_per_tensor(oracle.decode_input(wbits, "bf16"))  # offline, untimed
        t0 = time.perf_counter()
        aq, sa = oracle.quant_per_tensor(oracle.decode_input(abits, "bf16"))
        t1 = time.perf_counter()
        oracle.fp8_linear(aq, sa, wq, sw, rows=rows)
        t2 = time.perf_counter()
        t_quant += t1 - t0
        t_dot += t2 - t1
        flops += 2 * M * N * K
    est = t_quant + t_dot * (M / rows_per_shape)
    return {"value": round(flops / est / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle",
            "sample": f"all activations quantized; {rows_per_shape} of {M} output rows per linear "
                      f"computed ({t_quant + t_dot:.1f} s), dot-product time scaled to {M} rows"}


def f16_bits_to_f32(bits):
    return bits.view(np.float16).astype(np.float32)


def rotation(pw, bql, nbytes):
    """Device copies of a packed weight, enough that a pass over them moves
    more than ROTATE_BYTES."""
    n = max(2, -(-ROTATE_BYTES // nbytes))
    return [bql.PackedWeight(pw.packed.clone(), pw.scales.clone(), pw.N, pw.K, pw.fmt) for _ in range(n)]


def steps_per_graph(M, steps):
    """Steps per captured graph: SMALL_STEPS_PER_GRAPH for the small-M
    steps; otherwise the largest of 4, 2, 1 that divides the timed step count
    (so exactly that many steps are timed).  Consecutive replays of a graph
    leave a gap of a few microseconds on the device: at one step per graph
    the M = 1024 step measured 1.2 % slower than at four, a 20-30 us call
    10-15 % slower."""
    if M <= 16:
        return SMALL_STEPS_PER_GRAPH
    return next(g for g in (4, 2, 1) if steps % g == 0)


def timed_graphs(step, nslots, steps, warmup, per_graph=1, min_warm_s=ROW_WARM_S):
    return graph_step_time(step, nslots, steps, warmup, per_graph, min_warm_s)


def bench_w8a16(bql, dev, steps, warmup):
    """Weight-only fp8 decode GEMV: M in {1, 8}, K = N = 4096, E4M3 weight
    with per-channel fp16 scales, fp16 activations and output."""
    N = K = 4096
    g = wl.rng(2, 0)
    bits = wl.weight(g, N, K, "f16")
    sbits = wl.w8a16_channel_scales(g, f16_bits_to_f32(bits))
    w = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.float16)
    sc = torch.from_numpy(sbits.view(np.int16)).to(dev).view(torch.float16)
    rot = rotation(bql.prepack_weight(w, "fp8_channel", scales=sc), bql, N * K)
    out = {"workload": "W8A16 decode GEMV, K=N=4096, E4M3 weight with per-channel fp16 scales "
                       "u*amax_n/448 (u ~ U[0.5,2]), fp16 A N(0,1) and fp16 out",
           "weight_rotation_copies": len(rot)}
    for M in (1, 8):
        a = torch.from_numpy(wl.activation(wl.rng(2, M, 3), M, K, "f16").view(np.int16)).to(dev).view(torch.float16)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = torch.empty(max(256, bql.lib().bql_w8a16_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=dev)
        sec = timed_graphs(lambda i: bql.w8a16_linear(a, rot[i % len(rot)], out=y, ws=ws), len(rot), steps, warmup,
                           per_graph=SMALL_STEPS_PER_GRAPH * 2)
        byts = N * K + 2 * N + 2 * M * K + 2 * M * N
        gbs = byts / sec / 1e9
        out[f"M{M}"] = {"value": round(gbs, 1), "unit": "GB/s", "us_per_call": round(sec * 1e6, 2),
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    return out


def bench_w4a8(bql, dev, steps, warmup):
    """W4A8 per-channel integer linear over K = N in {4096, 5120, 6656, 8192}:
    int8 per-token activations (quantized before the timed region), int4
    weights with fp16 channel scales, int32 accumulation, fp16 out.  One step
    runs the four linears."""
    shapes = wl.CFG5_KN
    rots = []
    for idx, n in enumerate(shapes):
        g = wl.rng(5, idx, 1)
        w4 = wl.int4_weight(g, n, n)
        sbits = wl.w4a8_channel_scales(g, n)
        wpk = torch.from_numpy(wl.pack_int4(w4).reshape(n, n // 2)).to(dev)
        sc = torch.from_numpy(sbits.view(np.int16)).to(dev).view(torch.float16)
        rots.append(rotation(bql.prepack_weight(wpk, "int4_channel", scales=sc), bql, n * n // 2))
    nslots = max(len(r) for r in rots)
    out = {"workload": "W4A8 per-channel integer linears K=N in {4096,5120,6656,8192}: int4 weights "
                       "U{-8..7} with fp16 channel scales U[0.5,2]*2^-8, int8 per-token activations "
                       "from fp16 N(0,1), int32 accumulation, fp16 out",
           "weight_rotation_copies": [len(r) for r in rots]}
    for M in (1024, 1):
        aqs, sas, ys, wss = [], [], [], []
        for idx, n in enumerate(shapes):
            a = torch.from_numpy(wl.activation(wl.rng(5, idx, M, 3), M, n, "f16").view(np.int16)).to(dev)
            aq, sa = bql.int8_quantize_per_token(a.view(torch.float16))
            aqs.append(aq)
            sas.append(sa)
            ys.append(torch.empty((M, n), dtype=torch.float16, device=dev))
            wss.append(torch.empty(max(256, bql.lib().bql_w4a8_linear_workspace_size(M, n, n)),
                                   dtype=torch.uint8, device=dev))

        def step(i):
            for j in range(len(shapes)):
                r = rots[j]
                bql.w4a8_linear(aqs[j], sas[j], r[i % len(r)], out=ys[j], ws=wss[j])
        sec = timed_graphs(step, nslots, steps, warmup, per_graph=steps_per_graph(M, steps))
        ops = sum(2 * M * n * n for n in shapes)
        byts = sum(n * n // 2 + M * n + 4 * M + 2 * n + 2 * M * n for n in shapes)
        if M == 1:
            gbs = byts / sec / 1e9
            out["M1"] = {"value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(sec * 1e6, 2),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}
        else:
            tops = ops / sec / 1e12
            out[f"M{M}"] = {"value": round(tops, 1), "unit": "TOP/s", "us_per_step": round(sec * 1e6, 2),
                            "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": PEAK_I8_TOPS,
                                         "unit": "TOP/s", "frac": round(tops / PEAK_I8_TOPS, 4)}}
    return out


def bench_int4_group(bql, dev, steps, warmup, fp16_act=False):
    """Per-group int4 weights (one fp16 scale per channel and 128-k group)
    over the W4A8 shapes K = N in {4096, 5120, 6656, 8192}, with int8
    per-token activations (W4A8) or fp16 activations (weight-only W4A16):
    M = 1024 in TOP/s (TFLOP/s for fp16) and M = 1 in GB/s of algorithmic
    bytes (N*K/2 + N*K/128*4 group scales + the activations, their scales
    and the fp16 output)."""
    shapes = wl.CFG5_KN
    seed = 94 if fp16_act else 95
    rots = []
    for idx, n in enumerate(shapes):
        g = wl.rng(seed, idx, 1)
        w4 = wl.int4_weight(g, n, n)
        s = (g.uniform(0.5, 2.0, size=(n, n // 128)) * 2.0 ** -8).astype(np.float16)
        wpk = torch.from_numpy(wl.pack_int4(w4).reshape(n, n // 2)).to(dev)
        sc = torch.from_numpy(s).to(dev)
        pw = bql.prepack_weight(wpk, "int4_group", scales=sc)
        rots.append(rotation(pw, bql, n * n // 2))
    nslots = max(len(r) for r in rots)
    act = "fp16 N(0,1) activations" if fp16_act else "int8 per-token activations from fp16 N(0,1)"
    out = {"workload": f"per-group {'W4A16' if fp16_act else 'W4A8'} linears (g128) K=N in "
                       "{4096,5120,6656,8192}: int4 weights U{-8..7} with fp16 scales U[0.5,2]*2^-8 "
                       f"per channel and 128-k group, {act}, fp16 out"}
    for M in (1024, 1):
        acts, ys, wss = [], [], []
        for idx, n in enumerate(shapes):
            a = torch.from_numpy(wl.activation(wl.rng(seed, idx, M, 3), M, n, "f16").view(np.int16)).to(dev)
            acts.append(a.view(torch.float16) if fp16_act else bql.int8_quantize_per_token(a.view(torch.float16)))
            ys.append(torch.empty((M, n), dtype=torch.float16, device=dev))
            wsb = (bql.lib().bql_w4a16_linear_workspace_size(M, n, n) if fp16_act
                   else bql.lib().bql_w4a8_linear_workspace_size(M, n, n))
            wss.append(torch.empty(max(256, wsb), dtype=torch.uint8, device=dev))

        def step(i):
            for j in range(len(shapes)):
                r = rots[j]
                if fp16_act:
                    bql.w4a16_group_linear(acts[j], r[i % len(r)], out=ys[j], ws=wss[j])
                else:
                    bql.w4a8_group_linear(acts[j][0], acts[j][1], r[i % len(r)], out=ys[j], ws=wss[j])
        sec = timed_graphs(step, nslots, steps, warmup, per_graph=steps_per_graph(M, steps))
        ops = sum(2 * M * n * n for n in shapes)
        abytes = (lambda n: 2 * M * n) if fp16_act else (lambda n: M * n + 4 * M)
        byts = sum(n * n // 2 + n * (n // 128) * 4 + abytes(n) + 2 * M * n for n in shapes)
        if M == 1:
            gbs = byts / sec / 1e9
            out["M1"] = {"value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(sec * 1e6, 2),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                      "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}
        else:
            tops = ops / sec / 1e12
            peak = PEAK_F16_TFLOPS if fp16_act else PEAK_I8_TOPS
            unit = "TFLOP/s" if fp16_act else "TOP/s"
            out[f"M{M}"] = {"value": round(tops, 1), "unit": unit, "us_per_step": round(sec * 1e6, 2),
                            "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": peak,
                                         "unit": unit, "frac": round(tops / peak, 4)}}
    return out


def bench_small_n(bql, dev, steps, warmup):
    """The MoE router shape (gate_proj with 8 experts) at N = 8 < 16: M = 4096
    tokens, K = 4096, bf16 A with outlier channels, per-tensor weight, bf16
    out.  A is rotated over copies beyond twice the Infinity Cache.  GB/s of
    algorithmic bytes: end to end (dynamic quantization included: A read as
    bf16) and the GEMM alone on pre-quantized E4M3 A."""
    M, N, K = 4096, 8, 4096
    g = wl.rng(96, 9)
    wb = wl.weight(g, N, K, "bf16")
    pw = bql.prepack_weight(torch.from_numpy(wb.view(np.int16)).to(dev).view(torch.bfloat16),
                            "fp8_tensor")
    a0 = torch.from_numpy(wl.activation(g, M, K, "bf16", "channels").view(np.int16)).to(dev)
    copies = max(2, -(-ROTATE_BYTES // (2 * M * K)))
    xs = [a0.view(torch.bfloat16).clone() for _ in range(copies)]
    pre = [bql.quantize_dynamic(x) for x in xs]
    pre = [(q.view(torch.float8_e4m3fn), sc) for q, sc in pre]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8, device=dev)

    def e2e(i):
        bql.fp8_linear(xs[i % copies], pw, out_dtype=torch.bfloat16, out=y, ws=ws)

    def gemm(i):
        q, sc = pre[i % copies]
        bql.fp8_linear(q, pw, a_scale=sc, out_dtype=torch.bfloat16, out=y, ws=ws)
    out = {"workload": "MoE router fp8 linear at N = 8 experts (no padding of N in memory): "
                       "M = 4096 tokens, K = 4096, bf16 A N(0,1) with 1% outlier channels x20, "
                       "per-tensor E4M3 weight, bf16 out"}
    for tag, fn, byts in (("end_to_end", e2e, 2 * M * K + N * K + 2 * M * N + 8),
                          ("gemm_only", gemm, M * K + N * K + 2 * M * N + 8)):
        sec = timed_graphs(fn, copies, steps, warmup, per_graph=SMALL_STEPS_PER_GRAPH)
        gbs = byts / sec / 1e9
        out[tag] = {"value": round(gbs, 1), "unit": "GB/s", "us_per_call": round(sec * 1e6, 2),
                    "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    return out


def bench_rmsnorm_quant(bql, dev, steps, warmup):
    """RMSNorm fused with the activation quantizers: per-token int8 at the
    W4A8 activation shapes (M = 1024, K in {4096, 5120, 6656, 8192}, fp16)
    and per-tensor E4M3 at the Llama hidden sizes (M = 1024, K = 4096 and
    M = 4096, K = 8192, bf16 with outlier channels).  Inputs are rotated over
    copies beyond twice the Infinity Cache.  GB/s of algorithmic bytes: x
    read once, g, the codes and the scales written once."""
    out = {"workload": "RMSNorm (gain U[0.5,1.5], eps 1e-5) fused with per-token int8 (W4A8 "
                       "activations, fp16 N(0,1), M=1024, K in {4096,5120,6656,8192}) and with "
                       "per-tensor E4M3 (bf16 N(0,1) with 1% outlier channels x20; M=1024 K=4096, "
                       "M=4096 K=8192)"}

    def inputs(M, K, dtype, outliers, idx):
        g = wl.rng(98, idx, M, K)
        xb = wl.activation(g, M, K, dtype, outliers)
        gb = wl.norm_weight(g, K, dtype)
        tdt = torch.float16 if dtype == "f16" else torch.bfloat16
        x = torch.from_numpy(xb.view(np.int16)).to(dev).view(tdt)
        gw = torch.from_numpy(gb.view(np.int16)).to(dev).view(tdt)
        copies = max(2, -(-ROTATE_BYTES // (2 * M * K)))
        return [x.clone() for _ in range(copies)], gw

    # per-token int8, the four W4A8 activation shapes as one step
    M = 1024
    xs, gs, qs, ss = [], [], [], []
    for idx, K in enumerate(wl.CFG5_KN):
        x, gw = inputs(M, K, "f16", "none", idx)
        xs.append(x)
        gs.append(gw)
        qs.append(torch.empty((M, K), dtype=torch.int8, device=dev))
        ss.append(torch.empty(M, dtype=torch.float32, device=dev))
    L = bql.lib()

    def step8(i):
        for j, K in enumerate(wl.CFG5_KN):
            x = xs[j][i % len(xs[j])]
            bql._check("bql_rmsnorm_int8_quantize_per_token",
                       L.bql_rmsnorm_int8_quantize_per_token(
                           bql._ptr(x), bql._ptr(gs[j]), bql.F16, M, K, 1e-5, bql._ptr(qs[j]),
                           bql._ptr(ss[j]), None, bql._stream(dev)))
    nslots = max(len(x) for x in xs)
    sec = timed_graphs(step8, nslots, steps, warmup, per_graph=SMALL_STEPS_PER_GRAPH)
    byts = sum(2 * M * K + 2 * K + M * K + 4 * M for K in wl.CFG5_KN)
    gbs = byts / sec / 1e9
    out["int8_per_token_M1024"] = {
        "value": round(gbs, 1), "unit": "GB/s", "us_per_step": round(sec * 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4)}}

    # per-tensor E4M3 (two launches: row statistics, then the cast)
    for idx, (M, K) in enumerate([(1024, 4096), (4096, 8192)]):
        x, gw = inputs(M, K, "bf16", "channels", 10 + idx)
        q = torch.empty((M, K), dtype=torch.uint8, device=dev)
        sc = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(max(256, L.bql_rmsnorm_quantize_workspace_size(M)), dtype=torch.uint8,
                         device=dev)

        def stepf(i, x=x, gw=gw, q=q, sc=sc, ws=ws, M=M, K=K):
            xi = x[i % len(x)]
            bql._check("bql_rmsnorm_fp8_quantize_dynamic",
                       L.bql_rmsnorm_fp8_quantize_dynamic(
                           bql._ptr(xi), bql._ptr(gw), bql.BF16, M, K, 1e-5, bql._ptr(q),
                           bql._ptr(sc), None, bql._ptr(ws), ws.numel(), bql._stream(dev)))
        sec = timed_graphs(stepf, len(x), steps, warmup, per_graph=SMALL_STEPS_PER_GRAPH)
        byts = 2 * M * K + 2 * K + M * K + 4
        gbs = byts / sec / 1e9
        out[f"fp8_per_tensor_M{M}_K{K}"] = {
            "value": round(gbs, 1), "unit": "GB/s", "us_per_call": round(sec * 1e6, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def roof(bound, achieved, unit):
    peak = {"hbm": PEAK_HBM_GBS, "mfma_fp8": PEAK_FP8_TFLOPS, "mfma_i8": PEAK_I8_TOPS}[bound]
    return {"bound": "hbm" if bound == "hbm" else "mfma", "achieved": round(achieved, 1), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4)}


def oracle_rows(M, count):
    """Seeded output rows the oracle computes for a row's CPU time (first and
    last included); the dot-product time is scaled by M / count."""
    if M <= count:
        return np.arange(M, dtype=np.int64)
    g = np.random.Generator(np.random.PCG64(77 + M))
    r = set(g.choice(M, size=count - 2, replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(r), dtype=np.int64)


def bench_configs(bql, dev, steps, warmup, oracle_sample_rows):
    """One row per (configuration, shape, M, output): the end-to-end call
    through the C ABI, timed as the other legs (HIP graphs of back-to-back
    calls, weights rotated past the Infinity Cache where the row streams
    them), its rate against the roofline that bounds it (HBM at M <= 128,
    the matrix cores above), and the CPU oracle's time for the same call on
    a bounded sample (every activation quantized in full; `rows` output
    rows with all N columns computed, scaled to M rows; weights quantized
    offline, untimed on both sides)."""
    import oracle
    out = []

    def time_call(fn, nslots, M):
        return timed_graphs(fn, nslots, steps, warmup, per_graph=steps_per_graph(M, steps))

    def act_copies(t, nbytes):
        n = max(1, -(-ROTATE_BYTES // nbytes)) if nbytes >= 16 * 2 ** 20 else 1
        return [t] + [t.clone() for _ in range(n - 1)]

    def fp8_config(cfg, name, shapes, Ms, dtype, outliers, per_channel, out_kinds):
        tdt = torch.float16 if dtype == "f16" else torch.bfloat16
        for idx, (N, K) in enumerate(shapes):
            wbits = wl.weight(wl.rng(cfg, idx, 1), N, K, dtype)
            w = torch.from_numpy(wbits.view(np.int16)).to(dev).view(tdt)
            pw = bql.prepack_weight(w, "fp8_channel" if per_channel else "fp8_tensor")
            del w
            wrot = rotation(pw, bql, N * K) if min(Ms) <= 128 else [pw]
            wf = oracle.decode_input(wbits, dtype)
            wq, sw = oracle.quant_per_row(wf) if per_channel else oracle.quant_per_tensor(wf)
            sw = np.atleast_1d(np.asarray(sw, dtype=np.float32))
            del wf
            for M in Ms:
                abits = wl.activation(wl.rng(cfg, idx, M, 3), M, K, dtype, outliers)
                a0 = torch.from_numpy(abits.view(np.int16)).to(dev).view(tdt)
                acopies = act_copies(a0, 2 * M * K)
                ws = torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8,
                                 device=dev)
                # CPU oracle on a bounded sample of the same call
                # the Llama-70B prefill at M = 4096: 256 seeded rows
                rows = oracle_rows(M, 256 if M >= 4096 else oracle_sample_rows)
                t0 = time.perf_counter()
                aq, sa = oracle.quant_per_tensor(oracle.decode_input(abits, dtype))
                t1 = time.perf_counter()
                oracle.fp8_linear(aq, sa, wq, sw, rows=rows)
                t2 = time.perf_counter()
                oracle_s = (t1 - t0) + (t2 - t1) * M / len(rows)
                ybf = torch.empty((M, N), dtype=tdt, device=dev)
                bql.fp8_linear(a0, pw, out=ybf, out_dtype=tdt, ws=ws)
                torch.cuda.synchronize()
                for kind in out_kinds:
                    if kind == "fp8":
                        # output_scale of a calibrating quantizer: max|Y| / 448
                        osc = (ybf.float().abs().max() / 448.0).reshape(1).contiguous()
                        y = torch.empty((M, N), dtype=torch.uint8, device=dev)
                        fn = (lambda i, y=y, osc=osc: bql.fp8_linear(
                            acopies[i % len(acopies)], wrot[i % len(wrot)], out=y,
                            out_dtype=torch.float8_e4m3fn, output_scale=osc, ws=ws))
                        ysz = 1
                    else:
                        y = ybf
                        fn = (lambda i, y=y: bql.fp8_linear(acopies[i % len(acopies)], wrot[i % len(wrot)],
                                                            out=y, out_dtype=tdt, ws=ws))
                        ysz = 2
                    sec = time_call(fn, max(len(acopies), len(wrot)), M)
                    byts = N * K + 2 * M * K + ysz * M * N + 4 * (N if per_channel else 1) + 4
                    flops = 2 * M * N * K
                    row = {"config": name, "N": N, "K": K, "M": M, "out": kind if kind == "fp8" else dtype,
                           "us": round(sec * 1e6, 2)}
                    if M <= 128:
                        row["GBs"] = round(byts / sec / 1e9, 1)
                        row["roofline"] = roof("hbm", byts / sec / 1e9, "GB/s")
                    else:
                        row["TFLOPs"] = round(flops / sec / 1e12, 1)
                        row["roofline"] = roof("mfma_fp8", flops / sec / 1e12, "TFLOP/s")
                    row["oracle_s"] = round(oracle_s, 3)
                    row["oracle_sample"] = (f"A quantized in full; {len(rows)} of {M} rows x all {N} "
                                            f"columns, scaled to {M} rows" if len(rows) < M else "whole call")
                    out.append(row)
                    log(f"  {name} N={N} K={K} M={M} {row['out']}: {row['us']} us")
                del acopies, a0, ybf, ws
            del wrot, pw, wq

    log("config rows: fp8 linears ...")
    fp8_config(1, "cfg1", [(1024, 1024)], [16], "f16", "entries", False, ["f16"])
    fp8_config(3, "cfg3", wl.CFG3_SHAPES, wl.CFG3_M, "bf16", "channels", False, ["bf16"])
    fp8_config(4, "cfg4", wl.CFG4_SHAPES, wl.CFG4_M, "bf16", "channels", True, ["bf16", "fp8"])

    log("config rows: W8A16 ...")
    N = K = 4096
    g = wl.rng(2, 0)
    wbits = wl.weight(g, N, K, "f16")
    sbits = wl.w8a16_channel_scales(g, f16_bits_to_f32(wbits))
    pw = bql.prepack_weight(torch.from_numpy(wbits.view(np.int16)).to(dev).view(torch.float16),
                            "fp8_channel",
                            scales=torch.from_numpy(sbits.view(np.int16)).to(dev).view(torch.float16))
    wrot = rotation(pw, bql, N * K)
    s32 = oracle.decode_input(sbits, "f16")
    wq = oracle.quant_with_scales(oracle.decode_input(wbits, "f16"), s32)
    for M in (1, 8):
        abits = wl.activation(wl.rng(2, M, 3), M, K, "f16")
        a = torch.from_numpy(abits.view(np.int16)).to(dev).view(torch.float16)
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ws = torch.empty(max(256, bql.lib().bql_w8a16_linear_workspace_size(M, N, K)), dtype=torch.uint8,
                         device=dev)
        sec = time_call(lambda i: bql.w8a16_linear(a, wrot[i % len(wrot)], out=y, ws=ws), len(wrot), M)
        t0 = time.perf_counter()
        oracle.w8a16_linear(oracle.decode_input(abits, "f16"), wq, s32)
        oracle_s = time.perf_counter() - t0
        byts = N * K + 2 * N + 2 * M * K + 2 * M * N
        out.append({"config": "cfg2", "N": N, "K": K, "M": M, "out": "f16", "us": round(sec * 1e6, 2),
                    "GBs": round(byts / sec / 1e9, 1), "roofline": roof("hbm", byts / sec / 1e9, "GB/s"),
                    "oracle_s": round(oracle_s, 3), "oracle_sample": "whole call"})
    del wrot, pw

    log("config rows: W4A8 ...")
    for idx, n in enumerate(wl.CFG5_KN):
        g = wl.rng(5, idx, 1)
        w4 = wl.int4_weight(g, n, n)
        sbits = wl.w4a8_channel_scales(g, n)
        pw = bql.prepack_weight(torch.from_numpy(wl.pack_int4(w4).reshape(n, n // 2)).to(dev), "int4_channel",
                                scales=torch.from_numpy(sbits.view(np.int16)).to(dev).view(torch.float16))
        wrot = rotation(pw, bql, n * n // 2)
        s32 = oracle.decode_input(sbits, "f16")
        for M in wl.CFG5_M:
            abits = wl.activation(wl.rng(5, idx, M, 3), M, n, "f16")
            aq, sa = bql.int8_quantize_per_token(torch.from_numpy(abits.view(np.int16)).to(dev).view(torch.float16))
            y = torch.empty((M, n), dtype=torch.float16, device=dev)
            ws = torch.empty(max(256, bql.lib().bql_w4a8_linear_workspace_size(M, n, n)), dtype=torch.uint8,
                             device=dev)
            sec = time_call(lambda i: bql.w4a8_linear(aq, sa, wrot[i % len(wrot)], out=y, ws=ws), len(wrot), M)
            rows = oracle_rows(M, oracle_sample_rows)
            t0 = time.perf_counter()
            aq_ref, sa_ref = oracle.int8_quant_per_token(oracle.decode_input(abits, "f16"))
            t1 = time.perf_counter()
            acc = oracle.w4a8_acc(aq_ref, w4, rows=rows)
            oracle.w4a8_linear(acc, sa_ref, s32, rows=rows)
            t2 = time.perf_counter()
            oracle_s = (t1 - t0) + (t2 - t1) * M / len(rows)
            ops = 2 * M * n * n
            byts = n * n // 2 + M * n + 4 * M + 2 * n + 2 * M * n
            row = {"config": "cfg5", "N": n, "K": n, "M": M, "out": "f16", "us": round(sec * 1e6, 2)}
            if M <= 16:
                row["GBs"] = round(byts / sec / 1e9, 1)
                row["roofline"] = roof("hbm", byts / sec / 1e9, "GB/s")
            else:
                row["TOPs"] = round(ops / sec / 1e12, 1)
                row["roofline"] = roof("mfma_i8", ops / sec / 1e12, "TOP/s")
            row["oracle_s"] = round(oracle_s, 3)
            row["oracle_sample"] = (f"A quantized in full; {len(rows)} of {M} rows x all {n} columns, "
                                    f"scaled to {M} rows" if len(rows) < M else "whole call")
            out.append(row)
        del wrot, pw
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-config-rows", action="store_true",
                    help="skip the per-configuration rows (every shape and M of the five workloads)")
    ap.add_argument("--oracle-sample-rows", type=int, default=16,
                    help="output rows the CPU oracle computes per configuration row")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the per-configuration rows")
    ap.add_argument("--step-only", action="store_true",
                    help="only the M=1024 step (for a rocprofv3 run of its kernels)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the dominant-kernel launches (for a rocprofv3 run of that kernel)")
    ap.add_argument("--rmsnorm-only", action="store_true",
                    help="only the fused RMSNorm + quantization leg (for a rocprofv3 run of it)")
    ap.add_argument("--w4a8-only", action="store_true",
                    help="only the per-channel W4A8 leg (for a rocprofv3 run of it)")
    ap.add_argument("--w4a8-group-only", action="store_true",
                    help="only the per-group W4A8 and W4A16 legs (for a rocprofv3 run of them)")
    ap.add_argument("--small-n-only", action="store_true",
                    help="only the small-N (MoE router) leg (for a rocprofv3 run of it)")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="write the matrix-core counter summary from one rocprofv3 --pmc run")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc output folders")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import bit_quantized_linear_amd as bql
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bql.lib()
    if args.rmsnorm_only:
        print(json.dumps({"rmsnorm_quant": bench_rmsnorm_quant(bql, dev, args.steps, args.warmup)}),
              flush=True)
        return
    if args.w4a8_only:
        print(json.dumps({"w4a8": bench_w4a8(bql, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.w4a8_group_only:
        print(json.dumps({"w4a8_group": bench_int4_group(bql, dev, args.steps, args.warmup),
                          "w4a16_group": bench_int4_group(bql, dev, args.steps, args.warmup, True)}),
              flush=True)
        return
    if args.small_n_only:
        print(json.dumps({"small_n": bench_small_n(bql, dev, args.steps, args.warmup)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"configs": bench_configs(bql, dev, args.steps, args.warmup,
                                                   args.oracle_sample_rows)}), flush=True)
        return

    log("generating weights ...")
    host_w, rot = build_weights(bql, dev)
    nrot = len(rot)

    def run_pass(M, fast=False, prequant=False, timed=True, static=False):
        # activations rotate too where a set is large (M = 1024: 54.5 MB)
        abits, asets = build_activations(M, dev, rotate=M > 16)
        a = asets[0]
        nslots = max(nrot, len(asets))
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for N, K in SHAPES]
        wss = [torch.empty(max(256, bql.fp8_linear_workspace_size(M, N, K)), dtype=torch.uint8,
                           device=dev) for N, K in SHAPES]
        pre = None
        if prequant:
            pre = [[bql.quantize_dynamic(x) for x in aset] for aset in asets]
            pre = [[(q.view(torch.float8_e4m3fn), sc) for q, sc in ps] for ps in pre]
        if static:  # a calibrated input_scale per linear (here the tensor's own amax / 448)
            st = [bql.quantize_dynamic(x)[1] for x in a]

        def step(i):
            ws_set = rot[i % nrot]
            ai = i % len(asets)
            for j in range(len(SHAPES)):
                if static:
                    bql.fp8_linear_static(asets[ai][j], ws_set[j], st[j], out_dtype=torch.bfloat16,
                                          out=outs[j], ws=wss[j], fast_accum=fast)
                elif prequant:
                    q, sc = pre[ai][j]
                    bql.fp8_linear(q, ws_set[j], a_scale=sc, out_dtype=torch.bfloat16,
                                   out=outs[j], ws=wss[j], fast_accum=fast)
                else:
                    bql.fp8_linear(asets[ai][j], ws_set[j], out_dtype=torch.bfloat16, out=outs[j],
                                   ws=wss[j], fast_accum=fast)
        sec = sec_eager = float("nan")
        if timed:
            sec_eager = time_steps(step, args.steps, args.warmup, WARM_S)
            sec = graph_step_time(step, nslots, args.steps, args.warmup,
                                  per_graph=steps_per_graph(M, args.steps))
        flops = sum(2 * M * N * K for N, K in SHAPES)
        byts = sum(algorithmic_bytes(M, N, K) for N, K in SHAPES)
        return abits, pre, outs, wss, (sec, sec_eager), flops, byts, len(asets)

    # ---- headline: M = 1024, exact accumulation, dynamic activation quant
    M = 1024
    if not args.roofline_only:
        log("timing M=1024 exact ...")
        abits, _, _, _, (sec, sec_eager), flops, byts, a_copies = run_pass(M)
        value = flops / sec / 1e12
        if args.step_only:
            print(json.dumps({"value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(sec * 1e3, 4),
                              "eager_value": round(flops / sec_eager / 1e12, 2)}), flush=True)
            return

    # dominant kernel: the tiled GEMM of the (28672, 4096) linear, on
    # pre-quantized A packed beforehand, so that each call is that one kernel
    def kernel_roofline(fast):
        _, pre, outs, wss, _, _, _, _ = run_pass(M, fast=fast, prequant=True, timed=False)
        j = 2
        N, K = SHAPES[j]
        packed = [(bql.pack_activations(ps[j][0]), ps[j][1]) for ps in pre]

        def launch(i):
            pa, sc = packed[i % len(packed)]
            bql.fp8_linear(pa, rot[i % nrot][j], a_scale=sc, out_dtype=torch.bfloat16,
                           out=outs[j], ws=wss[j], fast_accum=fast)
        us = event_avg_us(launch, 50)
        fl = 2 * M * N * K
        ach = fl / us / 1e6
        # the method's contraction is E4M3 x E4M3: its peak is the fp8
        # matrix-core peak; the exact mode runs it on the f16 matrix cores,
        # whose peak (half of it) is given beside
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_FP8_TFLOPS, 4),
                "traffic": read_traffic("fast_hbm_bytes_per_launch" if fast else "exact_hbm_bytes_per_launch"),
                **({} if fast else {"frac_of_f16_mfma_peak": round(ach / PEAK_F16_TFLOPS, 4)}),
                "algorithmic_bytes_per_launch": algorithmic_bytes_gemm(M, N, K),
                "kernel": (f"gemm_kernel<V_FP8,256,256,4,4,2> M={M} N={N} K={K}" if fast else
                           f"gemm_exact_kernel<7, 2> (256x224 blocks, four waves) M={M} N={N} K={K}"),
                "avg_launch_us": round(us, 2), "flops_per_launch": fl}
    log("kernel rooflines ...")
    roof = kernel_roofline(False)
    roof_fast = kernel_roofline(True)
    if args.roofline_only:
        # plain device copy of known size: the calibration for HBM byte counters
        src = torch.empty(CALIBRATION_COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"roofline": roof, "fast_accum_roofline": roof_fast,
                          "calibration_copy_bytes": CALIBRATION_COPY_BYTES}), flush=True)
        return

    # fast accumulation (fp8 matrix cores' own accumulation), same step
    log("timing M=1024 fast ...")
    _, _, _, _, (sec_f, sec_f_eager), _, _, _ = run_pass(M, fast=True)

    # static activation scale (checkpoint input_scale): no amax pass
    log("timing M=1024 static scale ...")
    _, _, _, _, (sec_s, _), _, _, _ = run_pass(M, static=True)

    # ---- M = 1 decode pass
    log("timing M=1 ...")
    _, _, _, _, (sec1, sec1_eager), flops1, byts1, _ = run_pass(1)
    _, _, _, _, (sec1p, _), _, _, _ = run_pass(1, prequant=True)

    log("timing W8A16 decode ...")
    w8a16 = bench_w8a16(bql, dev, args.steps, args.warmup)
    log("timing W4A8 ...")
    w4a8 = bench_w4a8(bql, dev, args.steps, args.warmup)
    log("timing RMSNorm + quantization ...")
    norm_quant = bench_rmsnorm_quant(bql, dev, args.steps, args.warmup)
    log("timing small N ...")
    small_n = bench_small_n(bql, dev, args.steps, args.warmup)
    log("timing W4A8 per group ...")
    w4a8_group = bench_int4_group(bql, dev, args.steps, args.warmup)
    log("timing W4A16 per group ...")
    w4a16_group = bench_int4_group(bql, dev, args.steps, args.warmup, fp16_act=True)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3-8B-shaped W8A8 fp8 linears (N,K)=(6144,4096),(4096,4096),"
                        "(28672,4096),(4096,14336); bf16 A N(0,1) with 1% outlier channels x20, "
                        "dynamic per-tensor E4M3 activation scale, per-tensor E4M3 weights, "
                        "exact fp32 accumulation, bf16 out",
            "M": M, "accum": "exact", "weight_rotation_copies": nrot,
            "activation_rotation_copies": a_copies,
            "timing": f"HIP graph replay of whole steps, {steps_per_graph(M, args.steps)} consecutive "
                      f"steps per graph at M=1024 and {SMALL_STEPS_PER_GRAPH} at M=1 (each on its own "
                      "weight copy); eager-launch rates under 'eager'",
        },
        "eager": {"value": round(flops / sec_eager / 1e12, 2), "unit": "TFLOP/s",
                  "m1_GBs": round(byts1 / sec1_eager / 1e9, 1),
                  "note": "same steps launched from Python one call at a time"},
        "m1": {
            "value": round(byts1 / sec1 / 1e9, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(byts1 / sec1 / 1e9 / PEAK_HBM_GBS, 4),
            "ms_per_pass": round(sec1 * 1e3, 4),
            "gemm_only_GBs": round(byts1 / sec1p / 1e9, 1),
            "note": "M=1, four linears, dynamic quant included (one fused kernel per linear); "
                    "gemm_only = pre-quantized E4M3 A (the streaming kernel alone)",
        },
        "fast_accum": {
            "value": round(flops / sec_f / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(sec_f * 1e3, 4), "roofline": roof_fast,
        },
        "roofline": roof,
        "static_scale": {
            "value": round(flops / sec_s / 1e12, 2), "unit": "TFLOP/s",
            "ms_per_step": round(sec_s * 1e3, 4),
            "note": "same M=1024 step with a given per-tensor activation scale "
                    "(bql_fp8_linear_static: one cast launch per linear, no amax pass)"},
        "w8a16": w8a16,
        "w4a8": w4a8,
        "rmsnorm_quant": norm_quant,
        "small_n": small_n,
        "w4a8_group": w4a8_group,
        "w4a16_group": w4a16_group,
    }
    if not args.no_config_rows:
        out["configs"] = bench_configs(bql, dev, args.steps, args.warmup, args.oracle_sample_rows)
    out["host"] = {"cpu_model": cpu_model(), "oracle_threads": None}
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        out["cpu_baseline"] = cpu_baseline(host_w, abits, M, args.cpu_rows)
        out["cpu_baseline"]["cpu_model"] = out["host"]["cpu_model"]
    import oracle
    out["host"]["oracle_threads"] = oracle.threads()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
