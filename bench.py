"""Benchmark of the BitStack residual-block linear layer on one MI355X.

Headline (printed as one JSON line): HBM GB/s of single-token decode through the
seven linears of a Llama-3-8B-shaped decoder layer (q/o 4096x4096, k/v 1024x4096,
gate/up 14336x4096, down 4096x14336), each held as n = 8 residual blocks with k = 16
(synthetic Bernoulli(0.5) signs, U and V = |N(0,1)| * 0.05 in fp16, x ~ N(0,1) fp16).
One step is one grouped launch over the layer's seven linears.  Four distinct copies
of the layer are resident (about 0.96 GB) and the steps rotate over them, so the
256 MB last-level cache cannot serve the reads.  Bytes are the algorithmic bytes of
the loaded blocks, n * (m d / 8 + 2 k (m + d)) per weight, counted once.

Also reported: the same decode with every linear held as n = 8 equal-size vanilla-SVD
blocks (rank k' = 16 + m d / (16 (m + d)), fp16 factors, no signs: the "w/o AVD"
baseline, the same bytes per block); prefill at M = 2048 tokens through one such layer, on the tile path
(W_hat rebuilt per tile, then a GEMM; executed MFMA work (2 k n G + 2 M) m d per weight
with G = ceil(M / 512) token groups) and on the factored path (the S Z contraction,
2 n k M m d per weight); the decode kernel's roofline from per-launch HIP events; and
the CPU oracle (fp64 reconstruct-then-matmul) on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]
                       [--prefill-steps P] [--no-cpu] [--no-prefill] [--sweep] [--llama70b]
                       [--per-weight] [--calibrate-copy] [--load] [--cpu-layers C]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "BitStack linear HBM GB/s + MFMA TFLOP/s (% of peak), M=1 decode & M=2048 prefill"
HBM_PEAK_GBS = 8000.0
FP16_MFMA_PEAK_TFLOPS = 2516.6  # 256 CU x 4096 flop/clk x 2.4 GHz, dense
K_RANK = 16


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def block_bytes(m: int, d: int) -> int:
    return m * d // 8 + 2 * K_RANK * (m + d)


class Layers:
    """One bitstack stack holding `layers` copies of a decoder layer's linears.

    Every layer gets its own device blocks.  With `shared_sources` the host blocks of a
    weight shape are drawn once (as many as the largest count needs) and every layer loads
    its own count of them into its own slots, so large stacks are built without holding
    every layer's blocks on the host; layers are then loaded `batch` at a time."""

    def __init__(self, bsl, torch, shapes, counts, layers, seed, M, path=None, decode=None, shared_sources=False,
                 batch=8):
        self.bsl, self.torch = bsl, torch
        self.shapes = shapes
        self.layers = layers
        self.per = len(shapes)
        ms = [m for _ in range(layers) for (_, m, _) in shapes]
        ds = [d for _ in range(layers) for (_, _, d) in shapes]
        self.h = bsl.bsl_init(0, ms, ds, 16, 16, 0)
        if path is not None:
            bsl.bsl_set_path(self.h, path)
        if decode is not None:
            bsl.bsl_set_decode(self.h, decode)
        self.counts = [int(counts[l][j]) for l in range(layers) for j in range(self.per)]
        loaded = [0] * (layers * self.per)
        if shared_sources:
            nmax = [max(int(counts[l][j]) for l in range(layers)) for j in range(self.per)]
            src = [synth.synthetic_blocks(seed, m, d, nmax[j], 16, 0, j) for j, (_, m, d) in enumerate(shapes)]
            for l0 in range(0, layers, batch):
                for l in range(l0, min(layers, l0 + batch)):
                    for j in range(self.per):
                        bsl.bsl_set_source(self.h, l * self.per + j, src[j])
                        loaded[l * self.per + j] = self.counts[l * self.per + j]
                bsl.bsl_load_blocks(self.h, loaded, 0)
                log(f"  loaded layers {l0 + 1}..{min(layers, l0 + batch)}/{layers}")
        else:
            for l in range(layers):
                for j, (_, m, d) in enumerate(shapes):
                    n = self.counts[l * self.per + j]
                    blocks = synth.synthetic_blocks(seed, m, d, n, 16, l, j)
                    bsl.bsl_set_source(self.h, l * self.per + j, blocks)
                log(f"  generated layer {l + 1}/{layers}")
            bsl.bsl_load_blocks(self.h, self.counts, 0)
        # the host copies are no longer needed once loaded
        for key in [k for k in bsl._sources if k[0] == self.h]:
            del bsl._sources[key]
        self.x, self.y = [], []
        for l in range(layers):
            xs, ys = [], []
            for j, (_, m, d) in enumerate(shapes):
                x = synth.activations(seed + 1, M, d, l, j)
                xs.append(torch.from_numpy(x).cuda())
                ys.append(torch.empty((M, m), dtype=torch.float16, device="cuda"))
            self.x.append(xs)
            self.y.append(ys)
        self.M = M

    def launch(self, l: int, stream: int) -> None:
        ws = list(range(l * self.per, (l + 1) * self.per))
        self.bsl.bsl_forward_group(self.h, ws, [t.data_ptr() for t in self.x[l]], [t.data_ptr() for t in self.y[l]],
                                   self.M, False, stream)

    def bytes(self, l: int) -> int:
        return sum(self.counts[l * self.per + j] * block_bytes(m, d) for j, (_, m, d) in enumerate(self.shapes))

    def flops(self, l: int) -> int:
        """MFMA work of the factored formulation (the S Z contraction)."""
        return sum(2 * self.counts[l * self.per + j] * K_RANK * self.M * m * d for j, (_, m, d) in enumerate(self.shapes))

    def tile_flops(self, l: int) -> int:
        """MFMA work of the tile formulation: every group of up to 512 tokens rebuilds W_hat
        (K = k products, 2 k n m d) and multiplies it with its tokens (2 M m d)."""
        groups = -(-self.M // 512)
        return sum((2 * K_RANK * self.counts[l * self.per + j] * groups + 2 * self.M) * m * d
                   for j, (_, m, d) in enumerate(self.shapes))

    def product_flops(self, l: int) -> int:
        """MFMA work the product-index kernel executes: per block the K = k products
        (2 k n m d) and the sparse contraction with the tokens padded to 32 (2 * 32 n m d,
        counted as the instruction's useful work, half its dense equivalent)."""
        return sum((2 * K_RANK + 2 * 32) * self.counts[l * self.per + j] * m * d for j, (_, m, d) in enumerate(self.shapes))

    def gemm_flops(self, l: int) -> int:
        return sum(2 * self.M * m * d for (_, m, d) in self.shapes)

    def close(self):
        self.torch.cuda.synchronize()
        self.bsl.bsl_destroy(self.h)


WARM_S = 0.2  # seconds of untimed launches before a non-headline section's timing


def time_steps(torch, layers: Layers, steps: int, warmup: int, warm_s: float = 0.0):
    """Warm up, then time exactly `steps` steps (one grouped launch each) between two
    device synchronisations.  One HIP event pair on the launch stream brackets the same
    steps, so the average launch duration carries no per-launch event overhead.  With
    `warm_s`, the same launches first run for that many seconds (the sections other than
    the headline: each builds its layers on the host first, and launches that follow an
    idle GPU run slower while its clock ramps up)."""
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
    t_end, s = time.perf_counter() + warm_s, 0
    while time.perf_counter() < t_end:
        layers.launch(s % layers.layers, sp)
        s += 1
        if s % 16 == 0:
            torch.cuda.synchronize()
    for s in range(warmup):
        layers.launch(s % layers.layers, sp)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    total_bytes = total_flops = 0
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(steps):
        l = s % layers.layers
        layers.launch(l, sp)
        total_bytes += layers.bytes(l)
        total_flops += layers.flops(l)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = [e0.elapsed_time(e1) / steps]
    return wall, kern_ms, total_bytes, total_flops


def cpu_baseline(seed: int, layers: int = 4, single_layers: int = 1) -> dict:
    """The oracle, untouched, on a bounded sample of the decode workload: `layers`
    distinct 8B-shaped layers (all seven linears each) with n = 8 and M = 1, i.e.
    `layers` steps of the GPU benchmark (about 10-30 s of CPU work) with the BLAS library's
    own threads (one per host core the process may use), and `single_layers` more with
    BLAS limited to one thread."""
    import oracle

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_info = threadpool_limits = None
    host_cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1]) \
        if threadpool_info else host_cores

    def run(n_layers, tag):
        total_bytes, elapsed = 0, 0.0
        for l in range(n_layers):
            for j, (_, m, d) in enumerate(synth.LLAMA3_8B_LAYER):
                blocks = synth.synthetic_blocks(seed, m, d, 8, 16, tag, l, j)
                x = synth.activations(seed + 1, 1, d, tag, l, j)
                t0 = time.perf_counter()
                oracle.forward(x, blocks, 8)
                elapsed += time.perf_counter() - t0
                total_bytes += 8 * block_bytes(m, d)
        return total_bytes, elapsed

    tb, el = run(layers, 99)
    out = {
        "value": round(tb / el / 1e9, 4),
        "unit": "GB/s",
        "cores": int(blas_threads),
        "host_cores": int(host_cores),
        "kind": "oracle",
        "sample": f"{layers} Llama-3-8B-shaped layers (7 linears each), n=8, M=1: fp64 reconstruct-then-matmul per linear",
        "seconds": round(el, 2),
    }
    if threadpool_limits and single_layers > 0:
        with threadpool_limits(limits=1, user_api="blas"):
            tb1, el1 = run(single_layers, 98)
        out["one_thread"] = {"value": round(tb1 / el1 / 1e9, 4), "unit": "GB/s", "cores": 1, "seconds": round(el1, 2),
                             "sample": f"{single_layers} Llama-3-8B-shaped layer(s), n=8, M=1, BLAS limited to one thread"}
    return out


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_m1_kernel_llama3_8b_layer_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "bit_sign_rank_amd", "csrc", "bsl_kernels.hip")


def measured_traffic():
    """HBM bytes per decode launch from the committed counter summary (FETCH_SIZE +
    WRITE_SIZE, copy-calibrated), or None when the kernel source has changed since
    the counters were taken (the summary records the source's SHA-256)."""
    import hashlib

    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    fields = {}
    with open(TRAFFIC_SUMMARY) as f:
        for line in f:
            if ":" in line and not line.startswith(" "):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    with open(KERNEL_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest or "hbm_bytes_per_launch" not in fields:
        return None
    return int(fields["hbm_bytes_per_launch"])


PROFILE_KERNELS = (
    # (label, kernel name prefix, grid size of the profiled launch or None, algorithmic flops per launch)
    ("decode_m1_kernel (8B-shaped layer, n=8, M=1)", "void bsl::decode_m1_kernel", 256 * 1024,
     sum(2 * 8 * K_RANK * 1 * m * d for _, m, d in synth.LLAMA3_8B_LAYER)),
    ("decode_wp_kernel<8, 4> (8B-shaped layer, n=8, M=4)", "void bsl::decode_wp_kernel<8, 4>", None,
     sum(2 * 8 * K_RANK * 4 * m * d for _, m, d in synth.LLAMA3_8B_LAYER)),
    ("tile_split_kernel<8> (8B-shaped layer, n=8, M=2048)", "void bsl::tile_split_kernel<8>", None,
     sum((2 * K_RANK * 8 * 4 + 2 * 2048) * m * d for _, m, d in synth.LLAMA3_8B_LAYER)),
    ("product_kernel<2, 2> (8B-shaped layer, n=8, M=16)", "void bsl::product_kernel<2, 2>", None,
     sum((2 * K_RANK * 8 + 2 * 16 * 8) * m * d for _, m, d in synth.LLAMA3_8B_LAYER)),
)
# K = 16 rebuild MFMA work of the product-index kernel per launch of the profile set (rows and
# columns of the 8B-shaped layer are multiples of its 512-row groups and 512-column chunks)
PRODUCT_REBUILD_FLOPS = sum(2 * K_RANK * 8 * m * d for _, m, d in synth.LLAMA3_8B_LAYER)


def write_profile_summaries(trace_dir: str, sq1_dir: str, sq2_dir: str, fetch_dir: str, write_dir: str,
                            command: str, mem_dir: str | None = None) -> None:
    """Turn rocprofv3 outputs of `bench.py --profile-set` runs (one --kernel-trace --stats
    run, two --pmc passes of SQ counters, one FETCH_SIZE and one WRITE_SIZE pass, and
    optionally a pass of vector-memory-path counters) into the short text summaries kept
    under profiles/."""
    import csv
    import glob
    import hashlib
    import statistics

    def one(d, suffix):
        files = glob.glob(os.path.join(d, "*" + suffix))
        assert files, (d, suffix)
        return files[0]

    def pick(name, grid, want_name, want_grid):
        return name.startswith(want_name) and (want_grid is None or int(grid) == want_grid)

    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(KERNEL_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    cmd = command.split(";")
    # --- kernel trace: durations per (kernel, grid)
    durs = {}
    for r in csv.DictReader(open(one(trace_dir, "kernel_trace.csv"))):
        key = (r["Kernel_Name"], int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0))
        durs.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# rocprofv3 --kernel-trace --stats of bench.py --profile-set (Llama-3-8B-shaped layer, n=8, k=16):",
             "# decode M=1 (both single-token kernels), few-token M=4, product-index M=16 (against the tile path), tile-path prefill M=2048",
             f"command: {cmd[0].strip()}", f"kernel_source_sha256: {digest}", "",
             f"{'kernel':58s} {'grid':>8s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for (name, grid), v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        if not name.startswith(("void bsl::", "bsl::")):
            continue
        lines.append(f"{name[:58]:58s} {grid:8d} {len(v):6d} {statistics.mean(v):10.2f} {min(v):10.2f} {max(v):10.2f}")
    with open(os.path.join(ROOT, "profiles", "kernel_stats_llama3_8b_layer.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # --- counters: median per dispatch, per kernel of interest
    def counters(d):
        vals = {}
        for r in csv.DictReader(open(one(d, "counter_collection.csv"))):
            key = (r["Kernel_Name"], int(r["Grid_Size"]))
            e = vals.setdefault(key, {})
            e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            e.setdefault("_dur_us", {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        return vals

    med = statistics.median
    c1, c2 = counters(sq1_dir), counters(sq2_dir)
    c3 = counters(mem_dir) if mem_dir else {}
    out = ["# rocprofv3 --pmc SQ counters, two passes of bench.py --profile-set; medians per dispatch.",
           "# SQ counters are sums over the 32 shader engines (8 XCDs); the shader clock is SQ_BUSY_CYCLES / 32 over",
           "# the dispatch's duration in the counter run (dispatches run one at a time there); MFMA busy is",
           "# SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs over those cycles; MFMA flops are SQ_INSTS_VALU_MFMA_MOPS_F16 * 512",
           "# (the sparse 16x16x64 instruction counts at its dense-equivalent 32768 flops, twice the 16384 it does",
           "# for the layer; likewise the product kernel's sparse 32x32x32, with the tokens padded to 32).",
           f"pass 1: {cmd[1].strip() if len(cmd) > 1 else ''}", f"pass 2: {cmd[2].strip() if len(cmd) > 2 else ''}",
           *([f"pass 3 (vector memory path; busy fractions over GRBM_GUI_ACTIVE / 8 cycles and 256 CUs): {cmd[5].strip()}"]
             if mem_dir and len(cmd) > 5 else []),
           f"kernel_source_sha256: {digest}", ""]
    for label, prefix, grid, algo in PROFILE_KERNELS:
        k1 = [k for k in c1 if pick(k[0], k[1], prefix, grid)]
        k2 = [k for k in c2 if pick(k[0], k[1], prefix, grid)]
        if not k1 or not k2:
            continue
        a, b = c1[k1[0]], c2[k2[0]]
        dur = med(list(a["_dur_us"].values()))
        cyc = med(a["SQ_BUSY_CYCLES"]) / 32
        clock = cyc / (dur * 1e3)
        mfma = med(a["SQ_INSTS_MFMA"])
        flops_ctr = med(a["SQ_INSTS_VALU_MFMA_MOPS_F16"]) * 512
        busy = med(a["SQ_VALU_MFMA_BUSY_CYCLES"]) / 1024 / cyc
        waves = med(a["SQ_WAVES"])
        # the sparse instructions count at their dense equivalent, twice their useful work
        # (the product kernel's K = 16 rebuild MFMAs are dense)
        useful = (flops_ctr / 2 if "decode" in prefix else
                  (flops_ctr + PRODUCT_REBUILD_FLOPS) / 2 if "product" in prefix else flops_ctr)
        out += [f"## {label}",
                f"dispatch duration (counter run): {dur:.1f} us over {len(a['_dur_us'])} dispatches",
                f"shader clock: {clock:.3f} GHz",
                f"waves: {waves:.0f}",
                f"MFMA instructions: {mfma:.0f}",
                f"MFMA flops from counters: {flops_ctr:.4g} (useful for the layer: {useful:.4g}; algorithmic: {algo:.4g})",
                f"MFMA TFLOP/s (useful, counter run): {useful / dur / 1e6:.1f} = {useful / dur / 1e6 / FP16_MFMA_PEAK_TFLOPS:.3f} of {FP16_MFMA_PEAK_TFLOPS} TFLOP/s",
                f"MFMA busy: {busy:.3f} of the SIMD cycles",
                f"VALU instructions per wave: {med(a['SQ_INSTS_VALU']) / waves:.0f}",
                f"LDS instructions per wave: {med(a['SQ_INSTS_LDS']) / waves:.0f}",
                f"vector memory reads per wave: {med(b['SQ_INSTS_VMEM_RD']) / waves:.0f}",
                f"wave cycles waiting on dependencies (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES): {med(b['SQ_WAIT_INST_ANY']) / med(b['SQ_WAVE_CYCLES']):.3f}",
                f"VALU active / wave cycles: {med(b['SQ_ACTIVE_INST_VALU']) / med(b['SQ_WAVE_CYCLES']):.3f}",
                f"LDS active (SQ_LDS_IDX_ACTIVE / (32 x cycles x 8 CUs)): {med(b['SQ_LDS_IDX_ACTIVE']) / (cyc * 256):.3f}",
                f"LDS bank conflicts: {med(b['SQ_LDS_BANK_CONFLICT']):.0f}"]
        k3 = [k for k in c3 if pick(k[0], k[1], prefix, grid)]
        if k3:
            m = c3[k3[0]]
            gui = med(m["GRBM_GUI_ACTIVE"]) / 8
            req = med(m["TCP_TCC_READ_REQ_sum"])
            hit, miss = med(m["TCC_HIT_sum"]), med(m["TCC_MISS_sum"])
            out += [f"TA busy (address unit, per CU): {med(m['TA_TA_BUSY_sum']) / 256 / gui:.3f}",
                    f"TD busy (data return unit, per CU): {med(m['TD_TD_BUSY_sum']) / 256 / gui:.3f}",
                    f"L2 hit rate: {hit / (hit + miss):.3f}",
                    f"average L1-to-L2 read latency: {med(m['TCP_TCC_READ_REQ_LATENCY_sum']) / req:.0f} cycles"]
        out.append("")
    with open(os.path.join(ROOT, "profiles", "sq_counters_llama3_8b_layer.txt"), "w") as f:
        f.write("\n".join(out) + "\n")

    # --- HBM traffic of the decode kernel, copy-calibrated
    def tcc(d, name):
        vals = {}
        for r in csv.DictReader(open(one(d, "counter_collection.csv"))):
            if r["Counter_Name"] == name:
                vals.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = tcc(fetch_dir, "FETCH_SIZE"), tcc(write_dir, "WRITE_SIZE")
    copy_key = next(k for k in fetch if "neg_kernel" in k[0])  # the torch.neg copy of copy_calibration()
    dec_key = next(k for k in fetch if pick(k[0], k[1], PROFILE_KERNELS[0][1], PROFILE_KERNELS[0][2]))
    copy_bytes = 1024 * (1 << 20)  # each copy dispatch reads and writes exactly 1 GiB
    f_copy, w_copy = med(fetch[copy_key]), med(write[copy_key])
    f_scale, w_scale = copy_bytes / (f_copy * 1024), copy_bytes / (w_copy * 1024)
    f_dec = med(fetch[dec_key]) * 1024 * f_scale
    w_dec = med(write[dec_key]) * 1024 * w_scale
    algo = sum(8 * block_bytes(m, d) for _, m, d in synth.LLAMA3_8B_LAYER)
    text = f"""# HBM traffic of decode_m1_kernel, one grouped launch over a Llama-3-8B-shaped layer (n=8, k=16, M=1)
fetch command: {cmd[3].strip() if len(cmd) > 3 else ''}
write command: {cmd[4].strip() if len(cmd) > 4 else ''}
calibration: a 1 GiB fp16 elementwise copy (torch.neg) in the same runs reads FETCH_SIZE {f_copy:.1f} KiB and writes WRITE_SIZE {w_copy:.1f} KiB per dispatch
fetch_scale: {f_scale:.4f}
write_scale: {w_scale:.4f}
decode_fetch_kib_median: {med(fetch[dec_key]):.2f} over {len(fetch[dec_key])} dispatches
decode_write_kib_median: {med(write[dec_key]):.2f} over {len(write[dec_key])} dispatches
fetch_bytes_per_launch: {int(f_dec)}
write_bytes_per_launch: {int(w_dec)}
hbm_bytes_per_launch: {int(f_dec + w_dec)}
algorithmic_bytes_per_launch: {algo}
traffic_over_algorithmic: {(f_dec + w_dec) / algo:.4f}
kernel_source_sha256: {digest}
"""
    with open(TRAFFIC_SUMMARY, "w") as f:
        f.write(text)
    print(open(TRAFFIC_SUMMARY).read())


def block_streaming(bsl, torch, seed: int) -> dict:
    """Host -> device block loading (pack on the host into pinned staging, asynchronous
    copy) of one 8B-shaped layer at n = 8: its rate alone, and while single-token decode
    forwards of another stack run on a second stream (both rates reported)."""
    shapes = synth.LLAMA3_8B_LAYER
    src = [synth.synthetic_blocks(seed, m, d, 8, 16, 0, j) for j, (_, m, d) in enumerate(shapes)]
    layer_bytes = sum(8 * block_bytes(m, d) for _, m, d in shapes)
    h = bsl.bsl_init(0, [m for _, m, _ in shapes], [d for _, _, d in shapes], 16, 16, 0)
    for j, b in enumerate(src):
        bsl.bsl_set_source(h, j, b)
    s2 = torch.cuda.Stream()
    sp2 = int(s2.cuda_stream)

    def unload():  # (a shrink waits for the whole device, so it is done beforehand)
        bsl.bsl_load_blocks(h, [0] * 7, sp2)

    def load_all():
        t0 = time.perf_counter()
        bsl.bsl_load_blocks(h, [8] * 7, sp2)
        return time.perf_counter() - t0

    load_all()  # (first call allocates the pinned staging)
    times = []
    for _ in range(2):
        unload()
        times.append(load_all())
    alone = min(times)
    # one more block of the largest weight (gate, 14336 x 4096)
    bsl.bsl_load_blocks(h, [8, 8, 8, 8, 7, 8, 8], sp2)
    t0 = time.perf_counter()
    bsl.bsl_load_blocks(h, [8] * 7, sp2)
    one_block = time.perf_counter() - t0
    # decode on another stack and stream, alone and during a load
    dec = Layers(bsl, torch, shapes, [[8] * 7] * 2, 2, seed + 1, M=1)
    s1 = torch.cuda.current_stream()
    sp1 = int(s1.cuda_stream)

    def decode_span(k, during_load):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if during_load:
            unload()
        torch.cuda.synchronize()
        e0.record(s1)
        for i in range(k):
            dec.launch(i % 2, sp1)
        e1.record(s1)
        wall = load_all() if during_load else None
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k, wall

    k = max(200, int(alone / 80e-6))  # enough decode work to cover the load
    dec_alone, _ = decode_span(k, False)
    dec_during, load_during = decode_span(k, True)
    dec.close()
    bsl.bsl_destroy(h)
    return {
        "workload": "Llama-3-8B-shaped layer, 7 linears x 8 blocks (k=16): row-major sign bits copied to the device and repacked there by a kernel, factor layouts written on the host",
        "layer_bytes": layer_bytes,
        "load_ms": round(alone * 1e3, 1),
        "load_GB_per_s": round(layer_bytes / alone / 1e9, 2),
        "one_gate_block_ms": round(one_block * 1e3, 2),
        "one_gate_block_bytes": block_bytes(14336, 4096),
        "load_during_decode_ms": round(load_during * 1e3, 1),
        "load_during_decode_GB_per_s": round(layer_bytes / load_during / 1e9, 2),
        "decode_us_per_step_alone": round(dec_alone, 2),
        "decode_us_per_step_during_load": round(dec_during, 2),
    }


def equal_size_svd_decode(bsl, torch, seed: int, layers: int, steps: int, warmup: int) -> dict:
    """The "w/o AVD" baseline at equal bytes: every linear of the 8B-shaped layer held as
    n = 8 vanilla-SVD blocks of rank k' = 16 + m d / (16 (m + d)) (fp16 U', V', no signs),
    single-token decode through one grouped launch pair per step, `layers` resident
    copies rotated like the headline decode.  Bytes are 8 * 2 k' (m + d) per weight."""
    shapes = synth.LLAMA3_8B_LAYER
    kps = [bsl.bsl_lr_equal_rank(m, d, K_RANK) for _, m, d in shapes]
    h = bsl.bsl_lr_init(0, [m for _ in range(layers) for _, m, _ in shapes], [d for _ in range(layers) for _, _, d in shapes],
                        kps * layers, 8)
    for j, (_, m, d) in enumerate(shapes):
        g = synth.rng(seed, 50, j)
        blocks = [{"u": (g.standard_normal((m, kps[j]), dtype=np.float32) * 0.05).astype(np.float16),
                   "v": (g.standard_normal((d, kps[j]), dtype=np.float32) * 0.05).astype(np.float16)} for _ in range(8)]
        for l in range(layers):  # the same host factors, one device copy per layer
            bsl.bsl_lr_set_source(h, l * 7 + j, blocks)
    bsl.bsl_lr_load_blocks(h, [8] * (7 * layers), 0)
    for key in [k for k in bsl._sources if k[0] == "lr" and k[1] == h]:
        del bsl._sources[key]
    xs = [[torch.from_numpy(synth.activations(seed + 1, 1, d, l, j)).cuda() for j, (_, _, d) in enumerate(shapes)]
          for l in range(layers)]
    ys = [[torch.empty((1, m), dtype=torch.float16, device="cuda") for _, m, _ in shapes] for _ in range(layers)]
    layer_bytes = sum(8 * bsl.bsl_lr_block_bytes(m, d, kps[j]) for j, (_, m, d) in enumerate(shapes))
    st = torch.cuda.current_stream()
    sp = int(st.cuda_stream)

    def launch(l):
        bsl.bsl_lr_forward_group(h, list(range(l * 7, l * 7 + 7)), [t.data_ptr() for t in xs[l]],
                                 [t.data_ptr() for t in ys[l]], 1, False, sp)

    for i in range(warmup):
        launch(i % layers)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(steps):
        launch(i % layers)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = e0.elapsed_time(e1) * 1e3 / steps
    bsl.bsl_lr_destroy(h)
    return {
        "workload": "Llama-3-8B-shaped layer linears, n=8 vanilla-SVD blocks of the equal-size rank k' "
                    f"({', '.join(f'{nm} {kp}' for (nm, _, _), kp in zip(shapes, kps))}), M=1 decode, "
                    f"one grouped launch pair per step, {layers} resident layer copies rotated",
        "bytes_per_step": layer_bytes,
        "us_per_step": round(us, 2),
        "wall_us_per_step": round(wall * 1e6 / steps, 2),
        "GB_per_s": round(layer_bytes / (us * 1e-6) / 1e9, 1),
        "hbm_frac_of_peak": round(layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "kernels": "lowrank_xv_kernel + lowrank_tu_kernel",
    }


def copy_calibration(torch, mib: int = 1024, reps: int = 3) -> None:
    """A plain elementwise copy (y = -x, fp16) of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters: each dispatch reads and writes exactly `mib` MiB."""
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {mib} MiB")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--prefill-steps", type=int, default=2, help="timed steps of the factored M=2048 prefill")
    ap.add_argument("--tile-steps", type=int, default=20, help="timed steps of the tile-path M=2048 prefill")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-svd", action="store_true", help="skip the equal-size vanilla-SVD decode baseline")
    ap.add_argument("--no-few", action="store_true", help="skip the few-token (M = 2, 3, 4) decode runs")
    ap.add_argument("--decode", choices=["auto", "shared", "private"], default="auto",
                    help="single-token kernel of the headline (auto: the shared-operand kernel)")
    ap.add_argument("--no-sweep", action="store_true", help="skip variable block counts at M = 1, 4, 16")
    ap.add_argument("--no-70b", action="store_true", help="skip the 80-layer 70B-shaped decode stack")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured HBM / matrix-core peaks")
    ap.add_argument("--no-load", action="store_true", help="skip host -> device block streaming")
    ap.add_argument("--profile-set", action="store_true",
                    help="only the kernels the committed profiles cover: the decode headline (after the measured "
                         "peaks, as in the full run), the few-token kernel at M = 4, the product-index kernel at "
                         "M = 16 and the tile-path prefill, plus a 1 GiB copy for counter calibration")
    ap.add_argument("--per-weight", action="store_true", help="also time single-weight launches of each linear")
    ap.add_argument("--calibrate-copy", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--cpu-layers", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--write-profile-summaries", nargs=6,
                    metavar=("TRACE_DIR", "SQ1_DIR", "SQ2_DIR", "FETCH_DIR", "WRITE_DIR", "COMMANDS"),
                    help="write profiles/ summaries from rocprofv3 outputs (no GPU work)")
    ap.add_argument("--mem-dir", default=None,
                    help="with --write-profile-summaries: rocprofv3 output of the vector-memory-path counter pass")
    args = ap.parse_args()
    if args.profile_set:
        args.no_cpu = args.no_svd = args.no_sweep = args.no_70b = args.no_load = True
        args.calibrate_copy = True
    if args.write_profile_summaries:
        write_profile_summaries(*args.write_profile_summaries, mem_dir=args.mem_dir)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_sign_rank_amd as bsl

    bsl.lib()  # fails loudly if the HIP library is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.cuda.get_device_properties(0)
    log(f"device: {dev.name} ({getattr(dev, 'gcnArchName', '?')}), {dev.multi_processor_count} CUs")

    shapes = synth.LLAMA3_8B_LAYER
    result = {"metric": METRIC}

    # ---------------- decode (headline)
    log(f"decode: building {args.layers} resident 8B-shaped layers (n=8, k=16)")
    kinds = {"auto": bsl.BSL_DECODE_AUTO, "shared": bsl.BSL_DECODE_SHARED, "private": bsl.BSL_DECODE_PRIVATE}
    dec = Layers(bsl, torch, shapes, [[8] * 7] * args.layers, args.layers, args.seed, M=1, decode=kinds[args.decode])
    # The measured peaks of this GPU (HBM and matrix-core loops, about a second of GPU
    # work) run here, between building the layers (host work, GPU idle) and the decode
    # timing, so the timed launches do not start from an idle GPU's clock.
    pk = None
    if not args.no_peaks:
        from bit_sign_rank_amd import peaks as _peaks

        log("peaks: HBM read / copy, matrix-core loops")
        pk = _peaks.measure(torch, dev.multi_processor_count, reps=10, gib=1.0)
        torch.cuda.empty_cache()
    # the other single-token kernel on the same stack, for comparison
    private = args.decode == "private"
    bsl.bsl_set_decode(dec.h, bsl.BSL_DECODE_SHARED if private else bsl.BSL_DECODE_PRIVATE)
    w_o, k_o, b_o, _ = time_steps(torch, dec, args.steps, args.warmup)
    other = {"kernel": "decode_m1_kernel" if private else "decode_wp_kernel",
             "us_per_step": round(float(np.mean(k_o)) * 1e3, 2),
             "GB_per_s": round(dec.bytes(0) / (float(np.mean(k_o)) * 1e-3) / 1e9, 1)}
    bsl.bsl_set_decode(dec.h, kinds[args.decode])
    wall, kern_ms, tbytes, tflops = time_steps(torch, dec, args.steps, args.warmup)
    ms_per_step = wall * 1e3 / args.steps
    value = tbytes / wall / 1e9
    kavg = float(np.mean(kern_ms))
    per_launch_bytes = dec.bytes(0)
    achieved = per_launch_bytes / (kavg * 1e-3) / 1e9
    log(f"decode: {ms_per_step * 1e3:.1f} us/step, {value:.0f} GB/s wall, kernel avg {kavg * 1e3:.1f} us -> {achieved:.0f} GB/s")
    per_weight = []
    for j, (name, m, d) in enumerate(shapes if args.per_weight else []):
        # single-weight launches, for the per-shape picture
        h = dec.h
        x, y = dec.x[0][j], dec.y[0][j]
        st = torch.cuda.current_stream()
        for _ in range(5):
            bsl.bsl_forward(h, j, x.data_ptr(), y.data_ptr(), 1, False, int(st.cuda_stream))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 50
        e0.record(st)
        for r in range(reps):
            lw = (r % args.layers) * 7 + j
            bsl.bsl_forward(h, lw, dec.x[r % args.layers][j].data_ptr(), dec.y[r % args.layers][j].data_ptr(), 1, False,
                            int(st.cuda_stream))
        e1.record(st)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        b = 8 * block_bytes(m, d)
        per_weight.append({"weight": name, "m": m, "d": d, "us": round(us, 2), "GB/s": round(b / (us * 1e-6) / 1e9, 1)})
    dec.close()
    del dec
    torch.cuda.empty_cache()

    result.update(
        {
            "value": round(value, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f16",
            "data": "synthetic",
            "config": {
                "workload": "Llama-3-8B-shaped decoder-layer linears (q,k,v,o,gate,up,down), n=8 blocks, k=16, M=1 decode, "
                f"one grouped launch per step, {args.layers} resident layer copies rotated",
                "bytes_per_step": per_launch_bytes,
                "mfma_flops_per_step": int(tflops // args.steps),
                "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
                "mfma_tflops": round(tflops / wall / 1e12, 1),
            },
            "roofline": {
                "bound": "hbm",
                "kernel": "decode_wp_kernel" if args.decode == "private" else "decode_m1_kernel",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(),
                "avg_launch_us": round(kavg * 1e3, 2),
            },
        }
    )
    if per_weight:
        result["decode_single_weight_launches"] = per_weight
    result["decode_other_kernel"] = other

    # ---------------- measured peaks of this GPU (the roofline fractions are also given against them)
    if pk is not None:
        result["measured_peaks"] = {
            "hbm_read_GBs": pk["hbm_read_GBs"],
            "hbm_copy_GBs": pk["hbm_copy_GBs"],
            "fp16_dense_mfma_tflops": pk["mfma_v_mfma_f32_16x16x32_f16"]["tflops"],
            "fp16_dense_mfma_clock_ghz": round(pk["mfma_v_mfma_f32_16x16x32_f16"]["clock_ghz"] or 0, 3),
            "sparse_mfma_tflops": pk["mfma_v_smfmac_f32_16x16x64_f16"]["tflops"],
            "sparse_mfma_decode_operands_with_sign_stream": {
                k: pk["sparse_mfma_lds_r4_mode1_stream"][k] for k in ("tflops", "stream_GBs", "clock_ghz")},
            "note": "bench_peaks kernels (libbsl_peaks.so): grid-stride non-temporal 16-byte loads of 1 GiB; "
                    "16 independent MFMA chains per wave, 4 waves per SIMD; the last line is the sparse MFMA with "
                    "A = 1, B random fp16 from LDS and a matched 1 KiB-per-16-MFMA HBM stream (the single-token "
                    "kernel's operand profile and byte rate)",
        }
        rf = result["roofline"]
        rf["frac_of_measured_read_peak"] = round(rf["achieved"] / pk["hbm_read_GBs"], 4)

    # ---------------- resident bytes against the blocks' payload (one 8B-shaped layer, n = 8)
    probe = bsl.bsl_init(0, [m for _, m, _ in shapes], [d for _, _, d in shapes], 16, 16, 0)
    for j, (_, m, d) in enumerate(shapes):
        bsl.bsl_set_source(probe, j, synth.synthetic_blocks(args.seed + 61, m, d, 8, 16, j))
    bsl.bsl_load_blocks(probe, [8] * 7, 0)
    payload = sum(8 * block_bytes(m, d) for _, m, d in shapes)
    resident = bsl.bsl_resident_bytes(probe)
    vbytes = sorted((8 * d * 32 for _, _, d in shapes), reverse=True)[:8]
    result["resident_bytes"] = {"workload": "one Llama-3-8B-shaped layer, n=8", "payload_bytes": payload,
                                "resident_bytes": int(resident), "ratio": round(resident / payload, 4),
                                "stack_workspace_bytes": int(bsl.bsl_workspace_bytes(probe)),
                                "of_which_rank_major_v": int(sum(vbytes)),
                                "note": "blocks hold one copy of each factor; the tile path forms V in rank-major "
                                        "order per call in a stack workspace sized for the 8 weights with the most "
                                        "V bytes (one per stack, whatever the number of layers)"}
    torch.cuda.synchronize()
    bsl.bsl_destroy(probe)
    for key in [k for k in bsl._sources if k[0] == probe]:
        del bsl._sources[key]

    # ---------------- 1024 x 1024, n = 4, M = 1 (the parity workload's shape; launch-bound)
    if not args.profile_set:
        c1 = Layers(bsl, torch, [("w", 1024, 1024)], [[4]] * 64, 64, args.seed + 71, M=1)
        w1, k1, b1, _ = time_steps(torch, c1, 640, 64, warm_s=WARM_S)
        result["single_1024x1024_n4_decode"] = {
            "workload": "one 1024x1024 linear, n=4 blocks (k=16), M=1, 64 resident copies rotated; blocks synthetic of "
                        "the decomposed shape (the CPU decomposition is not on the timed path)",
            "us_per_launch": round(float(np.mean(k1)) * 1e3, 2), "bytes_per_launch": c1.bytes(0)}
        c1.close()
        del c1
        torch.cuda.empty_cache()

    # ---------------- prefill M = 2048: tile path (the default for batches), then factored
    # ---------------- a few tokens (batched decode): the wave-private kernel over T tokens
    if not args.no_few:
        few = []
        kern = {2: "decode_wp_kernel<8, 2>", 3: "decode_wp_kernel<8, 3>", 4: "decode_wp_kernel<8, 4>"}
        sets = (("8B", shapes, [8] * 7), ("70B", synth.LLAMA2_70B_LAYER, [3] * 7))
        for label, lshapes, counts in (sets[:1] if args.profile_set else sets):
            for M in ((4,) if args.profile_set else (2, 3, 4)):
                row = {"layer": label, "n": counts[0], "M": M,
                       "auto_takes": ("few-token" + (" (down projection: product-index)" if label == "70B" and M == 3 else ""))
                       if M < 4 else "product-index (product_kernel<2, 2>)"}
                paths = [("few_token", bsl.BSL_PATH_DECODE), ("factored", bsl.BSL_PATH_FACTORED)]
                if M >= 3 and not args.profile_set:  # (at 3 tokens AUTO differs from DECODE where a weight is wide)
                    paths.append(("auto", bsl.BSL_PATH_AUTO))
                for name, path in paths:
                    log(f"few tokens: {label}-shaped layer, n={counts[0]}, M={M}, {name} path")
                    lay = Layers(bsl, torch, lshapes, [counts] * 2, 2, args.seed + 5, M=M, path=path, shared_sources=True)
                    w_, k_, b_, f_ = time_steps(torch, lay, 60, 6, warm_s=WARM_S)
                    row[f"{name}_us_per_step"] = round(w_ * 1e6 / 60, 1)
                    row[f"{name}_kernel_us"] = round(float(np.mean(k_)) * 1e3, 1)
                    if name == "few_token":
                        kus = float(np.mean(k_)) * 1e-3
                        row["sz_flops_per_step"] = int(f_ // 60)
                        row["mfma_tflops"] = round(f_ / 60 / kus / 1e12, 1)
                        row["mfma_frac_of_peak"] = round(f_ / 60 / kus / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)
                        row["GB_per_s"] = round(b_ / 60 / kus / 1e9, 1)
                    lay.close()
                    del lay
                    torch.cuda.empty_cache()
                row["kernel"] = kern[M] + ("" if label == "8B" or M == 2 else " (down projection: prefill_kernel, second launch)")
                row["speedup_vs_factored"] = round(row["factored_kernel_us"] / row["few_token_kernel_us"], 2)
                few.append(row)
                log(f"few tokens: {row}")
        result["few_token_decode"] = {
            "workload": "decoder-layer linears (Llama-3-8B shapes at n=8; Llama-2-70B shapes at n=3), k=16, M tokens per "
                        "grouped launch, 2 rotated layers; the few-token kernel (BSL_PATH_DECODE) against the factored "
                        "path, and at M = 4 the product-index path AUTO takes there; MFMA work = the S Z contraction "
                        "2 n k M m d",
            "runs": few}

    # ---------------- 4 to 32 tokens: the product-index kernel against the tile kernel (and the
    # few-token kernel at M = 4) on the same stack
    if not args.no_few:
        prod = []
        lay = Layers(bsl, torch, shapes, [[8] * 7] * 2, 2, args.seed + 9, M=32, shared_sources=True)
        for M in ((16,) if args.profile_set else (4, 8, 16, 32)):
            lay.M = M  # (the first M rows of the layer's 32-token x and y)
            row = {"M": M}
            paths = [("product", bsl.BSL_PATH_PRODUCT), ("tile", bsl.BSL_PATH_TILE)]
            if M == 4:
                paths.append(("few_token", bsl.BSL_PATH_DECODE))
            for name, path in paths:
                bsl.bsl_set_path(lay.h, path)
                w_, k_, _, _ = time_steps(torch, lay, 40, 5, warm_s=WARM_S)
                row[f"{name}_us"] = round(float(np.mean(k_)) * 1e3, 1)
            kus = row["product_us"] * 1e-6
            row["auto_takes"] = "product" if 4 <= M <= 32 else ("few_token" if M <= 3 else "tile")
            row["product_roofline"] = {"bound": "mfma", "achieved": round(lay.product_flops(0) / kus / 1e12, 1),
                                       "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(lay.product_flops(0) / kus / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
                                       "flops": "executed MFMA work: (2 k + 2 * 32) n m d (tokens padded to 32)"}
            row["tokens_per_s"] = round(M / kus, 1)
            prod.append(row)
            log(f"product-index: {row}")
        bsl.bsl_set_path(lay.h, bsl.BSL_PATH_AUTO)
        lay.close()
        del lay
        torch.cuda.empty_cache()
        result["product_index"] = {
            "workload": "Llama-3-8B-shaped layer linears, n=8, k=16, M tokens per grouped launch, 2 rotated layers; "
                        "product_kernel (with its per-call V and x layout passes) against the tile path and, at M = 4, "
                        "the few-token kernel",
            "runs": prod}

    if not args.no_prefill:
        log("prefill: one 8B-shaped layer, n=8, M=2048, tile path")
        pre = Layers(bsl, torch, shapes, [[8] * 7], 1, args.seed + 7, M=2048, path=bsl.BSL_PATH_TILE)
        wall_t, kms_t, _, _ = time_steps(torch, pre, args.tile_steps, 2, warm_s=WARM_S)
        t_step = wall_t / args.tile_steps
        tfl_t = pre.tile_flops(0) / t_step / 1e12
        k_step = float(np.mean(kms_t)) * 1e-3
        result["prefill"] = {
            "workload": "Llama-3-8B-shaped layer linears, n=8, k=16, M=2048, one grouped launch per step, tile path",
            "ms_per_step": round(t_step * 1e3, 3),
            "tokens_per_s": round(2048 / t_step, 1),
            "kernel": "tile_split_kernel<8>",
            "mfma_flops_per_step": pre.tile_flops(0),
            "roofline": {"bound": "mfma", "achieved": round(pre.tile_flops(0) / k_step / 1e12, 1),
                         "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(pre.tile_flops(0) / k_step / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
                         "avg_launch_us": round(k_step * 1e6, 1)},
            "gemm_equivalent_tflops": round(pre.gemm_flops(0) / t_step / 1e12, 1),
        }
        log(f"prefill (tile): {t_step * 1e3:.2f} ms/step, {tfl_t:.1f} TFLOP/s executed MFMA work")
        pre.close()
        del pre
        torch.cuda.empty_cache()
    if not args.no_prefill and not args.profile_set:
        log("prefill: one 8B-shaped layer, n=8, M=2048, factored path")
        pre = Layers(bsl, torch, shapes, [[8] * 7], 1, args.seed + 7, M=2048, path=bsl.BSL_PATH_FACTORED)
        wall_p, kms_p, tb_p, tf_p = time_steps(torch, pre, args.prefill_steps, 1)
        tfl = tf_p / wall_p / 1e12
        result["prefill_factored"] = {
            "workload": "Llama-3-8B-shaped layer linears, n=8, k=16, M=2048, one grouped launch per step, factored path",
            "ms_per_step": round(wall_p * 1e3 / args.prefill_steps, 2),
            "mfma_tflops": round(tfl, 1),
            "mfma_frac_of_peak": round(tfl / FP16_MFMA_PEAK_TFLOPS, 4),
            "kernel": "prefill_kernel",
            "flops_per_step": int(tf_p // args.prefill_steps),
        }
        result["prefill"]["speedup_vs_factored"] = round(result["prefill_factored"]["ms_per_step"] / result["prefill"]["ms_per_step"], 1)
        log(f"prefill (factored): {wall_p * 1e3 / args.prefill_steps:.1f} ms/step, {tfl:.1f} TFLOP/s")
        pre.close()
        del pre
        torch.cuda.empty_cache()

    # ---------------- equal-size vanilla-SVD baseline ("w/o AVD"), decode
    if not args.no_svd:
        log("equal-size SVD baseline: 8B-shaped layer, n=8 blocks of rank k', M=1")
        result["equal_size_svd_decode"] = equal_size_svd_decode(bsl, torch, args.seed + 41, args.layers, args.steps,
                                                                args.warmup)
        r = result["equal_size_svd_decode"]
        r["bitstack_decode_us_per_step"] = result["roofline"]["avg_launch_us"]
        r["bitstack_speedup"] = round(r["us_per_step"] / result["roofline"]["avg_launch_us"], 2)
        log(f"equal-size SVD baseline: {r['us_per_step']} us/step, {r['GB_per_s']} GB/s")
        torch.cuda.empty_cache()

    # ---------------- variable block counts (n_w drawn in 1..16), M = 1, 4, 16
    if not args.no_sweep:
        sweep = []
        counts = synth.block_counts(13, 7, 1, 16)
        for M in (1, 4, 16):
            lay = Layers(bsl, torch, shapes, [counts] * 2, 2, args.seed + 11, M=M, shared_sources=True)
            steps = 100 if M < 16 else 50
            w_, k_, b_, f_ = time_steps(torch, lay, steps, 5, warm_s=WARM_S)
            kus = float(np.mean(k_)) * 1e-3
            row = {"M": M, "n_w": [int(c) for c in counts], "us_per_step": round(kus * 1e6, 1),
                   "path": "single-token (decode_m1_kernel)" if M == 1 else "product-index (product_kernel)",
                   "bytes_per_step": lay.bytes(0), "GB_per_s": round(lay.bytes(0) / kus / 1e9, 1)}
            if M == 1:
                row["roofline"] = {"bound": "hbm", "achieved": row["GB_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(row["GB_per_s"] / HBM_PEAK_GBS, 4)}
            else:
                fl = lay.product_flops(0)
                row["roofline"] = {"bound": "mfma", "achieved": round(fl / kus / 1e12, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(fl / kus / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4),
                                   "flops": "executed MFMA work of the path: (2 k + 2 * 32) n m d (tokens padded to 32)"}
                row["sz_work_frac"] = round(lay.flops(0) / kus / 1e12 / FP16_MFMA_PEAK_TFLOPS, 4)
                # on the same stack, for comparison: the few-token kernel at 4 tokens, the tile path at 16
                name, path = ("few_token", bsl.BSL_PATH_DECODE) if M == 4 else ("tile_path", bsl.BSL_PATH_TILE)
                bsl.bsl_set_path(lay.h, path)
                _, kt_, _, _ = time_steps(torch, lay, steps, 5, warm_s=WARM_S)
                bsl.bsl_set_path(lay.h, bsl.BSL_PATH_AUTO)
                row[f"{name}_us_per_step"] = round(float(np.mean(kt_)) * 1e3, 1)
            sweep.append(row)
            lay.close()
            del lay
            torch.cuda.empty_cache()
            log(f"sweep M={M}: {row}")
        result["variable_blocks_sweep"] = {
            "workload": "Llama-3-8B-shaped layer linears, n_w drawn in 1..16 per weight (seeded), k=16, 2 rotated layers, "
                        "M tokens per grouped launch", "runs": sweep}
    # ---------------- 80-layer Llama-2-70B-shaped stack, n_w drawn in 1..6, M = 1
    if not args.no_70b:
        counts = [synth.block_counts(18, 7, 1, 6, l) for l in range(synth.LLAMA2_70B_LAYERS)]
        log("llama70b: building 80 layers (device copies of shared host blocks, 8 layers per load)")
        lay = Layers(bsl, torch, synth.LLAMA2_70B_LAYER, counts, synth.LLAMA2_70B_LAYERS, args.seed + 21, M=1,
                     shared_sources=True, batch=8)
        tokens = 3
        w_, k_, b_, f_ = time_steps(torch, lay, synth.LLAMA2_70B_LAYERS * tokens, synth.LLAMA2_70B_LAYERS, warm_s=WARM_S)
        tok_us = float(np.mean(k_)) * 1e-3 * synth.LLAMA2_70B_LAYERS
        per_token = sum(lay.bytes(l) for l in range(synth.LLAMA2_70B_LAYERS))
        nsum = sum(int(c) for cc in counts for c in cc)
        result["llama2_70b_decode"] = {
            "workload": "80 Llama-2-70B-shaped decoder layers (q/o 8192x8192, k/v 1024x8192, gate/up 28672x8192, "
                        f"down 8192x28672), n_w drawn in 1..6 per weight (mean {nsum / 560:.2f}), k=16, M=1, one grouped "
                        "launch per layer, 80 launches per token; all 80 layers resident",
            "ms_per_token": round(tok_us * 1e3, 3),
            "bytes_per_token": per_token,
            "GB_per_s": round(per_token / tok_us / 1e9, 1),
            "roofline": {"bound": "hbm", "achieved": round(per_token / tok_us / 1e9, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(per_token / tok_us / 1e9 / HBM_PEAK_GBS, 4)},
            "resident_bytes": int(bsl.bsl_resident_bytes(lay.h)),
            "stack_workspace_bytes": int(bsl.bsl_workspace_bytes(lay.h)),
            "wall_ms_per_token": round(w_ * 1e3 / tokens, 3),
        }
        log(f"llama70b: {result['llama2_70b_decode']}")
        lay.close()
        del lay
        torch.cuda.empty_cache()

    if not args.no_load:
        log("block streaming: loading an 8B-shaped layer, alone and beside decode")
        result["block_streaming"] = block_streaming(bsl, torch, args.seed + 31)
        log(f"block streaming: {result['block_streaming']}")

    # ---------------- CPU oracle
    if not args.no_cpu:
        log("cpu baseline: oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(args.seed + 5, args.cpu_layers)
    if args.calibrate_copy:
        copy_calibration(torch)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
