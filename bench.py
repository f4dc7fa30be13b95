"""Benchmark of the BitStack residual-block linear layer on one MI355X.

Headline (printed as one JSON line): HBM GB/s of single-token decode through the
seven linears of a Llama-3-8B-shaped decoder layer (q/o 4096x4096, k/v 1024x4096,
gate/up 14336x4096, down 4096x14336), each held as n = 8 residual blocks with k = 16
(synthetic Bernoulli(0.5) signs, U and V = |N(0,1)| * 0.05 in fp16, x ~ N(0,1) fp16).
One step is one grouped launch over the layer's seven linears.  Four distinct copies
of the layer are resident (about 0.96 GB) and the steps rotate over them, so the
256 MB last-level cache cannot serve the reads.  Bytes are the algorithmic bytes of
the loaded blocks, n * (m d / 8 + 2 k (m + d)) per weight, counted once.

Also reported: prefill on the dense path (W_hat restored to a workspace, then a library
GEMM); the same decode with every linear held as n = 8 equal-size vanilla-SVD
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
    """One bitstack stack holding `layers` copies of a decoder layer's linears."""

    def __init__(self, bsl, torch, shapes, counts, layers, seed, M, path=None, decode=None):
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
        self.counts = []
        for l in range(layers):
            for j, (_, m, d) in enumerate(shapes):
                n = int(counts[l][j])
                blocks = synth.synthetic_blocks(seed, m, d, n, 16, l, j)
                bsl.bsl_set_source(self.h, l * self.per + j, blocks)
                self.counts.append(n)
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

    def gemm_flops(self, l: int) -> int:
        return sum(2 * self.M * m * d for (_, m, d) in self.shapes)

    def close(self):
        self.torch.cuda.synchronize()
        self.bsl.bsl_destroy(self.h)


def time_steps(torch, layers: Layers, steps: int, warmup: int):
    """Warm up, then time exactly `steps` steps (one grouped launch each) between two
    device synchronisations.  One HIP event pair on the launch stream brackets the same
    steps, so the average launch duration carries no per-launch event overhead."""
    stream = torch.cuda.current_stream()
    sp = int(stream.cuda_stream)
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


def cpu_baseline(seed: int, layers: int = 4) -> dict:
    """The oracle, untouched, on a bounded sample of the decode workload: `layers`
    distinct 8B-shaped layers (all seven linears each) with n = 8 and M = 1, i.e.
    `layers` steps of the GPU benchmark (about 10-30 s of CPU work)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    total_bytes = 0
    elapsed = 0.0
    for l in range(layers):
        for j, (_, m, d) in enumerate(synth.LLAMA3_8B_LAYER):
            blocks = synth.synthetic_blocks(seed, m, d, 8, 16, 99, l, j)
            x = synth.activations(seed + 1, 1, d, 99, l, j)
            t0 = time.perf_counter()
            oracle.forward(x, blocks, 8)
            elapsed += time.perf_counter() - t0
            total_bytes += 8 * block_bytes(m, d)
    return {
        "value": round(total_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{layers} Llama-3-8B-shaped layers (7 linears each), n=8, M=1: fp64 reconstruct-then-matmul per linear",
        "seconds": round(elapsed, 2),
    }


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


def write_profile_summaries(trace_dir: str, fetch_dir: str, write_dir: str, command: str) -> None:
    """Turn rocprofv3 outputs (kernel-trace --stats of a bench run, then one --pmc
    FETCH_SIZE and one --pmc WRITE_SIZE pass of a bench run with --calibrate-copy) into
    the short text summaries kept under profiles/."""
    import csv
    import glob
    import hashlib

    def one(pattern):
        files = glob.glob(os.path.join(pattern))
        assert files, pattern
        return files[0]

    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    stats = list(csv.DictReader(open(one(os.path.join(trace_dir, "*kernel_stats.csv")))))
    lines = [f"# rocprofv3 --kernel-trace --stats, Llama-3-8B-shaped layer (n=8, k=16): decode M=1 and prefill M=2048",
             f"command: {command.split(';')[0]}",
             "", f"{'kernel':58s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}"]
    for r in stats:
        lines.append(f"{r['Name'][:58]:58s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
    with open(os.path.join(ROOT, "profiles", "kernel_stats_llama3_8b_layer.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def counters(d, name):
        vals = {}
        for r in csv.DictReader(open(one(os.path.join(d, "*counter_collection.csv")))):
            if r["Counter_Name"] == name:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = counters(fetch_dir, "FETCH_SIZE"), counters(write_dir, "WRITE_SIZE")
    copy_name = next(k for k in fetch if "neg_kernel" in k)  # the torch.neg copy of copy_calibration()
    dec_name = next(k for k in fetch if "decode_m1_kernel" in k)
    med = lambda v: sorted(v)[len(v) // 2]
    copy_bytes = 1024 * (1 << 20)  # each copy dispatch reads and writes exactly 1 GiB
    f_copy = med(fetch[copy_name])
    w_copy = med(write[copy_name])
    f_scale = copy_bytes / (f_copy * 1024)
    w_scale = copy_bytes / (w_copy * 1024)
    f_dec = med(fetch[dec_name]) * 1024 * f_scale
    w_dec = med(write[dec_name]) * 1024 * w_scale
    with open(KERNEL_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    algo = sum(8 * block_bytes(m, d) for _, m, d in synth.LLAMA3_8B_LAYER)
    text = f"""# HBM traffic of decode_m1_kernel, one grouped launch over a Llama-3-8B-shaped layer (n=8, k=16, M=1)
fetch command: {command.split(';')[1].strip() if ';' in command else ''}
write command: {command.split(';')[2].strip() if command.count(';') > 1 else ''}
calibration: a 1 GiB fp16 elementwise copy (torch.neg) in the same runs reads FETCH_SIZE {f_copy:.1f} KiB and writes WRITE_SIZE {w_copy:.1f} KiB per dispatch
fetch_scale: {f_scale:.4f}
write_scale: {w_scale:.4f}
decode_fetch_kib_median: {med(fetch[dec_name]):.2f} over {len(fetch[dec_name])} dispatches
decode_write_kib_median: {med(write[dec_name]):.2f} over {len(write[dec_name])} dispatches
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
        "workload": "Llama-3-8B-shaped layer, 7 linears x 8 blocks (k=16), packed on the host and copied to the device",
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
    ap.add_argument("--no-few", action="store_true", help="skip the few-token (M = 2, 4) decode runs")
    ap.add_argument("--decode", choices=["auto", "shared", "private"], default="auto",
                    help="single-token kernel of the headline (auto: the shared-operand kernel)")
    ap.add_argument("--sweep", action="store_true", help="also run variable block counts at M = 1, 4, 16")
    ap.add_argument("--llama70b", action="store_true", help="also run the 80-layer 70B-shaped decode stack")
    ap.add_argument("--per-weight", action="store_true", help="also time single-weight launches of each linear")
    ap.add_argument("--calibrate-copy", action="store_true", help="also run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--load", action="store_true", help="also measure host -> device block streaming, alone and beside decode")
    ap.add_argument("--cpu-layers", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--write-profile-summaries", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "COMMANDS"),
                    help="write profiles/ summaries from rocprofv3 outputs (no GPU work)")
    args = ap.parse_args()
    if args.write_profile_summaries:
        write_profile_summaries(*args.write_profile_summaries)
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

    # ---------------- prefill M = 2048: tile path (the default for batches), then factored
    # ---------------- a few tokens (batched decode): the wave-private kernel over T tokens
    if not args.no_few:
        few = []
        for M in (2, 4):
            row = {"M": M}
            for name, path in (("auto", bsl.BSL_PATH_AUTO), ("factored", bsl.BSL_PATH_FACTORED)):
                log(f"few tokens: 8B-shaped layer, n=8, M={M}, {name} path")
                lay = Layers(bsl, torch, shapes, [[8] * 7] * 2, 2, args.seed + 5, M=M, path=path)
                w_, k_, b_, _ = time_steps(torch, lay, 100, 10)
                row[f"{name}_us_per_step"] = round(w_ * 1e6 / 100, 1)
                row[f"{name}_kernel_us"] = round(float(np.mean(k_)) * 1e3, 1)
                row[f"{name}_GB_per_s"] = round(b_ / w_ / 1e9, 1)
                lay.close()
                del lay
                torch.cuda.empty_cache()
            row["kernel"] = "decode_wp_kernel<8, 2>" if M == 2 else "decode_wp_kernel<4, 4>"
            row["speedup_vs_factored"] = round(row["factored_us_per_step"] / row["auto_us_per_step"], 2)
            few.append(row)
            log(f"few tokens M={M}: {row}")
        result["few_token_decode"] = {
            "workload": "Llama-3-8B-shaped layer linears, n=8, k=16, M tokens per grouped launch, 2 rotated layers",
            "runs": few}

    if not args.no_prefill:
        log("prefill: one 8B-shaped layer, n=8, M=2048, tile path")
        pre = Layers(bsl, torch, shapes, [[8] * 7], 1, args.seed + 7, M=2048, path=bsl.BSL_PATH_TILE)
        wall_t, kms_t, _, _ = time_steps(torch, pre, args.tile_steps, 2)
        t_step = wall_t / args.tile_steps
        tfl_t = pre.tile_flops(0) / t_step / 1e12
        k_step = float(np.mean(kms_t)) * 1e-3
        result["prefill"] = {
            "workload": "Llama-3-8B-shaped layer linears, n=8, k=16, M=2048, one grouped launch per step, tile path",
            "ms_per_step": round(t_step * 1e3, 3),
            "tokens_per_s": round(2048 / t_step, 1),
            "kernel": "tile_kernel",
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
        log("prefill: one 8B-shaped layer, n=8, M=2048, dense path (restore W_hat, then a rocBLAS GEMM)")
        pre = Layers(bsl, torch, shapes, [[8] * 7], 1, args.seed + 7, M=2048, path=bsl.BSL_PATH_DENSE)
        wall_d, kms_d, _, _ = time_steps(torch, pre, args.tile_steps, 2)
        d_step = wall_d / args.tile_steps
        result["prefill_dense"] = {
            "workload": "Llama-3-8B-shaped layer linears, n=8, k=16, M=2048, dense path: one restore launch "
                        "(W_hat in fp16, 436 MB) then one rocBLAS fp16 GEMM per linear",
            "ms_per_step": round(d_step * 1e3, 3),
            "tokens_per_s": round(2048 / d_step, 1),
            "gemm_equivalent_tflops": round(pre.gemm_flops(0) / d_step / 1e12, 1),
            "speedup_vs_tile": round(t_step / d_step, 2),
        }
        log(f"prefill (dense): {d_step * 1e3:.2f} ms/step")
        pre.close()
        del pre
        torch.cuda.empty_cache()
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

    # ---------------- optional sweeps
    if args.sweep:
        sweep = []
        counts = synth.block_counts(13, 7, 1, 16)
        for M in (1, 4, 16):
            lay = Layers(bsl, torch, shapes, [counts] * 2, 2, args.seed + 11, M=M)
            w_, k_, b_, f_ = time_steps(torch, lay, 50, 5)
            sweep.append({"M": M, "n_w": [int(c) for c in counts], "GB/s": round(b_ / w_ / 1e9, 1),
                          "path": "single-token" if M == 1 else ("tile" if M >= 5 else "few-token"),
                          "sz_equivalent_tflops": round(f_ / w_ / 1e12, 1), "us_per_step": round(w_ * 1e6 / 50, 1)})
            lay.close()
            del lay
            torch.cuda.empty_cache()
            log(f"sweep M={M}: {sweep[-1]}")
        result["variable_blocks_sweep"] = sweep
    if args.llama70b:
        counts = [synth.block_counts(18, 7, 1, 6, l) for l in range(synth.LLAMA2_70B_LAYERS)]
        log("llama70b: building 80 layers (this takes a while)")
        lay = Layers(bsl, torch, synth.LLAMA2_70B_LAYER, counts, synth.LLAMA2_70B_LAYERS, args.seed + 21, M=1)
        w_, k_, b_, f_ = time_steps(torch, lay, synth.LLAMA2_70B_LAYERS * 3, synth.LLAMA2_70B_LAYERS)
        tok_ms = w_ * 1e3 / 3
        result["llama2_70b_decode"] = {"ms_per_token": round(tok_ms, 3), "GB/s": round(b_ / w_ / 1e9, 1),
                                       "bytes_per_token": int(b_ // 3)}
        lay.close()

    if args.load:
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
