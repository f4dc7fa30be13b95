"""Measured peaks of the GPU the benchmark runs on (libbsl_peaks.so, built beside the
library): HBM read and copy rates, and the sustained issue rate of the matrix-core
instructions the layer's kernels use, alone and beside an HBM stream.  Each result
carries the average shader clock over the kernel (from s_memtime against the constant
100 MHz s_memrealtime counter).  torch supplies the device buffers and the stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

FLOP = {0: 16384, 1: 16384, 2: 32768}  # per instruction: dense 16x16x32, sparse 16x16x64 (useful), dense 32x32x16
NAMES = {0: "v_mfma_f32_16x16x32_f16", 1: "v_smfmac_f32_16x16x64_f16", 2: "v_mfma_f32_32x32x16_f16"}


def lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(_HERE, "libbsl_peaks.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with bit_sign_rank_amd/build.py")
        L = ctypes.CDLL(path)
        L.bslp_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.bslp_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.bslp_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        L.bslp_lds.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.bslp_mfma_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
        for f in (L.bslp_read, L.bslp_copy, L.bslp_mfma, L.bslp_lds, L.bslp_mfma_lds):
            f.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what}: hip error {rc}")


def _clock_ghz(clocks):
    """Average shader clock (GHz) over the workgroups' own start/end stamps."""
    c = clocks.cpu().numpy().reshape(-1, 4).astype("float64")
    cyc = c[:, 1] - c[:, 0]
    real = (c[:, 3] - c[:, 2]) / 100e6  # s_memrealtime counts at 100 MHz
    ok = real > 0
    if not ok.any():
        return None
    return float((cyc[ok] / real[ok]).mean() / 1e9)


def _time(torch, launch, reps):
    st = torch.cuda.current_stream()
    launch()  # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        launch()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / reps


def measure(torch, cus: int, reps: int = 20, gib: float = 2.0) -> dict:
    """All peaks on the current device.  Buffers: 2 x `gib` GiB."""
    L = lib()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = int(gib * (1 << 30))
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    grid = cus * 8
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(grid * 4, dtype=torch.int64, device="cuda")
    res = {}

    t = _time(torch, lambda: _check(L.bslp_read(src.data_ptr(), nbytes, out.data_ptr(), clocks.data_ptr(), grid, st), "read"), reps)
    res["hbm_read_GBs"] = round(nbytes / t / 1e9, 1)
    t = _time(torch, lambda: _check(L.bslp_copy(src.data_ptr(), dst.data_ptr(), nbytes, clocks.data_ptr(), grid, st), "copy"), reps)
    res["hbm_copy_GBs"] = round(2 * nbytes / t / 1e9, 1)  # bytes read + bytes written

    # matrix-core loops: 4 waves per workgroup, 4 workgroups per CU (4 waves per SIMD)
    mgrid = cus * 4
    mout = torch.empty(mgrid * 256, dtype=torch.float32, device="cuda")
    mclk = torch.zeros(mgrid * 4, dtype=torch.int64, device="cuda")
    iters = 2048
    n16 = 1
    while n16 * 2 * 16 <= nbytes:
        n16 *= 2
    for wps, g in ((4, mgrid), (1, cus)):  # waves per SIMD
        for kind in (0, 1, 2):
            per_iter = 16
            flops = FLOP[kind] * per_iter * iters * g * 4
            t = _time(torch, lambda: _check(L.bslp_mfma(kind, iters, mout.data_ptr(), mclk.data_ptr(), None, 0, g, st), "mfma"), reps // 4 + 1)
            key = f"mfma_{NAMES[kind]}" + ("" if wps == 4 else "_1wave_per_simd")
            ck = _clock_ghz(mclk[: g * 4])
            res[key] = {"tflops": round(flops / t / 1e12, 1), "clock_ghz": ck,
                        "cycles_per_instr": round(t * ck * 1e9 / (wps * per_iter * iters), 2) if ck else None}
    # LDS reads: 16 KiB per wave per round
    lds_bytes = 16 * 1024 * iters * mgrid * 4
    t = _time(torch, lambda: _check(L.bslp_lds(iters, out.data_ptr(), mclk.data_ptr(), mgrid, st), "lds"), reps // 4 + 1)
    ck = _clock_ghz(mclk)
    res["lds_read"] = {"TBs": round(lds_bytes / t / 1e12, 1), "clock_ghz": ck,
                       "bytes_per_clk_per_cu": round(lds_bytes / t / (ck * 1e9) / cus, 1) if ck else None}
    # sparse MFMAs whose B operand (2 KiB per wave) is read from LDS every r instructions,
    # with three operand profiles (mode 0: A = 1, B ~ 1; mode 1: A = 1, B random; mode 2:
    # both random), alone and beside the matched sign-byte stream
    for r in (4, 8, 16):
        for mode in (0, 1, 2):
            for stream in (False, True):
                it = iters // 4
                n_instr = 16 * r * it
                flops = FLOP[1] * n_instr * mgrid * 4
                sp, sb = (src.data_ptr(), n16 * 16) if stream else (None, 0)
                t = _time(torch, lambda: _check(L.bslp_mfma_lds(r, mode, it, mout.data_ptr(), mclk.data_ptr(), sp, sb, mgrid, st), "mfma_lds"), reps // 4 + 1)
                ck = _clock_ghz(mclk)
                key = f"sparse_mfma_lds_r{r}_mode{mode}" + ("_stream" if stream else "")
                res[key] = {"tflops": round(flops / t / 1e12, 1), "clock_ghz": ck,
                            "cycles_per_instr": round(t * ck * 1e9 / (4 * n_instr), 2) if ck else None}
                if stream:
                    res[key]["stream_GBs"] = round(n_instr // 16 * 1024 * mgrid * 4 / t / 1e9, 1)
    # the sparse loop beside an HBM stream of 1 KiB per wave per 16 instructions
    flops = FLOP[1] * 16 * iters * mgrid * 4
    streamed = 16 * 64 * iters * mgrid * 4
    t = _time(torch, lambda: _check(L.bslp_mfma(1, iters, mout.data_ptr(), mclk.data_ptr(), src.data_ptr(), n16 * 16, mgrid, st), "mfma+stream"), reps // 4 + 1)
    res["sparse_mfma_with_stream"] = {"tflops": round(flops / t / 1e12, 1), "stream_GBs": round(streamed / t / 1e9, 1),
                                      "clock_ghz": _clock_ghz(mclk)}
    del src, dst
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    import json

    import torch

    props = torch.cuda.get_device_properties(0)
    print(json.dumps(measure(torch, props.multi_processor_count), indent=1))
