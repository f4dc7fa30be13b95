"""Python binding of libbitstack_linear (ctypes; argument marshalling only).

Every function here forwards to the C entry point of the same name declared in
``include/bitstack_linear.h``; all arithmetic of the layer runs in the library's HIP
kernels.  Device buffers and streams are passed as integer addresses (for torch
tensors: ``t.data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``).  If the
library has not been built, importing works but every call raises ``RuntimeError``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitstack_linear.so")

BSL_OK = 0
BSL_EINVAL = -1
BSL_ENOMEM = -2
BSL_EHIP = -3
BSL_EUNSUPPORTED = -4
BSL_PATH_AUTO = 0
BSL_PATH_FACTORED = 1
BSL_PATH_TILE = 2
BSL_PATH_PRODUCT = 3
BSL_PATH_DECODE = 4
BSL_DECODE_AUTO = 0
BSL_DECODE_SHARED = 1
BSL_DECODE_PRIVATE = 2
BSL_KERNEL_KINDS = 5

EXPORTED = (
    "bsl_block_bytes",
    "bsl_packed_sign_bytes",
    "bsl_pack_signs",
    "bsl_unpack_signs",
    "bsl_init",
    "bsl_set_path",
    "bsl_set_decode",
    "bsl_set_source",
    "bsl_set_input_scale",
    "bsl_load_blocks",
    "bsl_active_blocks",
    "bsl_resident_bytes",
    "bsl_workspace_bytes",
    "bsl_launch_counts",
    "bsl_forward",
    "bsl_forward_group",
    "bsl_forward_group_static",
    "bsl_debug_unpack",
    "bsl_last_error",
    "bsl_destroy",
    # equal-size vanilla-SVD baseline (bitstack_lowrank.h)
    "bsl_lr_equal_rank",
    "bsl_lr_block_bytes",
    "bsl_lr_init",
    "bsl_lr_set_source",
    "bsl_lr_load_blocks",
    "bsl_lr_resident_bytes",
    "bsl_lr_forward",
    "bsl_lr_forward_group",
    "bsl_lr_destroy",
)


class BslError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (code {code})")
        self.code = code


class _BlockSrc(ctypes.Structure):
    _fields_ = [("sign_bits", ctypes.c_void_p), ("u", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class _LrBlockSrc(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("v", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        c_i32, c_i64, c_u64, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p
        L.bsl_block_bytes.restype = c_sz
        L.bsl_block_bytes.argtypes = [c_i64, c_i64, c_i32]
        L.bsl_packed_sign_bytes.restype = c_sz
        L.bsl_packed_sign_bytes.argtypes = [c_i64, c_i64]
        L.bsl_pack_signs.argtypes = [c_vp, c_i64, c_i64, c_vp]
        L.bsl_unpack_signs.argtypes = [c_vp, c_i64, c_i64, c_vp]
        L.bsl_init.argtypes = [ctypes.POINTER(c_vp), ctypes.c_int, c_i32, c_vp, c_vp, c_i32, c_i32, c_u64]
        L.bsl_set_source.argtypes = [c_vp, c_i32, c_i32, c_vp]
        L.bsl_set_input_scale.argtypes = [c_vp, c_i32, c_vp]
        L.bsl_load_blocks.argtypes = [c_vp, c_vp, c_vp]
        L.bsl_active_blocks.argtypes = [c_vp, c_i32, ctypes.POINTER(c_i32)]
        L.bsl_resident_bytes.restype = c_u64
        L.bsl_resident_bytes.argtypes = [c_vp]
        L.bsl_workspace_bytes.restype = c_u64
        L.bsl_workspace_bytes.argtypes = [c_vp]
        L.bsl_launch_counts.argtypes = [c_vp, c_vp]
        L.bsl_forward.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp]
        L.bsl_forward_group.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp]
        L.bsl_forward_group_static.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp]
        L.bsl_set_path.argtypes = [c_vp, c_i32]
        L.bsl_set_decode.argtypes = [c_vp, c_i32]
        L.bsl_debug_unpack.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]
        L.bsl_last_error.restype = ctypes.c_char_p
        L.bsl_last_error.argtypes = []
        L.bsl_destroy.restype = None
        L.bsl_destroy.argtypes = [c_vp]
        L.bsl_lr_equal_rank.restype = c_i32
        L.bsl_lr_equal_rank.argtypes = [c_i64, c_i64, c_i32]
        L.bsl_lr_block_bytes.restype = c_sz
        L.bsl_lr_block_bytes.argtypes = [c_i64, c_i64, c_i32]
        L.bsl_lr_init.argtypes = [ctypes.POINTER(c_vp), ctypes.c_int, c_i32, c_vp, c_vp, c_vp, c_i32]
        L.bsl_lr_set_source.argtypes = [c_vp, c_i32, c_i32, c_vp]
        L.bsl_lr_load_blocks.argtypes = [c_vp, c_vp, c_vp]
        L.bsl_lr_resident_bytes.restype = c_u64
        L.bsl_lr_resident_bytes.argtypes = [c_vp]
        L.bsl_lr_forward.argtypes = [c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp]
        L.bsl_lr_forward_group.argtypes = [c_vp, c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp]
        L.bsl_lr_destroy.restype = None
        L.bsl_lr_destroy.argtypes = [c_vp]
        for f in ("bsl_pack_signs", "bsl_unpack_signs", "bsl_init", "bsl_set_source", "bsl_load_blocks",
                  "bsl_active_blocks", "bsl_launch_counts", "bsl_forward", "bsl_forward_group", "bsl_forward_group_static", "bsl_set_path", "bsl_debug_unpack", "bsl_set_decode",
                  "bsl_set_input_scale", "bsl_lr_init", "bsl_lr_set_source", "bsl_lr_load_blocks", "bsl_lr_forward",
                  "bsl_lr_forward_group"):
            getattr(L, f).restype = c_i32
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != BSL_OK:
        raise BslError(rc, lib().bsl_last_error().decode(errors="replace"))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ------------------------------------------------------------------ host helpers
def bsl_block_bytes(m: int, d: int, k: int = 16) -> int:
    return int(lib().bsl_block_bytes(m, d, k))


def bsl_packed_sign_bytes(m: int, d: int) -> int:
    return int(lib().bsl_packed_sign_bytes(m, d))


def bsl_pack_signs(bits: np.ndarray, m: int, d: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    if bits.size != m * (d // 8):
        raise ValueError("bits must hold m * d / 8 bytes")
    out = np.empty(max(1, bsl_packed_sign_bytes(m, d)), dtype=np.uint8)
    _check(lib().bsl_pack_signs(_ptr(bits), m, d, _ptr(out)))
    return out


def bsl_unpack_signs(tiled: np.ndarray, m: int, d: int) -> np.ndarray:
    tiled = np.ascontiguousarray(tiled, dtype=np.uint8)
    if tiled.size < bsl_packed_sign_bytes(m, d):
        raise ValueError("tiled buffer too small")
    out = np.empty((m, d), dtype=np.int8)
    _check(lib().bsl_unpack_signs(_ptr(tiled), m, d, _ptr(out)))
    return out


# ------------------------------------------------------------------ stack
_sources: dict = {}  # keeps host block arrays alive while a stack may read them


def bsl_init(device: int, m, d, k: int = 16, n_cap: int = 16, budget_bytes: int = 0) -> int:
    m = np.ascontiguousarray(m, dtype=np.int32)
    d = np.ascontiguousarray(d, dtype=np.int32)
    if m.shape != d.shape or m.ndim != 1:
        raise ValueError("m and d must be 1-D of equal length")
    h = ctypes.c_void_p()
    _check(lib().bsl_init(ctypes.byref(h), device, m.size, _ptr(m), _ptr(d), k, n_cap, budget_bytes))
    return int(h.value)


def bsl_set_source(stack: int, w: int, blocks) -> None:
    """blocks: sequence of dicts with ``bits`` (uint8 [m, d/8]), ``u`` (fp16 [m, 16]), ``v`` (fp16 [d, 16])."""
    keep = []
    arr = (_BlockSrc * max(1, len(blocks)))()
    for i, b in enumerate(blocks):
        bits = np.ascontiguousarray(b["bits"], dtype=np.uint8)
        u = np.ascontiguousarray(b["u"], dtype=np.float16)
        v = np.ascontiguousarray(b["v"], dtype=np.float16)
        keep.append((bits, u, v))
        arr[i].sign_bits, arr[i].u, arr[i].v = _ptr(bits), _ptr(u), _ptr(v)
    _check(lib().bsl_set_source(stack, w, len(blocks), ctypes.addressof(arr)))
    _sources[(stack, w)] = keep


def bsl_set_input_scale(stack: int, w: int, inv_scale) -> None:
    """inv_scale: ``d`` positive floats (1 / the per-input-channel scale), or None."""
    if inv_scale is None:
        _check(lib().bsl_set_input_scale(stack, w, None))
        return
    a = np.ascontiguousarray(inv_scale, dtype=np.float32)
    _check(lib().bsl_set_input_scale(stack, w, _ptr(a)))


def bsl_load_blocks(stack: int, n_per_weight, stream: int = 0) -> None:
    n = np.ascontiguousarray(n_per_weight, dtype=np.int32)
    _check(lib().bsl_load_blocks(stack, _ptr(n), stream))


def bsl_active_blocks(stack: int, w: int) -> int:
    n = ctypes.c_int32()
    _check(lib().bsl_active_blocks(stack, w, ctypes.byref(n)))
    return int(n.value)


def bsl_resident_bytes(stack: int) -> int:
    return int(lib().bsl_resident_bytes(stack))


def bsl_workspace_bytes(stack: int) -> int:
    return int(lib().bsl_workspace_bytes(stack))


def bsl_launch_counts(stack: int) -> list:
    """Forward launches so far per kernel: [shared single-token, wave-private single- and
    few-token, factored multi-token, tile-reconstruct]."""
    c = np.zeros(BSL_KERNEL_KINDS, dtype=np.uint64)
    _check(lib().bsl_launch_counts(stack, _ptr(c)))
    return [int(v) for v in c]


def bsl_forward(stack: int, w: int, x_ptr: int, y_ptr: int, M: int, y_is_fp32: bool, stream: int = 0) -> None:
    _check(lib().bsl_forward(stack, w, x_ptr, y_ptr, M, 1 if y_is_fp32 else 0, stream))


def bsl_forward_group(stack: int, weights, x_ptrs, y_ptrs, M: int, y_is_fp32: bool, stream: int = 0) -> None:
    n = len(weights)
    ws = (ctypes.c_int32 * n)(*weights)
    xs = (ctypes.c_void_p * n)(*x_ptrs)
    ys = (ctypes.c_void_p * n)(*y_ptrs)
    _check(lib().bsl_forward_group(stack, n, ctypes.addressof(ws), ctypes.addressof(xs), ctypes.addressof(ys), M,
                                   1 if y_is_fp32 else 0, stream))


def bsl_forward_group_static(stack: int, weights, x_ptrs, y_ptrs, M: int, y_is_fp32: bool, stream: int = 0) -> None:
    n = len(weights)
    ws = (ctypes.c_int32 * n)(*weights)
    xs = (ctypes.c_void_p * n)(*x_ptrs)
    ys = (ctypes.c_void_p * n)(*y_ptrs)
    _check(lib().bsl_forward_group_static(stack, n, ctypes.addressof(ws), ctypes.addressof(xs), ctypes.addressof(ys), M,
                                          1 if y_is_fp32 else 0, stream))


def bsl_set_path(stack: int, path: int) -> None:
    _check(lib().bsl_set_path(stack, path))


def bsl_set_decode(stack: int, kind: int) -> None:
    _check(lib().bsl_set_decode(stack, kind))


def bsl_debug_unpack(stack: int, w: int, i: int, path: int, out_ptr: int, stream: int = 0) -> None:
    _check(lib().bsl_debug_unpack(stack, w, i, path, out_ptr, stream))


def bsl_last_error() -> str:
    return lib().bsl_last_error().decode(errors="replace")


def bsl_destroy(stack: int) -> None:
    if stack:
        lib().bsl_destroy(stack)
        for key in [k for k in _sources if k[0] == stack]:
            del _sources[key]


# ---------------------------------------------------------------- vanilla-SVD baseline (bitstack_lowrank.h)
def bsl_lr_equal_rank(m: int, d: int, k: int = 16) -> int:
    return int(lib().bsl_lr_equal_rank(m, d, k))


def bsl_lr_block_bytes(m: int, d: int, k_prime: int) -> int:
    return int(lib().bsl_lr_block_bytes(m, d, k_prime))


def bsl_lr_init(device: int, m, d, k_prime, n_cap: int = 16) -> int:
    m = np.ascontiguousarray(m, dtype=np.int32)
    d = np.ascontiguousarray(d, dtype=np.int32)
    kp = np.ascontiguousarray(k_prime, dtype=np.int32)
    if m.shape != d.shape or m.shape != kp.shape or m.ndim != 1:
        raise ValueError("m, d and k_prime must be 1-D of equal length")
    h = ctypes.c_void_p()
    _check(lib().bsl_lr_init(ctypes.byref(h), device, m.size, _ptr(m), _ptr(d), _ptr(kp), n_cap))
    return int(h.value)


def bsl_lr_set_source(stack: int, w: int, blocks) -> None:
    """blocks: sequence of dicts with ``u`` (fp16 [m, k']) and ``v`` (fp16 [d, k'])."""
    keep = []
    arr = (_LrBlockSrc * max(1, len(blocks)))()
    for i, b in enumerate(blocks):
        u = np.ascontiguousarray(b["u"], dtype=np.float16)
        v = np.ascontiguousarray(b["v"], dtype=np.float16)
        keep.append((u, v))
        arr[i].u, arr[i].v = _ptr(u), _ptr(v)
    _check(lib().bsl_lr_set_source(stack, w, len(blocks), ctypes.addressof(arr)))
    _sources[("lr", stack, w)] = keep


def bsl_lr_load_blocks(stack: int, n_per_weight, stream: int = 0) -> None:
    n = np.ascontiguousarray(n_per_weight, dtype=np.int32)
    _check(lib().bsl_lr_load_blocks(stack, _ptr(n), stream))


def bsl_lr_resident_bytes(stack: int) -> int:
    return int(lib().bsl_lr_resident_bytes(stack))


def bsl_lr_forward(stack: int, w: int, x_ptr: int, y_ptr: int, M: int, y_is_fp32: bool, stream: int = 0) -> None:
    _check(lib().bsl_lr_forward(stack, w, x_ptr, y_ptr, M, 1 if y_is_fp32 else 0, stream))


def bsl_lr_forward_group(stack: int, weights, x_ptrs, y_ptrs, M: int, y_is_fp32: bool, stream: int = 0) -> None:
    n = len(weights)
    ws = (ctypes.c_int32 * n)(*weights)
    xs = (ctypes.c_void_p * n)(*x_ptrs)
    ys = (ctypes.c_void_p * n)(*y_ptrs)
    _check(lib().bsl_lr_forward_group(stack, n, ctypes.addressof(ws), ctypes.addressof(xs), ctypes.addressof(ys), M,
                                      1 if y_is_fp32 else 0, stream))


def bsl_lr_destroy(stack: int) -> None:
    if stack:
        lib().bsl_lr_destroy(stack)
        for key in [k for k in _sources if k[0] == "lr" and k[1] == stack]:
            del _sources[key]
