"""Helpers for the GPU parity tests: a stack built through the C-ABI binding, torch
used only for device buffers and the stream, and error metrics against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import bit_sign_rank_amd as bsl

REL_TOL = 5e-3  # relative Frobenius error bound of the layer output vs the fp64 oracle


def stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


class Stack:
    """A bitstack_linear stack over the given weights (list of (m, d, blocks))."""

    def __init__(self, weights, n_cap=16, budget=0, device=0, path=None, decode=None):
        self.shapes = [(m, d) for m, d, _ in weights]
        self.blocks = [b for _, _, b in weights]
        self.h = bsl.bsl_init(device, [m for m, _ in self.shapes], [d for _, d in self.shapes], 16, n_cap, budget)
        if path is not None:
            bsl.bsl_set_path(self.h, path)
        if decode is not None:
            bsl.bsl_set_decode(self.h, decode)
        for w, blocks in enumerate(self.blocks):
            bsl.bsl_set_source(self.h, w, blocks)

    def load(self, counts, stream=None):
        bsl.bsl_load_blocks(self.h, counts, stream_ptr(stream))

    def forward(self, w, x: np.ndarray, fp32=True, stream=None) -> np.ndarray:
        m, d = self.shapes[w]
        xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).reshape(-1, d).cuda()
        M = xt.shape[0]
        y = torch.empty((M, m), dtype=torch.float32 if fp32 else torch.float16, device="cuda")
        bsl.bsl_forward(self.h, w, xt.data_ptr(), y.data_ptr(), M, fp32, stream_ptr(stream))
        torch.cuda.synchronize()
        return y.cpu().numpy().astype(np.float64)

    def forward_group(self, ws, xs, fp32=True) -> list:
        xts, ys = [], []
        for w, x in zip(ws, xs):
            m, d = self.shapes[w]
            xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).reshape(-1, d).cuda()
            xts.append(xt)
            ys.append(torch.empty((xt.shape[0], m), dtype=torch.float32 if fp32 else torch.float16, device="cuda"))
        M = xts[0].shape[0]
        bsl.bsl_forward_group(self.h, list(ws), [t.data_ptr() for t in xts], [t.data_ptr() for t in ys], M, fp32,
                              stream_ptr())
        torch.cuda.synchronize()
        return [y.cpu().numpy().astype(np.float64) for y in ys]

    def close(self):
        if self.h:
            torch.cuda.synchronize()
            bsl.bsl_destroy(self.h)
            self.h = 0

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


U16 = 2.0**-11  # unit roundoff of fp16
U32 = 2.0**-24  # unit roundoff of fp32


def abs_bound(x, blocks, n):
    """A[t, j] = sum_c |x[t, c]| sum_i (|U_i| |V_i|^T)[j, c]: the scale of every rounding."""
    d = x.shape[1]
    m = blocks[0]["u"].shape[0] if blocks else 0
    W = np.zeros((m, d))
    for b in blocks[:n]:
        W += np.abs(b["u"].astype(np.float64)) @ np.abs(b["v"].astype(np.float64)).T
    return np.abs(x.astype(np.float64)) @ W.T


def elem_factor(kernel, n, d):
    """Per-element error bound / A for each kernel's arithmetic (fp32 output):
    factored paths round Z = V x to fp16 once (U16) then sum in fp32 over d + 16 n terms;
    the wave-private kernels multiply V and x exactly inside the matrix core; the tile
    path rounds each block's U_i V_i^T and each running sum of W_hat to fp16 (n + 1 U16);
    the product-index kernel rounds each block's U_i V_i^T to fp16 once (U16) and sums
    all n d products in fp32."""
    acc = (d + 16 * n) * U32
    return {"z16": U16 + acc, "exact": acc, "tile": (n + 1) * U16 + acc,
            "product": U16 + (n * d + 16 * n) * U32}[kernel]


def assert_elementwise(y, ref, bound, ctx=""):
    """|y - ref| <= bound everywhere (bound: per-element array)."""
    ratio = np.abs(y - ref) / np.maximum(bound, 1e-300)
    worst = np.unravel_index(int(ratio.argmax()), ratio.shape) if ratio.size else None
    assert ratio.size == 0 or ratio.max() <= 1.0, f"{ctx}: worst element {worst} at {ratio.max():.3f} of its bound"
