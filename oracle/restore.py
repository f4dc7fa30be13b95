"""Dense fp64 reconstruct-then-matmul: the plain definition of the layer.

Restoration (OpenReview discussion page, the authors' reply giving the weight
restoration code): start from a zero ``out_features x in_features`` matrix and,
for every loaded block, add the unpacked sign matrix times ``u_k @ vt_k``:

    W_hat_n = sum_{i < n} S_i * (U_i V_i^T)          (elementwise *)

and the layer output is ``y = x W_hat_n^T``.  Everything here is fp64 from the
stored values (fp16 U, V and x upcast exactly, S as +-1).  With n = 0 the sum is
empty and y = 0.

Block size (paper-review page, Figure 5 caption, and the OpenReview reply A1.A):
a block stores the m x d signs at 1 bit each and the two rank-k factors at
16 bits per entry, so it takes m*d/8 + 2*k*(m + d) bytes.
"""
from __future__ import annotations

import numpy as np

from .signs import signs_from_bits


def reconstruct(blocks, n: int | None = None, rows=None) -> np.ndarray:
    """fp64 ``W_hat`` from the first ``n`` blocks (all rows, or the listed rows)."""
    n = len(blocks) if n is None else n
    u0 = np.asarray(blocks[0]["u"])
    v0 = np.asarray(blocks[0]["v"])
    m, d = u0.shape[0], v0.shape[0]
    sel = np.arange(m) if rows is None else np.asarray(rows)
    W = np.zeros((sel.size, d), dtype=np.float64)
    for i in range(n):
        b = blocks[i]
        U = np.asarray(b["u"], dtype=np.float64)[sel]
        V = np.asarray(b["v"], dtype=np.float64)
        if "signs" in b and b["signs"] is not None:
            S = np.asarray(b["signs"], dtype=np.float64)[sel]
        else:
            S = signs_from_bits(np.asarray(b["bits"])[sel], d).astype(np.float64)
        W += S * (U @ V.T)
    return W


def forward(x: np.ndarray, blocks, n: int | None = None) -> np.ndarray:
    """``y[M, m] = x W_hat_n^T`` in fp64 (``x`` is ``[M, d]`` or ``[d]``)."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n = len(blocks) if n is None else n
    if n == 0:
        m = np.asarray(blocks[0]["u"]).shape[0]
        return np.zeros((x64.shape[0], m), dtype=np.float64)
    return x64 @ reconstruct(blocks, n).T


def forward_rows(x: np.ndarray, blocks, rows, n: int | None = None) -> np.ndarray:
    """The listed output columns of ``forward`` (rows of W_hat), ``[M, len(rows)]``."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n = len(blocks) if n is None else n
    rows = np.asarray(rows)
    if n == 0:
        return np.zeros((x64.shape[0], rows.size), dtype=np.float64)
    return x64 @ reconstruct(blocks, n, rows=rows).T


def block_bytes(m: int, d: int, k: int) -> int:
    """Bytes of one residual block: 1-bit signs plus two fp16 rank-k factors."""
    return m * d // 8 + 2 * k * (m + d)
