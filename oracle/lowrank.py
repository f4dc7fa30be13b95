"""Vanilla-SVD residual blocks: the equal-size low-rank baseline ("w/o AVD").

TEST INFRASTRUCTURE ONLY (see the package docstring).

Paper-review page "BitStack: Fine-Grained Size Control ...", Figure 5 caption: in the
"w/o AVD" ablation a plain SVD replaces the absolute value decomposition, and its rank
is raised to k' = k + m n / (16 (m + n)) so that a block takes as many bytes as an AVD
block (16-bit factor entries: 2 k' (m + n) bytes against m n / 8 + 2 k (m + n)).

Readings (the caption gives only the rank):
  * k' is rounded down to an integer, so a block never exceeds an AVD block.
  * The iteration is the AVD one without signs: the block is the rank-k' truncated SVD
    of the residual itself, U = P sqrt(Sigma), V = Q sqrt(Sigma), and the next residual
    subtracts U V^T (taken with the fp16-rounded factors, as for AVD).
  * The layer with n blocks is y = x (sum_i U_i V_i^T)^T = sum_i (x V_i) U_i^T.
"""
from __future__ import annotations

import numpy as np


def equal_bytes_rank(m: int, d: int, k: int = 16) -> int:
    """Integer rank k' of a vanilla-SVD block no larger than an AVD block of rank k."""
    return k + (m * d) // (16 * (m + d))


def lowrank_block_bytes(m: int, d: int, kp: int) -> int:
    """Bytes of one vanilla-SVD block: two fp16 factors of rank ``kp``."""
    return 2 * kp * (m + d)


def svd_step(R: np.ndarray, kp: int, round_fp16: bool = True):
    """One block: the rank-``kp`` truncated SVD of the residual ``R`` (no signs).
    Returns ``(block, R_next, sigma)``; ``block`` has keys ``u`` (m x kp) and ``v``
    (d x kp), fp16 unless ``round_fp16`` is False."""
    R = np.asarray(R, dtype=np.float64)
    P, sigma, Qt = np.linalg.svd(R, full_matrices=False)
    kp = min(kp, sigma.size)
    root = np.sqrt(sigma[:kp])
    U = P[:, :kp] * root
    V = Qt[:kp].T * root
    if round_fp16:
        U = U.astype(np.float16)
        V = V.astype(np.float16)
    R_next = R - U.astype(np.float64) @ V.astype(np.float64).T
    return {"u": U, "v": V}, R_next, sigma


def decompose_svd(W: np.ndarray, kp: int, n: int, round_fp16: bool = True):
    """``n`` vanilla-SVD blocks of rank ``kp`` from ``W``.  Returns ``(blocks, norms)``
    with ``norms[i]`` the Frobenius norm of the residual after ``i`` blocks."""
    R = np.asarray(W, dtype=np.float64)
    blocks, norms = [], [float(np.linalg.norm(R))]
    for _ in range(n):
        b, R, _ = svd_step(R, kp, round_fp16=round_fp16)
        blocks.append(b)
        norms.append(float(np.linalg.norm(R)))
    return blocks, norms


def forward_lowrank(x: np.ndarray, blocks, n: int | None = None) -> np.ndarray:
    """``y[M, m] = sum_{i < n} (x V_i) U_i^T`` in fp64."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    n = len(blocks) if n is None else n
    m = np.asarray(blocks[0]["u"]).shape[0]
    y = np.zeros((x64.shape[0], m), dtype=np.float64)
    for i in range(n):
        U = np.asarray(blocks[i]["u"], dtype=np.float64)
        V = np.asarray(blocks[i]["v"], dtype=np.float64)
        y += (x64 @ V) @ U.T
    return y
