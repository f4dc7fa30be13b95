"""Iterated absolute value decomposition (AVD), fp64, step by step.

What is computed (OpenReview discussion page, reply A3; paper-review page,
Figure 3 caption; abstract on the codewithpapers page):

  R_0 = W
  for i = 0 .. n-1:
      S_i = sign(R_i)                       (kept as a packed +-1 matrix)
      |R_i| ~= U_i V_i^T                    (rank-k truncated SVD of |R_i|)
      R_{i+1} = R_i - S_i * (U_i V_i^T)     (elementwise product)

Readings where the pages are silent (each listed in the design notes):
  * sign(0) is +1 (also for -0.0): a +-1 matrix has no zero.
  * The singular values are split evenly, U = P_k sqrt(Sigma_k) and
    V = Q_k sqrt(Sigma_k): the restoration code multiplies only ``u_k @ vt_k``.
  * Each singular pair is oriented so that the entry of largest magnitude in
    the right vector is positive (the SVD fixes a pair only up to a joint sign).
  * U and V are stored as fp16 (round to nearest even), and the residual is
    taken with the rounded factors, so the stored blocks and the residuals agree.
  * No activation-aware scaling is applied (the pages do not print it).
"""
from __future__ import annotations

import numpy as np

from .signs import bits_from_signs


def _orient(P: np.ndarray, Q: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Flip each singular pair so the largest-|.| entry of the right vector is > 0."""
    idx = np.argmax(np.abs(Q), axis=0)
    flip = np.where(Q[idx, np.arange(Q.shape[1])] < 0, -1.0, 1.0)
    return P * flip, Q * flip


def avd_step(R: np.ndarray, k: int, round_fp16: bool = True):
    """One AVD step on the fp64 residual ``R[m, d]``.

    Returns ``(block, R_next, sigma)`` where ``block`` has keys ``signs``
    (int8 +-1), ``bits`` (packed, set = -1), ``u`` and ``v`` (fp16, or fp64 when
    ``round_fp16`` is False), and ``sigma`` holds all singular values of |R|.
    """
    R = np.asarray(R, dtype=np.float64)
    S = np.where(R >= 0, 1, -1).astype(np.int8)
    A = np.abs(R)
    P, sigma, Qt = np.linalg.svd(A, full_matrices=False)
    Q = Qt.T
    k = min(k, sigma.size)
    Pk, Qk = _orient(P[:, :k], Q[:, :k])
    root = np.sqrt(sigma[:k])
    U = Pk * root
    V = Qk * root
    if round_fp16:
        U = U.astype(np.float16)
        V = V.astype(np.float16)
    L = U.astype(np.float64) @ V.astype(np.float64).T
    R_next = R - S * L
    block = {"signs": S, "bits": bits_from_signs(S) if R.shape[1] % 8 == 0 else None, "u": U, "v": V}
    return block, R_next, sigma


def decompose(W: np.ndarray, k: int, n: int, round_fp16: bool = True):
    """Run ``n`` AVD steps on ``W``.  Returns ``(blocks, residual_norms)`` where
    ``residual_norms[i]`` is the Frobenius norm of R_i (i = 0..n)."""
    R = np.asarray(W, dtype=np.float64)
    blocks = []
    norms = [float(np.linalg.norm(R))]
    for _ in range(n):
        block, R, _ = avd_step(R, k, round_fp16=round_fp16)
        blocks.append(block)
        norms.append(float(np.linalg.norm(R)))
    return blocks, norms
