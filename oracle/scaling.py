"""Activation-aware scaling of the input channels: the layer with a scaled stack.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Paper-review page "BitStack: Fine-Grained Size Control ...", Figure 5 caption: the
"w/o scaling" ablation leaves out the activation-aware scaling of Eq. 4 before the
decomposition.  The equation is not printed on the pages; the reading taken here is
the plainest one consistent with "activation-aware": every input channel c has a
factor s[c] > 0 drawn from activation statistics, the decomposition is run on
``W diag(s)``, and the layer undoes the factor on the activations:

    W_hat_n approximates W diag(s)
    y = x W^T  ~=  (x diag(s)^-1) W_hat_n^T = (x (.) inv_scale) W_hat_n^T,
    inv_scale[c] = 1 / s[c].

The factor is given here as ``inv_scale`` (what the layer multiplies by).
"""
from __future__ import annotations

import numpy as np

from .avd import decompose
from .restore import forward


def forward_scaled(x: np.ndarray, blocks, inv_scale, n: int | None = None) -> np.ndarray:
    """``y[M, m] = (x (.) inv_scale) W_hat_n^T`` in fp64 (``inv_scale`` has one entry per
    input channel, i.e. per column of ``W_hat`` and per entry of a token)."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    s = np.asarray(inv_scale, dtype=np.float64)
    if s.shape != (x64.shape[1],):
        raise ValueError("inv_scale needs one entry per input channel")
    return forward(x64 * s[None, :], blocks, n)


def decompose_scaled(W: np.ndarray, scale, k: int, n: int, round_fp16: bool = True):
    """The decomposition of ``W diag(scale)`` (``scale`` = s, one factor per input
    channel): the blocks to use with ``forward_scaled(x, blocks, 1 / scale)``."""
    W64 = np.asarray(W, dtype=np.float64) * np.asarray(scale, dtype=np.float64)[None, :]
    return decompose(W64, k, n, round_fp16=round_fp16)
