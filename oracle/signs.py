"""Sign matrix <-> packed sign bits, the oracle's own conversion.

The residual block's sign matrix holds only +1 and -1 and is stored packed
(paper-review page, Figure 3 caption).  The pages do not fix the bit order or
polarity; the reading used here (and by the input generators) is: row-major,
``d/8`` bytes per row, least significant bit = lowest column, bit set = -1.
"""
from __future__ import annotations

import numpy as np


def signs_from_bits(bits: np.ndarray, d: int | None = None) -> np.ndarray:
    """``uint8[m, d/8]`` packed bits -> ``int8[m, d]`` matrix of +1 / -1."""
    bits = np.asarray(bits, dtype=np.uint8)
    flags = np.unpackbits(bits, axis=1, bitorder="little")
    if d is not None:
        flags = flags[:, :d]
    return (1 - 2 * flags.astype(np.int8)).astype(np.int8)


def bits_from_signs(signs: np.ndarray) -> np.ndarray:
    """``[m, d]`` matrix of +1 / -1 -> ``uint8[m, d/8]`` packed bits (set = -1)."""
    signs = np.asarray(signs)
    if signs.shape[1] % 8:
        raise ValueError("d must be a multiple of 8")
    return np.packbits(signs < 0, axis=1, bitorder="little")
