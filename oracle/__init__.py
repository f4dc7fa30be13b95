"""CPU oracle for the BitStack residual-block linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
imports, links or calls it, and it shares no code, header, table or constant
with the HIP library: it is a plain, slow, fp64 statement of what the layer
computes, written from the pages that describe the method:

* "BitStack" GitHub README (xinghaow99/BitStack), sections "Decomposition" and
  "Evaluation": ``--niter`` decomposition iterations and ``--k`` singular vectors.
* Paper-review page "BitStack: Fine-Grained Size Control for Compressed Large
  Language Models in Variable Memory Environments", Figure 3 caption: a residual
  block is a +-1 sign matrix (packed into GPU data types) plus singular vectors
  from an absolute value decomposition (AVD); Figure 5 caption: the equal-size
  rank k' of a vanilla-SVD block.
* Same page, Figure 5 caption: the "w/o scaling" ablation (activation-aware scaling
  of Eq. 4, whose formula the pages do not print; see ``scaling`` for the reading).
* Abstract (codewithpapers page "BitStack: Any-Size Compression of Large Language
  Models in Variable Memory Environments"): each decomposition iteration yields an
  approximately 1-bit-per-parameter residual block.
* OpenReview discussion (paperhub page for the ICLR 2025 submission), reply A3:
  SVD is applied to the absolute value of the previous approximation error, and
  the sign matrix is kept; the later reply on weight restoration: the weight is
  the sum over blocks of the unpacked signs times ``u_k @ vt_k``; reply A1.A: the
  largest residual block of an 8B model is 7.56 MB.

Modules:
  signs    -- row-major sign-bit <-> +-1 conversion (the input format)
  avd      -- one absolute-value-decomposition step and the iterated decomposition
  restore  -- dense fp64 reconstruct-then-matmul forward, block byte count
  scaling  -- the layer with an input-channel scale (activation-aware scaling)
  lowrank  -- vanilla-SVD blocks of the equal-size rank k' and their forward

Parity status: every function is pinned by ``tests/test_oracle.py`` against
closed forms, invariants, special cases and brute force (see the list there).
"""
from .signs import signs_from_bits, bits_from_signs  # noqa: F401
from .avd import avd_step, decompose  # noqa: F401
from .restore import reconstruct, forward, forward_rows, block_bytes  # noqa: F401
from .scaling import forward_scaled, decompose_scaled  # noqa: F401
from .lowrank import equal_bytes_rank, lowrank_block_bytes, svd_step, decompose_svd, forward_lowrank  # noqa: F401
