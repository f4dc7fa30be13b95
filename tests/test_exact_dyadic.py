"""CPU checks of the exactness argument behind the GPU's bit-exact full-size pins.

The pins use residual blocks whose factor entries are 1/4 or 1/2 (``synth.dyadic_factor``,
drawn per row, column and rank) and integer activations.  Then, with rank k = 16:

  * every entry of U_i V_i^T is a sum of 16 products in {1/16, 1/8, 1/4}: a multiple of
    1/16 in [1, 4], exact in fp16 (at most 7 significant bits);
  * every partial sum of W_hat = sum_i S_i (U_i V_i^T) over n <= 16 blocks is a multiple
    of 1/16 of magnitude <= 4 n <= 64, exact in fp16 (at most 11 significant bits);
  * every Z = V x is an fp16 number exactly (|x| <= 2);
  * every partial sum of y is a multiple of 1/16 of magnitude <= max|x| 4 n d, so while
    max|x| 4 n d < 2^20 every one is exact in fp32 (24 significant bits), whatever the
    summation order, split or path.

So the GPU must reproduce the fp64 oracle bit for bit in fp32 output, on every path.
These tests check each claim with plain numpy on small and on the largest shapes the
GPU pins use, and that such a pin, unlike one with constant factors, is sensitive to
the rank pairing and to the row / column indexing of the factors.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

K = 16


def test_factor_entries_are_quarter_or_half():
    u = synth.dyadic_factor(1, 1000, K, 3)
    assert set(np.unique(u.astype(np.float64)).tolist()) == {0.25, 0.5}
    # both values occur in every rank column and the draw differs per tag
    assert all(len(np.unique(u[:, r])) == 2 for r in range(K))
    assert not np.array_equal(u, synth.dyadic_factor(1, 1000, K, 4))


def test_low_rank_product_is_on_the_sixteenth_grid_and_exact_in_fp16():
    u = synth.dyadic_factor(2, 256, K, 0).astype(np.float64)
    v = synth.dyadic_factor(2, 512, K, 1).astype(np.float64)
    L = u @ v.T
    assert L.min() >= 1.0 and L.max() <= 4.0
    assert np.array_equal(L * 16, np.round(L * 16))
    assert np.array_equal(L.astype(np.float16).astype(np.float64), L)


def test_running_fp16_sum_over_sixteen_blocks_is_exact():
    m, d, n = 64, 256, 16
    blocks = synth.dyadic_blocks(3, m, d, n)
    acc16 = np.zeros((m, d), np.float16)
    for i in range(n):
        L = (blocks[i]["u"].astype(np.float64) @ blocks[i]["v"].astype(np.float64).T).astype(np.float16)
        S = oracle.signs_from_bits(blocks[i]["bits"], d).astype(np.float16)
        acc16 = (acc16 + S * L).astype(np.float16)  # each step rounded to fp16, as the tile path does
    assert np.array_equal(acc16.astype(np.float64), oracle.reconstruct(blocks, n))


def _fp32_sum_orders(x, blocks, n, chunk):
    """y accumulated in fp32 from fp64-exact products in two orders: columns forward per
    block, and blocks and column chunks reversed."""
    m = blocks[0]["u"].shape[0]
    d = x.shape[1]
    terms = []
    for i in range(n):
        L = blocks[i]["u"].astype(np.float64) @ blocks[i]["v"].astype(np.float64).T
        S = oracle.signs_from_bits(blocks[i]["bits"], d).astype(np.float64)
        terms.append(x.astype(np.float64)[:, None, :] * (S * L)[None, :, :])  # [M, m, d] exact products
    fwd = np.zeros((x.shape[0], m), np.float32)
    for t in terms:
        for c in range(d):
            fwd = (fwd + t[:, :, c].astype(np.float32)).astype(np.float32)
    rev = np.zeros((x.shape[0], m), np.float32)
    for t in reversed(terms):
        for c0 in range(d - chunk, -1, -chunk):
            part = np.zeros((x.shape[0], m), np.float32)
            for c in range(c0, c0 + chunk):
                part = (part + t[:, :, c].astype(np.float32)).astype(np.float32)
            rev = (rev + part).astype(np.float32)
    return fwd, rev


def test_fp32_accumulation_is_order_independent_under_the_bound():
    m, d, n, M = 8, 512, 16, 2
    blocks = synth.dyadic_blocks(4, m, d, n)
    x = synth.integer_activations(4, M, d, -1, 1)
    assert 1 * 4 * n * d < 2**20
    ref = oracle.forward(x, blocks, n)
    fwd, rev = _fp32_sum_orders(x, blocks, n, chunk=64)
    assert np.array_equal(fwd.astype(np.float64), ref)
    assert np.array_equal(rev.astype(np.float64), ref)


def test_exactness_bound_holds_for_the_full_size_pins():
    # (max |x|, largest block count, largest d) of each GPU pin: 8B-shaped layer at n = 8
    # with x in [-2, 2]; 8B-shaped variable counts (n <= 16) and the 70B-shaped layer
    # (n <= 6, d up to 28672) with x in [-1, 1]
    for xmax, n, d in ((2, 8, 14336), (1, 16, 14336), (1, 6, 28672)):
        assert xmax * 4 * n * d < 2**20


def test_dyadic_pin_sees_rank_pairing_and_factor_indexing():
    # A kernel that paired U's rank r with V's rank r' != r, read U transposed within a
    # tile, or took V from a neighbouring column would still pass a pin with constant
    # factors (U V^T == 1 whatever the indexing); with dyadic factors the exact output
    # changes.
    m, d, n = 32, 64, 2
    blocks = synth.dyadic_blocks(5, m, d, n)
    x = synth.integer_activations(5, 2, d)
    ref = oracle.forward(x, blocks, n)
    perm = np.roll(np.arange(K), 1)
    swapped_rank = [{**b, "u": b["u"][:, perm]} for b in blocks]
    row_shift = [{**b, "u": np.roll(b["u"], 1, axis=0)} for b in blocks]
    col_shift = [{**b, "v": np.roll(b["v"], 1, axis=0)} for b in blocks]
    for wrong in (swapped_rank, row_shift, col_shift):
        assert not np.array_equal(oracle.forward(x, wrong, n), ref)
    const = [{**b, "u": np.full((m, K), 0.25, np.float16), "v": np.full((d, K), 0.25, np.float16)} for b in blocks]
    const_rank = [{**b, "u": b["u"][:, perm]} for b in const]
    assert np.array_equal(oracle.forward(x, const_rank, n), oracle.forward(x, const, n))
