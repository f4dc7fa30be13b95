"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value:
  * values printed on the pages (block size 7.56 MB; the equal-size rank k'),
  * closed forms (energy drop of one AVD step, Eckart-Young),
  * invariants (non-increasing residual, sign/magnitude split, Perron-Frobenius),
  * special cases that reduce to a textbook routine (full rank, signed rank 1,
    non-negative weight, integer forward),
  * brute force with exact rational arithmetic on tiny shapes.
A plausible mistake in the oracle (SVD of R instead of |R|, a dropped sign, a
transposed factor, a wrong residual update, wrong bit order) fails at least one
of them; ``test_planted_mistakes_are_caught`` checks that for a few mutants.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import avd as oavd
from oracle import lowrank as olowrank
from oracle import restore as orest
from oracle import scaling as oscaling
from oracle import signs as osigns
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- block bytes
def _golden_block_sizes():
    rows = []
    with open(os.path.join(GOLDEN, "residual_block_size.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                m, d, k, mb = line.split()
                rows.append((int(m), int(d), int(k), float(mb)))
    return rows


@pytest.mark.parametrize("m,d,k,mb", _golden_block_sizes())
def test_block_bytes_match_printed_size(m, d, k, mb):
    b = oracle.block_bytes(m, d, k)
    assert b == 7_929_856
    assert round(b / 2**20, 2) == mb


@pytest.mark.parametrize("m,d", [(4096, 4096), (1024, 4096), (14336, 4096), (8192, 28672), (1024, 1024)])
def test_block_bytes_equal_vanilla_svd_rank(m, d):
    # Figure 5 caption: a vanilla-SVD block of rank k' = k + m d / (16 (m + d)) has the
    # same size as an AVD block, with 16-bit factor entries: 2 k' (m + d) bytes.
    k = 16
    kp = Fraction(k) + Fraction(m * d, 16 * (m + d))
    assert 2 * kp * (m + d) == oracle.block_bytes(m, d, k)


# ---------------------------------------------------------------- sign bits
def _bit_order_pin_holds():
    # bit order: LSB of byte 0 is column 0, set bit is -1
    one = np.zeros((1, 2), np.uint8)
    one[0, 0] = 0b0000_0101
    one[0, 1] = 0b1000_0000
    s1 = osigns.signs_from_bits(one)[0]
    return s1.tolist() == [-1, 1, -1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, -1]


def test_sign_bits_round_trip_and_order():
    bits = synth.sign_bits(3, 5, 24)
    s = osigns.signs_from_bits(bits)
    assert s.dtype == np.int8 and set(np.unique(s)) <= {-1, 1}
    assert np.array_equal(osigns.bits_from_signs(s), bits)
    assert _bit_order_pin_holds()


def test_sign_of_zero_is_plus_one():
    R = np.array([[0.0, -0.0, 1e-300, -1e-300, 2.0, -3.0, 0.0, -0.0]])
    blk, _, _ = oavd.avd_step(R, 1)
    assert blk["signs"].tolist() == [[1, 1, 1, -1, 1, -1, 1, 1]]


# ---------------------------------------------------------------- one AVD step
def test_avd_step_energy_drop_closed_form():
    # With exact factors, R_next = S * (|R| - L) and L is the best rank-k approximation
    # of |R| (Eckart-Young), so ||R_next||^2 = ||R||^2 - sum_{j<k} sigma_j(|R|)^2.
    R = synth.gaussian_weight(11, 40, 28).astype(np.float64)
    for k in (1, 3, 7):
        _, Rn, sigma = oavd.avd_step(R, k, round_fp16=False)
        lhs = np.sum(Rn**2)
        rhs = np.sum(R**2) - np.sum(sigma[:k] ** 2)
        assert abs(lhs - rhs) <= 1e-10 * np.sum(R**2)


def test_sign_magnitude_split_is_exact():
    R = synth.gaussian_weight(5, 33, 16).astype(np.float64)
    blocks, _ = oavd.decompose(R, 4, 3)
    Ri = R
    for b in blocks:
        assert np.array_equal(b["signs"] * np.abs(Ri), Ri)
        L = b["u"].astype(np.float64) @ b["v"].astype(np.float64).T
        Ri = Ri - b["signs"] * L


def test_singular_values_match_eigh():
    # textbook route: sigma(A) = sqrt(eig(A^T A))
    R = synth.gaussian_weight(7, 9, 6).astype(np.float64)
    _, _, sigma = oavd.avd_step(R, 2, round_fp16=False)
    ev = np.sort(np.linalg.eigvalsh(np.abs(R).T @ np.abs(R)))[::-1]
    assert np.allclose(sigma, np.sqrt(np.clip(ev, 0, None)), rtol=1e-10, atol=1e-12)


def test_top_vectors_nonnegative_perron_frobenius():
    # |R| is entrywise non-negative, so its top singular vectors can be taken >= 0
    # (Perron-Frobenius).  An SVD of R itself would give mixed signs.
    R = synth.gaussian_weight(9, 64, 48).astype(np.float64)
    blk, _, _ = oavd.avd_step(R, 4, round_fp16=False)
    assert np.all(blk["u"][:, 0] >= 0) and np.all(blk["v"][:, 0] >= 0)


def test_residual_nonincreasing_with_fp16_factors():
    W = synth.gaussian_weight(0, 96, 128)
    _, norms = oracle.decompose(W, 8, 6)
    assert all(b <= a * (1 + 1e-12) for a, b in zip(norms, norms[1:]))
    assert norms[-1] < 0.5 * norms[0]


def test_gaussian_first_step_ratio():
    # For W with i.i.d. N(0, s^2) entries, |W| has mean s sqrt(2/pi); the rank-1 mean
    # part already leaves ||W|| sqrt(1 - 2/pi), and rank 16 removes a little more.
    W = synth.gaussian_weight(0, 256, 256)
    _, norms = oracle.decompose(W, 16, 1)
    r = norms[1] / norms[0]
    assert 0.50 < r < np.sqrt(1 - 2 / np.pi) + 0.005


# ---------------------------------------------------------------- special cases
def test_full_rank_single_block_reproduces_weight():
    W = synth.gaussian_weight(2, 12, 16).astype(np.float64)
    blocks, _ = oracle.decompose(W, 12, 1)
    What = orest.reconstruct(blocks, 1)
    # only fp16 rounding of the factors remains: |err| <= sum_r |u_r v_r| 2^-10
    U = blocks[0]["u"].astype(np.float64)
    V = blocks[0]["v"].astype(np.float64)
    bound = (np.abs(U) @ np.abs(V).T) * 2.0**-10 + 1e-12
    assert np.all(np.abs(What - W) <= bound)
    assert np.abs(What - W).max() < 1e-2 * np.abs(W).max()


def test_signed_rank_one_is_exact_for_avd_not_for_svd():
    g = synth.rng(4)
    a = 0.5 + g.random(10)
    b = 0.5 + g.random(16)
    s = np.where(g.random((10, 16)) < 0.5, -1.0, 1.0)
    W = s * np.outer(a, b)
    blocks, norms = oracle.decompose(W, 1, 1)
    assert norms[1] < 2e-3 * norms[0]  # only fp16 rounding left
    # vanilla rank-1 SVD of W itself cannot capture the random signs
    Ps, ss, Qs = np.linalg.svd(W)
    assert np.linalg.norm(W - ss[0] * np.outer(Ps[:, 0], Qs[0])) > 0.5 * norms[0]


def test_nonnegative_weight_is_plain_low_rank():
    g = synth.rng(8)
    W = g.random((20, 24))
    blocks, _ = oracle.decompose(W, 3, 1)
    assert np.all(blocks[0]["signs"] == 1)
    x = synth.activations(1, 3, 24)
    U = blocks[0]["u"].astype(np.float64)
    V = blocks[0]["v"].astype(np.float64)
    expect = (x.astype(np.float64) @ V) @ U.T  # x (U V^T)^T, associated the other way
    assert np.allclose(oracle.forward(x, blocks, 1), expect, rtol=1e-12, atol=1e-12)


def _integer_pin_holds():
    # U = V = 0.25 with k = 16 gives U V^T == 1, so W_hat = sum_i S_i and y = x sum_i S_i^T
    # (the expected value uses numpy's own unpacking, not the oracle's).
    m, d, n, k = 48, 64, 3, 16
    blocks = []
    for i in range(n):
        bits = synth.sign_bits(21, m, d, i)
        blocks.append({"bits": bits, "u": np.full((m, k), 0.25, np.float16), "v": np.full((d, k), 0.25, np.float16)})
    x = synth.integer_activations(3, 2, d)
    Ssum = sum(1 - 2 * np.unpackbits(b["bits"], axis=1, bitorder="little").astype(np.int64) for b in blocks)
    expect = x.astype(np.int64) @ Ssum.T
    return np.array_equal(oracle.forward(x, blocks, n), expect.astype(np.float64))


def test_integer_forward_is_exact_sign_sum():
    assert _integer_pin_holds()


def test_zero_blocks_give_zero_output():
    blocks = synth.synthetic_blocks(1, 16, 32, 2, 4)
    y = oracle.forward(synth.activations(1, 2, 32), blocks, 0)
    assert y.shape == (2, 16) and not y.any()


# ---------------------------------------------------------------- brute force
def _brute_force(x, blocks, n, inv_scale=None):
    M, d = x.shape
    m, k = blocks[0]["u"].shape
    sf = [Fraction(1)] * d if inv_scale is None else [Fraction(float(v)) for v in inv_scale]
    xf = [[Fraction(float(v)) * sf[c] for c, v in enumerate(row)] for row in x]
    out = []
    for t in range(M):
        row = []
        for j in range(m):
            acc = Fraction(0)
            for i in range(n):
                S = osigns.signs_from_bits(blocks[i]["bits"], d)
                for c in range(d):
                    w = sum(Fraction(float(blocks[i]["u"][j, r])) * Fraction(float(blocks[i]["v"][c, r])) for r in range(k))
                    acc += int(S[j, c]) * w * xf[t][c]
            row.append(acc)
        out.append(row)
    return out


@pytest.mark.parametrize("m,d,k,n,M", [(3, 8, 1, 1, 1), (5, 8, 2, 3, 2), (8, 16, 2, 2, 1)])
def test_forward_matches_exact_rational_brute_force(m, d, k, n, M):
    blocks = synth.synthetic_blocks(17, m, d, n, k)
    x = synth.activations(2, M, d)
    exact = _brute_force(x, blocks, n)
    y = oracle.forward(x, blocks, n)
    for t in range(M):
        for j in range(m):
            e = float(exact[t][j])
            assert abs(y[t, j] - e) <= 1e-15 * max(1.0, abs(e)) * d * n


def test_forward_rows_agrees_with_full_forward():
    blocks = synth.synthetic_blocks(5, 64, 32, 3, 4)
    x = synth.activations(5, 3, 32)
    rows = synth.sample_rows(5, 64, 9)
    assert np.array_equal(oracle.forward_rows(x, blocks, rows), oracle.forward(x, blocks)[:, rows])


# ---------------------------------------------------------------- input-channel scale
@pytest.mark.parametrize("m,d,k,n,M", [(3, 8, 1, 1, 1), (5, 16, 2, 3, 2), (8, 8, 2, 2, 2)])
def test_forward_scaled_matches_exact_rational_brute_force(m, d, k, n, M):
    blocks = synth.synthetic_blocks(19, m, d, n, k)
    x = synth.activations(4, M, d)
    s = synth.inv_input_scale(6, d)
    exact = _brute_force(x, blocks, n, inv_scale=s)
    y = oracle.forward_scaled(x, blocks, s, n)
    for t in range(M):
        for j in range(m):
            e = float(exact[t][j])
            assert abs(y[t, j] - e) <= 1e-15 * max(1.0, abs(e)) * d * n


def test_forward_scaled_with_unit_scale_is_the_layer():
    blocks = synth.synthetic_blocks(3, 48, 64, 3)
    x = synth.activations(3, 5, 64)
    assert np.array_equal(oracle.forward_scaled(x, blocks, np.ones(64, np.float32)), oracle.forward(x, blocks))
    assert np.array_equal(oracle.forward_scaled(x, blocks, np.ones(64), 0), np.zeros((5, 48)))


def test_input_scale_folds_into_v_exactly():
    """Column scaling commutes with the elementwise sign product:
    (S (.) U V^T) diag(t) = S (.) U (diag(t) V)^T.  With power-of-two factors (and no
    underflow) the folded V is exact in fp16, so both sides agree to fp64 rounding."""
    m, d, n = 40, 96, 3
    blocks = synth.synthetic_blocks(8, m, d, n)
    # factors 1..8 (dividing could push small V entries into fp16 subnormals)
    t = np.ldexp(1.0, synth.rng(8, 99).integers(0, 4, size=d)).astype(np.float32)
    folded = [{"bits": b["bits"], "u": b["u"], "v": (b["v"].astype(np.float64) * t[:, None]).astype(np.float16)} for b in blocks]
    for b, f in zip(blocks, folded):
        assert np.array_equal(f["v"].astype(np.float64), b["v"].astype(np.float64) * t[:, None])
    x = synth.activations(8, 4, d)
    ref = oracle.forward_scaled(x, blocks, t)
    assert np.abs(oracle.forward(x, folded) - ref).max() <= 1e-13 * np.abs(ref).max()
    # the same factors on the output channels instead give another layer
    assert np.abs(oracle.forward(x, blocks) * 1.0 - ref).max() > 1e-3 * np.abs(ref).max()


def test_scaled_decomposition_restores_w():
    """decompose_scaled stores W diag(s): undoing s on the columns of its restoration
    gives back W within the residual left after n blocks."""
    W = synth.gaussian_weight(12, 64, 96)
    s = 1.0 / synth.inv_input_scale(12, 96).astype(np.float64)
    blocks, norms = oracle.decompose_scaled(W, s, 16, 6, round_fp16=False)
    R = W.astype(np.float64) * s[None, :] - orest.reconstruct(blocks)
    assert abs(np.linalg.norm(R) - norms[-1]) <= 1e-9 * norms[0]
    assert norms[-1] < 0.5 * norms[0]


def test_scaling_lowers_output_error_under_outlier_channels():
    """The direction of the "w/o scaling" ablation (Figure 5 caption) on synthetic
    activations with outlier channels: at the same block count, decomposing W diag(s)
    with s = channel magnitude^0.5 and undoing s on x leaves a smaller output error
    than decomposing W itself."""
    m = d = 256
    W = synth.gaussian_weight(14, m, d)
    mag = synth.channel_magnitudes(14, d, outlier_frac=0.03)
    x = synth.outlier_activations(14, 64, d, mag)
    y = x.astype(np.float64) @ W.astype(np.float64).T
    s = np.sqrt(mag.astype(np.float64))
    plain, _ = oracle.decompose(W, 16, 4)
    scaled, _ = oracle.decompose_scaled(W, s, 16, 4)
    err_plain = np.linalg.norm(oracle.forward(x, plain) - y)
    err_scaled = np.linalg.norm(oracle.forward_scaled(x, scaled, 1.0 / s) - y)
    assert err_scaled < 0.9 * err_plain


# ---------------------------------------------------------------- vanilla-SVD blocks ("w/o AVD")
def _brute_force_lowrank(x, blocks, n):
    M, d = x.shape
    m, kp = blocks[0]["u"].shape
    xf = [[Fraction(float(v)) for v in row] for row in x]
    out = []
    for t in range(M):
        row = []
        for j in range(m):
            acc = Fraction(0)
            for i in range(n):
                for c in range(d):
                    for r in range(kp):
                        acc += Fraction(float(blocks[i]["u"][j, r])) * Fraction(float(blocks[i]["v"][c, r])) * xf[t][c]
            row.append(acc)
        out.append(row)
    return out


def _lowrank_blocks(seed, m, d, kp, n):
    return [{"u": synth.factor(seed, m, kp, i, 0), "v": (synth.factor(seed, d, kp, i, 1) * np.float16(-1) ** i)} for i in range(n)]


@pytest.mark.parametrize("m,d,kp,n,M", [(3, 8, 2, 1, 1), (5, 8, 3, 2, 2), (6, 6, 2, 2, 1)])
def test_forward_lowrank_matches_exact_rational_brute_force(m, d, kp, n, M):
    blocks = _lowrank_blocks(9, m, d, kp, n)
    x = synth.activations(9, M, d)
    exact = _brute_force_lowrank(x, blocks, n)
    y = oracle.forward_lowrank(x, blocks, n)
    for t in range(M):
        for j in range(m):
            e = float(exact[t][j])
            assert abs(y[t, j] - e) <= 1e-15 * max(1.0, abs(e)) * d * n * kp


@pytest.mark.parametrize("m,d", [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (8192, 28672), (37, 520)])
def test_equal_bytes_rank_is_the_largest_that_fits(m, d):
    kp = oracle.equal_bytes_rank(m, d, 16)
    assert oracle.lowrank_block_bytes(m, d, kp) <= oracle.block_bytes(m, d, 16) < oracle.lowrank_block_bytes(m, d, kp + 1)


def test_equal_bytes_rank_values():
    # k' for the 8B-shaped layer's q/o, k/v and gate/up/down shapes
    assert [oracle.equal_bytes_rank(m, d) for m, d in [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]] == [144, 67, 215, 215]


def test_svd_iteration_follows_eckart_young():
    """With exact factors the i-th residual is W minus its best rank i k' approximation:
    ||R_i||^2 = sum of the squared singular values of W past index i k'."""
    W = synth.gaussian_weight(15, 48, 40).astype(np.float64)
    sig = np.linalg.svd(W, compute_uv=False)
    kp, n = 5, 8  # n kp = 40 = rank of W: the last residual is zero
    blocks, norms = oracle.decompose_svd(W, kp, n, round_fp16=False)
    for i in range(n + 1):
        assert abs(norms[i] ** 2 - np.sum(sig[i * kp:] ** 2)) <= 1e-10 * np.sum(sig ** 2)
    x = synth.activations(15, 3, 40)
    full = x.astype(np.float64) @ W.T
    assert np.abs(oracle.forward_lowrank(x, blocks) - full).max() <= 1e-10 * np.abs(full).max()


def test_svd_block_of_a_low_rank_weight_is_exact():
    g = synth.rng(16, 1)
    W = g.standard_normal((30, 3)) @ g.standard_normal((3, 24))
    blocks, norms = oracle.decompose_svd(W, 4, 1, round_fp16=False)
    assert norms[1] <= 1e-12 * norms[0]
    assert blocks[0]["u"].shape == (30, 4) and blocks[0]["v"].shape == (24, 4)


def test_avd_beats_svd_at_equal_bytes_on_a_gaussian_weight():
    """The direction of the "w/o AVD" ablation (Figure 5 caption) on a synthetic
    Gaussian weight: at the same block count and block size, AVD blocks leave a smaller
    output error than vanilla-SVD blocks of rank k'."""
    m = d = 256
    W = synth.gaussian_weight(17, m, d)
    x = synth.activations(17, 16, d)
    y = x.astype(np.float64) @ W.astype(np.float64).T
    n = 4
    avd, _ = oracle.decompose(W, 16, n)
    svd, _ = oracle.decompose_svd(W, oracle.equal_bytes_rank(m, d), n)
    e_avd = np.linalg.norm(oracle.forward(x, avd) - y)
    e_svd = np.linalg.norm(oracle.forward_lowrank(x, svd) - y)
    assert e_avd < 0.5 * e_svd


# ---------------------------------------------------------------- planted mistakes
def _mutant_svd_of_R(R, k, round_fp16=True):
    R = np.asarray(R, dtype=np.float64)
    S = np.where(R >= 0, 1, -1).astype(np.int8)
    P, sigma, Qt = np.linalg.svd(R, full_matrices=False)  # mistake: R instead of |R|
    U = (P[:, :k] * np.sqrt(sigma[:k])).astype(np.float16)
    V = (Qt.T[:, :k] * np.sqrt(sigma[:k])).astype(np.float16)
    L = U.astype(np.float64) @ V.astype(np.float64).T
    return {"signs": S, "bits": None, "u": U, "v": V}, R - S * L, sigma


def _mutant(module, old: str, new: str):
    """A copy of an oracle module with one planted mistake: its source with `old`
    (which must occur exactly once) replaced by `new`, run as a fresh module."""
    import inspect
    import types
    src = inspect.getsource(module)
    assert src.count(old) == 1, old
    m = types.ModuleType(module.__name__ + "_mutant")
    m.__package__ = module.__package__
    exec(compile(src.replace(old, new), module.__file__ + " (mutant)", "exec"), m.__dict__)
    return m


def test_planted_mistakes_are_caught(monkeypatch):
    # 1) SVD of R instead of |R| breaks Perron-Frobenius orientation / energy pin.
    monkeypatch.setattr(oavd, "avd_step", _mutant_svd_of_R)
    R = synth.gaussian_weight(9, 64, 48).astype(np.float64)
    blk, Rn, sigma = oavd.avd_step(R, 4)
    assert not (np.all(blk["u"][:, 0] >= 0) and np.all(blk["v"][:, 0] >= 0))
    monkeypatch.undo()
    # 2) a restoration that drops the sign matrix fails the integer pin
    monkeypatch.setattr(orest, "signs_from_bits", lambda bits, d=None: np.ones_like(osigns.signs_from_bits(bits, d)))
    assert not _integer_pin_holds()
    monkeypatch.undo()
    assert _integer_pin_holds()
    # 3) an unpacking with the opposite bit order (most significant bit first) fails the
    # bit-order pin, and so does one with the opposite polarity
    real = osigns.signs_from_bits
    monkeypatch.setattr(osigns, "signs_from_bits", lambda bits, d=None: real(np.asarray(bits)[:, ::-1], d)[:, ::-1])
    assert not _bit_order_pin_holds()
    monkeypatch.setattr(osigns, "signs_from_bits", lambda bits, d=None: -real(bits, d))
    assert not _bit_order_pin_holds()
    monkeypatch.undo()
    assert _bit_order_pin_holds()
    # 4) a transposed product (x W instead of x W^T) fails brute force on a square shape
    blocks = synth.synthetic_blocks(17, 8, 8, 2, 2)
    xx = synth.activations(2, 1, 8)
    exact = np.array([[float(v) for v in row] for row in _brute_force(xx, blocks, 2)])
    mut = _mutant(orest, "return x64 @ reconstruct(blocks, n).T", "return x64 @ reconstruct(blocks, n)")
    assert np.abs(mut.forward(xx, blocks, 2) - exact).max() > 1e-3 * np.abs(exact).max()
    assert np.abs(oracle.forward(xx, blocks, 2) - exact).max() <= 1e-13 * np.abs(exact).max()
    # 5) the input-channel factor applied to the output channels fails brute force
    t = synth.inv_input_scale(6, 8)
    exact = np.array([[float(v) for v in row] for row in _brute_force(xx, blocks, 2, inv_scale=t)])
    mut = _mutant(oscaling, "return forward(x64 * s[None, :], blocks, n)", "return forward(x64, blocks, n) * s[None, :]")
    assert np.abs(mut.forward_scaled(xx, blocks, t, 2) - exact).max() > 1e-3 * np.abs(exact).max()
    assert np.abs(oracle.forward_scaled(xx, blocks, t, 2) - exact).max() <= 1e-13 * np.abs(exact).max()
    # 6) a low-rank forward with the factors swapped (x U V^T) fails brute force
    lb = _lowrank_blocks(9, 6, 6, 2, 2)
    xs = synth.activations(9, 1, 6)
    exact = np.array([[float(v) for v in row] for row in _brute_force_lowrank(xs, lb, 2)])
    mut = _mutant(olowrank, "y += (x64 @ V) @ U.T", "y += (x64 @ U) @ V.T")
    assert np.abs(mut.forward_lowrank(xs, lb, 2) - exact).max() > 1e-3 * np.abs(exact).max()
    assert np.abs(olowrank.forward_lowrank(xs, lb, 2) - exact).max() <= 1e-13 * np.abs(exact).max()
