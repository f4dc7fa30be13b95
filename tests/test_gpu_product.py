"""GPU parity of the product-index kernel (BSL_PATH_PRODUCT, 2 to 32 tokens) against the
fp64 CPU oracle, through the C-ABI.

The kernel restores each block's products U_i V_i^T (rounded to fp16) per 32 x 32 tile
and plane and lets the stored sign bits select +x or -x inside the 2:4 sparse MFMA.
Pins: dyadic factors with integer activations are bit-exact (every product, fp16 value
and fp32 partial sum is exact, tests/test_exact_dyadic.py), on shapes with ragged rows
(m not a multiple of 32), a partial last chunk and a partial last plane (d not a
multiple of 512 or 32), block counts that leave a batch of four part-filled, one to 32
tokens; float blocks within a per-element bound from the kernel's arithmetic.  Each
mistake below fails one of them: a transposed or shifted U or V row (dyadic factors vary
by row, column and rank), a wrong sign-word group or plane half (Bernoulli signs), a
B-operand column order that does not match the A values (every column differs), a
token or row mapped to the wrong output, a missing zero past d or past M, a part-filled
batch whose spare slots add a block again, a row tile whose shares are not all added.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_sign_rank_amd as bsl  # noqa: E402  (no skip: a missing library must fail here)
from gpu_util import REL_TOL, Stack, abs_bound, assert_elementwise, elem_factor, rel_err  # noqa: E402

PRODUCT = bsl.BSL_PATH_PRODUCT


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    bsl.lib()
    yield


@pytest.mark.parametrize("m,d,n", [(64, 1024, 3), (37, 520, 2), (200, 2560, 4), (1024, 4096, 16), (16, 8, 1),
                                   (3000, 1544, 5), (100, 512, 7), (33, 1064, 9)])
@pytest.mark.parametrize("M", [2, 3, 5, 16, 17, 31, 32])
def test_product_integer_bit_exact(m, d, n, M):
    blocks = synth.dyadic_blocks(61, m, d, n)
    x = synth.integer_activations(62, M, d)
    with Stack([(m, d, blocks)], path=PRODUCT) as st:
        st.load([n])
        before = bsl.bsl_launch_counts(st.h)[4]
        y = st.forward(0, x, fp32=True)
        assert bsl.bsl_launch_counts(st.h)[4] == before + 1  # the product-index kernel ran
    ref = oracle.forward(x, blocks, n)
    if not np.array_equal(y, ref):
        bad = np.argwhere(y != ref)
        t, j = bad[0]
        raise AssertionError(f"m={m} d={d} n={n} M={M}: {len(bad)} of {y.size} differ; first token {t} row {j}: "
                             f"got {y[t, j]!r}, oracle {ref[t, j]!r}")


@pytest.mark.parametrize("M", [4, 16, 32])
def test_product_grouped_with_empty_weights_between(M):
    shapes = [(512, 1024), (1024, 512), (300, 1536), (64, 2048), (2048, 1024), (96, 4104)]
    counts = [0, 3, 0, 2, 5, 6]
    ws = [(m, d, synth.synthetic_blocks(63, m, d, 6, 16, j)) for j, (m, d) in enumerate(shapes)]
    xs = [synth.activations(64, M, d, j) for j, (_, d) in enumerate(shapes)]
    with Stack(ws, path=PRODUCT) as st:
        st.load(counts)
        for fp32 in (True, False):
            ys = st.forward_group(list(range(len(shapes))), xs, fp32=fp32)
            for j, (m, d, blocks) in enumerate(ws):
                if counts[j] == 0:
                    assert not ys[j].any()
                    continue
                ref = oracle.forward(xs[j], blocks, counts[j])
                assert rel_err(ys[j], ref) <= REL_TOL
                if fp32:
                    bound = elem_factor("product", counts[j], d) * abs_bound(xs[j], blocks, counts[j])
                    assert_elementwise(ys[j], ref, bound, f"weight {j} M={M}")


@pytest.mark.parametrize("M", [2, 8, 32])
def test_product_float_decomposed_weight(M):
    W = synth.gaussian_weight(0, 1024, 1024)
    blocks, _ = oracle.decompose(W, 16, 4)
    x = synth.activations(65, M, 1024)
    with Stack([(1024, 1024, blocks)], path=PRODUCT) as st:
        for n in (1, 2, 3, 4):
            st.load([n])
            y = st.forward(0, x)
            ref = oracle.forward(x, blocks, n)
            assert rel_err(y, ref) <= REL_TOL
            assert_elementwise(y, ref, elem_factor("product", n, 1024) * abs_bound(x, blocks, n), f"n={n} M={M}")


def test_product_same_bits_run_to_run_and_grouped_vs_single():
    # every workgroup stores its fp32 share of a row group in a slot of its own and the
    # finishing pass adds the slots in workgroup order: the same launch gives the same
    # bits every time, and a grouped launch (another split of the units over the
    # workgroups) the same bits as single-weight launches when every share is exact
    # (dyadic pins)
    shapes = [(1000, 1544), (256, 4096), (4096, 512)]
    n = 6
    ws = [(m, d, synth.dyadic_blocks(66, m, d, n, 16, j)) for j, (m, d) in enumerate(shapes)]
    xs = [synth.integer_activations(67, 24, d, -2, 2, j) for j, (_, d) in enumerate(shapes)]
    with Stack(ws, path=PRODUCT) as st:
        st.load([n] * 3)
        g1 = st.forward_group([0, 1, 2], xs)
        g2 = st.forward_group([0, 1, 2], xs)
        for j in range(3):
            ref = oracle.forward(xs[j], ws[j][2], n)
            assert np.array_equal(g1[j], ref) and np.array_equal(g2[j], ref)
            assert np.array_equal(st.forward(j, xs[j]), ref)


def test_product_rejects_more_than_32_tokens():
    blocks = synth.synthetic_blocks(68, 64, 512, 2)
    with Stack([(64, 512, blocks)], path=PRODUCT) as st:
        st.load([2])
        x = torch.zeros((33, 512), dtype=torch.float16, device="cuda")
        y = torch.empty((33, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_forward(st.h, 0, x.data_ptr(), y.data_ptr(), 33, True, 0)
        assert e.value.code == bsl.BSL_EUNSUPPORTED


@pytest.mark.parametrize("M,kind", [(2, 1), (3, 1), (4, 4), (5, 4), (32, 4), (33, 3)])
def test_auto_takes_the_documented_kernel(M, kind):
    # BSL_PATH_AUTO: the few-token kernel at 2 and 3 tokens, the product-index kernel from
    # 4 to 32, the tile kernel from 33 (launch-count kinds 1, 4 and 3); exact either way
    m, d, n = 200, 1544, 3
    blocks = synth.dyadic_blocks(90, m, d, n, 16)
    x = synth.integer_activations(91, M, d, -2, 2)
    with Stack([(m, d, blocks)]) as st:
        st.load([n])
        before = np.array(bsl.bsl_launch_counts(st.h))
        y = st.forward(0, x)
        delta = np.array(bsl.bsl_launch_counts(st.h)) - before
    assert delta.tolist() == [1 if i == kind else 0 for i in range(bsl.BSL_KERNEL_KINDS)]
    assert np.array_equal(y, oracle.forward(x, blocks, n))


def test_decode_path_rejects_more_than_4_tokens():
    blocks = synth.synthetic_blocks(92, 64, 512, 2)
    with Stack([(64, 512, blocks)], path=bsl.BSL_PATH_DECODE) as st:
        st.load([2])
        x = torch.zeros((5, 512), dtype=torch.float16, device="cuda")
        y = torch.empty((5, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_forward(st.h, 0, x.data_ptr(), y.data_ptr(), 5, True, 0)
        assert e.value.code == bsl.BSL_EUNSUPPORTED


def test_product_smaller_call_after_larger_leaves_no_stale_shares():
    # the share slots keep the last call's contents and a call stores only the lanes of
    # its own tokens: a 5-token call after a 32-token one on the same stack must not pick
    # up the earlier call's tokens 5..31 (exact on dyadic blocks)
    shapes = [(1000, 1544), (256, 4096)]
    n = 5
    ws = [(m, d, synth.dyadic_blocks(93, m, d, n, 16, j)) for j, (m, d) in enumerate(shapes)]
    with Stack(ws, path=PRODUCT) as st:
        st.load([n] * 2)
        for M, seed in ((32, 94), (5, 95), (7, 96)):
            xs = [synth.integer_activations(seed, M, d, -2, 2, j) for j, (_, d) in enumerate(shapes)]
            ys = st.forward_group([0, 1], xs)
            for j in range(2):
                assert np.array_equal(ys[j], oracle.forward(xs[j], ws[j][2], n)), (M, j)
