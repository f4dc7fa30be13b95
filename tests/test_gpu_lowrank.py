"""GPU parity of the equal-size vanilla-SVD baseline (bitstack_lowrank.h) against the
fp64 oracle (``oracle.forward_lowrank``), through the C-ABI.

Bars: an integer-valued case is bit-exact (every product and partial sum is an integer
below 2^24, exact in fp32 in any order); everything else is within the layer's relative
Frobenius error of 5e-3.  The low-rank oracle is cheap at full size, so the 8B-shaped
layer is checked whole.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_sign_rank_amd as bsl  # noqa: E402
from gpu_util import REL_TOL, rel_err, stream_ptr  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    bsl.lib()
    yield


class LrStack:
    def __init__(self, weights, n_cap=16):
        """weights: list of (m, d, k', blocks)."""
        self.shapes = [(m, d) for m, d, _, _ in weights]
        self.h = bsl.bsl_lr_init(0, [w[0] for w in weights], [w[1] for w in weights], [w[2] for w in weights], n_cap)
        for i, (_, _, _, blocks) in enumerate(weights):
            bsl.bsl_lr_set_source(self.h, i, blocks)

    def load(self, counts):
        bsl.bsl_lr_load_blocks(self.h, counts, stream_ptr())

    def forward(self, w, x, fp32=True):
        m, d = self.shapes[w]
        xt = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).reshape(-1, d).cuda()
        y = torch.empty((xt.shape[0], m), dtype=torch.float32 if fp32 else torch.float16, device="cuda")
        bsl.bsl_lr_forward(self.h, w, xt.data_ptr(), y.data_ptr(), xt.shape[0], fp32, stream_ptr())
        torch.cuda.synchronize()
        return y.cpu().numpy().astype(np.float64)

    def forward_group(self, ws, xs, fp32=True):
        xts, ys = [], []
        for w, x in zip(ws, xs):
            m, d = self.shapes[w]
            xts.append(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).reshape(-1, d).cuda())
            ys.append(torch.empty((xts[-1].shape[0], m), dtype=torch.float32 if fp32 else torch.float16, device="cuda"))
        bsl.bsl_lr_forward_group(self.h, list(ws), [t.data_ptr() for t in xts], [t.data_ptr() for t in ys],
                                 xts[0].shape[0], fp32, stream_ptr())
        torch.cuda.synchronize()
        return [y.cpu().numpy().astype(np.float64) for y in ys]

    def close(self):
        if self.h:
            torch.cuda.synchronize()
            bsl.bsl_lr_destroy(self.h)
            self.h = 0

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()


def lr_blocks(seed, m, d, kp, n):
    """Synthetic vanilla-SVD blocks: fp16 factors of mixed sign."""
    out = []
    for i in range(n):
        g = synth.rng(seed, 40, m, d, kp, i)
        out.append({"u": (g.standard_normal((m, kp)) * 0.05).astype(np.float16),
                    "v": (g.standard_normal((d, kp)) * 0.05).astype(np.float16)})
    return out


def test_equal_rank_and_block_bytes_match_the_oracle():
    for m, d in [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (37, 520)]:
        kp = bsl.bsl_lr_equal_rank(m, d, 16)
        assert kp == oracle.equal_bytes_rank(m, d, 16)
        assert bsl.bsl_lr_block_bytes(m, d, kp) == oracle.lowrank_block_bytes(m, d, kp)


@pytest.mark.parametrize("m,d,kp,n", [(64, 512, 8, 2), (37, 520, 5, 3), (200, 1544, 67, 2)])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 9, 17])
def test_integer_lowrank_forward_bit_exact(m, d, kp, n, M):
    g = synth.rng(31, m, d, kp, n)
    blocks = [{"u": g.integers(-2, 3, size=(m, kp)).astype(np.float16),
               "v": g.integers(-2, 3, size=(d, kp)).astype(np.float16)} for _ in range(n)]
    x = synth.integer_activations(31, M, d)
    with LrStack([(m, d, kp, blocks)]) as st:
        st.load([n])
        y = st.forward(0, x)
    assert np.array_equal(y, oracle.forward_lowrank(x, blocks, n))


@pytest.mark.parametrize("m,d,kp,n", [(1000, 1544, 67, 3), (37, 520, 5, 1), (4096, 4096, 144, 2), (16, 8, 1, 2)])
@pytest.mark.parametrize("M", [1, 4, 8, 13])
@pytest.mark.parametrize("fp32", [True, False])
def test_lowrank_forward_ragged(m, d, kp, n, M, fp32):
    blocks = lr_blocks(32, m, d, kp, n)
    x = synth.activations(32, M, d)
    with LrStack([(m, d, kp, blocks)]) as st:
        st.load([n])
        y = st.forward(0, x, fp32=fp32)
    assert rel_err(y, oracle.forward_lowrank(x, blocks, n)) <= REL_TOL


def test_svd_decomposition_all_block_counts():
    m = d = 1024
    W = synth.gaussian_weight(33, m, d)
    kp = oracle.equal_bytes_rank(m, d)
    blocks, _ = oracle.decompose_svd(W, kp, 4)
    x = synth.activations(33, 3, d)
    with LrStack([(m, d, kp, blocks)], n_cap=4) as st:
        for n in (0, 1, 2, 4, 3, 0, 4):
            st.load([n])
            assert bsl.bsl_lr_resident_bytes(st.h) == n * oracle.lowrank_block_bytes(m, d, kp)
            y = st.forward(0, x)
            if n == 0:
                assert not y.any()
            else:
                assert rel_err(y, oracle.forward_lowrank(x, blocks, n)) <= REL_TOL


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 8])
def test_llama3_8b_layer_equal_size_grouped(M):
    """The 8B-shaped layer with equal-size ranks k' and n = 8 blocks per weight, all
    seven weights in one grouped launch pair, checked whole."""
    shapes = synth.LLAMA3_8B_LAYER
    weights = []
    for j, (_, m, d) in enumerate(shapes):
        kp = oracle.equal_bytes_rank(m, d)
        weights.append((m, d, kp, lr_blocks(34 + j, m, d, kp, 8)))
    xs = [synth.activations(34, M, d, j) for j, (_, _, d) in enumerate(shapes)]
    with LrStack(weights, n_cap=8) as st:
        st.load([8] * len(shapes))
        total = sum(8 * oracle.lowrank_block_bytes(m, d, kp) for m, d, kp, _ in weights)
        assert bsl.bsl_lr_resident_bytes(st.h) == total
        ys = st.forward_group(list(range(len(shapes))), xs)
        for j, (m, d, kp, blocks) in enumerate(weights):
            assert rel_err(ys[j], oracle.forward_lowrank(xs[j], blocks, 8)) <= REL_TOL
        # single-weight launches give the same result bit for bit (same per-row order)
        assert np.array_equal(st.forward(6, xs[6]), ys[6])


def test_lowrank_grouped_with_empty_weight():
    weights = [(300, 1032, 20, lr_blocks(35, 300, 1032, 20, 2)), (64, 512, 8, lr_blocks(36, 64, 512, 8, 2)),
               (130, 2048, 33, lr_blocks(37, 130, 2048, 33, 3))]
    counts = [2, 0, 3]
    xs = [synth.activations(35, 6, d, j) for j, (_, d, _, _) in enumerate(weights)]
    with LrStack(weights, n_cap=4) as st:
        st.load(counts)
        ys = st.forward_group([2, 0, 1], [xs[2], xs[0], xs[1]])
    assert rel_err(ys[0], oracle.forward_lowrank(xs[2], weights[2][3], 3)) <= REL_TOL
    assert rel_err(ys[1], oracle.forward_lowrank(xs[0], weights[0][3], 2)) <= REL_TOL
    assert not ys[2].any()


def test_lowrank_argument_errors():
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_lr_init(0, [64], [100], [8])  # d not a multiple of 8
    assert e.value.code == bsl.BSL_EUNSUPPORTED
    with pytest.raises(bsl.BslError) as e:
        bsl.bsl_lr_init(0, [64], [512], [0])
    assert e.value.code == bsl.BSL_EUNSUPPORTED
    blocks = lr_blocks(38, 64, 512, 8, 2)
    with LrStack([(64, 512, 8, blocks), (64, 512, 8, blocks)], n_cap=2) as st:
        with pytest.raises(bsl.BslError) as e:
            st.load([3, 0])
        assert e.value.code == bsl.BSL_EINVAL
        st.load([2, 1])
        x = torch.zeros((1, 512 + 8), dtype=torch.float16, device="cuda")
        y = torch.zeros((1, 64), dtype=torch.float32, device="cuda")
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_lr_forward(st.h, 0, x.data_ptr() + 2, y.data_ptr(), 1, True, 0)
        assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_lr_forward_group(st.h, [1, 1], [x.data_ptr()] * 2, [y.data_ptr()] * 2, 1, True, 0)
        assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_lr_forward(st.h, 2, x.data_ptr(), y.data_ptr(), 1, True, 0)
        assert e.value.code == bsl.BSL_EINVAL
        xx = synth.activations(38, 2, 512)
        assert rel_err(st.forward(1, xx), oracle.forward_lowrank(xx, blocks, 1)) <= REL_TOL
