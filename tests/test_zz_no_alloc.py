"""The allocation-free forward (bsl_forward_group_static) against bsl_forward_group
under BSL_PATH_DECODE (the single- and few-token kernels at 1 to 4 tokens).

Two calls in a row on one device, the second with a smaller input, each compared with
the existing entry point's output (same kernels, same launch configuration: identical
bits) and with the fp64 oracle (bit-exact on dyadic blocks, relative Frobenius 5e-3 on
float blocks); and the calls it refuses are refused before anything runs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_sign_rank_amd as bsl  # noqa: E402
from gpu_util import REL_TOL, Stack, rel_err, stream_ptr  # noqa: E402

SHAPES = [(2048, 1024), (512, 2048), (1024, 1536), (300, 520)]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    bsl.lib()
    yield


def _buffers(st, ws, xs, fp32=True):
    xts, yts = [], []
    for w, x in zip(ws, xs):
        m, d = st.shapes[w]
        xts.append(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)).cuda())
        yts.append(torch.full((x.shape[0], m), float("nan"), dtype=torch.float32 if fp32 else torch.float16, device="cuda"))
    return xts, yts


def _call(fn, st, ws, xts, yts, fp32=True):
    fn(st.h, list(ws), [t.data_ptr() for t in xts], [t.data_ptr() for t in yts], xts[0].shape[0], fp32, stream_ptr())
    torch.cuda.synchronize()
    return [y.cpu().numpy().astype(np.float64) for y in yts]


@pytest.mark.parametrize("decode", [bsl.BSL_DECODE_SHARED, bsl.BSL_DECODE_PRIVATE], ids=["shared", "private"])
@pytest.mark.parametrize("kind", ["dyadic", "float"])
def test_static_forward_matches_group_forward(decode, kind):
    n = 3
    if kind == "dyadic":
        weights = [(m, d, synth.dyadic_blocks(61, m, d, n, 16, j)) for j, (m, d) in enumerate(SHAPES)]
        make_x = lambda M, d, j: synth.integer_activations(62, M, d, -2, 2, j)  # noqa: E731
    else:
        weights = [(m, d, synth.synthetic_blocks(63, m, d, n, 16, j)) for j, (m, d) in enumerate(SHAPES)]
        make_x = lambda M, d, j: synth.activations(64, M, d, j)  # noqa: E731
    with Stack(weights, path=bsl.BSL_PATH_DECODE, decode=decode) as st:
        st.load([n] * len(SHAPES))
        # first call: every weight, 4 tokens; second call: a smaller input (2 weights, 1 token)
        for ws, M in (([0, 1, 2, 3], 4), ([3, 1], 1)):
            xs = [make_x(M, SHAPES[w][1], w) for w in ws]
            xts, y_static = _buffers(st, ws, xs)
            _, y_group = _buffers(st, ws, xs)
            got = _call(bsl.bsl_forward_group_static, st, ws, xts, y_static)
            ref_gpu = _call(bsl.bsl_forward_group, st, ws, xts, y_group)
            for w, x, a, b in zip(ws, xs, got, ref_gpu):
                assert np.array_equal(a, b), (kind, decode, M, w)
                ref = oracle.forward(x, weights[w][2], n)
                if kind == "dyadic":
                    assert np.array_equal(a, ref), (kind, decode, M, w)
                else:
                    assert rel_err(a, ref) <= REL_TOL, (kind, decode, M, w, rel_err(a, ref))


def test_static_forward_repeated_calls_agree():
    # the scratch keeps the last call's contents; the counters are cleared by each call
    weights = [(m, d, synth.synthetic_blocks(65, m, d, 2, 16, j)) for j, (m, d) in enumerate(SHAPES)]
    with Stack(weights) as st:
        st.load([2] * len(SHAPES))
        xs = [synth.activations(66, 2, d, j) for j, (_, d) in enumerate(SHAPES)]
        xts, yts = _buffers(st, range(4), xs)
        first = _call(bsl.bsl_forward_group_static, st, range(4), xts, yts)
        for _ in range(3):
            again = _call(bsl.bsl_forward_group_static, st, range(4), xts, yts)
            assert all(np.array_equal(a, b) for a, b in zip(first, again))


def test_static_forward_refusals():
    # more than 4 tokens
    weights = [(m, d, synth.synthetic_blocks(67, m, d, 1, 16, j)) for j, (m, d) in enumerate(SHAPES[:1])]
    with Stack(weights) as st:
        st.load([1])
        x = synth.activations(68, 5, SHAPES[0][1])
        xts, yts = _buffers(st, [0], [x])
        with pytest.raises(bsl.BslError) as e:
            _call(bsl.bsl_forward_group_static, st, [0], xts, yts)
        assert e.value.code == bsl.BSL_EUNSUPPORTED
    # activations that do not fit the few-token kernel's LDS (4 x 20480 fp16 = 160 KiB)
    with Stack([(96, 20480, synth.synthetic_blocks(69, 96, 20480, 1))]) as st:
        st.load([1])
        x = synth.activations(70, 4, 20480)
        xts, yts = _buffers(st, [0], [x])
        with pytest.raises(bsl.BslError) as e:
            _call(bsl.bsl_forward_group_static, st, [0], xts, yts)
        assert e.value.code == bsl.BSL_EUNSUPPORTED
        # the same call through bsl_forward_group works (it falls back to another kernel)
        _call(bsl.bsl_forward_group, st, [0], xts, yts)
    # a launch whose partial sums exceed the scratch: 8 weights of 131072 rows at 4 tokens
    # (16384 row groups of 64 rows, 256 floats each); no block needs to be loaded
    h = bsl.bsl_init(0, [131072] * 8, [8] * 8, 16, 1, 0)
    try:
        xt = torch.zeros((4, 8), dtype=torch.float16, device="cuda")
        yt = [torch.zeros((4, 131072), dtype=torch.float32, device="cuda") for _ in range(8)]
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_forward_group_static(h, list(range(8)), [xt.data_ptr()] * 8, [t.data_ptr() for t in yt], 4, True,
                                         stream_ptr())
        assert e.value.code == bsl.BSL_EUNSUPPORTED and "static scratch" in str(e.value)
    finally:
        torch.cuda.synchronize()
        bsl.bsl_destroy(h)
