"""GPU parity of the HIP path (through the C-ABI) against the fp64 CPU oracle.

Bars: sign unpacking and the integer-valued forward are bit-exact; every other output
is within a relative Frobenius error of 5e-3 of the oracle (the layer's stated
tolerance).  Large shapes are checked on seeded row samples that the oracle computes
one by one, in the same launch configuration the benchmark times.  Both formulations
are covered: FACTORED (S_i Z_i on the matrix cores, never forming W_hat) and TILE
(W_hat rebuilt per tile in registers, then a GEMM with the activations).
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

PATHS = [bsl.BSL_PATH_FACTORED, bsl.BSL_PATH_TILE]
PATH_IDS = ["factored", "tile"]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    bsl.lib()  # raises if the library is missing
    yield


def integer_blocks(m, d, n, seed=21):
    # dyadic factors (entries 1/4 or 1/2 per row, column and rank) and Bernoulli signs:
    # with integer activations every partial sum of every path is exact in fp32 while
    # max|x| 4 n d < 2^20 (tests/test_exact_dyadic.py), so outputs are compared bit for bit
    return synth.dyadic_blocks(seed, m, d, n)


# ---------------------------------------------------------------- sign unpack
@pytest.mark.parametrize("m,d", [(1024, 1024), (48, 1536), (37, 520), (4096, 4096), (16, 8)])
@pytest.mark.parametrize("path", [0, 1, 2])
def test_debug_unpack_bit_exact(m, d, path):
    blocks = synth.synthetic_blocks(5, m, d, 2, 16, m, d)
    with Stack([(m, d, blocks)]) as st:
        st.load([2])
        for i in range(2):
            out = torch.empty((m, d), dtype=torch.int8, device="cuda")
            bsl.bsl_debug_unpack(st.h, 0, i, path, out.data_ptr(), 0)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), oracle.signs_from_bits(blocks[i]["bits"], d))


# ---------------------------------------------------------------- exact integer forward
@pytest.mark.parametrize("m,d,n", [(64, 1024, 3), (37, 520, 2), (200, 2560, 4), (1024, 4096, 16), (16, 8, 1)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 17, 130])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_integer_forward_bit_exact(m, d, n, M, path):
    # U V^T is a multiple of 1/16 in [1, 4], W_hat a multiple of 1/16 below 64 (exact in
    # fp16 on the tile path), y a multiple of 1/16 below 2^20: exact in fp32 in any order.
    blocks = integer_blocks(m, d, n)
    x = synth.integer_activations(9, M, d)
    with Stack([(m, d, blocks)], path=path) as st:
        st.load([n])
        y = st.forward(0, x, fp32=True)
    assert np.array_equal(y, oracle.forward(x, blocks, n))


# ---------------------------------------------------------------- decomposed 1024 x 1024
@pytest.fixture(scope="module")
def cfg1_blocks():
    W = synth.gaussian_weight(0, 1024, 1024)
    blocks, _ = oracle.decompose(W, 16, 4)
    return blocks


@pytest.mark.parametrize("fp32", [True, False])
@pytest.mark.parametrize("path", [bsl.BSL_PATH_AUTO] + PATHS, ids=["auto"] + PATH_IDS)
def test_decomposed_weight_all_block_counts(cfg1_blocks, fp32, path):
    x1 = synth.activations(1, 1, 1024)
    x8 = synth.activations(2, 8, 1024)
    with Stack([(1024, 1024, cfg1_blocks)], path=path) as st:
        for n in (1, 2, 3, 4):  # grow one block at a time, no repacking of the others
            st.load([n])
            assert bsl.bsl_active_blocks(st.h, 0) == n
            for x in (x1, x8):
                y = st.forward(0, x, fp32=fp32)
                ref = oracle.forward(x, cfg1_blocks, n)
                assert rel_err(y, ref) <= REL_TOL


def test_grow_shrink_and_zero_blocks(cfg1_blocks):
    x = synth.activations(3, 1, 1024)
    with Stack([(1024, 1024, cfg1_blocks)]) as st:
        for n in (4, 2, 3, 0, 1, 4):
            st.load([n])
            y = st.forward(0, x)
            if n == 0:
                assert not y.any()
            else:
                assert rel_err(y, oracle.forward(x, cfg1_blocks, n)) <= REL_TOL
        resident = bsl.bsl_resident_bytes(st.h)
        # aligned shapes: the four slots hold the blocks' payload and nothing else
        assert resident == 4 * bsl.bsl_block_bytes(1024, 1024, 16)
        st.load([0])
        assert bsl.bsl_resident_bytes(st.h) == 0


def test_non_default_stream(cfg1_blocks):
    x = synth.activations(4, 1, 1024)
    s = torch.cuda.Stream()
    with Stack([(1024, 1024, cfg1_blocks)]) as st:
        st.load([4], stream=s)
        with torch.cuda.stream(s):
            y = st.forward(0, x, stream=s)
    assert rel_err(y, oracle.forward(x, cfg1_blocks, 4)) <= REL_TOL


def test_load_overlaps_forwards_on_another_stream(cfg1_blocks):
    # Forwards of weight 0 with 2 blocks are queued on one stream; while they run, weight 0
    # grows to 4 blocks and weight 1 is loaded on a second stream.  The queued forwards
    # keep their block count (the load writes only new table entries), later ones see the
    # new counts.
    other = synth.synthetic_blocks(33, 1024, 1024, 3, 16, 1)
    x = synth.activations(34, 8, 1024)
    xt = torch.from_numpy(x).cuda()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with Stack([(1024, 1024, cfg1_blocks), (1024, 1024, other)]) as st:
        st.load([2, 0])
        torch.cuda.synchronize()
        before = []
        with torch.cuda.stream(s1):
            for _ in range(16):
                y = torch.empty((8, 1024), dtype=torch.float32, device="cuda")
                bsl.bsl_forward(st.h, 0, xt.data_ptr(), y.data_ptr(), 8, True, int(s1.cuda_stream))
                before.append(y)
        bsl.bsl_load_blocks(st.h, [4, 3], int(s2.cuda_stream))
        with torch.cuda.stream(s1):
            y0 = torch.empty((8, 1024), dtype=torch.float32, device="cuda")
            y1 = torch.empty((8, 1024), dtype=torch.float32, device="cuda")
            bsl.bsl_forward(st.h, 0, xt.data_ptr(), y0.data_ptr(), 8, True, int(s1.cuda_stream))
            bsl.bsl_forward(st.h, 1, xt.data_ptr(), y1.data_ptr(), 8, True, int(s1.cuda_stream))
        torch.cuda.synchronize()
        ref2 = oracle.forward(x, cfg1_blocks, 2)
        for y in before:
            assert rel_err(y.cpu().numpy().astype(np.float64), ref2) <= REL_TOL
        assert rel_err(y0.cpu().numpy().astype(np.float64), oracle.forward(x, cfg1_blocks, 4)) <= REL_TOL
        assert rel_err(y1.cpu().numpy().astype(np.float64), oracle.forward(x, other, 3)) <= REL_TOL


def test_tile_rank_major_v_workspace():
    # A block keeps V only in the tiled order; the tile path forms the launch's V in rank-
    # major order in a workspace sized at load for the 8 weights with the most V bytes.
    # Ten weights: a group of exactly those 8 fits and matches the oracle, and the
    # workspace does not grow with the other two.
    ds = [512, 1024, 1536, 2048, 2560, 3072, 3584, 4096, 512, 1024]
    ns = [2, 3, 1, 2, 2, 1, 2, 1, 3, 1]
    weights = [(256, d, synth.synthetic_blocks(40 + j, 256, d, n, 16, 0, j)) for j, (d, n) in enumerate(zip(ds, ns))]
    vbytes = [n * d * 32 for d, n in zip(ds, ns)]  # (d is a multiple of 512: no column padding)
    top = sorted(range(len(ds)), key=lambda j: -vbytes[j])[:8]
    with Stack(weights, path=bsl.BSL_PATH_TILE) as st:
        before = bsl.bsl_workspace_bytes(st.h)
        st.load(ns)
        grown = bsl.bsl_workspace_bytes(st.h) - before
        raw = max(256 * d // 8 for d in ds)  # plus the load's two device buffers of raw sign bits
        assert sum(vbytes[j] for j in top) <= grown <= sum(vbytes[j] for j in top) + 2 * raw
        assert bsl.bsl_resident_bytes(st.h) == sum(n * bsl.bsl_block_bytes(256, d, 16) + n * (1024 - 256) * (d // 8 + 32)
                                                   for d, n in zip(ds, ns))
        tiles = bsl.bsl_launch_counts(st.h)[3]
        xs = [synth.activations(41, 24, ds[j], j) for j in top]
        ys = st.forward_group(top, xs)  # 24 tokens: the tile path
        assert bsl.bsl_launch_counts(st.h)[3] == tiles + 1
        for k, j in enumerate(top):
            blocks = weights[j][2]
            ref = oracle.forward(xs[k], blocks, ns[j])
            assert_elementwise(ys[k], ref, elem_factor("tile", ns[j], ds[j]) * abs_bound(xs[k], blocks, ns[j]), f"weight {j} d={ds[j]}")


def test_multi_token_workspace_shared_by_groups():
    # The factored multi-token path cuts its items along the (block, chunk) sequence when
    # there are few of them and sums the pieces from a partial-sum workspace that the
    # stack shares among its weights (room for the 8 weights needing the most).  Ten
    # weights: groups of 8 in two different orders, twice each, all match the oracle (the
    # arrival counters are back at zero after every launch).
    ms = [512, 1024, 1536, 2048, 2560, 3072, 3584, 4096, 1024, 2048]
    weights = [(m, 1536, synth.synthetic_blocks(50 + j, m, 1536, 2, 16, 0, j)) for j, m in enumerate(ms)]
    groups = [[7, 6, 5, 4, 3, 2, 9, 1], [0, 8, 1, 9, 2, 3, 4, 5]]
    with Stack(weights, path=bsl.BSL_PATH_FACTORED) as st:
        st.load([2] * len(ms))
        for rep in range(2):
            for g, ws in enumerate(groups):
                xs = [synth.activations(51 + g, 6, 1536, j) for j in ws]
                ys = st.forward_group(ws, xs)
                for k, j in enumerate(ws):
                    blocks = weights[j][2]
                    ref = oracle.forward(xs[k], blocks, 2)
                    assert_elementwise(ys[k], ref, elem_factor("z16", 2, 1536) * abs_bound(xs[k], blocks, 2),
                                       f"group {g} weight {j} pass {rep}")


# ---------------------------------------------------------------- 8B decoder layer
def layer_blocks(shapes, counts, seed, layer=0):
    return [(m, d, synth.synthetic_blocks(seed, m, d, int(n), 16, layer, j)) for j, ((_, m, d), n) in enumerate(zip(shapes, counts))]


def check_sampled(weights, counts, ys, xs, rows_per_weight=48, seed=0):
    for j, ((m, d, blocks), n, y, x) in enumerate(zip(weights, counts, ys, xs)):
        rows = synth.sample_rows(seed, m, rows_per_weight, j)
        ref = oracle.forward_rows(x, blocks, rows, int(n))
        err = rel_err(y[:, rows], ref)
        assert err <= REL_TOL, (j, m, d, n, err)


@pytest.mark.slow
def test_llama3_8b_layer_decode_grouped():
    shapes = synth.LLAMA3_8B_LAYER
    counts = [8] * 7
    weights = layer_blocks(shapes, counts, seed=11)
    xs = [synth.activations(12, 1, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(weights) as st:
        st.load(counts)
        ys = st.forward_group(list(range(7)), xs)
        check_sampled(weights, counts, ys, xs)
        # the same launch again gives the same bits (the pieces are summed in a fixed order)
        again = st.forward_group(list(range(7)), xs)
        assert all(np.array_equal(a, b) for a, b in zip(ys, again))
        # a single-weight launch splits the blocks over workgroups differently, so only
        # the fp32 summation order differs
        for j in (1, 4, 6):
            assert rel_err(st.forward(j, xs[j]), ys[j]) <= 1e-5


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("path", [bsl.BSL_PATH_AUTO, bsl.BSL_PATH_FACTORED], ids=["auto", "factored"])
def test_llama3_8b_variable_block_counts(M, path):
    if M == 1 and path == bsl.BSL_PATH_FACTORED:
        pytest.skip("M = 1 takes the same kernel under both settings")
    shapes = synth.LLAMA3_8B_LAYER
    counts = synth.block_counts(13, 7, 1, 16)
    weights = layer_blocks(shapes, counts, seed=14)
    xs = [synth.activations(15, M, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(weights, path=path) as st:
        st.load(counts)
        ys = st.forward_group(list(range(7)), xs)
        check_sampled(weights, counts, ys, xs, rows_per_weight=32)


@pytest.mark.slow
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_llama3_8b_prefill_2048_tokens(path):
    shapes = [("q", 4096, 4096), ("down", 4096, 14336)]
    counts = [8, 8]
    weights = layer_blocks(shapes, counts, seed=16)
    xs = [synth.activations(17, 2048, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(weights, path=path) as st:
        st.load(counts)
        ys = [st.forward(j, xs[j], fp32=False) for j in range(2)]
        check_sampled(weights, counts, ys, xs, rows_per_weight=24)


@pytest.mark.slow
def test_llama3_8b_layer_prefill_grouped_tile():
    # the benchmark's prefill launch: all seven linears of a layer in one grouped launch,
    # n = 8, M = 2048, default (AUTO -> tile) path, fp16 y
    shapes = synth.LLAMA3_8B_LAYER
    counts = [8] * 7
    weights = layer_blocks(shapes, counts, seed=29)
    xs = [synth.activations(30, 2048, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(weights) as st:
        st.load(counts)
        ys = st.forward_group(list(range(7)), xs, fp32=False)
        check_sampled(weights, counts, ys, xs, rows_per_weight=16)


@pytest.mark.slow
def test_llama2_70b_layer_decode():
    shapes = synth.LLAMA2_70B_LAYER
    counts = synth.block_counts(18, 7, 1, 6)
    weights = layer_blocks(shapes, counts, seed=19)
    xs = [synth.activations(20, 1, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(weights) as st:
        st.load(counts)
        ys = st.forward_group(list(range(7)), xs, fp32=False)
        check_sampled(weights, counts, ys, xs, rows_per_weight=32)


# ---------------------------------------------------------------- ragged shapes
@pytest.mark.parametrize("m,d,M", [(37, 520, 1), (37, 520, 5), (300, 11008 // 4, 1), (1000, 1544, 9), (16, 8, 2)])
def test_ragged_shapes_random_blocks(m, d, M):
    blocks = synth.synthetic_blocks(23, m, d, 3, 16, m, d)
    x = synth.activations(24, M, d)
    with Stack([(m, d, blocks)]) as st:
        st.load([3])
        y = st.forward(0, x)
    assert rel_err(y, oracle.forward(x, blocks, 3)) <= REL_TOL


# ---------------------------------------------------------------- many tokens (the 32x32 prefill path)
@pytest.mark.parametrize("m,d,M", [(1000, 1544, 133), (37, 520, 64), (512, 1024, 256)])
@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_prefill_ragged_shapes(m, d, M, path):
    blocks = synth.synthetic_blocks(25, m, d, 3, 16, m, d)
    x = synth.activations(26, M, d)
    with Stack([(m, d, blocks)], path=path) as st:
        st.load([3])
        y = st.forward(0, x, fp32=False)
    assert rel_err(y, oracle.forward(x, blocks, 3)) <= REL_TOL


# token-group edges of the tile path (groups of 64, 128, 256 and 512 tokens; the last group
# partial), one and two 8-block batches, ragged rows / columns
@pytest.mark.parametrize("m,d,M,n", [(130, 1032, 511, 3), (256, 512, 512, 9), (37, 520, 513, 1), (300, 1536, 1100, 11),
                                     (1024, 2048, 7, 16), (16, 8, 40, 2), (200, 1536, 100, 5), (72, 2560, 128, 9),
                                     (300, 2560, 250, 9), (64, 512, 256, 2)])
def test_tile_token_groups_and_batches(m, d, M, n):
    blocks = synth.synthetic_blocks(31, m, d, n, 16, m, d)
    x = synth.activations(32, M, d)
    with Stack([(m, d, blocks)], path=bsl.BSL_PATH_TILE) as st:
        st.load([n])
        y = st.forward(0, x)
        y16 = st.forward(0, x, fp32=False)
    ref = oracle.forward(x, blocks, n)
    assert rel_err(y, ref) <= REL_TOL
    assert rel_err(y16, ref) <= REL_TOL
    assert_elementwise(y, ref, elem_factor("tile", n, d) * abs_bound(x, blocks, n), f"tile m={m} d={d} M={M} n={n}")


@pytest.mark.parametrize("path", PATHS, ids=PATH_IDS)
def test_prefill_grouped_launch_and_zero_blocks(path):
    shapes = [(1024, 1024, 2), (512, 2048, 0), (1536, 512, 4)]
    weights = [(m, d, synth.synthetic_blocks(27, m, d, max(n, 1), 16, j)) for j, (m, d, n) in enumerate(shapes)]
    xs = [synth.activations(28, 256, d, j) for j, (_, d, _) in enumerate(shapes)]
    with Stack(weights, path=path) as st:
        st.load([n for _, _, n in shapes])
        ys = st.forward_group([0, 1, 2], xs)
    for (m, d, blocks), (_, _, n), y, x in zip(weights, shapes, ys, xs):
        if n == 0:
            assert not y.any()
        else:
            assert rel_err(y, oracle.forward(x, blocks, n)) <= REL_TOL


# ---------------------------------------------------------------- single-token kernels
DECODES = [bsl.BSL_DECODE_SHARED, bsl.BSL_DECODE_PRIVATE]
DECODE_IDS = ["shared", "private"]


@pytest.mark.parametrize("m,d,n", [(64, 1024, 3), (37, 520, 2), (200, 2560, 4), (1024, 4096, 16), (16, 8, 1),
                                   (3000, 1544, 5)])
@pytest.mark.parametrize("decode", DECODES, ids=DECODE_IDS)
def test_integer_decode_bit_exact_both_kernels(m, d, n, decode):
    blocks = integer_blocks(m, d, n)
    x = synth.integer_activations(3, 1, d)
    with Stack([(m, d, blocks)], decode=decode) as st:
        st.load([n])
        y = st.forward(0, x)
    assert np.array_equal(y, oracle.forward(x, blocks, n))


@pytest.mark.parametrize("decode", [bsl.BSL_DECODE_AUTO] + DECODES, ids=["auto"] + DECODE_IDS)
def test_decode_grouped_with_empty_weights_between(decode):
    """Weights without blocks in the middle and at the ends of a grouped single-token
    launch: their y is zero and their row groups do not disturb their neighbours'."""
    shapes = [(512, 1024), (1024, 512), (300, 1536), (64, 2048), (2048, 1024)]
    counts = [0, 3, 0, 2, 0]
    ws = [(m, d, synth.synthetic_blocks(41, m, d, 3, 16, j)) for j, (m, d) in enumerate(shapes)]
    xs = [synth.activations(41, 1, d, j) for j, (_, d) in enumerate(shapes)]
    with Stack(ws, decode=decode) as st:
        st.load(counts)
        ys = st.forward_group(list(range(len(shapes))), xs)
    for j, (m, d, blocks) in enumerate(ws):
        if counts[j] == 0:
            assert not ys[j].any()
        else:
            assert rel_err(ys[j], oracle.forward(xs[j], blocks, counts[j])) <= REL_TOL


def test_decode_kernels_agree(cfg1_blocks):
    x = synth.activations(43, 1, 1024)
    outs = []
    for decode in DECODES:
        with Stack([(1024, 1024, cfg1_blocks)], decode=decode) as st:
            st.load([4])
            outs.append(st.forward(0, x))
    ref = oracle.forward(x, cfg1_blocks, 4)
    for y in outs:
        assert rel_err(y, ref) <= REL_TOL
    assert rel_err(outs[0], outs[1]) <= 1e-3


@pytest.mark.slow
@pytest.mark.parametrize("layer", ["llama3_8b", "llama2_70b"])
def test_private_decode_fits_the_layer_shapes(layer):
    """The wave-private kernel takes the whole 8B- and 70B-shaped layers in one grouped
    launch (BSL_DECODE_PRIVATE fails rather than falling back)."""
    shapes = synth.LLAMA3_8B_LAYER if layer == "llama3_8b" else synth.LLAMA2_70B_LAYER
    counts = [2] * len(shapes)
    ws = [(m, d, synth.synthetic_blocks(44, m, d, 2, 16, j)) for j, (_, m, d) in enumerate(shapes)]
    xs = [synth.activations(44, 1, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(ws, decode=bsl.BSL_DECODE_PRIVATE) as st:
        st.load(counts)
        ys = st.forward_group(list(range(len(shapes))), xs)
    for j, (m, d, blocks) in enumerate(ws):
        rows = synth.sample_rows(44, m, 64, j)
        assert rel_err(ys[j][:, rows], oracle.forward_rows(xs[j], blocks, rows, 2)) <= REL_TOL


# ---------------------------------------------------------------- a few tokens (wave-private kernel)
# Under BSL_PATH_DECODE (and BSL_PATH_AUTO at 2 and 3 tokens), 2 to 4 tokens run on the
# wave-private kernel with every operand but the activations shared by the tokens whenever
# the activations fit its LDS, else on the factored multi-token kernel.
@pytest.mark.parametrize("m,d,n", [(64, 1024, 3), (37, 520, 2), (200, 2560, 4), (1024, 4096, 16), (16, 8, 1),
                                   (3000, 1544, 5)])
@pytest.mark.parametrize("M", [2, 3, 4])
def test_integer_few_tokens_bit_exact(m, d, n, M):
    blocks = integer_blocks(m, d, n)
    x = synth.integer_activations(4, M, d)
    with Stack([(m, d, blocks)], path=bsl.BSL_PATH_DECODE) as st:
        st.load([n])
        y = st.forward(0, x)
    assert np.array_equal(y, oracle.forward(x, blocks, n))


@pytest.mark.parametrize("M", [2, 3, 4])
def test_few_tokens_grouped_with_empty_weights_between(M):
    shapes = [(512, 1024), (1024, 512), (300, 1536), (64, 2048), (2048, 1024)]
    counts = [0, 3, 0, 2, 0]
    ws = [(m, d, synth.synthetic_blocks(45, m, d, 3, 16, j)) for j, (m, d) in enumerate(shapes)]
    xs = [synth.activations(45, M, d, j) for j, (_, d) in enumerate(shapes)]
    with Stack(ws, path=bsl.BSL_PATH_DECODE) as st:
        st.load(counts)
        for fp32 in (True, False):
            ys = st.forward_group(list(range(len(shapes))), xs, fp32=fp32)
            for j, (m, d, blocks) in enumerate(ws):
                if counts[j] == 0:
                    assert not ys[j].any()
                else:
                    assert rel_err(ys[j], oracle.forward(xs[j], blocks, counts[j])) <= REL_TOL


@pytest.mark.parametrize("M", [2, 3, 4])
def test_few_tokens_agree_with_the_factored_kernel(cfg1_blocks, M):
    x = synth.activations(46, M, 1024)
    outs = []
    for path in (bsl.BSL_PATH_DECODE, bsl.BSL_PATH_FACTORED):
        with Stack([(1024, 1024, cfg1_blocks)], path=path) as st:
            st.load([4])
            outs.append(st.forward(0, x))
    ref = oracle.forward(x, cfg1_blocks, 4)
    for y in outs:
        assert rel_err(y, ref) <= REL_TOL
    assert rel_err(outs[0], outs[1]) <= 1e-3
    # each token's row equals that token run alone (the tokens share no arithmetic)
    with Stack([(1024, 1024, cfg1_blocks)]) as st:
        st.load([4])
        for t in range(M):
            assert rel_err(st.forward(0, x[t:t + 1]), outs[0][t:t + 1]) <= 1e-3


@pytest.mark.parametrize("M", [2, 4])
def test_few_tokens_wide_input_falls_back(M):
    """A weight whose activations for 4 tokens exceed the kernel's LDS (d = 20480: 160 KiB)
    takes the factored kernel at 4 tokens and the wave-private one at 2; both are exact."""
    m, d, n = 96, 20480, 2
    blocks = integer_blocks(m, d, n)
    x = synth.integer_activations(5, M, d)
    with Stack([(m, d, blocks)], path=bsl.BSL_PATH_DECODE) as st:
        st.load([n])
        y = st.forward(0, x)
    assert np.array_equal(y, oracle.forward(x, blocks, n))


# A grouped few-token call whose activations do not fit the wave-private kernel's LDS
# (148 KiB per workgroup): the weights taking at most half of it (narrow) go to that kernel
# in one launch, the rest (wide) to the factored multi-token kernel in a second one.
# d = 28672 needs 168 / 224 KiB at 3 / 4 tokens.  The zero-block weight writes zeros.
SPLIT_SHAPES = [(96, 1024), (200, 28672), (64, 2560), (300, 512), (1024, 4096)]
SPLIT_COUNTS = [3, 2, 0, 4, 2]


def _counts(st):
    return np.array(bsl.bsl_launch_counts(st.h))


@pytest.mark.parametrize("M,path,launches", [(3, "decode", [0, 1, 1, 0, 0]), (4, "decode", [0, 1, 1, 0, 0]),
                                             (3, "auto", [0, 1, 0, 0, 1]),
                                             (4, "auto", [0, 0, 0, 0, 1])])
def test_few_tokens_grouped_split_bit_exact(M, path, launches):
    # DECODE: the weight that does not fit the few-token kernel takes the factored
    # multi-token kernel; AUTO: the product-index path (and every weight from 4 tokens on)
    ws = [(m, d, integer_blocks(m, d, max(n, 1), 60 + j)) for j, ((m, d), n) in enumerate(zip(SPLIT_SHAPES, SPLIT_COUNTS))]
    xs = [synth.integer_activations(61, M, d, -1, 1, j) for j, (_, d) in enumerate(SPLIT_SHAPES)]
    with Stack(ws, path=bsl.BSL_PATH_DECODE if path == "decode" else bsl.BSL_PATH_AUTO) as st:
        st.load(SPLIT_COUNTS)
        before = _counts(st)
        ys = st.forward_group(list(range(5)), xs)
        assert (_counts(st) - before).tolist() == launches
    for j, ((m, d, blocks), n) in enumerate(zip(ws, SPLIT_COUNTS)):
        assert np.array_equal(ys[j], oracle.forward(xs[j], blocks, n)), (j, SPLIT_SHAPES[j], n)


@pytest.mark.parametrize("M,path", [(3, "decode"), (4, "decode"), (3, "auto")])
def test_few_tokens_grouped_split_float_all_rows(M, path):
    ws = [(m, d, synth.synthetic_blocks(62, m, d, max(n, 1), 16, j)) for j, ((m, d), n) in enumerate(zip(SPLIT_SHAPES, SPLIT_COUNTS))]
    xs = [synth.activations(63, M, d, j) for j, (_, d) in enumerate(SPLIT_SHAPES)]
    with Stack(ws, path=bsl.BSL_PATH_DECODE if path == "decode" else bsl.BSL_PATH_AUTO) as st:
        st.load(SPLIT_COUNTS)
        ys = st.forward_group(list(range(5)), xs)
    for j, ((m, d, blocks), n) in enumerate(zip(ws, SPLIT_COUNTS)):
        ref = oracle.forward(xs[j], blocks, n)
        if n == 0:
            assert not ys[j].any()
            continue
        assert rel_err(ys[j], ref) <= REL_TOL
        # exact products in the wave-private kernel; fp16 Z in the multi-token kernel, fp16
        # U V^T products in the product-index kernel
        kind = ("z16" if path == "decode" else "product") if d == 28672 else "exact"
        assert_elementwise(ys[j], ref, elem_factor(kind, n, d) * abs_bound(xs[j], blocks, n), f"weight {j} {SPLIT_SHAPES[j]}")


def test_few_tokens_narrow_subset_that_does_not_fit_falls_back():
    """Narrow weights (64 KiB of activations each at 4 tokens) whose units are so few that
    one workgroup's range spans three of them plus the start of a long one: that workgroup
    would need 208 KiB of LDS, so the narrow subset runs on the multi-token kernel too (one
    launch), and the wide weight in a second one; results stay exact."""
    shapes = [(64, 8192), (64, 8192), (64, 8192), (16384, 2048), (200, 20480)]
    counts = [1, 0, 1, 16, 2]
    ws = [(m, d, integer_blocks(m, d, max(n, 1), 70 + j)) for j, ((m, d), n) in enumerate(zip(shapes, counts))]
    xs = [synth.integer_activations(71, 4, d, -1, 1, j) for j, (_, d) in enumerate(shapes)]
    with Stack(ws, path=bsl.BSL_PATH_DECODE) as st:
        st.load(counts)
        before = _counts(st)
        ys = st.forward_group(list(range(5)), xs)
        assert (_counts(st) - before).tolist() == [0, 0, 2, 0, 0]
    for j, ((m, d, blocks), n) in enumerate(zip(ws, counts)):
        assert np.array_equal(ys[j], oracle.forward(xs[j], blocks, n)), (j, shapes[j], n)


@pytest.mark.slow
@pytest.mark.parametrize("M", [2, 3])
def test_llama3_8b_layer_few_tokens_grouped(M):
    shapes = synth.LLAMA3_8B_LAYER
    counts = [8] * 7
    weights = layer_blocks(shapes, counts, seed=47)
    xs = [synth.activations(47, M, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(weights, path=bsl.BSL_PATH_DECODE) as st:
        st.load(counts)
        ys = st.forward_group(list(range(7)), xs)
        check_sampled(weights, counts, ys, xs)
        again = st.forward_group(list(range(7)), xs)
        assert all(np.array_equal(a, b) for a, b in zip(ys, again))


@pytest.mark.slow
@pytest.mark.parametrize("M", [2, 3, 4])
def test_llama2_70b_layer_few_tokens(M):
    """The 70B-shaped layer in one grouped call: 2 tokens fit the wave-private kernel;
    at 3 and 4 the down projection's activations (M x 28672 fp16) exceed its LDS, so the
    call splits: the other six weights take the wave-private kernel and the down
    projection the factored kernel.  All are checked on sampled rows."""
    shapes = synth.LLAMA2_70B_LAYER
    counts = [2] * len(shapes)
    ws = [(m, d, synth.synthetic_blocks(48, m, d, 2, 16, j)) for j, (_, m, d) in enumerate(shapes)]
    xs = [synth.activations(48, M, d, j) for j, (_, _, d) in enumerate(shapes)]
    with Stack(ws, path=bsl.BSL_PATH_DECODE) as st:
        st.load(counts)
        ys = st.forward_group(list(range(len(shapes))), xs)
    check_sampled(ws, counts, ys, xs, rows_per_weight=32, seed=48)


# ---------------------------------------------------------------- input-channel scale
@pytest.mark.parametrize("m,d,n", [(1024, 1536, 3), (37, 520, 2)])
@pytest.mark.parametrize("M", [1, 3, 4, 40])
@pytest.mark.parametrize("path,decode", [(p, None) for p in PATHS] + [(bsl.BSL_PATH_AUTO, bsl.BSL_DECODE_PRIVATE),
                                                                       (bsl.BSL_PATH_DECODE, bsl.BSL_DECODE_PRIVATE)],
                         ids=PATH_IDS + ["auto-private", "decode-private"])
def test_input_scale_folded_at_load(m, d, n, M, path, decode):
    # (auto-private: the wave-private kernel at M = 1, the few-token kernel at M = 3, the
    # product-index kernel at M = 4; decode-private: the few-token kernel at M = 3 and 4,
    # reading the B-operand copy of the scaled V)
    if path == bsl.BSL_PATH_DECODE and M > 4:
        pytest.skip("BSL_PATH_DECODE takes at most 4 tokens")
    blocks = synth.synthetic_blocks(23, m, d, n, 16, m, d)
    t = synth.inv_input_scale(23, d)
    x = synth.outlier_activations(23, M, d, synth.channel_magnitudes(23, d))
    with Stack([(m, d, blocks)], path=path, decode=decode) as st:
        bsl.bsl_set_input_scale(st.h, 0, t)
        st.load([n])
        y = st.forward(0, x)
    assert rel_err(y, oracle.forward_scaled(x, blocks, t, n)) <= REL_TOL


@pytest.mark.parametrize("M", [1, 4, 40])
def test_scaled_decomposition_forward(M):
    """A stack decomposed from W diag(s), with 1/s folded in at load, against the
    oracle's scaled layer and (looser) against x W^T itself."""
    m = d = 1024
    W = synth.gaussian_weight(25, m, d)
    mag = synth.channel_magnitudes(25, d, outlier_frac=0.03)
    s = np.sqrt(mag.astype(np.float64))
    blocks, _ = oracle.decompose_scaled(W, s, 16, 4)
    t = (1.0 / s).astype(np.float32)
    x = synth.outlier_activations(25, M, d, mag)
    with Stack([(m, d, blocks)]) as st:
        bsl.bsl_set_input_scale(st.h, 0, t)
        st.load([4])
        y = st.forward(0, x)
    assert rel_err(y, oracle.forward_scaled(x, blocks, t, 4)) <= REL_TOL


def test_input_scale_errors_and_reset():
    m, d = 64, 1024
    blocks = synth.synthetic_blocks(24, m, d, 2)
    t = synth.inv_input_scale(24, d)
    x = synth.activations(24, 3, d)
    with Stack([(m, d, blocks)]) as st:
        for bad in (0.0, -1.0, np.inf, np.nan):
            tt = t.copy()
            tt[7] = bad
            with pytest.raises(bsl.BslError) as e:
                bsl.bsl_set_input_scale(st.h, 0, tt)
            assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_set_input_scale(st.h, 1, t)  # no such weight
        assert e.value.code == bsl.BSL_EINVAL
        # a factor that overflows fp16 in V: nothing is loaded
        bsl.bsl_set_input_scale(st.h, 0, np.full(d, 1e6, np.float32))
        with pytest.raises(bsl.BslError) as e:
            st.load([2])
        assert e.value.code == bsl.BSL_EINVAL
        assert bsl.bsl_active_blocks(st.h, 0) == 0 and bsl.bsl_resident_bytes(st.h) == 0
        bsl.bsl_set_input_scale(st.h, 0, t)
        st.load([1])
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_set_input_scale(st.h, 0, None)  # blocks are loaded
        assert e.value.code == bsl.BSL_EINVAL
        assert rel_err(st.forward(0, x), oracle.forward_scaled(x, blocks, t, 1)) <= REL_TOL
        st.load([0])
        bsl.bsl_set_input_scale(st.h, 0, None)
        st.load([2])
        assert rel_err(st.forward(0, x), oracle.forward(x, blocks, 2)) <= REL_TOL


def test_input_scale_overflow_after_a_queued_copy():
    """The second new block overflows once scaled while the first one's copy is in
    flight: the load is undone as a whole."""
    m, d = 64, 1024
    blocks = synth.synthetic_blocks(26, m, d, 2)
    blocks[0]["v"] = np.full((d, 16), 0.01, np.float16)
    blocks[1]["v"] = np.full((d, 16), 1.0, np.float16)
    with Stack([(m, d, blocks)]) as st:
        bsl.bsl_set_input_scale(st.h, 0, np.full(d, 1e5, np.float32))
        with pytest.raises(bsl.BslError) as e:
            st.load([2])
        assert e.value.code == bsl.BSL_EINVAL
        assert bsl.bsl_active_blocks(st.h, 0) == 0 and bsl.bsl_resident_bytes(st.h) == 0
        st.load([1])
        x = synth.activations(26, 2, d)
        ref = oracle.forward_scaled(x, blocks, np.full(d, 1e5), 1)
        assert rel_err(st.forward(0, x), ref) <= REL_TOL


# ---------------------------------------------------------------- error handling
def test_errors_leave_state_unchanged(cfg1_blocks):
    x = torch.zeros((1, 1024 + 8), dtype=torch.float16, device="cuda")
    y = torch.zeros((1, 1024), dtype=torch.float32, device="cuda")
    with Stack([(1024, 1024, cfg1_blocks)]) as probe:
        probe.load([1])
        slot = bsl.bsl_resident_bytes(probe.h)  # device bytes of one loaded block
    budget = 2 * slot + slot // 2  # room for 2 blocks, not 3
    with Stack([(1024, 1024, cfg1_blocks)], budget=budget) as st:
        st.load([2])
        before = bsl.bsl_resident_bytes(st.h)
        with pytest.raises(bsl.BslError) as e:
            st.load([3])
        assert e.value.code == bsl.BSL_ENOMEM
        assert bsl.bsl_active_blocks(st.h, 0) == 2 and bsl.bsl_resident_bytes(st.h) == before
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_forward(st.h, 0, x.data_ptr() + 2, y.data_ptr(), 1, True, 0)  # misaligned x
        assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_forward(st.h, 1, x.data_ptr(), y.data_ptr(), 1, True, 0)  # no such weight
        assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_load_blocks(st.h, [5], 0)  # only 4 source blocks
        assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_set_path(st.h, 5)  # no such formulation
        assert e.value.code == bsl.BSL_EINVAL
        with pytest.raises(bsl.BslError) as e:
            bsl.bsl_set_decode(st.h, 3)  # no such kernel
        assert e.value.code == bsl.BSL_EINVAL
        assert bsl.bsl_active_blocks(st.h, 0) == 2
        # still works after the failures
        xx = synth.activations(5, 1, 1024)
        assert rel_err(st.forward(0, xx), oracle.forward(xx, cfg1_blocks, 2)) <= REL_TOL
