"""Forwards recorded in a HIP graph and replayed.

A forward only enqueues kernels (no allocation, no synchronisation, no memset: the
allocation-free entry point clears its accumulators with a kernel, and the row
accumulators of the other entry points clear themselves), so a caller may capture it.
The graph below holds single- and few-token forwards through both entry points, a
product-index forward and a tile-path forward; it is replayed several times with ordinary forwards and
synchronisations between the replays, and every replay must give the eager results bit
for bit (the launches are deterministic).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import bit_sign_rank_amd as bsl  # noqa: E402
from gpu_util import REL_TOL, Stack, rel_err  # noqa: E402

SHAPES = [(2048, 1024), (1024, 1536), (512, 2048)]


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    bsl.lib()
    yield


def test_graph_replay_matches_eager():
    n = 3
    weights = [(m, d, synth.synthetic_blocks(71, m, d, n, 16, j)) for j, (m, d) in enumerate(SHAPES)]
    ws = list(range(len(SHAPES)))
    calls = [  # (entry point, tokens)
        (bsl.bsl_forward_group, 1),
        (bsl.bsl_forward_group_static, 1),
        (bsl.bsl_forward_group, 3),
        (bsl.bsl_forward_group_static, 4),
        (bsl.bsl_forward_group, 12),  # product-index path: the layout passes, then the product kernel
        (bsl.bsl_forward_group, 40),  # tile path: the rank-major V pass, then the tile kernel
    ]
    with Stack(weights) as st:
        st.load([n] * len(SHAPES))
        xs = [[torch.from_numpy(synth.activations(72 + k, M, d, j)).cuda() for j, (_, d) in enumerate(SHAPES)]
              for k, (_, M) in enumerate(calls)]
        ys = [[torch.zeros((M, m), dtype=torch.float32, device="cuda") for (m, _) in SHAPES] for (_, M) in calls]
        side_x = [torch.from_numpy(synth.activations(90, 2, d, j)).cuda() for j, (_, d) in enumerate(SHAPES)]
        side_y = [torch.zeros((2, m), dtype=torch.float32, device="cuda") for (m, _) in SHAPES]
        s = torch.cuda.Stream()

        def issue(stream):
            for k, (fn, M) in enumerate(calls):
                fn(st.h, ws, [t.data_ptr() for t in xs[k]], [t.data_ptr() for t in ys[k]], M, True, stream.cuda_stream)

        with torch.cuda.stream(s):
            issue(s)
        torch.cuda.synchronize()
        eager = [[y.clone() for y in row] for row in ys]
        # the eager results are right (fp64 oracle over full rows)
        for k, (_, M) in enumerate(calls):
            for j in ws:
                ref = oracle.forward(xs[k][j].cpu().numpy(), weights[j][2], n)
                assert rel_err(eager[k][j].cpu().numpy().astype(np.float64), ref) <= REL_TOL, (k, j)

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            issue(s)
        torch.cuda.synchronize()
        for rep in range(3):
            for row in ys:
                for y in row:
                    y.zero_()
            # ordinary work between the replays: another forward and a synchronisation
            bsl.bsl_forward_group(st.h, ws, [t.data_ptr() for t in side_x], [t.data_ptr() for t in side_y], 2, True, 0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k in range(len(calls)):
                for j in ws:
                    assert torch.equal(ys[k][j], eager[k][j]), (rep, k, j)
