"""Graph replay: layer calls captured in a HIP graph give, on every replay, the
same bytes as the same calls launched one by one.

The throughput figures come from replays of such a graph, so each path (split-K
small M, the single kernel, large M, and the FP8 layer at small and large M) is
captured with two consecutive calls that share one workspace, replayed several
times with unrelated eager work and synchronizations in between, and compared
with its eager result after every replay: Y, the outlier count and, where
asked for, the bias and the Y column absmax (which the kernels clear and
rebuild on each call).
"""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

# (variant, M, K, N, bias and Y column absmax)
CASES = [
    ("int8", 32, 1024, 520, True),   # split-K small M
    ("int8", 8, 1024, 264, False),   # single kernel
    ("int8", 300, 1024, 520, True),  # large M
    ("int8", 300, 4096, 520, True),  # large M, split-K tiles (arrival counters reset per call)
    ("fp8", 32, 1024, 520, False),
    ("fp8", 300, 512, 264, True),
]


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("variant,M,K,N,extras", CASES)
def test_graph_replays_match_eager(variant, M, K, N, extras):
    import torch
    import bit_quantized_matmul_col_amd as lm
    say(f"case graph replay {variant} M={M} K={K} N={N} extras={extras}")
    cuda = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    X0, W, _ = workloads.random_case(M, K, N, 31, n_out=6)
    X1, _, _ = workloads.random_case(M, K, N, 32, n_out=3)
    Xs, Wd = [cuda(X0), cuda(X1)], cuda(W)
    if variant == "int8":
        Wq, s = lm.llmint8_quantize_colwise(Wd)
        layer, ws_bytes = lm.llmint8_linear, lm.llmint8_workspace_size(M, K, N)
    else:
        Wq, s = lm.llmint8_quantize_colwise_fp8(Wd)
        layer, ws_bytes = lm.llmint8_linear_fp8, lm.llmint8_linear_fp8_workspace_size(M, K, N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    bias = (torch.randn(N, generator=torch.Generator().manual_seed(5)) * 0.5).half().cuda() \
        if extras else None

    def outputs():
        return ([torch.empty((M, N), dtype=torch.float16, device="cuda") for _ in Xs],
                [torch.empty(1, dtype=torch.int32, device="cuda") for _ in Xs],
                [torch.empty(N, dtype=torch.float32, device="cuda") if extras else None
                 for _ in Xs])

    def calls(Y, cnt, ycm):
        for i, X in enumerate(Xs):
            layer(X, Wq, s, Wd, 6.0, Y=Y[i], workspace=ws, outlier_count=cnt[i],
                  bias=bias, y_col_absmax=ycm[i])

    Yr, cr, mr = outputs()
    calls(Yr, cr, mr)
    torch.cuda.synchronize()
    assert cr[0].item() > 0

    Yg, cg, mg = outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(Yg, cg, mg)
    other = torch.randn((M, K), generator=torch.Generator().manual_seed(9)).half().cuda()
    for rep in range(4):
        for i in range(len(Xs)):  # stale values that a replay must overwrite
            Yg[i].fill_(7.0)
            cg[i].fill_(-1)
            if extras:
                mg[i].fill_(1e9)
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(Xs)):
            assert torch.equal(Yg[i].view(torch.int16), Yr[i].view(torch.int16)), (rep, i)
            assert torch.equal(cg[i], cr[i]), (rep, i)
            if extras:
                assert torch.equal(mg[i], mr[i]), (rep, i)
        # eager work on the same workspace between replays
        layer(other, Wq, s, Wd, 2.0, workspace=ws)
        torch.cuda.synchronize()
