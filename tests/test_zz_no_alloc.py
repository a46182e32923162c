"""The allocation-free layer entry point (llmint8_linear_noalloc) against
llmint8_linear on the same inputs: Y, the int32 accumulators and the outlier
count must be identical, call after call, with the shared per-GPU scratch
keeping the previous call's contents (the second call of each pair is
smaller than the first). Shapes whose workspace exceeds the scratch are
refused with LLMINT8_ERR_WORKSPACE."""
import sys

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import bit_quantized_matmul_col_amd as lm
    lm.lib()
    return torch, lm


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def both(torch, lm, M, K, N, seed, threshold=6.0):
    X, W, _ = workloads.random_case(M, K, N, seed=seed, n_out=3)
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W).cuda()
    Wq, s = lm.llmint8_quantize_colwise(Wd)
    C0 = torch.empty((M, N), dtype=torch.int32, device="cuda")
    C1 = torch.full((M, N), 7, dtype=torch.int32, device="cuda")
    c0 = torch.empty(1, dtype=torch.int32, device="cuda")
    c1 = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    Y1 = torch.full((M, N), 3.0, dtype=torch.float16, device="cuda")
    Y0 = lm.llmint8_linear(Xd, Wq, s, Wd, threshold, C_debug=C0, outlier_count=c0)
    lm.llmint8_linear_noalloc(Xd, Wq, s, Wd, threshold, Y=Y1, C_debug=C1, outlier_count=c1)
    Y2 = lm.llmint8_linear_noalloc(Xd, Wq, s, Wd, threshold)  # production form, no C_debug
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16)), "Y differs"
    assert torch.equal(Y0.view(torch.int16), Y2.view(torch.int16)), "Y (no C_debug) differs"
    assert torch.equal(C0, C1), "C differs"
    assert int(c0.item()) == int(c1.item()) >= 0


# pairs of consecutive calls, the second smaller: split-K small M (two K
# splits and more), the single kernel (M <= 16, K in {1024, 2048, 4096}), and
# a large-M call whose workspace fits in the scratch (the last pair: one that
# the workspace call runs with split-K tiles and the scratch call without)
PAIRS = [((64, 4096, 4096), (20, 1024, 520)),
         ((16, 4096, 11008), (3, 1024, 136)),
         ((300, 1024, 520), (70, 256, 64)),
         ((300, 4096, 520), (70, 256, 64)),
         ((48, 8192, 4096), (1, 16, 8)),
         ((192, 2048, 2048), (129, 4096, 520))]  # small-M kernels in three and four row groups


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_equals_linear_on_two_calls(dev, first, second):
    torch, lm = dev
    for i, (M, K, N) in enumerate((first, second)):
        say(f"case noalloc call {i} M={M} K={K} N={N}")
        assert lm.llmint8_workspace_size(M, K, N) <= lm.LLMINT8_NOALLOC_SCRATCH_BYTES
        both(torch, lm, M, K, N, seed=M + K + N + i)


def test_noalloc_refuses_shapes_beyond_its_scratch(dev):
    torch, lm = dev
    say("case noalloc beyond the scratch")
    M, K, N = 2048, 4096, 11008
    assert lm.llmint8_workspace_size(M, K, N) > lm.LLMINT8_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    Wq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    s = torch.ones(N, dtype=torch.float32, device="cuda")
    with pytest.raises(lm.Llmint8Error) as e:
        lm.llmint8_linear_noalloc(X, Wq, s, None, float("inf"))
    assert e.value.status == lm.LLMINT8_ERR_WORKSPACE
    # and a fitting call still works afterwards
    both(torch, lm, 32, 2048, 1032, seed=5)
