"""awq_search_static, the search entry point that allocates nothing (its workspace is the
library's static device array), against awq_search with a caller workspace, through the C ABI.
Two calls in a row share the one array; the second layer is smaller, and each call must be
bit-identical to the workspace search of the same layer (the same kernels and fixed-order
reductions run on the same inputs)."""
import pytest
import torch

from post_weight_quantization_mean_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def awq():
    from post_weight_quantization_mean_amd import awq as a
    a.lib()
    return a


def run_case(awq, M, K, N, dtype, seed):
    print(f"[gpu-case] search_static M={M} K={K} N={N} {dtype} seed={seed}", flush=True)
    _, X, W = synth.custom_layer(M, K, N, dtype=dtype, seed=seed)
    Xd, Wd = X.to(DEV), W.to(DEV)
    a = awq.stats(Xd)
    got = awq.search(Xd, Wd, a, return_table=True, no_alloc=True)
    ref = awq.search(Xd, Wd, a, return_table=True)
    torch.cuda.synchronize()
    assert torch.equal(got.losses.view(torch.int64), ref.losses.view(torch.int64)), (got.losses, ref.losses)
    assert got.best_index == ref.best_index
    assert torch.equal(got.s_best.view(torch.int32), ref.s_best.view(torch.int32))
    assert torch.equal(got.s_table.view(torch.int32), ref.s_table.view(torch.int32))
    return got


def test_static_search_twice_second_smaller(awq):
    # 4 token tiles x 6 output tiles x 8 groups, then a ragged layer that fits in less of the array
    first = run_case(awq, 2048, 1024, 768, "bf16", 41)
    second = run_case(awq, 600, 512, 200, "bf16", 42)
    assert not torch.equal(first.losses, second.losses)


def test_static_search_fp32_layer(awq):
    # the tiny fp32 configuration takes the fp32 kernel through the same static workspace
    run_case(awq, 64, 256, 128, "f32", 0)
