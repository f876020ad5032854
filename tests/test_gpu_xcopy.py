"""The persistent search kernel reads X from a copy in matrix-core operand order placed at the end
of the workspace; with a workspace too short for that copy the search runs the kernel that
stages X through LDS itself.  Both evaluate the candidate loss of "AWQ：为什么 4-bit 权重量化要先
观察 Activation" (§4: the module output error of each scaled, quantized weight) with the same
products summed in the same order, so their losses, choice and scales must agree bit for bit
on every shape: ragged token and output counts, strided X, several weights, the smallest and a
large K.  Parity of either kernel with the oracle is covered by the parity suites."""
import pytest
import torch

from post_weight_quantization_mean_amd import synth
from tests.test_abi import xcopy_bytes
from tests.test_gpu_parity import DEV, banner

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_mean_amd import awq as _awq
    _awq.lib()
    return _awq


def both(awq, X, W, a):
    """(persistent result, staged-X result): the full workspace, then one xcopy bytes short."""
    M, K = X.shape
    N = [w.shape[0] for w in W] if isinstance(W, list) else W.shape[0]
    full = awq.search_workspace_bytes(M, K, N)
    short = full - xcopy_bytes(M, K)
    assert xcopy_bytes(M, K) > 0
    r_full = awq.search(X, W, a, return_table=True,
                        workspace=torch.empty(full, dtype=torch.uint8, device=DEV))
    r_short = awq.search(X, W, a, return_table=True,
                         workspace=torch.empty(short, dtype=torch.uint8, device=DEV))
    return r_full, r_short


def assert_same(r1, r2):
    assert torch.equal(r1.losses, r2.losses)
    assert torch.equal(r1.best, r2.best)
    assert torch.equal(r1.s_best, r2.s_best) and torch.equal(r1.s_table, r2.s_table)
    assert torch.isfinite(r1.losses).all() and (r1.losses > 0).all()


@pytest.mark.parametrize("M,K,N", [
    (2048, 4096, 2048),   # several token tiles, whole tiles everywhere
    (1000, 512, 2048),    # the smallest K; the last token tile ragged (rows 1000..1023 zero in the copy)
    (1537, 1024, 2000),   # ragged tokens (one row into a fourth tile) and ragged outputs
    (512, 14336, 4096),   # one token tile, the decoder block's down-projection K
])
def test_persistent_matches_staged(awq, M, K, N):
    banner(f"persistent vs staged-X search M={M} K={K} N={N}")
    _, X, W = synth.custom_layer(M, K, N, dtype="bf16", seed=M + K + N)
    Xd, Wd = X.to(DEV), W.to(DEV)
    a = awq.stats(Xd)
    assert_same(*both(awq, Xd, Wd, a))


def test_persistent_strided_x(awq):
    """X as a view with row stride K + 128: the copy is gathered from the strided rows."""
    banner("persistent vs staged-X search, strided X")
    M, K, N = 1024, 1024, 3072
    _, X, W = synth.custom_layer(M, K + 128, N, dtype="bf16", seed=5)
    Xd = X.to(DEV)[:, :K]
    Wd = W[:, :K].contiguous().to(DEV)
    a = awq.stats(Xd)
    r_full, r_short = both(awq, Xd, Wd, a)
    assert_same(r_full, r_short)
    r_dense = awq.search(Xd.contiguous(), Wd, a)
    assert torch.equal(r_full.losses, r_dense.losses)


def test_persistent_several_weights(awq):
    banner("persistent vs staged-X search, three weights")
    M, K = 1536, 1024
    _, X, _ = synth.custom_layer(M, K, 1, dtype="bf16", seed=7)
    Ws = [synth.custom_layer(1, K, n, dtype="bf16", seed=8 + i)[2].to(DEV) for i, n in enumerate((1024, 300, 512))]
    Xd = X.to(DEV)
    a = awq.stats(Xd)
    assert_same(*both(awq, Xd, Ws, a))


def test_persistent_twice_in_a_row(awq):
    """A second call with fewer tokens into the same workspace: rows of the first call's copy
    past the second call's M must not leak into its products."""
    banner("persistent search, larger then smaller M in one workspace")
    K, N = 1024, 4096
    _, X, W = synth.custom_layer(2048, K, N, dtype="bf16", seed=9)
    Xd, Wd = X.to(DEV), W.to(DEV)
    ws = torch.empty(awq.search_workspace_bytes(2048, K, N), dtype=torch.uint8, device=DEV)
    awq.search(Xd, Wd, awq.stats(Xd), workspace=ws)
    Xs = Xd[:1500]
    a = awq.stats(Xs)
    r_reused = awq.search(Xs, Wd, a, workspace=ws)
    _, r_short = both(awq, Xs, Wd, a)
    assert torch.equal(r_reused.losses, r_short.losses) and torch.equal(r_reused.best, r_short.best)
