"""GPU parity of the grouped search (awq_search_multi): projections that read one X and share
one scale vector ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §6: Q, K and V all consume
the normalized input) searched as one layer from a list of weights, without concatenating
them.  With every weight's rows a multiple of 128 the result must be bit-identical to
awq_search on the concatenated weight (same tiles, same fixed-order sums); with ragged row
counts each weight is padded separately, and the losses are checked against the oracle on the
concatenation with the same tolerance as the single-weight search."""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as o
from post_weight_quantization_mean_amd import synth
from tests.test_gpu_parity import DEV, banner, check_choice, loss_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_mean_amd import awq as _awq
    _awq.lib()
    return _awq


def weights(K, Ns, dtype, seed):
    return [synth.custom_layer(1, K, n, dtype=dtype, seed=seed + i)[2] for i, n in enumerate(Ns)]


@pytest.mark.parametrize("Ns,wd", [((256, 128, 384), "bf16"), ((128, 128), "f32"), ((512,), "bf16")])
def test_multi_matches_concatenated(awq, Ns, wd):
    banner(f"search multi vs concatenated N={Ns} {wd}")
    M, K = 700, 384
    _, X, _ = synth.custom_layer(M, K, 1, dtype="bf16", seed=11)
    Ws = [w.to(DEV) for w in weights(K, Ns, wd, 20)]
    Xd = X.to(DEV)
    a = awq.stats(Xd)
    r_cat = awq.search(Xd, torch.cat(Ws, dim=0), a)
    r_multi = awq.search(Xd, Ws, a)
    assert torch.equal(r_multi.losses, r_cat.losses)
    assert torch.equal(r_multi.best, r_cat.best) and torch.equal(r_multi.s_best, r_cat.s_best)


@pytest.mark.parametrize("Ns", [(100, 37, 200), (1, 129)])
def test_multi_ragged_vs_oracle(awq, Ns):
    banner(f"search multi ragged N={Ns}")
    M, K = 600, 384
    _, X, _ = synth.custom_layer(M, K, 1, dtype="bf16", seed=12)
    Wl = weights(K, Ns, "bf16", 30)
    X64 = synth.to_f64(X)
    W32 = np.concatenate([synth.to_f32(w) for w in Wl], axis=0)
    a32 = o.activation_stat(X64).astype(np.float32)
    ref = o.search(X64, W32, a32)
    res = awq.search(X.to(DEV), [w.to(DEV) for w in Wl], torch.from_numpy(a32).to(DEV), return_table=True)
    assert np.array_equal(res.s_table.cpu().numpy().view(np.int32), ref["s_table"].view(np.int32))
    L = res.losses.cpu().numpy()
    tol = loss_tolerance(X64, W32, ref["s_table"], ref["losses"], False)
    err = np.abs(L - ref["losses"])
    assert np.all(err <= tol), f"loss error {err / ref['losses']} (rel) above tolerance"
    print(f"[gpu-case] max rel err {np.max(err / ref['losses']):.2e}", flush=True)
    check_choice(res.best_index, ref["losses"], ref["best"], tol, n_out=M * W32.shape[0])


def test_multi_strided_views(awq):
    """Weights given as views with row strides larger than K (and different per weight)."""
    banner("search multi strided views")
    M, K = 512, 256
    _, X, _ = synth.custom_layer(M, K, 1, dtype="bf16", seed=13)
    Wl = weights(K, (128, 256), "bf16", 40)
    pads = (8, 64)
    views = []
    for w, p in zip(Wl, pads):
        big = torch.zeros((w.shape[0], K + p), dtype=w.dtype)
        big[:, :K] = w
        views.append(big.to(DEV)[:, :K])
    Xd = X.to(DEV)
    a = awq.stats(Xd)
    r_multi = awq.search(Xd, views, a)
    r_cat = awq.search(Xd, torch.cat([w.to(DEV) for w in Wl], dim=0), a)
    assert torch.equal(r_multi.losses, r_cat.losses) and torch.equal(r_multi.best, r_cat.best)


def test_multi_rejects_mixed_dtypes_and_k(awq):
    Xd = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    a = torch.ones(256, device=DEV)
    with pytest.raises(ValueError, match="dtype"):
        awq.search(Xd, [torch.zeros((128, 256), dtype=torch.bfloat16, device=DEV),
                        torch.zeros((128, 256), device=DEV)], a)
    with pytest.raises(ValueError, match="disagree on K"):
        awq.search(Xd, [torch.zeros((128, 384), dtype=torch.bfloat16, device=DEV)], a)
