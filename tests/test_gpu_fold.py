"""GPU parity of applying the chosen scales ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §6):
folding S^-1 into a producer (rows divided by s) and scaling a consumer's columns by s must be
bit-exact against the oracle (one rounding of the exact result, fp32 or bf16); act(x) / s is
within a few fp32 ulps (device erfc / exp), one bf16 ulp after bf16 rounding."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import awq_oracle as o
from tests.conftest import GOLDEN

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_mean_amd import awq as _awq
    _awq.lib()
    return _awq


def _tensor(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def _scales(n, seed):
    return np.exp(0.5 * np.random.default_rng(seed).standard_normal(n)).astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fold_norm_and_previous_linear(awq, dtype):
    K, Kin = 1000, 300  # 1000 rows: vectors and ragged row tails
    rng = np.random.default_rng(1)
    s = _scales(K, 2)
    sd = torch.from_numpy(s).to(DEV)
    gamma = _tensor(rng.standard_normal(K), dtype)
    beta = _tensor(rng.standard_normal(K), dtype)
    full = _tensor(rng.standard_normal((K, Kin + 20)), dtype)  # row stride Kin + 20
    Wp = full[:, :Kin]
    for host in (gamma, beta, Wp):
        dev = host.to(DEV) if host.is_contiguous() else full.to(DEV)[:, :Kin]
        awq.fold_rows(dev, sd)
        ref = o.fold_rows(_np(host), s, dtype)
        assert np.array_equal(_np(dev), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,K,pad", [(256, 4096, 0), (77, 1000, 8), (3, 5, 3)])
def test_scale_cols(awq, dtype, N, K, pad):
    rng = np.random.default_rng(3)
    s = _scales(K, 4)
    full = _tensor(rng.standard_normal((N, K + pad)), dtype)
    W = full.to(DEV)[:, :K]
    awq.scale_cols(W, torch.from_numpy(s).to(DEV))
    assert np.array_equal(_np(W), o.scale_cols(_np(full[:, :K]), s, dtype))
    if pad:  # the padding columns are untouched
        assert np.array_equal(_np(full.to(DEV)[:, K:]), _np(full[:, K:]))


def _ulp32(x):
    return np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)


@pytest.mark.parametrize("act", ["gelu", "silu"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scaled_act(awq, act, dtype):
    rng = np.random.default_rng(5)
    M, K = 64, 1000
    X = _tensor(rng.standard_normal((M, K)) * 4.0, dtype)
    s = _scales(K, 6)
    Y = awq.scaled_act(X.to(DEV), torch.from_numpy(s).to(DEV), act)
    ref = o.scaled_activation(_np(X).astype(np.float64), s, act)
    got = _np(Y).astype(np.float64)
    if dtype == "f32":
        # the device erfc / exp (a few ulps), the fp32 roundings of the argument and of the
        # quotient, and for GELU the argument's rounding magnified by the slope of erfc:
        # d ln erfc(z) / dz ~ -2z, so 2^-24 |z| in z costs ~2 z^2 2^-24 relative
        z = np.abs(_np(X).astype(np.float64)) / np.sqrt(2.0)
        k = 16 + (2 * z * z if act == "gelu" else 2 * z)
        assert np.all(np.abs(got - ref) <= k * _ulp32(ref) + 1e-37)
    else:
        r16 = o._round_to(ref, "bf16").astype(np.float64)
        one = np.abs(r16) * 2.0 ** -7 + 1e-37  # one bf16 ulp (8 significand bits) or less
        assert np.all(np.abs(got - r16) <= one)


def test_gelu_example_on_gpu(awq):
    """The page's §6 example: act(h) / s followed by the s-scaled weight gives the reference."""
    ex = json.load(open(os.path.join(GOLDEN, "explainer_fold_example.json")))
    h = torch.tensor([ex["h"]], dtype=torch.float32, device=DEV)
    s = torch.tensor(ex["scales"], dtype=torch.float32, device=DEV)
    W = torch.tensor(ex["weights_k_by_n"], dtype=torch.float32).T.contiguous().to(DEV)  # [N, K]
    ref = o.gelu(np.array([ex["h"]])) @ np.array(ex["weights_k_by_n"])
    hs = awq.scaled_act(h, s, "gelu")
    Ws = awq.scale_cols(W.clone(), s)
    out = (hs.double() @ Ws.double().T).cpu().numpy()
    assert np.max(np.abs(out - ref)) <= 1e-6  # fp32 parameters and activation


def test_bf16_midpoint_ties(awq):
    """fp32 results that fall exactly halfway between two bf16 values while the exact product
    or quotient does not (s has 24 significand bits): the exact residual decides."""
    w = torch.tensor([[-2.171875, 1.0859375, -0.54296875, 0.033935546875]], dtype=torch.bfloat16)
    s = np.full(4, 1.7446043, np.float32)
    W = w.to(DEV)
    awq.scale_cols(W, torch.from_numpy(s).to(DEV))
    ref = o.scale_cols(_np(w), s, "bf16")
    assert np.array_equal(_np(W), ref)
    assert _np(W)[0, 0] == -3.796875  # the fp32 product -3.7890625 is the midpoint; exact is beyond it


def test_fold_flags(awq):
    s = torch.ones(16, device=DEV)
    s[3] = 0.0
    with pytest.raises(ValueError, match="scales"):
        awq.fold_rows(torch.ones(16, device=DEV), s)
    with pytest.raises(ValueError, match="scales"):
        awq.scale_cols(torch.ones((2, 16), device=DEV), s)
