"""The seeded input generator: determinism, shapes, dtypes and the outlier recipe."""
import numpy as np
import torch

from post_weight_quantization_mean_amd import synth


def test_deterministic_and_shapes():
    s1, X1, W1 = synth.make_layer("tiny")
    s2, X2, W2 = synth.make_layer("tiny")
    assert torch.equal(X1, X2) and torch.equal(W1, W2)
    assert X1.shape == (64, 256) and W1.shape == (128, 256) and X1.dtype == torch.float32
    _, X3, _ = synth.make_layer("tiny", seed=1)
    assert not torch.equal(X1, X3)


def test_row_prefix_sampling_matches_full_draw():
    spec, X, W = synth.make_layer("tiny")
    assert torch.equal(synth.make_x(spec, 0, 0, 0, rows=16), X[:16])
    assert torch.equal(synth.make_w(spec, 0, 0, 0, rows=8), W[:8])


def test_outlier_channels_recipe():
    spec = synth.CONFIGS["tiny"].layers[0]
    c = synth.channel_magnitudes(spec, synth._rng(0, 0, 0))
    base = synth._rng(0, 0, 0).lognormal(0.0, 0.5, size=spec.K)
    ratio = c / base.astype(np.float32)
    assert np.sum(np.isclose(ratio, 20.0, rtol=1e-6)) == 3
    assert np.sum(np.isclose(ratio, 1.0, rtol=1e-6)) == spec.K - 3


def test_config_table_matches_workloads():
    L = {c: [(l.name, l.M, l.K, l.N, l.dtype, l.n_out) for l in cfg.layers] for c, cfg in synth.CONFIGS.items()}
    assert L["tiny"] == [("tiny", 64, 256, 128, "f32", 3)]
    assert L["attn"] == [("attn", 4096, 4096, 4096, "bf16", 41)]
    assert L["down"] == [("down", 4096, 11008, 4096, "bf16", 110)]
    assert L["gate_up"] == [("gate_up", 8192, 5120, 27648, "bf16", 51)]
    assert [x[:4] for x in L["block"]] == [("qkv", 16384, 4096, 6144), ("o_proj", 16384, 4096, 4096),
                                           ("gate_up", 16384, 4096, 28672), ("down", 16384, 14336, 4096)]


def test_sparse_rows_mostly_near_zero():
    spec, X, _ = synth.custom_layer(64, 256, 8, x_kind="sparse", n_out=2, out_mult=("const", 30.0))
    c = synth.channel_magnitudes(spec, synth._rng(0, 100, 0))
    small = (X.abs().float().numpy() < 0.05 * c[None, :]).mean()
    assert 0.65 < small < 0.8
