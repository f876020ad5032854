"""Pins of the artefact decoder and the W4A16 product ("AWQ：为什么 4-bit 权重量化要先观察 Activation",
§7: decode the artefact's codes, scales and zero points and compare with the Q/DQ reference the
search used; §8: 4-bit weights times 16-bit activations)."""
from fractions import Fraction

import numpy as np

from oracle import awq_oracle as o


def test_artefact_matches_search_qdq_within_fp16_rounding():
    """§7's alignment check: the decoded artefact equals the search's Delta (q - z) up to the
    fp16 rounding of Delta (relative 2^-11), and exactly where Delta is an fp16 number."""
    rng = np.random.default_rng(0)
    W = (rng.standard_normal((32, 512)) * 0.05).astype(np.float32)
    s = (rng.random(512) + 0.5).astype(np.float32)
    art = o.pack(W, s)
    ref = o.dequant_scaled(art["codes"], art["z"], art["delta"])
    got = o.dequant_artefact(art["qweight"], art["scales"], art["zeros"])
    assert np.all(np.abs(got - ref) <= 2.0 ** -11 * np.abs(ref) + 1e-30)
    # groups whose range is a power of two times 15: Delta is exact in fp16, decoding is exact
    W2 = np.tile(np.linspace(-0.5, 1.375, 16, dtype=np.float32), (4, 8))  # range 1.875 = 15/8
    art2 = o.pack(W2, np.ones(128, np.float32))
    assert np.all(art2["delta"] == np.float32(0.125))
    assert np.array_equal(o.dequant_artefact(art2["qweight"], art2["scales"], art2["zeros"]),
                          o.dequant_scaled(art2["codes"], art2["z"], art2["delta"]))


def test_w4a16_exact_rational():
    rng = np.random.default_rng(1)
    W = (rng.standard_normal((3, 256)) * 0.1).astype(np.float32)
    art = o.pack(W, np.ones(256, np.float32))
    X = rng.standard_normal((2, 256)).astype(np.float32)
    Y = o.w4a16_matmul(X, art["qweight"], art["scales"], art["zeros"])
    q = o.unpack_words(art["qweight"])
    for m in range(2):
        for n in range(3):
            tot = Fraction(0)
            for k in range(256):
                g = k // 128
                d = Fraction(float(np.float16(art["scales"][n, g])))
                tot += Fraction(float(X[m, k])) * d * (int(q[n, k]) - int(np.float16(art["zeros"][n, g])))
            assert abs(float(tot) - Y[m, n]) <= 1e-12 * max(abs(float(tot)), 1e-30)


def test_w4a16_undoes_the_scaling():
    """With X' = X / s and the artefact of S W, X' W_hat^T approximates X W^T (the layer the
    search started from) to within the quantization error bound of §3 (|E| <= Delta / (2 s))."""
    rng = np.random.default_rng(2)
    K, N = 256, 8
    W = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    s = np.exp2(rng.integers(-2, 3, K)).astype(np.float32)
    X = rng.standard_normal((4, K))
    art = o.pack(W, s)
    Y = o.w4a16_matmul(X / s[None, :].astype(np.float64), art["qweight"], art["scales"], art["zeros"])
    # each weight is off by at most Delta/2 / s in the original units (codes in range), plus
    # |q - z| <= 15 times the fp16 rounding of Delta (2^-11 relative)
    dW = (art["scales"].astype(np.float64).repeat(128, axis=1) * (0.5 + 16 * 2.0 ** -11)) / s[None, :]
    bound = np.abs(X) @ dW.T
    assert np.all(np.abs(Y - X @ W.astype(np.float64).T) <= bound + 1e-12)
