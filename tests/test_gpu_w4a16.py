"""GPU parity of the W4A16 product over the packed artefact ("AWQ：为什么 4-bit 权重量化要先观察
Activation", §7, §8) against the oracle's exact product, on artefacts the oracle packed.
Decode (<= 8 bf16 tokens, or fp32 tokens): products exact in fp32, fp32 sums, the group scale
applied to partial sums, so the bound is a few dozen fp32 roundings of sum |x| Delta (q + z + 1)
(with bf16 tokens the sums carry a bias of 128 per code: q + z + 257).
Prefill (> 8 bf16 tokens): the decoded weight is rounded once to bf16 for the matrix cores,
so the bound adds 2^-8 sum |x| |W_hat| and K 2^-24 of fp32 accumulation."""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as o

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_mean_amd import awq as _awq
    _awq.lib()
    return _awq


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)


def artefact(N, K, seed):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)
    s = np.exp(0.3 * rng.standard_normal(K)).astype(np.float32)
    return o.pack(W, s)


def run(awq, art, X, prefill, biased=None):
    """biased: the decode variant for bf16 activations sums x (128 + q) and removes the bias
    per 32 channels, so its fp32 roundings scale with sum |x| Delta (q + z + 257)."""
    if biased is None:
        biased = X.dtype == torch.bfloat16 and not prefill
    q = torch.from_numpy(art["qweight"]).to(DEV)
    sc = torch.from_numpy(art["scales"].view(np.float16)).to(DEV)
    zz = torch.from_numpy(art["zeros"].view(np.float16)).to(DEV)
    Y = awq.w4a16(X.to(DEV), q, sc, zz).cpu().numpy().astype(np.float64)
    return check(Y, X.float().numpy().astype(np.float64), art, prefill, biased)


def check(Y, X64, art, prefill, biased):
    """Y [m, n] against the oracle's exact product of X64 [m, K] and the artefact's n rows."""
    ref = o.w4a16_matmul(X64, art["qweight"], art["scales"], art["zeros"])
    Wh = o.dequant_artefact(art["qweight"], art["scales"], art["zeros"])
    K = X64.shape[1]
    codes = o.unpack_words(art["qweight"]).astype(np.float64)
    d = art["scales"].astype(np.float64).repeat(128, axis=1)
    z = art["zeros"].astype(np.float64).repeat(128, axis=1)
    mag = np.abs(X64) @ (d * (codes + z + (257.0 if biased else 1.0))).T  # sum |x| Delta (q + z + 1 [+ 256])
    tol = 64 * 2.0 ** -24 * mag
    if prefill:
        tol = tol + (2.0 ** -8 + K * 2.0 ** -24) * (np.abs(X64) @ np.abs(Wh).T)
    err = np.abs(Y - ref)
    bad = np.argwhere(err > tol + 1e-30)
    assert bad.size == 0, f"{len(bad)} outputs outside tolerance, first {bad[:4].tolist()}"
    return float(np.max(err / (tol + 1e-30)))  # the largest error as a fraction of its tolerance


# dot kernel: one token, or K not a multiple of 1024; matrix-core kernel: 2-8 tokens with K a
# multiple of 1024 (8 x 14336: two K passes; ragged last tiles of 16 rows)
@pytest.mark.parametrize("M,K,N", [(1, 4096, 256), (3, 14336, 130), (8, 384, 64), (2, 5120, 4),
                                   (4, 2048, 33), (6, 3072, 50), (8, 4096, 100), (8, 14336, 70)])
def test_decode_bf16(awq, M, K, N):
    banner(f"w4a16 decode M={M} K={K} N={N}")
    art = artefact(N, K, 1)
    X = torch.from_numpy(np.random.default_rng(2).standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    run(awq, art, X, prefill=False)


def test_decode_fp32_many_tokens(awq):
    """fp32 activations take the decode kernel at any M, eight tokens per launch."""
    art = artefact(96, 1024, 3)
    X = torch.from_numpy(np.random.default_rng(4).standard_normal((20, 1024)).astype(np.float32))
    run(awq, art, X, prefill=False)


# K / 32 chunks: 16 (one unrolled run of 12, tail 4), 128 (tail 8), 32 (tail 8), 4 (tail only),
# 12 and 48 (no tail), 64 (tail 4); M and N ragged against the 512 x 128 tile
@pytest.mark.parametrize("M,K,N", [(9, 512, 128), (600, 4096, 200), (1024, 1024, 384), (520, 128, 130),
                                   (513, 384, 64), (700, 1536, 256), (40, 2048, 129)])
def test_prefill_bf16(awq, M, K, N):
    banner(f"w4a16 prefill M={M} K={K} N={N}")
    art = artefact(N, K, 5)
    X = torch.from_numpy(np.random.default_rng(6).standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    run(awq, art, X, prefill=True)


def test_strided_activations_and_output(awq):
    art = artefact(64, 512, 7)
    full = torch.from_numpy(np.random.default_rng(8).standard_normal((4, 640)).astype(np.float32)).to(torch.bfloat16)
    Xd = full.to(DEV)[:, :512]  # row stride 640
    q = torch.from_numpy(art["qweight"]).to(DEV)
    sc = torch.from_numpy(art["scales"].view(np.float16)).to(DEV)
    zz = torch.from_numpy(art["zeros"].view(np.float16)).to(DEV)
    Yfull = torch.full((4, 80), -7.0, device=DEV)
    awq.w4a16(Xd, q, sc, zz, out=Yfull[:, :64])
    ref = o.w4a16_matmul(full[:, :512].float().numpy(), art["qweight"], art["scales"], art["zeros"])
    assert np.allclose(Yfull[:, :64].cpu().numpy(), ref, rtol=1e-4, atol=1e-5)
    assert torch.all(Yfull[:, 64:] == -7.0)  # outside the output view: untouched


def test_prefill_strided_activations_and_output(awq):
    """The prefill (more than 8 bf16 tokens) on an X view with row stride K + 72 and an output
    view with row stride N + 40: the X copies address rows by their stride, and nothing outside
    the output view is written."""
    banner("w4a16 prefill strided")
    M, K, N = 600, 1024, 200
    art = artefact(N, K, 11)
    full = torch.from_numpy(np.random.default_rng(12).standard_normal((M, K + 72)).astype(np.float32)).to(torch.bfloat16)
    Xd = full.to(DEV)[:, :K]
    q = torch.from_numpy(art["qweight"]).to(DEV)
    sc = torch.from_numpy(art["scales"].view(np.float16)).to(DEV)
    zz = torch.from_numpy(art["zeros"].view(np.float16)).to(DEV)
    Yfull = torch.full((M, N + 40), -7.0, device=DEV)
    awq.w4a16(Xd, q, sc, zz, out=Yfull[:, :N])
    check(Yfull[:, :N].cpu().numpy().astype(np.float64), full[:, :K].float().numpy().astype(np.float64), art,
          prefill=True, biased=False)
    assert torch.all(Yfull[:, N:] == -7.0)


def test_scaled_inputs_recover_the_layer(awq):
    """GPU chain: pack S W on the GPU, feed X / s: the W4A16 output approximates X W^T within the
    quantization error bound |E| <= Delta / (2 s), plus |q - z| times the fp16 rounding of Delta."""
    rng = np.random.default_rng(9)
    M, K, N = 16, 1024, 256
    W = torch.from_numpy((rng.standard_normal((N, K)) / np.sqrt(K)).astype(np.float32)).to(torch.bfloat16)
    s = torch.from_numpy(np.exp(0.3 * rng.standard_normal(K)).astype(np.float32))
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    q, sc, zz = awq.pack(W.to(DEV), s.to(DEV))
    Xs = (X / s[None, :]).to(DEV)  # fp32 activations carrying S^-1
    Y = awq.w4a16(Xs, q, sc, zz).cpu().double()
    exact = X.double() @ W.double().T
    # |v - Delta16 (q - z)| <= Delta / 2 + |q - z| Delta 2^-11 <= Delta16 (1/2 + 16 2^-11)
    dW = sc.cpu().double().repeat_interleave(128, dim=1) * (0.5 + 16 * 2.0 ** -11) / s.double()[None, :]
    bound = X.double().abs() @ dW.T + 1e-4 * (X.double().abs() @ W.double().abs().T)
    assert torch.all((Y - exact).abs() <= bound)


def test_prefill_full_size_sampled(awq):
    """The prefill in the shape the benchmark times: 4096 bf16 tokens against a 28672 x 4096
    artefact (synthetic: uniformly random code words, positive fp16 scales, integer zeros), all
    outputs computed on the GPU, a 24 x 96 sample of them (tokens and outputs from every tile
    row and column, the last of each included) checked against the oracle."""
    banner("w4a16 prefill full size 4096 x 28672 x 4096, sampled")
    M, K, N = 4096, 4096, 28672
    rng = np.random.default_rng(10)
    art = {"qweight": rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint32).view(np.int32),
           "scales": (np.abs(rng.standard_normal((N, K // 128))) * 0.01 + 1e-3).astype(np.float16),
           "zeros": rng.integers(0, 16, size=(N, K // 128)).astype(np.float16)}
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(art["qweight"]).to(DEV)
    sc = torch.from_numpy(art["scales"]).to(DEV)
    zz = torch.from_numpy(art["zeros"]).to(DEV)
    Y = awq.w4a16(X.to(DEV), q, sc, zz)
    rows = np.unique(np.concatenate([rng.choice(M, 23, replace=False), [M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 95, replace=False), [N - 1]]))
    Ys = Y[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    sub = {k: v[cols] for k, v in art.items()}
    X64 = X.float().numpy().astype(np.float64)[rows]
    frac = check(Ys, X64, sub, prefill=True, biased=False)
    print(f"[gpu-case] full-size prefill sample: largest error {frac:.3f} of its tolerance", flush=True)


@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_decode_full_size_sampled(awq, M):
    """The decode in the shape the benchmark times: M bf16 tokens against a 28672 x 4096
    artefact (synthetic: uniformly random code words, positive fp16 scales, integer zeros).  The
    grid sweeps the rows several times (one token: each wave owns several row groups; eight
    tokens: one block per CU, so waves loop over several 16-row tiles), so every wave's later rows
    are covered; a sample of 256 outputs (the first and last rows included) is checked against the
    oracle."""
    banner(f"w4a16 decode full size M={M} x 28672 x 4096, sampled")
    K, N = 4096, 28672
    rng = np.random.default_rng(20 + M)
    art = {"qweight": rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint32).view(np.int32),
           "scales": (np.abs(rng.standard_normal((N, K // 128))) * 0.01 + 1e-3).astype(np.float16),
           "zeros": rng.integers(0, 16, size=(N, K // 128)).astype(np.float16)}
    X = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(art["qweight"]).to(DEV)
    sc = torch.from_numpy(art["scales"]).to(DEV)
    zz = torch.from_numpy(art["zeros"]).to(DEV)
    Y = awq.w4a16(X.to(DEV), q, sc, zz)
    cols = np.unique(np.concatenate([rng.choice(N, 254, replace=False), [0, N - 1]]))
    Ys = Y[:, torch.from_numpy(cols).to(DEV)].cpu().numpy().astype(np.float64)
    sub = {k: v[cols] for k, v in art.items()}
    frac = check(Ys, X.float().numpy().astype(np.float64), sub, prefill=False, biased=True)
    print(f"[gpu-case] full-size decode M={M} sample: largest error {frac:.3f} of its tolerance", flush=True)


def test_decode_unaligned_scales_take_the_dot_kernel(awq):
    """The matrix-core decode reads scales and zeros 16 bytes at a time; tensors that are only
    2-byte aligned (a contiguous view one element into a buffer) go to the dot kernel instead, with
    the same result bound, for several token counts."""
    banner("w4a16 decode, scales and zeros 2-byte aligned")
    N, K = 96, 2048
    art = artefact(N, K, 4)
    q = torch.from_numpy(art["qweight"]).to(DEV)
    G = K // 128
    sbuf = torch.empty(N * G + 1, dtype=torch.float16, device=DEV)
    zbuf = torch.empty(N * G + 1, dtype=torch.float16, device=DEV)
    sc = sbuf[1:].view(N, G)
    zz = zbuf[1:].view(N, G)
    sc.copy_(torch.from_numpy(art["scales"].view(np.float16)))
    zz.copy_(torch.from_numpy(art["zeros"].view(np.float16)))
    assert sc.data_ptr() % 16 != 0 and zz.data_ptr() % 16 != 0
    for M in (1, 2, 5):
        X = torch.from_numpy(np.random.default_rng(30 + M).standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
        Y = awq.w4a16(X.to(DEV), q, sc, zz).cpu().numpy().astype(np.float64)
        check(Y, X.float().numpy().astype(np.float64), art, prefill=False, biased=True)


# matrix-core decode edges: one row, rows around one 16-row tile, one 1024-channel round, five
# rounds (tiles start at rotated rounds), 257 tiles with a partial last one
@pytest.mark.parametrize("M,K,N", [(2, 1024, 1), (3, 1024, 15), (8, 1024, 17), (5, 5120, 33), (2, 3072, 4100)])
def test_decode_mfma_edges(awq, M, K, N):
    banner(f"w4a16 decode (matrix cores) M={M} K={K} N={N}")
    art = artefact(N, K, 5)
    X = torch.from_numpy(np.random.default_rng(40 + M).standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    run(awq, art, X, prefill=False)


def test_prefill_unaligned_scales_odd_groups(awq):
    """The prefill reads each row's fp16 scale and zero with 2-byte loads: scales and zeros that
    are only 2-byte aligned (a view one element into a buffer) with an odd number of groups per
    row (K = 1152: every other row starts at an odd element) give the same result bound, on a
    ragged M and N (two token tiles, two output tiles, the K loop's 4-step tail)."""
    banner("w4a16 prefill, scales and zeros 2-byte aligned, K / 128 odd")
    N, K, M = 200, 1152, 700
    art = artefact(N, K, 8)
    q = torch.from_numpy(art["qweight"]).to(DEV)
    G = K // 128
    sbuf = torch.empty(N * G + 1, dtype=torch.float16, device=DEV)
    zbuf = torch.empty(N * G + 1, dtype=torch.float16, device=DEV)
    sc = sbuf[1:].view(N, G)
    zz = zbuf[1:].view(N, G)
    sc.copy_(torch.from_numpy(art["scales"].view(np.float16)))
    zz.copy_(torch.from_numpy(art["zeros"].view(np.float16)))
    assert sc.data_ptr() % 4 != 0 and zz.data_ptr() % 4 != 0
    X = torch.from_numpy(np.random.default_rng(41).standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    Y = awq.w4a16(X.to(DEV), q, sc, zz).cpu().numpy().astype(np.float64)
    check(Y, X.float().numpy().astype(np.float64), art, prefill=True, biased=False)


@pytest.mark.parametrize("M,K,N,stride", [(9, 512, 128, 0), (600, 4096, 200, 0), (1000, 1152, 130, 0),
                                          (4096, 4096, 1024, 0), (700, 1024, 256, 72)])
def test_prefill_copy_of_x_matches_staged(awq, M, K, N, stride):
    """The prefill reading X from its copy in matrix-core operand order (the default, with a
    workspace) against the same kernel staging X through LDS (no workspace): the same products
    in the same order, so Y must agree bit for bit, on ragged M (rows past M zero in the copy),
    K / 128 odd, ragged N and X with row stride K + 72; and a reused, larger workspace gives
    the same Y again."""
    banner(f"w4a16 prefill copy vs staged M={M} K={K} N={N} stride+{stride}")
    art = artefact(N, K, 13)
    q = torch.from_numpy(art["qweight"]).to(DEV)
    sc = torch.from_numpy(art["scales"].view(np.float16)).to(DEV)
    zz = torch.from_numpy(art["zeros"].view(np.float16)).to(DEV)
    full = torch.from_numpy(np.random.default_rng(14).standard_normal((M, K + stride)).astype(np.float32))
    Xd = full.to(torch.bfloat16).to(DEV)[:, :K]
    need = awq.w4a16_workspace_bytes(M, K)
    assert need == 2 * (-(-M // 32) * 32) * K
    Y_copy = awq.w4a16(Xd, q, sc, zz)
    Y_staged = awq.w4a16(Xd, q, sc, zz, staged=True)
    assert torch.equal(Y_copy, Y_staged)
    ws = torch.full((need + 4096,), 0x7f, dtype=torch.uint8, device=DEV)  # stale bytes in the workspace
    assert torch.equal(awq.w4a16(Xd, q, sc, zz, workspace=ws), Y_staged)
