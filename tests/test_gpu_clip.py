"""GPU parity of the clipping search ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §5) and the
clipped pack: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.  Bars: every candidate's error within max(1e-3 relative, a bound derived from the
kernel's arithmetic); the chosen threshold identical unless the oracle's own errors of the two
choices are within those bounds; the chosen thresholds bitwise; the clipped pack bit-exact
given the same thresholds."""
import numpy as np
import pytest
import torch

from oracle import awq_oracle as o
from post_weight_quantization_mean_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
RTOL = 1e-3


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_mean_amd import awq as _awq
    _awq.lib()
    return _awq


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)


def clip_tolerance(X64, W32, s, ref, x_is_f32):
    """Per (candidate, row, group): max(1e-3 relative, bound).  Each partial output
    y = sum_{k in g} x_k e_k is formed from e rounded once to bf16 (8 significand bits, so
    |de| <= 2^-8 |e|), fp32
    products and reciprocals (<= 2^-21 |w|), an fp32 X split into two bf16 terms (<= 2^-16 |x|)
    and fp32 accumulation over the group's 128 terms (<= 128 2^-24); so
    |dy| <= cA sum|x||e| + cB sum|x||w| and |d mean(y^2)| <= mean(2|y||dy| + dy^2)."""
    cA = 2.0 ** -8 + 128 * 2.0 ** -24 + (2.0 ** -16 if x_is_f32 else 0.0)
    cB = 2.0 ** -21
    n_clip, N, G = ref["err"].shape
    tol = np.empty_like(ref["err"])
    absX = np.abs(X64)
    Wabs = np.abs(W32.astype(np.float64))
    for i in range(n_clip):
        q, z, d = o.quantize_clipped(W32, s, ref["thresholds"][i])
        E = W32.astype(np.float64) - o.effective_weight(q, z, d, s)
        for g in range(G):
            sl = slice(128 * g, 128 * (g + 1))
            Y = X64[:, sl] @ E[:, sl].T
            dy = cA * (absX[:, sl] @ np.abs(E[:, sl]).T) + cB * (absX[:, sl] @ Wabs[:, sl].T)
            bound = np.mean(2 * np.abs(Y) * dy + dy * dy, axis=0)
            tol[i, :, g] = np.maximum(RTOL * ref["err"][i, :, g], bound)
    return tol


def check_clip(awq, X, W, s, n_clip=10, rows=None, Xd=None):
    """Run the GPU search on the whole layer and compare rows ``rows`` (all by default).
    ``Xd``: the device tokens when they are a view (otherwise X is copied)."""
    Xd = X.to(DEV) if Xd is None else Xd
    Wd = W.to(DEV)
    res = awq.clip(Xd, Wd, torch.from_numpy(s).to(DEV), n_clip=n_clip, return_err=True)
    X64, W32 = synth.to_f64(X), synth.to_f32(W)
    if rows is None:
        rows = np.arange(W32.shape[0])
    ref = o.clip_errors(X64, W32[rows], s, n_clip=n_clip)
    err = res.err.cpu().numpy()[:, rows, :]
    best = res.best.cpu().numpy()[rows]
    mv = res.max_val.cpu().numpy()[rows]
    tol = clip_tolerance(X64, W32[rows], s, ref, X.dtype == torch.float32)
    bad = np.argwhere(np.abs(err - ref["err"]) > tol)
    assert bad.size == 0, f"{len(bad)} errors outside tolerance, first {bad[:4].tolist()}"
    # the chosen threshold: the oracle's, or one the bounds cannot separate from it
    diff = np.argwhere(best != ref["best"])
    for n, g in diff:
        bg, bo = best[n, g], ref["best"][n, g]
        gap = ref["err"][bg, n, g] - ref["err"][bo, n, g]
        assert gap <= tol[bg, n, g] + tol[bo, n, g], f"(n={n}, g={g}) gpu {bg} oracle {bo} gap {gap:.3e}"
    # the threshold of the chosen candidate, bit for bit
    chosen = np.take_along_axis(ref["thresholds"], best[None].astype(np.int64), axis=0)[0]
    assert np.array_equal(mv.view(np.uint32), chosen.view(np.uint32))
    return res, ref, len(diff)


@pytest.mark.parametrize("M,K,N,xd,wd", [
    (512, 512, 256, "bf16", "bf16"),   # one token tile, two row tiles, four groups
    (700, 384, 200, "bf16", "bf16"),   # two ragged token tiles, ragged rows, three groups
    (64, 256, 128, "f32", "f32"),      # fp32 X split into two bf16 terms
    (1, 128, 1, "bf16", "bf16"),       # one token, one group, one row
    (300, 1152, 130, "f32", "bf16"),   # nine groups: three blocks of four groups, the last short
    (200, 640, 70, "bf16", "f32"),
])
def test_clip_parity(awq, M, K, N, xd, wd):
    banner(f"clip M={M} K={K} N={N} {xd}/{wd}")
    _, X, _ = synth.custom_layer(M, K, N, dtype=xd, seed=11)
    _, _, W = synth.custom_layer(M, K, N, dtype=wd, seed=12)
    a32 = o.activation_stat(synth.to_f64(X)).astype(np.float32)
    tab, _ = o.scale_table_f32(a32)
    _, _, ndiff = check_clip(awq, X, W, tab[10])
    banner(f"clip M={M}: {ndiff} choices differ within tolerance")


def test_clip_full_size_sampled_tokens(awq):
    """The attention-projection layer with every 8th token (512 of 4096, a strided view), all
    4096 rows on the GPU, 48 rows against the oracle."""
    banner("clip attn 4096x4096, tokens ::8")
    spec, X, W = synth.make_layer("attn")
    a32 = o.activation_stat(synth.to_f64(X)).astype(np.float32)
    tab, _ = o.scale_table_f32(a32)
    rows = np.random.default_rng(0).choice(spec.N, 48, replace=False)
    Xd = X.to(DEV)[::8]  # row stride 8 K: no copy
    assert Xd.stride(0) == 8 * spec.K
    check_clip(awq, X[::8], W, tab[7], rows=np.sort(rows), Xd=Xd)


def test_clip_n_clip_sizes(awq):
    _, X, W = synth.custom_layer(256, 256, 64, seed=13)
    s = np.ones(256, np.float32)
    for n_clip in (1, 20):
        res, ref, _ = check_clip(awq, X, W, s, n_clip=n_clip)
        if n_clip == 1:
            assert np.all(res.best.cpu().numpy() == 0)


def test_pack_clipped_bit_exact(awq):
    banner("pack clipped")
    _, X, W = synth.custom_layer(256, 512, 300, dtype="bf16", seed=14)
    s = (np.random.default_rng(1).random(512) + 0.5).astype(np.float32)
    W32 = synth.to_f32(W)
    for i in (0, 3, 9):
        mv = o.clip_thresholds(W32, s)[i]
        qw, sc, zz = awq.pack(W.to(DEV), torch.from_numpy(s).to(DEV), max_val=torch.from_numpy(mv).to(DEV))
        art = o.pack_clipped(W32, s, mv)
        assert np.array_equal(qw.cpu().numpy(), art["qweight"])
        assert np.array_equal(sc.cpu().numpy(), art["scales"])
        assert np.array_equal(zz.cpu().numpy(), art["zeros"])


def test_clip_then_pack_end_to_end(awq):
    """awq_clip's thresholds fed to awq_pack_clipped give the oracle's clipped artefact."""
    _, X, W = synth.custom_layer(512, 384, 128, dtype="bf16", seed=15)
    s = np.ones(384, np.float32)
    Xd, Wd, sd = X.to(DEV), W.to(DEV), torch.from_numpy(s).to(DEV)
    res = awq.clip(Xd, Wd, sd)
    qw, sc, zz = awq.pack(Wd, sd, max_val=res.max_val)
    art = o.pack_clipped(synth.to_f32(W), s, res.max_val.cpu().numpy())
    assert np.array_equal(qw.cpu().numpy(), art["qweight"]) and np.array_equal(zz.cpu().numpy(), art["zeros"])
    plain = awq.pack(Wd, sd)[0]
    assert not torch.equal(qw, plain)  # some groups are clipped


def test_clip_is_deterministic(awq):
    _, X, W = synth.custom_layer(600, 256, 300, seed=16)
    s = torch.ones(256, device=DEV)
    r1 = awq.clip(X.to(DEV), W.to(DEV), s, return_err=True)
    r2 = awq.clip(X.to(DEV), W.to(DEV), s, return_err=True)
    assert torch.equal(r1.err, r2.err) and torch.equal(r1.max_val, r2.max_val)


def test_clip_flags(awq):
    _, X, W = synth.custom_layer(64, 256, 64, seed=17)
    Wn = W.clone()
    Wn[3, 7] = float("nan")
    with pytest.raises(ValueError, match="weights"):
        awq.clip(X.to(DEV), Wn.to(DEV), torch.ones(256, device=DEV))
    s = torch.ones(256, device=DEV)
    s[5] = 0.0
    with pytest.raises(ValueError, match="scales"):
        awq.clip(X.to(DEV), W.to(DEV), s)
    mv = torch.full((64, 2), -1.0, device=DEV)
    with pytest.raises(ValueError, match="thresholds"):
        awq.pack(W.to(DEV), torch.ones(256, device=DEV), max_val=mv)
