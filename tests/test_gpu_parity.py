"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded
inputs.  Bars: statistic rel <= 1e-6; scale table bitwise; per-candidate loss rel <= 1e-3
(bf16 matrix-core product vs fp64 oracle); chosen candidate identical unless the oracle's
losses of the two choices differ by less than 1e-3 relative; codes, zero points, fp16
scales and packed words bit-exact given the same scales."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import awq_oracle as o
from post_weight_quantization_mean_amd import synth
from tests.conftest import GOLDEN

pytestmark = pytest.mark.gpu

LOSS_RTOL = 1e-3
STAT_RTOL = 1e-6


@pytest.fixture(scope="module")
def awq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_mean_amd import awq as _awq
    _awq.lib()
    return _awq


DEV = "cuda:0"


def banner(msg):
    print(f"[gpu-case] {msg}", flush=True)


def check_choice(best_gpu, losses_oracle, best_oracle, tol=None, n_out=None):
    """The chosen candidate must be the oracle's unless the two are within 1e-3 relative in
    the oracle's own losses (several choices are then correct).  For layers with fewer than
    TINY_OUTPUTS outputs (n_out), whose per-candidate error bound ``tol`` is wider than 1e-3,
    any choice those bounds cannot separate is correct."""
    if n_out is not None and n_out >= TINY_OUTPUTS:
        tol = None
    if best_gpu == best_oracle:
        return
    gap = losses_oracle[best_gpu] - losses_oracle[best_oracle]
    rel = abs(gap) / losses_oracle[best_oracle]
    if rel < LOSS_RTOL:
        return
    assert tol is not None and gap <= tol[best_gpu] + tol[best_oracle], \
        f"gpu picked {best_gpu}, oracle {best_oracle}, gap {rel:.2e}"


# Below this many outputs (M N) no averaging hides the bf16 rounding of E, and the per-candidate
# tolerance is the bound derived below; from it on every candidate is held to 1e-3 relative.
# Measured on the small cases of this file: M N >= 6144 stay within 6.5e-4; the one-token,
# one-output cases (M N = 1) are at 3e-2.
TINY_OUTPUTS = 4096


def loss_tolerance(X64, W32, s_table, ref_losses, x_is_f32):
    """Per-candidate tolerance: 1e-3 relative (the rule for the search), except for layers with
    fewer than TINY_OUTPUTS outputs, which take max(1e-3 relative, a bound derived from the
    kernel's arithmetic).  Each output y = sum_k x_k e_k is formed from e rounded once to bf16
    (8 significand bits: |de| <= 2^-8 |e|), fp32 quantities rounded a few times (<= 2^-21 |w|),
    an fp32 split of fp32 X into two bf16 terms (<= 2^-16 |x|) and fp32 accumulation over K
    (<= K 2^-24).  So |dy| <= c_A sum|x||e| + c_B sum|x||w| and |d(y^2)| <= 2|y||dy| + dy^2."""
    M, K = X64.shape
    if M * W32.shape[0] >= TINY_OUTPUTS:
        return LOSS_RTOL * np.asarray(ref_losses)
    cA = 2.0 ** -8 + K * 2.0 ** -24 + (2.0 ** -16 if x_is_f32 else 0.0)
    cB = 2.0 ** -21
    absX = np.abs(X64)
    B = absX @ np.abs(W32.astype(np.float64)).T
    tol = np.empty(len(s_table))
    for i, s in enumerate(s_table):
        q, z, d = o.quantize(W32, s, 128)
        E = W32.astype(np.float64) - o.effective_weight(q, z, d, s, 128)
        Y = X64 @ E.T
        dy = cA * (absX @ np.abs(E).T) + cB * B
        bound = np.mean(2 * np.abs(Y) * dy + dy * dy) + 1e-5 * ref_losses[i]
        tol[i] = max(LOSS_RTOL * ref_losses[i], bound)
    return tol


def run_search_case(awq, X, W, n_grid=20):
    X64, W32 = synth.to_f64(X), synth.to_f32(W)
    a32 = o.activation_stat(X64).astype(np.float32)
    ref = o.search(X64, W32, a32, n_grid=n_grid)
    res = awq.search(X.to(DEV), W.to(DEV), torch.from_numpy(a32).to(DEV), n_grid=n_grid, return_table=True)
    L = res.losses.cpu().numpy()
    # scale table: same a in, bitwise same s out
    tab = res.s_table.cpu().numpy()
    mism = np.nonzero(tab.view(np.int32) != ref["s_table"].view(np.int32))
    assert mism[0].size == 0, f"scale table differs at {mism[0].size} entries, first {list(zip(*mism))[:4]}"
    tol = loss_tolerance(X64, W32, ref["s_table"], ref["losses"], X.dtype == torch.float32)
    err = np.abs(L - ref["losses"])
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"loss error {err[bad] / ref['losses'][bad]} (rel) above tolerance at {bad}"
    check_choice(res.best_index, ref["losses"], ref["best"], tol, n_out=X.shape[0] * W.shape[0])
    assert np.array_equal(res.s_best.cpu().numpy(), ref["s_table"][res.best_index])
    rel = err / ref["losses"]
    print(f"[gpu-case] max rel err {rel.max():.2e}, tolerance used {np.max(tol / ref['losses']):.2e} rel",
          flush=True)
    return res, ref, rel


# ------------------------------------------------------------------------------ statistic
@pytest.mark.parametrize("shape,dtype", [((64, 256), "f32"), ((1000, 640), "bf16"), ((3, 128), "f32"),
                                         ((1, 128), "bf16"), ((4096, 4096), "bf16"), ((700, 11008), "bf16"),
                                         ((1001, 1024), "bf16")])  # 15 interleaved splits, one-row tail
def test_stats_parity(awq, shape, dtype):
    M, K = shape
    banner(f"stats {shape} {dtype}")
    spec, X, _ = synth.custom_layer(M, K, 8, dtype=dtype, x_kind="sparse" if K == 11008 else "gauss")
    a = awq.stats(X.to(DEV)).cpu().numpy()
    ref = o.activation_stat(synth.to_f64(X))
    assert np.all(np.abs(a - ref) <= STAT_RTOL * ref)
    # fp64 accumulation is exact here, so the fp32 result is the correctly rounded mean
    assert np.mean(a == ref.astype(np.float32)) > 0.999


def test_stats_tiny_config_closed_form(awq):
    spec, X, _ = synth.make_layer("tiny")
    c = synth.channel_magnitudes(spec, synth._rng(0, 0, 0))
    assert np.array_equal(awq.stats(X.to(DEV)).cpu().numpy(), c)


# ------------------------------------------------------------------------------ search
def test_search_tiny_config(awq):
    banner("search tiny config")
    spec, X, W = synth.make_layer("tiny")
    res, ref, rel = run_search_case(awq, X, W)
    banner(f"tiny: best gpu {res.best_index} oracle {ref['best']} max rel {rel.max():.2e}")
    assert rel.max() <= LOSS_RTOL


@pytest.mark.parametrize("M,K,N,xd,wd", [
    (700, 384, 200, "bf16", "bf16"),   # two M tiles and two N tiles, both ragged; 3 groups
    (1, 128, 1, "f32", "f32"),
    (1, 128, 1, "bf16", "bf16"),       # degenerate: one token, one group, one output
    (513, 256, 129, "bf16", "bf16"),   # one row / one column past a tile
    (96, 256, 64, "f32", "f32"),
    (130, 384, 140, "bf16", "f32"),
    (200, 128, 130, "f32", "bf16"),
])
def test_search_ragged(awq, M, K, N, xd, wd):
    banner(f"search ragged M={M} K={K} N={N} {xd}/{wd}")
    _, X, _ = synth.custom_layer(M, K, N, dtype=xd, seed=1)
    _, _, W = synth.custom_layer(M, K, N, dtype=wd, seed=2)
    run_search_case(awq, X, W)


@pytest.mark.parametrize("n_grid", [1, 7, 64])
def test_search_grid_sizes(awq, n_grid):
    banner(f"search n_grid={n_grid}")
    _, X, W = synth.custom_layer(256, 256, 128, seed=3)
    res, ref, _ = run_search_case(awq, X, W, n_grid=n_grid)
    if n_grid == 1:
        assert res.best_index == 0


def test_search_is_deterministic(awq):
    _, X, W = synth.custom_layer(600, 256, 300, seed=4)
    Xd, Wd = X.to(DEV), W.to(DEV)
    a = awq.stats(Xd)
    r1 = awq.search(Xd, Wd, a)
    r2 = awq.search(Xd, Wd, a)
    assert torch.equal(r1.losses, r2.losses) and torch.equal(r1.s_best, r2.s_best)


def test_search_timed_matches_search(awq):
    """awq_search_timed returns exactly what awq_search returns, and its two events bracket a
    positive time no longer than the whole call."""
    banner("search_timed")
    _, X, W = synth.custom_layer(1024, 512, 384, seed=6)
    Xd, Wd = X.to(DEV), W.to(DEV)
    a = awq.stats(Xd)
    r1 = awq.search(Xd, Wd, a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    r2 = awq.search(Xd, Wd, a, fused_events=(ev[1], ev[2]))
    ev[3].record()
    torch.cuda.synchronize()
    assert torch.equal(r1.losses, r2.losses) and torch.equal(r1.best, r2.best)
    assert torch.equal(r1.s_best, r2.s_best)
    fused, whole = ev[1].elapsed_time(ev[2]), ev[0].elapsed_time(ev[3])
    assert 0.0 < fused <= whole


GOLDEN_LOSSES = os.path.join(GOLDEN, "oracle_losses.json")


def golden_keys():
    if not os.path.exists(GOLDEN_LOSSES):
        return []
    return sorted(json.load(open(GOLDEN_LOSSES)))


@pytest.mark.parametrize("key", golden_keys())
def test_search_full_size_vs_stored_oracle(awq, key):
    """Full-size layers in the benchmark's launch configuration against the oracle's losses,
    stored by tests/golden/make_oracle_losses.py (oracle + generator only)."""
    g = json.load(open(GOLDEN_LOSSES))[key]
    cfg, name = key.split("/")
    li = [l.name for l in synth.CONFIGS[cfg].layers].index(name)
    banner(f"full-size search {key} M={g['M']} K={g['K']} N={g['N']}")
    spec, X, W = synth.make_layer(cfg, li)
    a32 = o.activation_stat(synth.to_f64(X)).astype(np.float32)
    import hashlib
    assert hashlib.sha256(a32.tobytes()).hexdigest()[:16] == g["a_sha"], "generator drift"
    Xd, Wd = X.to(DEV), W.to(DEV)
    del X
    res = awq.search(Xd, Wd, torch.from_numpy(a32).to(DEV))
    L = res.losses.cpu().numpy()
    ref = np.array(g["losses"])
    rel = np.abs(L - ref) / ref
    banner(f"{key}: best gpu {res.best_index} oracle {g['best']} max rel {rel.max():.2e}")
    assert rel.max() <= LOSS_RTOL
    check_choice(res.best_index, ref, g["best"])
    # the statistic on the same input
    a_gpu = awq.stats(Xd).cpu().numpy()
    assert np.all(np.abs(a_gpu - a32) <= STAT_RTOL * a32)
    # sampled rows of the packed artefact, bit-exact against the oracle at the oracle's winner
    s_best = o.scale_table_f32(a32)[0][g["best"]]
    rows = np.random.default_rng(0).choice(spec.N, 48, replace=False)
    qw, sc, zz = awq.pack(Wd, torch.from_numpy(s_best).to(DEV))
    art = o.pack(synth.to_f32(W)[rows], s_best)
    assert np.array_equal(qw.cpu().numpy()[rows], art["qweight"])
    assert np.array_equal(sc.cpu().numpy()[rows], art["scales"])
    assert np.array_equal(zz.cpu().numpy()[rows], art["zeros"])


# ------------------------------------------------------------------------------ pack
@pytest.mark.parametrize("N,K,wd", [(128, 256, "f32"), (300, 384, "bf16"), (1, 128, "bf16"), (77, 640, "f32")])
def test_pack_bit_exact(awq, N, K, wd):
    banner(f"pack N={N} K={K} {wd}")
    _, X, W = synth.custom_layer(64, K, N, dtype=wd, seed=5)
    a32 = o.activation_stat(synth.to_f64(X)).astype(np.float32)
    tab, _ = o.scale_table_f32(a32)
    Wd = W.to(DEV)
    W32 = synth.to_f32(W)
    for i in (0, 5, 13, 19):
        qw, sc, zz = awq.pack(Wd, torch.from_numpy(tab[i]).to(DEV))
        art = o.pack(W32, tab[i])
        assert np.array_equal(qw.cpu().numpy(), art["qweight"]), f"qweight differs at candidate {i}"
        assert np.array_equal(sc.cpu().numpy(), art["scales"])
        assert np.array_equal(zz.cpu().numpy(), art["zeros"])


def test_pack_bf16_many_rows_strided(awq):
    """bf16 W with more rows than one sweep of the pack grid covers (several iterations, a
    partial last one) and a row stride larger than K: every code, scale and zero point of all
    2500 rows against the oracle."""
    banner("pack bf16 N=2500 K=4096 ldw=4160")
    g = torch.Generator().manual_seed(21)
    full = (torch.randn(2500, 4160, generator=g) / 64).to(torch.bfloat16)
    W = full[:, :4096]  # ldw = 4160
    s = (torch.rand(4096, generator=g) + 0.5).to(torch.float32)
    qw, sc, zz = awq.pack(full.to(DEV)[:, :4096], s.to(DEV))
    art = o.pack(synth.to_f32(W.contiguous()), s.numpy())
    assert np.array_equal(qw.cpu().numpy(), art["qweight"])
    assert np.array_equal(sc.cpu().numpy(), art["scales"])
    assert np.array_equal(zz.cpu().numpy(), art["zeros"])


def test_pack_bf16_row_slabs(awq):
    """A bf16 W of more than 2^30 bytes (131073 rows of 4096): the pack runs in row slabs of
    2^30 bytes (32-bit offsets inside each), here one full slab and a one-row slab.  Rows on
    both sides of the slab boundary, the first and the last, bit-exact against the oracle
    (the pack is row-independent)."""
    banner("pack bf16 row slabs N=131073 K=4096")
    N, K = 131073, 4096
    g = torch.Generator(device=DEV).manual_seed(22)
    Wd = (torch.randn((N, K), generator=g, device=DEV) / 64).to(torch.bfloat16)
    s = (torch.rand(K, generator=torch.Generator().manual_seed(23)) + 0.5).to(torch.float32)
    qw, sc, zz = awq.pack(Wd, s.to(DEV))
    rows = [0, 1, 65536, 131070, 131071, 131072]
    Ws = synth.to_f32(Wd[rows].cpu())
    art = o.pack(Ws, s.numpy())
    assert np.array_equal(qw[rows].cpu().numpy(), art["qweight"])
    assert np.array_equal(sc[rows].cpu().numpy(), art["scales"])
    assert np.array_equal(zz[rows].cpu().numpy(), art["zeros"])
    del Wd, qw, sc, zz
    torch.cuda.empty_cache()


def test_pack_hand_vectors(awq):
    # groups built from the oracle's hand-derived fp32 vectors, padded to 128 with copies of
    # their own values (min, max and so Delta, z unchanged)
    rows = []
    for v in ([-1.0, 0.5, 0.25, 1.0], [-11.5, 3.5], [0.1, 1.0], [-0.7, -0.2], [0.0, 0.0]):
        rows.append(np.resize(np.array(v, np.float32), 128))
    W = np.stack(rows).astype(np.float32)
    s = np.ones(128, np.float32)
    qw, sc, zz = awq.pack(torch.from_numpy(W).to(DEV), torch.from_numpy(s).to(DEV))
    art = o.pack(W, s)
    assert np.array_equal(qw.cpu().numpy(), art["qweight"])
    assert zz.cpu().numpy()[:, 0].tolist() == [7, 12, 0, 15, 0]
    assert np.array_equal(sc.cpu().numpy(), art["scales"])


def test_pack_near_tie_quotients(awq):
    """Values whose quotient v / Delta lies within a few ulps of a half-integer: the codes
    depend on the correctly rounded fp32 quotient, which the kernel forms from a reciprocal and
    FMA corrections; they must equal the oracle's, which divides exactly."""
    rng = np.random.default_rng(11)
    rows = []
    for _ in range(256):
        lo, hi = np.float32(-rng.uniform(0.1, 4.0)), np.float32(rng.uniform(0.1, 4.0))
        delta = np.float32(np.float32(hi - lo) / np.float32(15.0))
        v = [lo, hi]
        for _ in range(126):
            k = rng.integers(-15, 15)
            x = np.float32((k + 0.5) * float(delta))
            for _ in range(int(rng.integers(-4, 5))):
                x = np.nextafter(x, np.float32(np.inf) if rng.random() < 0.5 else np.float32(-np.inf))
            v.append(np.float32(np.clip(x, lo, hi)))
        rows.append(np.array(v, np.float32))
    W = np.stack(rows)
    W = np.concatenate([W, W[:, ::-1]], axis=1).astype(np.float32)  # K = 256, two groups
    s = np.ones(256, np.float32)
    qw, sc, zz = awq.pack(torch.from_numpy(W).to(DEV), torch.from_numpy(s).to(DEV))
    art = o.pack(W, s)
    assert np.array_equal(qw.cpu().numpy(), art["qweight"])
    assert np.array_equal(zz.cpu().numpy(), art["zeros"])
    assert np.array_equal(sc.cpu().numpy(), art["scales"])


# ------------------------------------------------------------------------------ data errors
def test_pack_bf16_group_categories(awq):
    """bf16 groups of every kind the quantizer distinguishes, with random per-channel scales:
    ranges containing 0 (z from the rounding alone), groups of one sign far from 0 (z clamped to
    0 or 15, codes clamped), groups that touch 0 (min or max exactly 0), constant groups (the
    1e-5 range floor) and narrow ones; codes, scales and zeros bit-exact against the oracle."""
    rng = np.random.default_rng(12)
    N, K = 512, 512
    W = np.empty((N, K), np.float32)
    kinds = ("mixed", "positive", "negative", "touch_lo", "touch_hi", "constant", "narrow")
    for n in range(N):
        for g in range(K // 128):
            kind = kinds[rng.integers(len(kinds))]
            sl = slice(128 * g, 128 * g + 128)
            if kind == "mixed":
                W[n, sl] = rng.uniform(-rng.uniform(0.01, 2), rng.uniform(0.01, 2), 128)
            elif kind == "positive":
                lo = rng.uniform(0.05, 1.0)
                W[n, sl] = rng.uniform(lo, lo * rng.uniform(1.01, 8.0), 128)
            elif kind == "negative":
                hi = -rng.uniform(0.05, 1.0)
                W[n, sl] = rng.uniform(hi * rng.uniform(1.01, 8.0), hi, 128)
            elif kind == "touch_lo":
                W[n, sl] = rng.uniform(0, 1, 128)
                W[n, 128 * g + rng.integers(128)] = 0.0
            elif kind == "touch_hi":
                W[n, sl] = rng.uniform(-1, 0, 128)
                W[n, 128 * g + rng.integers(128)] = 0.0
            elif kind == "constant":
                W[n, sl] = rng.uniform(-1, 1)
            else:
                c = rng.uniform(-1, 1)
                W[n, sl] = c + rng.uniform(-1e-3, 1e-3, 128)
    Wb = torch.from_numpy(W).to(torch.bfloat16)
    s = np.exp(0.5 * rng.standard_normal(K)).astype(np.float32)
    qw, sc, zz = awq.pack(Wb.to(DEV), torch.from_numpy(s).to(DEV))
    art = o.pack(synth.to_f32(Wb), s)
    assert np.array_equal(qw.cpu().numpy(), art["qweight"])
    assert np.array_equal(zz.cpu().numpy(), art["zeros"])
    assert np.array_equal(sc.cpu().numpy(), art["scales"])
    zeros = art["zeros"].astype(np.float32)
    assert np.any(zeros == 0) and np.any(zeros == 15) and np.any((zeros > 0) & (zeros < 15))


def test_strided_inputs_match_contiguous(awq):
    """Row strides larger than K (X: K + 64, W: K + 128): stats, the direct search and the Gram
    search read rows by their stride and give the same bits as on contiguous copies."""
    banner("stats / search / gram on strided views")
    M, K, N = 1500, 512, 300
    _, X, W = synth.custom_layer(M, K, N, dtype="bf16", seed=24)
    Xbig = torch.zeros((M, K + 64), dtype=X.dtype)
    Xbig[:, :K] = X
    Wbig = torch.zeros((N, K + 128), dtype=W.dtype)
    Wbig[:, :K] = W
    Xv, Wv = Xbig.to(DEV)[:, :K], Wbig.to(DEV)[:, :K]
    Xc, Wc = X.to(DEV), W.to(DEV)
    assert Xv.stride(0) == K + 64 and Wv.stride(0) == K + 128
    a_v, a_c = awq.stats(Xv), awq.stats(Xc)
    assert torch.equal(a_v, a_c)
    for gram in (False, True):
        r_v = awq.search(Xv, Wv, a_c, gram=gram)
        r_c = awq.search(Xc, Wc, a_c, gram=gram)
        assert torch.equal(r_v.losses, r_c.losses) and r_v.best_index == r_c.best_index, gram
        assert torch.equal(r_v.s_best, r_c.s_best)


def test_flags_nonfinite(awq):
    _, X, W = synth.custom_layer(64, 256, 64, seed=6)
    Xn = X.clone()
    Xn[3, 17] = float("nan")
    with pytest.raises(ValueError, match="activations"):
        awq.stats(Xn.to(DEV))
    Xi = X.clone()
    Xi[0, 0] = float("inf")
    with pytest.raises(ValueError, match="activations"):
        awq.stats(Xi.to(DEV))
    a = awq.stats(X.to(DEV))
    Wn = W.clone()
    Wn[5, 100] = float("nan")
    with pytest.raises(ValueError, match="loss"):
        awq.search(X.to(DEV), Wn.to(DEV), a)
    with pytest.raises(ValueError, match="weights"):
        awq.pack(Wn.to(DEV), torch.ones(256, device=DEV))


def test_flags_scale_and_f16_range(awq):
    _, X, W = synth.custom_layer(64, 256, 64, seed=7)
    s = torch.ones(256, device=DEV)
    s[9] = 0.0
    with pytest.raises(ValueError, match="scale"):
        awq.pack(W.to(DEV), s)
    a = awq.stats(X.to(DEV))
    a[3] = -1.0
    with pytest.raises(ValueError, match="scale"):
        awq.search(X.to(DEV), W.to(DEV), a)
    Wbig = torch.full((2, 128), 2.0e6)
    Wbig[:, 0] = -2.0e6
    with pytest.raises(ValueError, match="fp16"):
        awq.pack(Wbig.to(DEV), torch.ones(128, device=DEV))


def test_no_silent_fallback(awq):
    # the binding is the C library: no CPU path exists behind it
    import post_weight_quantization_mean_amd.awq as mod
    assert mod._lib is not None and os.path.basename(mod._LIB_PATH) == "libawq.so"
