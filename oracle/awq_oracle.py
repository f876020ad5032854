"""Plain, slow CPU oracle for the AWQ activation-aware INT4 scale search and packing.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module: only the
tests, the smoke check and the CPU-baseline leg of the benchmark call it.  It shares no
code, constants table or helper with the HIP library; the only thing the two sides share
is the seeded input generator, which holds none of the method's arithmetic.

Sources (cited by page title and section):

* [EXPLAINER] "AWQ：为什么 4-bit 权重量化要先观察 Activation" (charlestar.github.io):
  §1 (error measured through the input, the per-channel statistic a_j),
  §2 (the symmetric [-7, 7] teaching quantizer), §3 (equivalent scaling XW = (XS^-1)(SW),
  the worked two-channel examples and the 20-candidate search, the per-element error bound),
  §4 (the candidate family s = a^alpha, alpha in {0, 0.05, ..., 0.95}, clamp 1e-4 before the
  sqrt(max*min) normalisation, the per-candidate module-output MSE, first minimum wins),
  §7 (the asymmetric group pseudo-quantizer actually used for the artefact: round w/Delta,
  add z, clamp to [0, 15], reconstruct Delta(q - z); group size divides K; K-axis grouping
  of a PyTorch [N, K] weight), §8 (g128 + fp16 scale + fp16 zero = 4.25 bits/weight),
  §5 (the clipping search that follows the scale search: ten thresholds 1, 0.95, ..., 0.55
  of each group's absmax, chosen per output channel and input group by the squared error of
  the group's partial output on the calibration tokens; the symmetric counterexample),
  §6 (where S^-1 goes: a LayerNorm's gamma and beta, an RMSNorm's gamma, a preceding Linear's
  output rows and bias, or act(x) / s after a non-linearity, never through it; every
  consuming projection's input columns take s); §7 and §8 for using the artefact: decode
  scales * (q - zeros) and multiply with 16-bit activations that carry S^-1 (W4A16).
* [DREAMVFIA] "AWQ salient weight / GGUF compilation" report (dreamvfia.cn), §二: the
  statistic (1/B) sum_b |X_bk| and the scale-equivalence algebra.
* [MODULES] "5. 核心模块：校准器、压缩算法、格式封装与 kernel 后端" (ai-infra.cypggs.com), §5.3:
  INT4 codes are usually packed eight per int32.

Readings where the pages are silent (each is listed in the design doc):

* The asymmetric formulas themselves were lost from the explainer's §7; the text gives the
  order of operations and says a positive floor prevents division by zero.  This oracle uses
  Delta = max(max - min, 1e-5) / 15, z = clamp(rne(-min / Delta), 0, 15),
  q = clamp(rne(v / Delta) + z, 0, 15).  The 1e-5 floor is our choice.
* Working precision of the quantizer: IEEE fp32, each operation rounded once (numpy float32
  has no fused multiply-add), correctly rounded division, ties-to-even rounding.  The
  scale table is computed in fp64 and rounded once to fp32.  The loss is fp64.
* The loss of a candidate is the mean over the M x N outputs of (X E)^2 with
  E = W - S^-1 Q(S W): the module-output MSE of §4 for a single linear layer.  Its Gram form
  sum_n E[n] (X^T X) E[n]^T / (M N) (§1: the exact error carries the cross terms of X^T X) is
  the same number in exact arithmetic.
* Clipping: the threshold of candidate i is fp32(absmax * fp32(1 - i/20)) of the scaled
  weight v = fp32(W s); the clipped group clamp(v, -c, c) goes through the same asymmetric
  quantizer; the error of (n, g) is the mean over the given tokens of
  (sum_{k in g} X[m,k] e[n,k])^2 with e = W - S^-1 Q(clamp(S W)), in float64; the first
  minimum wins.  Which tokens are sampled is the caller's choice.
* Folding: every folded or scaled parameter is the exact quotient or product rounded once
  to its storage type (fp32, or bf16 with ties to even).
* Packing: qweight int32 [N, K/8], nibble i of word j holds the code of k = 8j + i (least
  significant nibble first); scales fp16 [N, K/g] hold Delta (round-to-nearest-even);
  zeros fp16 [N, K/g] hold the integer z.

Every function here is pinned by tests (worked examples printed on the pages, closed forms,
invariants, brute force on tiny inputs).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

from math import fsum, isfinite, sqrt
from typing import Dict, List, Sequence, Tuple

import numpy as np

N_GRID = 20          # [EXPLAINER §4] twenty ratios 0, 0.05, ..., 0.95 (1 excluded)
SCALE_FLOOR = 1e-4   # [EXPLAINER §4] clamp applied after the power, before normalising
RANGE_FLOOR = np.float32(1e-5)  # positive floor on max - min (our reading of §7)
QMAX = 15            # [EXPLAINER §7] unsigned 4-bit codes 0..15
GROUP = 128          # [EXPLAINER §8], quant config group 128 (g128)


# ---------------------------------------------------------------------------------------
# Step 1: the activation statistic  [EXPLAINER §1], [DREAMVFIA §二]
# ---------------------------------------------------------------------------------------
def activation_stat(X: np.ndarray) -> np.ndarray:
    """a_j = mean over the M calibration rows of |X[m, j]|, in float64.

    X holds the exact input values (fp32 or bf16 values embed exactly in float64)."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2 or X.shape[0] == 0:
        raise ValueError("X must be a non-empty [M, K] matrix")
    if not np.all(np.isfinite(X)):
        raise ValueError("activations must be finite")
    return np.abs(X).sum(axis=0) / X.shape[0]


# ---------------------------------------------------------------------------------------
# Step 2: the scale candidates  [EXPLAINER §3 listing and §4]
# ---------------------------------------------------------------------------------------
def alpha_grid(n_grid: int = N_GRID) -> List[float]:
    """alpha_i = i / n_grid for i = 0 .. n_grid-1 (the value 1 itself is not a candidate)."""
    return [i / n_grid for i in range(n_grid)]


def candidate_scales(a: Sequence[float], alpha: float) -> np.ndarray:
    """s = r / sqrt(max(r) * min(r)) with r_j = max(a_j ** alpha, 1e-4), in float64.

    The clamp comes before the normalisation, so a final s_j may be below 1e-4; at
    alpha = 0 every r_j is 1 (0 ** 0 = 1) and s is all ones."""
    a = np.asarray(a, dtype=np.float64)
    if a.ndim != 1 or a.size == 0 or not np.all(np.isfinite(a)) or np.any(a < 0):
        raise ValueError("the statistic must be a finite non-negative vector")
    r = np.maximum(np.power(a, alpha), SCALE_FLOOR)
    return r / sqrt(float(r.max()) * float(r.min()))


def scale_table_f32(a32: np.ndarray, n_grid: int = N_GRID) -> Tuple[np.ndarray, np.ndarray]:
    """The fp32 table used by the production contract: s[i] = fp32(candidate_scales(a, i/n))
    and its reciprocal rs[i] = fp32(1 / s[i]) (both rounded once from float64)."""
    a64 = np.asarray(a32, dtype=np.float32).astype(np.float64)
    s = np.stack([candidate_scales(a64, al).astype(np.float32) for al in alpha_grid(n_grid)])
    if not np.all(np.isfinite(s)) or np.any(s <= 0):
        raise ValueError("a scale candidate is outside fp32 range")
    rs = (1.0 / s.astype(np.float64)).astype(np.float32)
    return s, rs


def first_argmin(losses: Sequence[float]) -> int:
    """Index of the first minimum (the earliest, i.e. smallest-alpha, candidate wins ties)."""
    best = 0
    for i, v in enumerate(losses):
        if v < losses[best]:
            best = i
    return best


# ---------------------------------------------------------------------------------------
# Step 3: group-wise asymmetric INT4 pseudo-quantization  [EXPLAINER §7]
# ---------------------------------------------------------------------------------------
def asym_params(v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per group (last axis) of fp32 values: Delta (fp32) and the integer zero point z."""
    v = np.asarray(v, dtype=np.float32)
    mx = v.max(axis=-1)
    mn = v.min(axis=-1)
    delta = np.maximum(mx - mn, RANGE_FLOOR) / np.float32(QMAX)
    if not np.all(np.isfinite(delta)):
        raise ValueError("group range outside fp32 range")
    z = np.clip(np.rint(-mn / delta), 0, QMAX)
    return delta.astype(np.float32), z.astype(np.int32)


def asym_codes(v: np.ndarray, delta: np.ndarray, z: np.ndarray) -> np.ndarray:
    """q = clamp(rne(v / Delta) + z, 0, 15) with Delta, z broadcast over the group axis."""
    v = np.asarray(v, dtype=np.float32)
    t = v / delta[..., None]
    q = np.clip(np.rint(t) + z[..., None].astype(np.float32), 0, QMAX)
    return q.astype(np.uint8)


def quantize(W32: np.ndarray, s32: np.ndarray, group: int = GROUP
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantize S W for a [N, K] weight whose rows are output channels.

    v[n, k] = fp32(W[n, k] * s[k]); groups of ``group`` consecutive k per row n.
    Returns codes uint8 [N, K], zero points int32 [N, K/g], steps fp32 [N, K/g]."""
    W32 = np.asarray(W32, dtype=np.float32)
    s32 = np.asarray(s32, dtype=np.float32)
    N, K = W32.shape
    if group <= 0 or K % group != 0:
        raise ValueError("the group size must divide K")
    if not np.all(np.isfinite(W32)):
        raise ValueError("weights must be finite")
    if s32.shape != (K,) or not np.all(np.isfinite(s32)) or np.any(s32 <= 0):
        raise ValueError("scales must be finite and positive")
    v = (W32 * s32[None, :]).reshape(N, K // group, group)
    if not np.all(np.isfinite(v)):
        raise ValueError("scaled weight outside fp32 range")
    delta, z = asym_params(v)
    q = asym_codes(v, delta, z)
    return q.reshape(N, K), z, delta


def dequant_scaled(q: np.ndarray, z: np.ndarray, delta: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Reconstruction in the scaled domain, Delta (q - z), in float64 [N, K]."""
    N, K = q.shape
    qg = q.reshape(N, K // group, group).astype(np.float64)
    out = delta.astype(np.float64)[..., None] * (qg - z.astype(np.float64)[..., None])
    return out.reshape(N, K)


def effective_weight(q, z, delta, s32, group: int = GROUP) -> np.ndarray:
    """S^-1 Q(S W): the weight the candidate actually applies to the unchanged X (float64)."""
    return dequant_scaled(q, z, delta, group) / np.asarray(s32, dtype=np.float64)[None, :]


# ---------------------------------------------------------------------------------------
# Step 4: candidate loss  [EXPLAINER §1, §3, §4]
# ---------------------------------------------------------------------------------------
def candidate_loss(X64: np.ndarray, W64: np.ndarray, What64: np.ndarray, chunk: int = 4096) -> float:
    """mean over the M x N outputs of (X E^T)^2 with E = W - What, all in float64.

    W and What are [N, K]; the output Y = X W^T is [M, N].  Chunked over N only to bound
    memory; the sum of squares is accumulated in float64."""
    M = X64.shape[0]
    N = W64.shape[0]
    sse = 0.0
    for n0 in range(0, N, chunk):
        E = W64[n0:n0 + chunk] - What64[n0:n0 + chunk]
        Y = X64 @ E.T
        sse += float(np.einsum("ij,ij->", Y, Y))
    return sse / (M * N)


def search(X: np.ndarray, W: np.ndarray, a32: np.ndarray, group: int = GROUP, n_grid: int = N_GRID,
           chunk: int = 4096) -> Dict[str, object]:
    """The full candidate search of [EXPLAINER §4] for one linear layer.

    X: exact activations [M, K]; W: exact weights [N, K] (fp32-representable);
    a32: the fp32 statistic fed to the scale table.  Every candidate is evaluated exactly
    (fp64 loss) and the first minimum wins."""
    X64 = np.asarray(X, dtype=np.float64)
    W32 = np.asarray(W, dtype=np.float32)
    if not np.array_equal(W32.astype(np.float64), np.asarray(W, dtype=np.float64)):
        raise ValueError("weights must be fp32-representable")
    if not np.all(np.isfinite(X64)):
        raise ValueError("activations must be finite")
    N, K = W32.shape
    if X64.shape[1] != K:
        raise ValueError("X and W disagree on K")
    W64 = W32.astype(np.float64)
    s_tab, rs_tab = scale_table_f32(a32, n_grid)
    losses = np.zeros(n_grid, dtype=np.float64)
    for i in range(n_grid):
        sse = 0.0
        for n0 in range(0, N, chunk):
            q, z, d = quantize(W32[n0:n0 + chunk], s_tab[i], group)
            What = effective_weight(q, z, d, s_tab[i], group)
            E = W64[n0:n0 + chunk] - What
            Y = X64 @ E.T
            sse += float(np.einsum("ij,ij->", Y, Y))
        losses[i] = sse / (X64.shape[0] * N)
    best = first_argmin(list(losses))
    return {"losses": losses, "best": best, "s_table": s_tab, "rs_table": rs_tab,
            "s_best": s_tab[best].copy(), "alpha_best": alpha_grid(n_grid)[best]}


def gram_matrix(X: np.ndarray) -> np.ndarray:
    """G = X^T X [K x K] in float64 ([EXPLAINER §1]: the cross terms of the inputs that the
    exact layer-output squared error depends on, beyond the per-channel statistic)."""
    X64 = np.asarray(X, dtype=np.float64)
    return X64.T @ X64


def gram_loss(G: np.ndarray, M: int, E: np.ndarray) -> float:
    """mean over the M x N outputs of (X E^T)^2 written through G = X^T X:
    sum_n E[n,:] G E[n,:]^T / (M N), all in float64 (E [N, K])."""
    E64 = np.asarray(E, dtype=np.float64)
    return float(np.einsum("nk,nk->", E64 @ G, E64)) / (M * E64.shape[0])


def gram_search_losses(X: np.ndarray, W: np.ndarray, s_table: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Every candidate's loss (the scale table s_table [n_grid, K]) in the Gram form: the same
    quantities as ``search``'s losses, evaluated through G = X^T X formed once."""
    X64 = np.asarray(X, dtype=np.float64)
    W32 = np.asarray(W, dtype=np.float32)
    G = gram_matrix(X64)
    out = np.empty(len(s_table))
    for i, s in enumerate(s_table):
        q, z, d = quantize(W32, s, group)
        out[i] = gram_loss(G, X64.shape[0], W32.astype(np.float64) - effective_weight(q, z, d, s, group))
    return out


def search_tiles(X: np.ndarray, W: np.ndarray, s32: np.ndarray, rows: Tuple[int, int],
                 cols: Tuple[int, int], group: int = GROUP) -> float:
    """Sum of squared output errors over the output block rows x cols for one candidate s
    (a sampled piece of the loss, for checks at sizes where the full search is slow)."""
    m0, m1 = rows
    n0, n1 = cols
    q, z, d = quantize(np.asarray(W, dtype=np.float32)[n0:n1], s32, group)
    E = np.asarray(W, dtype=np.float64)[n0:n1] - effective_weight(q, z, d, s32, group)
    Y = np.asarray(X, dtype=np.float64)[m0:m1] @ E.T
    return float(np.einsum("ij,ij->", Y, Y))


# ---------------------------------------------------------------------------------------
# Step 5: packing the winning codes  [EXPLAINER §7, §8], [MODULES §5.3]
# ---------------------------------------------------------------------------------------
def pack_words(q: np.ndarray) -> np.ndarray:
    """Eight 4-bit codes per int32: nibble i of word j <- code of k = 8j + i."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    if K % 8 != 0:
        raise ValueError("K must be a multiple of 8")
    if np.any(q > QMAX):
        raise ValueError("codes must be 4-bit")
    q8 = q.reshape(N, K // 8, 8)
    word = np.zeros((N, K // 8), dtype=np.uint32)
    for i in range(8):
        word |= q8[:, :, i] << np.uint32(4 * i)
    return word.view(np.int32)


def unpack_words(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words, dtype=np.int32).view(np.uint32)
    N, J = w.shape
    out = np.zeros((N, J, 8), dtype=np.uint8)
    for i in range(8):
        out[:, :, i] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(N, J * 8)


def pack(W: np.ndarray, s32: np.ndarray, group: int = GROUP) -> Dict[str, np.ndarray]:
    """The artefact for one layer: qweight int32 [N, K/8], scales fp16 [N, K/g] (Delta,
    round-to-nearest-even), zeros fp16 [N, K/g] (integer z), plus the codes themselves."""
    q, z, d = quantize(W, s32, group)
    scales = d.astype(np.float16)
    if not np.all(np.isfinite(scales)):
        raise ValueError("a group step overflows fp16")
    return {"qweight": pack_words(q), "scales": scales, "zeros": z.astype(np.float16),
            "codes": q, "z": z, "delta": d}


def artefact_bits_per_weight(N: int, K: int, group: int = GROUP) -> float:
    """Storage of the artefact per weight: 4-bit codes + one fp16 scale and one fp16 zero per
    group ([EXPLAINER §8]; padding and unquantized modules are not counted)."""
    payload_bits = N * K * 4 + (N * K // group) * (16 + 16)
    return payload_bits / (N * K)


# ---------------------------------------------------------------------------------------
# Teaching mode: the symmetric [-7, 7] quantizer and scaled forward  [EXPLAINER §2, §3]
# Written from the definitions (vectorised, float64); it exists only to reproduce the numbers
# the page prints for its two-channel example.
# ---------------------------------------------------------------------------------------
TEACH_QMAX = 7  # [EXPLAINER §2] symmetric codes -7 .. 7


def _finite_vector(values, what: str) -> np.ndarray:
    v = np.asarray(values, dtype=np.float64).reshape(-1)
    if v.size == 0 or not np.all(np.isfinite(v)):
        raise ValueError(f"{what} needs finite values")
    return v


def teaching_qdq(values: Sequence[float]) -> Tuple[List[int], List[float], float]:
    """The symmetric absmax quantizer of [EXPLAINER §2] on one group: step = max|v| / 7 (the
    page uses step 1 for an all-zero group), code = v / step rounded to the nearest integer
    with ties to even and limited to [-7, 7], reconstruction = step * code.
    Returns (codes, reconstruction, step)."""
    v = _finite_vector(values, "a group")
    peak = float(np.max(np.abs(v)))
    step = peak / TEACH_QMAX if peak > 0.0 else 1.0
    if not 0.0 < step < np.inf:
        raise ValueError("the step is outside the float range")
    codes = np.clip(np.rint(v / step), -TEACH_QMAX, TEACH_QMAX)
    return [int(c) for c in codes], [float(r) for r in codes * step], step


def _kept_in_range(original: np.ndarray, scaled: np.ndarray) -> bool:
    """A scaled copy is usable when every value stays finite and no non-zero value vanishes."""
    return bool(np.all(np.isfinite(scaled)) and not np.any((original != 0) & (scaled == 0)))


def teaching_forward(x: Sequence[float], w: Sequence[float], scales: Sequence[float]
                     ) -> Tuple[float, List[int], float]:
    """One output of the scaled layer of [EXPLAINER §3], all channels in one teaching group:
    y = sum_j (x_j / s_j) * Q(w_j * s_j), the sum rounded once (math.fsum of the products).
    Without quantization this is x.w exactly (XW = (XS^-1)(SW)).  Rejects mismatched or empty
    vectors, non-finite values, non-positive scales, and scalings that overflow or flush a
    value to zero.  Returns (y, codes, step)."""
    xv = np.asarray(x, dtype=np.float64).reshape(-1)
    wv = np.asarray(w, dtype=np.float64).reshape(-1)
    sv = np.asarray(scales, dtype=np.float64).reshape(-1)
    if xv.size == 0 or xv.shape != wv.shape or xv.shape != sv.shape:
        raise ValueError("x, w and the scales need the same non-zero length")
    if not (np.all(np.isfinite(xv)) and np.all(np.isfinite(wv))):
        raise ValueError("inputs must be finite")
    if not np.all(np.isfinite(sv) & (sv > 0)):
        raise ValueError("scales must be finite and positive")
    xs, ws = xv / sv, wv * sv
    if not (_kept_in_range(xv, xs) and _kept_in_range(wv, ws)):
        raise ValueError("the scaling left the float range")
    codes, restored, step = teaching_qdq(ws)
    y = fsum(xs * np.asarray(restored))
    if not isfinite(y):
        raise ValueError("the output is not finite")
    return y, codes, step


def teaching_search(x: Sequence[float], w: Sequence[float], n_grid: int = N_GRID) -> Dict[str, object]:
    """The candidate search of [EXPLAINER §3, §4] on a single token with the teaching quantizer:
    the statistic of one calibration row is |x|, candidate i uses candidate_scales(|x|, i/n),
    and its loss is (y_i - x.w)^2.  Returns the arrays alpha, y and loss over the candidates and
    ``best``, the first index of the least loss."""
    xv = _finite_vector(x, "x")
    wv = _finite_vector(w, "w")
    target = fsum(xv * wv)
    alphas = alpha_grid(n_grid)
    ys = np.array([teaching_forward(xv, wv, candidate_scales(np.abs(xv), al))[0] for al in alphas])
    losses = (ys - target) ** 2
    return {"alpha": np.array(alphas), "y": ys, "loss": losses, "best": first_argmin(list(losses)),
            "target": target}


# ---------------------------------------------------------------------------------------
# After the scale search: clipping search  [EXPLAINER §5]
# ---------------------------------------------------------------------------------------
CLIP_CANDIDATES = 10  # [EXPLAINER §5] thresholds 1, 0.95, ..., 0.55 of the group absmax


def clip_factors(n_clip: int = CLIP_CANDIDATES) -> np.ndarray:
    """Shrink factors f_i = 1 - i/20 for i < n_clip (the value 0.5 itself is not tried), as the
    fp32 numbers the thresholds are multiplied with."""
    if not 1 <= n_clip <= 20:
        raise ValueError("between 1 and 20 clipping candidates")
    return np.array([1.0 - i / 20.0 for i in range(n_clip)], dtype=np.float32)


def teaching_clip_qdq(values: Sequence[float], factor: float) -> List[float]:
    """The teaching quantizer of [EXPLAINER §5] with a clipping threshold: t = factor * max|v|,
    step = t / 7, each value clamped to [-t, t] and then reconstructed as step times its code
    (nearest, ties to even, limited to [-7, 7]).  An all-zero group stays zero.  Finite values
    and 0 < factor <= 1 only.  Returns the reconstruction."""
    v = _finite_vector(values, "a group")
    if not (isfinite(factor) and 0.0 < factor <= 1.0):
        raise ValueError("the clipping factor must lie in (0, 1]")
    peak = float(np.max(np.abs(v)))
    if peak == 0.0:
        return [0.0] * v.size
    thr = peak * factor
    step = thr / TEACH_QMAX
    if not 0.0 < step < np.inf:
        raise ValueError("the threshold is outside the float range")
    codes = np.clip(np.rint(np.clip(v, -thr, thr) / step), -TEACH_QMAX, TEACH_QMAX)
    return [float(r) for r in codes * step]


def teaching_clip_search(groups: Sequence[Tuple[Sequence[float], Sequence[float]]],
                         n_clip: int = CLIP_CANDIDATES) -> List[Tuple[float, float, float]]:
    """The per-group threshold choice of [EXPLAINER §5] on one token: group g's partial output
    x_g.w_g is the reference, candidate i predicts x_g.Q_i(w_g) with factor 1 - i/20, and the
    first factor with the least squared difference wins, independently per group.  Sums are
    rounded once (math.fsum).  Returns, per group, (factor, prediction, reference)."""
    factors = [1.0 - i / 20.0 for i in range(n_clip)]
    out = []
    for x, w in groups:
        xv = _finite_vector(x, "x")
        ref = fsum(xv * _finite_vector(w, "w"))
        preds = np.array([fsum(xv * np.asarray(teaching_clip_qdq(w, f))) for f in factors])
        i = first_argmin(list((preds - ref) ** 2))
        out.append((factors[i], float(preds[i]), ref))
    return out


def clip_thresholds(W32: np.ndarray, s32: np.ndarray, n_clip: int = CLIP_CANDIDATES,
                    group: int = GROUP) -> np.ndarray:
    """Candidate thresholds c[i, n, g] = fp32(absmax_g |v[n, .]| * f_i) of the scaled weight
    v = fp32(W s) ([EXPLAINER §5]: a shrink of the original group absmax)."""
    W32 = np.asarray(W32, dtype=np.float32)
    N, K = W32.shape
    if group <= 0 or K % group != 0:
        raise ValueError("the group size must divide K")
    v = (W32 * np.asarray(s32, dtype=np.float32)[None, :]).reshape(N, K // group, group)
    peak = np.abs(v).max(axis=-1)
    return (clip_factors(n_clip)[:, None, None] * peak[None, :, :]).astype(np.float32)


def quantize_clipped(W32: np.ndarray, s32: np.ndarray, c: np.ndarray, group: int = GROUP
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantize clamp(S W, -c, c) with the asymmetric group quantizer, c [N, K/g] one threshold
    per (row, group).  Same returns as ``quantize``; the clamp is exact in fp32."""
    W32 = np.asarray(W32, dtype=np.float32)
    s32 = np.asarray(s32, dtype=np.float32)
    N, K = W32.shape
    if group <= 0 or K % group != 0:
        raise ValueError("the group size must divide K")
    if not np.all(np.isfinite(W32)):
        raise ValueError("weights must be finite")
    if s32.shape != (K,) or not np.all(np.isfinite(s32)) or np.any(s32 <= 0):
        raise ValueError("scales must be finite and positive")
    c = np.asarray(c, dtype=np.float32)
    if c.shape != (N, K // group) or not np.all(np.isfinite(c)) or np.any(c < 0):
        raise ValueError("thresholds must be finite and non-negative, one per (row, group)")
    v = (W32 * s32[None, :]).reshape(N, K // group, group)
    v = np.minimum(np.maximum(v, -c[..., None]), c[..., None])
    delta, z = asym_params(v)
    q = asym_codes(v, delta, z)
    return q.reshape(N, K), z, delta


def clip_errors(X: np.ndarray, W32: np.ndarray, s32: np.ndarray, n_clip: int = CLIP_CANDIDATES,
                group: int = GROUP) -> Dict[str, np.ndarray]:
    """The clipping search of [EXPLAINER §5] for one linear layer after its scales s: for every
    output channel n, input group g and candidate i, the mean over the given tokens of the
    squared error of the group's partial output,
        err[i, n, g] = mean_m ( sum_{k in g} X[m, k] e_i[n, k] )^2,
    e_i = W - S^-1 Q(clamp(S W, -c_i, c_i)), in float64 from the fp32 codes.  Each (n, g)
    keeps the first candidate with the least error.  Returns err, best [N, K/g] and the
    chosen thresholds max_val [N, K/g] (fp32)."""
    X64 = np.asarray(X, dtype=np.float64)
    W32 = np.asarray(W32, dtype=np.float32)
    M, K = X64.shape
    N = W32.shape[0]
    if not np.all(np.isfinite(X64)):
        raise ValueError("activations must be finite")
    G = K // group
    cs = clip_thresholds(W32, s32, n_clip, group)
    err = np.empty((n_clip, N, G))
    for i in range(n_clip):
        q, z, d = quantize_clipped(W32, s32, cs[i], group)
        E = W32.astype(np.float64) - effective_weight(q, z, d, s32, group)
        for g in range(G):
            Y = X64[:, g * group:(g + 1) * group] @ E[:, g * group:(g + 1) * group].T  # [M, N]
            err[i, :, g] = np.mean(Y * Y, axis=0)
    best = np.argmin(err, axis=0)  # numpy argmin returns the first minimum
    max_val = np.take_along_axis(cs, best[None], axis=0)[0]
    return {"err": err, "best": best.astype(np.int32), "max_val": max_val, "thresholds": cs}


def pack_clipped(W: np.ndarray, s32: np.ndarray, max_val: np.ndarray, group: int = GROUP
                 ) -> Dict[str, np.ndarray]:
    """The artefact of ``pack`` for the clipped weight clamp(S W, -max_val, max_val)."""
    q, z, d = quantize_clipped(W, s32, max_val, group)
    scales = d.astype(np.float16)
    if not np.all(np.isfinite(scales)):
        raise ValueError("a group step overflows fp16")
    return {"qweight": pack_words(q), "scales": scales, "zeros": z.astype(np.float16),
            "codes": q, "z": z, "delta": d}


# ---------------------------------------------------------------------------------------
# Applying the scales: folding S^-1 into the producer of X  [EXPLAINER §6]
# ---------------------------------------------------------------------------------------
def _round_to(values64: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to the storage type ("f32", or "bf16" returned as float32
    holding bf16 values, round to nearest even)."""
    v32 = np.asarray(values64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return v32
    if dtype != "bf16":
        raise ValueError("dtype is f32 or bf16")
    # bf16 rounding of the exact value: round the float64 value directly to 8 significand bits
    x = np.asarray(values64, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # nearest with ties to even at 8 bits
    return r.astype(np.float32)


def fold_rows(A: np.ndarray, s32: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """Row k of A divided by s_k, rounded once to the storage type.  This is the fold of
    [EXPLAINER §6] for every producer whose output channel k feeds input channel k of the
    scaled layers: a LayerNorm's gamma and beta (A = [K] or [K, 1]), an RMSNorm's gamma, or a
    preceding Linear's output rows and bias (A = W_prev [K, K_in])."""
    A64 = np.asarray(A, dtype=np.float64)
    s64 = np.asarray(s32, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(s64)) or np.any(s64 <= 0):
        raise ValueError("scales must be finite and positive")
    shape = (-1,) + (1,) * (A64.ndim - 1)
    return _round_to(A64 / s64.reshape(shape), dtype)


def scale_cols(W: np.ndarray, s32: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """Column k of a consuming Linear weight W [N, K] multiplied by s_k, rounded once: every
    projection that reads the folded X takes its s ([EXPLAINER §6]: Q, K and V together)."""
    W64 = np.asarray(W, dtype=np.float64)
    s64 = np.asarray(s32, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(s64)) or np.any(s64 <= 0):
        raise ValueError("scales must be finite and positive")
    return _round_to(W64 * s64[None, :], dtype)


def gelu(x):
    """The exact GELU of [EXPLAINER §6], 0.5 x (1 + erf(x / sqrt 2)), evaluated as
    0.5 x erfc(-x / sqrt 2) (the same function: 1 + erf(z) = erfc(-z)), so that large negative
    x keep their relative precision in float64 instead of cancelling to zero."""
    from math import erfc
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * np.vectorize(erfc)(-x / sqrt(2.0))


def silu(x):
    """x sigmoid(x) = x / (1 + exp(-x)), float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def scaled_activation(X: np.ndarray, s32: np.ndarray, act: str = "gelu") -> np.ndarray:
    """act(X) / s per input channel, float64: the runtime form where the inverse scaling
    cannot be folded into parameters; the division comes after the activation, never before
    it ([EXPLAINER §6])."""
    f = {"gelu": gelu, "silu": silu}[act]
    s64 = np.asarray(s32, dtype=np.float32).astype(np.float64)
    return f(X) / s64[None, :]


# ---------------------------------------------------------------------------------------
# Using the artefact: W4A16 products over the packed weight  [EXPLAINER §7, §8]
# ---------------------------------------------------------------------------------------
def dequant_artefact(qweight: np.ndarray, scales16: np.ndarray, zeros16: np.ndarray,
                     group: int = GROUP) -> np.ndarray:
    """The weight the artefact encodes, in float64 [N, K]: scales[n, g] * (q[n, k] - zeros[n, g])
    with the fp16 scale and the integer zero point ([EXPLAINER §7]: reconstruct Delta (q - z);
    this is what a deployed kernel multiplies with the inputs that carry S^-1)."""
    q = unpack_words(np.asarray(qweight)).astype(np.float64)
    N, K = q.shape
    d = np.asarray(scales16, dtype=np.float16).astype(np.float64)
    z = np.asarray(zeros16, dtype=np.float16).astype(np.float64)
    if d.shape != (N, K // group) or z.shape != d.shape:
        raise ValueError("scales and zeros must be [N, K / group]")
    return (d[..., None] * (q.reshape(N, K // group, group) - z[..., None])).reshape(N, K)


def w4a16_matmul(Xs: np.ndarray, qweight: np.ndarray, scales16: np.ndarray, zeros16: np.ndarray,
                 group: int = GROUP) -> np.ndarray:
    """Y = X' W_hat^T in float64 for activations X' [M, K] that already carry S^-1 (the folded
    producer's output) and the artefact's weight W_hat [N, K]: the W4A16 product of
    [EXPLAINER §8] (4-bit weights, 16-bit activations) with exact arithmetic."""
    X64 = np.asarray(Xs, dtype=np.float64)
    return X64 @ dequant_artefact(qweight, scales16, zeros16, group).T
