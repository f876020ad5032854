"""CPU tests of the C-ABI boundary: the library loads without a GPU, exports every entry point
the header declares, and reports every argument error synchronously, before any HIP call
(no compute call is made here)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "awq.h")


@pytest.fixture(scope="module")
def L():
    from post_weight_quantization_mean_amd import awq
    if not os.path.exists(awq._LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return awq.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"AWQ_API\s+[\w\s\*]+?\b(awq_\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == {"awq_abi_version", "awq_status_string", "awq_stats_workspace_bytes", "awq_stats",
                          "awq_search_workspace_bytes", "awq_search", "awq_search_timed", "awq_pack",
                          "awq_search_multi_workspace_bytes", "awq_search_multi",
                          "awq_search_gram_workspace_bytes", "awq_search_gram",
                          "awq_pack_clipped", "awq_clip_workspace_bytes", "awq_clip", "awq_fold_rows",
                          "awq_scale_cols", "awq_scaled_act", "awq_w4a16", "awq_search_static",
                          "awq_w4a16_workspace_bytes", "awq_w4a16_ws"}


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_version_and_status_strings(L):
    assert L.awq_abi_version() == 8
    for st in range(7):
        assert L.awq_status_string(st)
    assert L.awq_status_string(99) == b"unknown status"


OK, INVALID, SHAPE, UNSUP, WS, HIP, SCRATCH = 0, 1, 2, 3, 4, 5, 6
BF16, F32 = 1, 0
P = 1 << 20  # a fake, 16-byte aligned device address: never dereferenced on these paths


def test_workspace_size_functions(L):
    assert L.awq_stats_workspace_bytes(0, 256) == 0
    assert L.awq_stats_workspace_bytes(4096, 4096) > 0
    assert L.awq_search_workspace_bytes(4096, 4096, 4096, 128, 20) > 4096 * 20 * 8
    assert L.awq_search_workspace_bytes(4096, 4096, 4096, 64, 20) == 0
    assert L.awq_search_workspace_bytes(4096, 4000, 4096, 128, 20) == 0
    assert L.awq_search_workspace_bytes(4096, 4096, 4096, 128, 0) == 0
    assert L.awq_search_workspace_bytes(4096, 4096, 4096, 128, 65) == 0
    # clip: thresholds (16 B) + partial column sums (4 B) per (candidate, group, row, token tile)
    assert L.awq_clip_workspace_bytes(512, 4096, 4096, 128, 10) >= 10 * 32 * 4096 * 20
    assert L.awq_clip_workspace_bytes(1024, 4096, 4096, 128, 10) > L.awq_clip_workspace_bytes(512, 4096, 4096, 128, 10)
    assert L.awq_clip_workspace_bytes(512, 4096, 4096, 64, 10) == 0
    assert L.awq_clip_workspace_bytes(512, 4096, 4096, 128, 0) == 0
    assert L.awq_clip_workspace_bytes(512, 4096, 4096, 128, 21) == 0
    assert L.awq_clip_workspace_bytes(512, 4000, 4096, 128, 10) == 0


def stats(L, X=P, dt=BF16, M=64, K=256, ldx=256, a=P, ws=P, wsb=1 << 30, fl=P):
    return L.awq_stats(X, dt, M, K, ldx, a, ws, wsb, fl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(a=None), INVALID), (dict(fl=None), INVALID),
    (dict(M=0), INVALID), (dict(K=0), INVALID), (dict(ldx=128), INVALID),
    (dict(K=200, ldx=200), SHAPE), (dict(dt=7), UNSUP), (dict(X=P + 8), INVALID),
    (dict(ldx=260), INVALID),  # 520-byte rows break 16-byte alignment
    (dict(ws=None), WS), (dict(wsb=16), WS), (dict(M=1 << 62, ldx=1 << 10, K=256), SHAPE),
])
def test_stats_argument_errors(L, kw, status):
    assert stats(L, **kw) == status


def search(L, X=P, xt=BF16, M=64, K=256, ldx=256, W=P, wt=BF16, N=128, ldw=256, a=P, group=128, n_grid=20,
           losses=P, best=P, sb=P, tab=None, ws=P, wsb=1 << 30, fl=P):
    return L.awq_search(X, xt, M, K, ldx, W, wt, N, ldw, a, group, n_grid, losses, best, sb, tab, ws, wsb, fl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(W=None), INVALID), (dict(a=None), INVALID), (dict(losses=None), INVALID),
    (dict(best=None), INVALID), (dict(sb=None), INVALID), (dict(fl=None), INVALID),
    (dict(N=0), INVALID), (dict(ldw=128), INVALID), (dict(K=384, ldx=384, ldw=200), INVALID),
    (dict(K=192, ldx=192, ldw=192), SHAPE), (dict(group=64), UNSUP), (dict(group=256), UNSUP),
    (dict(n_grid=0), INVALID), (dict(n_grid=65), INVALID), (dict(xt=3), UNSUP), (dict(wt=-1), UNSUP),
    (dict(ws=None), WS), (dict(wsb=1000), WS), (dict(a=P + 4), INVALID), (dict(tab=P + 4), INVALID),
    (dict(ldx=1 << 21, K=256), SHAPE),  # 512 rows of X would span more than 2^31 bytes
    (dict(K=1 << 17, ldx=1 << 17, ldw=1 << 17, N=1 << 21), SHAPE),  # group ranges span 2^31 bytes
])
def test_search_argument_errors(L, kw, status):
    assert search(L, **kw) == status


@pytest.mark.parametrize("kw,status", [(dict(X=None), INVALID), (dict(group=64), UNSUP), (dict(wsb=1000), WS)])
def test_search_timed_argument_errors(L, kw, status):
    # the timed variant validates exactly like awq_search, before recording any event
    a = dict(X=P, xt=BF16, M=64, K=256, ldx=256, W=P, wt=BF16, N=128, ldw=256, a=P, group=128, n_grid=20,
             losses=P, best=P, sb=P, tab=None, ws=P, wsb=1 << 30, fl=P)
    a.update(kw)
    assert L.awq_search_timed(a["X"], a["xt"], a["M"], a["K"], a["ldx"], a["W"], a["wt"], a["N"], a["ldw"],
                              a["a"], a["group"], a["n_grid"], a["losses"], a["best"], a["sb"], a["tab"],
                              a["ws"], a["wsb"], a["fl"], None, None, None) == status


def search_static(L, X=P, xt=BF16, M=64, K=256, ldx=256, W=P, wt=BF16, N=128, ldw=256, a=P, group=128,
                  n_grid=20, losses=P, best=P, sb=P, tab=None, fl=P):
    return L.awq_search_static(X, xt, M, K, ldx, W, wt, N, ldw, a, group, n_grid, losses, best, sb, tab, fl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(W=None), INVALID), (dict(a=None), INVALID), (dict(losses=None), INVALID),
    (dict(fl=None), INVALID), (dict(N=0), INVALID), (dict(K=192, ldx=192, ldw=192), SHAPE),
    (dict(group=64), UNSUP), (dict(n_grid=65), INVALID), (dict(xt=3), UNSUP), (dict(a=P + 4), INVALID),
    # the workspace of a 4096 x 28672 weight (147 MB of group ranges) exceeds the 128 MiB array
    (dict(K=4096, ldx=4096, ldw=4096, N=28672), SCRATCH),
    (dict(K=14336, ldx=14336, ldw=14336, N=8192), SCRATCH),
])
def test_search_static_argument_errors(L, kw, status):
    """The allocation-free search validates every argument and its size limit before its first
    HIP call (the lookup of the static array), so all of these return on the CPU."""
    assert search_static(L, **kw) == status


def xcopy_bytes(M, K):
    """The fragment-ordered copy of X at the end of a search workspace (header formula)."""
    if K % 256 or K < 512:
        return 0
    return -(-2 * (-(-M // 32) * 32) * K // 256) * 256


def test_search_static_limit_matches_the_workspace_size(L):
    from post_weight_quantization_mean_amd import awq
    assert awq.STATIC_SCRATCH_BYTES == 128 * 1024 * 1024
    ws = lambda M, K, N: L.awq_search_workspace_bytes(M, K, N, 128, 20) - xcopy_bytes(M, K)
    # the decoder block's down projection (K = 14336, N = 4096) fits, its fused gate+up does not
    assert ws(16384, 14336, 4096) <= awq.STATIC_SCRATCH_BYTES
    assert ws(16384, 4096, 28672) > awq.STATIC_SCRATCH_BYTES
    assert search_static(L, M=16384, K=4096, ldx=4096, ldw=4096, N=28672) == SCRATCH


@pytest.mark.parametrize("M,M2,K", [(4096, 3585, 4096), (1000, 513, 512), (16384, 15873, 14336), (64, 1, 256),
                                     (4096, 3585, 384), (33, 1, 1024)])
def test_search_workspace_ends_with_the_copy_of_x(L, M, M2, K):
    """Between two token counts with the same number of 512-row tiles (the same partial sums),
    the workspace differs by the copy of X exactly where K takes the persistent kernel (a
    multiple of 256, at least 512), for one weight and for several."""
    assert -(-M // 512) == -(-M2 // 512)
    one = lambda m: L.awq_search_workspace_bytes(m, K, 4096, 128, 20)
    assert one(M) - one(M2) == xcopy_bytes(M, K) - xcopy_bytes(M2, K)
    ns = (ctypes.c_int64 * 2)(2048, 2048)
    multi = lambda m: L.awq_search_multi_workspace_bytes(m, K, ns, 2, 128, 20)
    assert multi(M) - multi(M2) == xcopy_bytes(M, K) - xcopy_bytes(M2, K)
    if xcopy_bytes(M, K):
        assert xcopy_bytes(M, K) > xcopy_bytes(M2, K)


def search_multi(L, X=P, xt=BF16, M=64, K=256, ldx=256, Ws=(P, P + 4096), wt=BF16, Ns=(128, 64), ldws=(256, 256),
                 count=None, a=P, group=128, n_grid=20, losses=P, best=P, sb=P, tab=None, ws=P, wsb=1 << 30, fl=P):
    n = 2 if count is None else count
    arr = lambda typ, v: None if v is None else (typ * max(len(v), 1))(*v)
    return L.awq_search_multi(X, xt, M, K, ldx, arr(ctypes.c_void_p, Ws), wt, arr(ctypes.c_int64, Ns),
                              arr(ctypes.c_int64, ldws), n, a, group, n_grid, losses, best, sb, tab, ws, wsb, fl,
                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(Ws=None), INVALID), (dict(Ns=None), INVALID), (dict(ldws=None), INVALID),
    (dict(count=0), INVALID), (dict(count=9, Ws=(P,) * 9, Ns=(128,) * 9, ldws=(256,) * 9), INVALID),
    (dict(Ws=(P, None)), INVALID), (dict(Ns=(128, 0)), INVALID), (dict(ldws=(256, 128)), INVALID),
    (dict(Ws=(P, P + 8)), INVALID),  # the second weight is not 16-byte aligned
    (dict(ldws=(256, 1 << 24)), SHAPE),  # 128 rows of the second weight span 2^32 bytes
    (dict(group=64), UNSUP), (dict(wt=2), UNSUP), (dict(n_grid=0), INVALID), (dict(a=None), INVALID),
    (dict(ws=None), WS), (dict(wsb=1000), WS),
])
def test_search_multi_argument_errors(L, kw, status):
    assert search_multi(L, **kw) == status


def test_search_multi_workspace_pads_each_weight(L):
    ns = lambda *v: (ctypes.c_int64 * len(v))(*v)
    one = L.awq_search_multi_workspace_bytes(4096, 4096, ns(4096), 1, 128, 20)
    assert one == L.awq_search_workspace_bytes(4096, 4096, 4096, 128, 20)
    # three 4096-row weights take the space of one 12288-row weight
    assert L.awq_search_multi_workspace_bytes(4096, 4096, ns(4096, 4096, 4096), 3, 128, 20) == \
        L.awq_search_workspace_bytes(4096, 4096, 12288, 128, 20)
    # 100 + 100 rows pad to two tiles, more than one 200-row weight (also two tiles) never less
    assert L.awq_search_multi_workspace_bytes(512, 256, ns(100, 100), 2, 128, 20) >= \
        L.awq_search_workspace_bytes(512, 256, 200, 128, 20)
    assert L.awq_search_multi_workspace_bytes(512, 256, ns(100, 0), 2, 128, 20) == 0
    assert L.awq_search_multi_workspace_bytes(512, 256, None, 2, 128, 20) == 0
    assert L.awq_search_multi_workspace_bytes(512, 256, ns(*([128] * 9)), 9, 128, 20) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(W=None), INVALID), (dict(xt=F32), UNSUP), (dict(wt=F32), UNSUP),
    (dict(group=64), UNSUP), (dict(n_grid=0), INVALID), (dict(a=None), INVALID), (dict(ws=None), WS),
    (dict(wsb=1000), WS), (dict(K=1 << 20, ldx=1 << 20, ldw=1 << 20), SHAPE),  # 512 rows of T span 2^31
])
def test_search_gram_argument_errors(L, kw, status):
    a = dict(X=P, xt=BF16, M=64, K=256, ldx=256, W=P, wt=BF16, N=128, ldw=256, a=P, group=128, n_grid=20,
             losses=P, best=P, sb=P, tab=None, ws=P, wsb=1 << 30, fl=P)
    a.update(kw)
    assert L.awq_search_gram(a["X"], a["xt"], a["M"], a["K"], a["ldx"], a["W"], a["wt"], a["N"], a["ldw"],
                             a["a"], a["group"], a["n_grid"], a["losses"], a["best"], a["sb"], a["tab"],
                             a["ws"], a["wsb"], a["fl"], None) == status


def test_search_gram_workspace(L):
    # the search workspace for K rows of the left operand (T as K x 2K: hi and lo interleaved;
    # no copy of X) plus that K x 2K bf16 matrix
    K, N = 4096, 4096
    direct = lambda k: L.awq_search_workspace_bytes(k, k, N, 128, 20) - xcopy_bytes(k, k)
    assert L.awq_search_gram_workspace_bytes(16384, K, N, 128, 20) >= direct(K) + 2 * K * K * 2
    assert L.awq_search_gram_workspace_bytes(16384, 4000, N, 128, 20) == 0
    assert L.awq_search_gram_workspace_bytes(16384, K, N, 128, 65) == 0
    # plus the fp32 sums of the G tiles split along the tokens: at K = 4096, 528 upper-triangle
    # tiles of 128 x 128, the 16 past the first 512 split into 16 slices of 1024 tokens
    base = direct(K) + 2 * K * K * 2
    assert L.awq_search_gram_workspace_bytes(16384, K, N, 128, 20) >= base + 16 * 16 * 128 * 128 * 4
    # K = 5120: 820 tiles; the 308 past the first 512 would get one slice each, so none is split
    base = direct(5120) + 2 * 5120 * 5120 * 2
    assert base <= L.awq_search_gram_workspace_bytes(16384, 5120, N, 128, 20) < base + 4096


def pack(L, W=P, wt=BF16, N=128, K=256, ldw=256, s=P, group=128, q=P, sc=P, z=P, fl=P):
    return L.awq_pack(W, wt, N, K, ldw, s, group, q, sc, z, fl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), INVALID), (dict(s=None), INVALID), (dict(q=None), INVALID), (dict(sc=None), INVALID),
    (dict(z=None), INVALID), (dict(fl=None), INVALID), (dict(N=-1), INVALID), (dict(K=100, ldw=100), SHAPE),
    (dict(group=32), UNSUP), (dict(wt=5), UNSUP), (dict(s=P + 2), INVALID),
])
def test_pack_argument_errors(L, kw, status):
    assert pack(L, **kw) == status


def test_python_binding_rejects_host_tensors():
    import torch
    from post_weight_quantization_mean_amd import awq
    with pytest.raises(ValueError):
        awq.stats(torch.zeros(4, 128))
    with pytest.raises(TypeError):
        awq._dtype_code(torch.zeros(2, dtype=torch.float16))


def pack_clipped(L, W=P, wt=BF16, N=128, K=256, ldw=256, s=P, mv=P, group=128, q=P, sc=P, z=P, fl=P):
    return L.awq_pack_clipped(W, wt, N, K, ldw, s, mv, group, q, sc, z, fl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), INVALID), (dict(s=None), INVALID), (dict(q=None), INVALID), (dict(fl=None), INVALID),
    (dict(K=100, ldw=100), SHAPE), (dict(group=32), UNSUP), (dict(wt=5), UNSUP), (dict(s=P + 2), INVALID),
])
def test_pack_clipped_argument_errors(L, kw, status):
    assert pack_clipped(L, **kw) == status


def clip(L, X=P, xt=BF16, M=64, K=256, ldx=256, W=P, wt=BF16, N=128, ldw=256, s=P, group=128, n_clip=10,
         mv=P, best=None, err=None, ws=P, wsb=1 << 30, fl=P):
    return L.awq_clip(X, xt, M, K, ldx, W, wt, N, ldw, s, group, n_clip, mv, best, err, ws, wsb, fl, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(W=None), INVALID), (dict(s=None), INVALID), (dict(mv=None), INVALID),
    (dict(fl=None), INVALID), (dict(M=0), INVALID), (dict(ldw=128), INVALID), (dict(K=192, ldx=192, ldw=192), SHAPE),
    (dict(group=64), UNSUP), (dict(n_clip=0), INVALID), (dict(n_clip=21), INVALID), (dict(xt=3), UNSUP),
    (dict(ws=None), WS), (dict(wsb=1000), WS), (dict(s=P + 4), INVALID), (dict(ws=P + 8), INVALID),
    (dict(ldx=1 << 21, K=256), SHAPE),  # 512 rows of X would span more than 2^31 bytes
])
def test_clip_argument_errors(L, kw, status):
    assert clip(L, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), INVALID), (dict(s=None), INVALID), (dict(fl=None), INVALID), (dict(rows=0), INVALID),
    (dict(cols=0), INVALID), (dict(ld=3, cols=4), INVALID), (dict(dt=9), UNSUP), (dict(A=P + 1), INVALID),
    (dict(s=P + 2), INVALID), (dict(rows=1 << 62, ld=1 << 10, cols=4), SHAPE),
])
def test_fold_and_scale_argument_errors(L, kw, status):
    a = dict(A=P, dt=BF16, rows=64, cols=4, ld=4, s=P, fl=P)
    a.update(kw)
    assert L.awq_fold_rows(a["A"], a["dt"], a["rows"], a["cols"], a["ld"], a["s"], a["fl"], None) == status
    assert L.awq_scale_cols(a["A"], a["dt"], a["rows"], a["cols"], a["ld"], a["s"], a["fl"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(Y=None), INVALID), (dict(act=2), UNSUP), (dict(act=-1), UNSUP),
    (dict(Y=P + 1), INVALID), (dict(M=0), INVALID),
])
def test_scaled_act_argument_errors(L, kw, status):
    a = dict(X=P, Y=P, dt=F32, M=8, K=16, ld=16, act=0, s=P, fl=P)
    a.update(kw)
    assert L.awq_scaled_act(a["X"], a["Y"], a["dt"], a["M"], a["K"], a["ld"], a["act"], a["s"], a["fl"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), INVALID), (dict(q=None), INVALID), (dict(sc=None), INVALID), (dict(z=None), INVALID),
    (dict(Y=None), INVALID), (dict(N=0), INVALID), (dict(ldy=127), INVALID), (dict(q=P + 4), INVALID),
    (dict(sc=P + 1), INVALID), (dict(Y=P + 2), INVALID), (dict(group=64), UNSUP), (dict(xt=4), UNSUP),
    (dict(K=200, ldx=200), SHAPE), (dict(ldx=1 << 21), SHAPE),
    (dict(ldy=1 << 20), SHAPE),  # 512 rows of Y span 2^31 bytes (32-bit offsets in a prefill tile)
])
def test_w4a16_argument_errors(L, kw, status):
    a = dict(X=P, xt=BF16, M=4, K=256, ldx=256, q=P, sc=P, z=P, N=128, group=128, Y=P, ldy=128)
    a.update(kw)
    assert L.awq_w4a16(a["X"], a["xt"], a["M"], a["K"], a["ldx"], a["q"], a["sc"], a["z"], a["N"], a["group"],
                       a["Y"], a["ldy"], None) == status
    # the workspace form checks the same arguments first (prefill-sized M: it would use the copy)
    a["M"] = 64 if a["M"] == 4 else a["M"]
    assert L.awq_w4a16_ws(a["X"], a["xt"], a["M"], a["K"], a["ldx"], a["q"], a["sc"], a["z"], a["N"],
                          a["group"], a["Y"], a["ldy"], P, 1 << 30, None) == status


def test_w4a16_ws_rejects_a_misaligned_workspace(L):
    assert L.awq_w4a16_ws(P, BF16, 64, 256, 256, P, P, P, 128, 128, P, 128, P + 8, 1 << 20, None) == INVALID


@pytest.mark.parametrize("name,skipped", [
    ("model.layers.0.self_attn.q_proj", True), ("model.layers.0.self_attn.k_proj", True),
    ("transformer.h.3.attn.Wqkv", True), ("encoder.layer.1.attention.self.query", True),
    ("encoder.layer.1.attention.self.key", True),
    ("model.layers.0.self_attn.v_proj", False), ("model.layers.0.self_attn.o_proj", False),
    ("model.layers.0.mlp.gate_proj", False), ("model.layers.0.mlp.down_proj", False),
    ("encoder.layer.1.attention.self.value", False),
])
def test_clip_skips_query_and_key_modules(name, skipped):
    """The clipping search skips Linear modules whose name contains q_, k_, query, key or Wqkv
    ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §5); every other projection is clipped."""
    from post_weight_quantization_mean_amd import awq
    assert awq.clip_skipped(name) is skipped


@pytest.mark.parametrize("M,K,dt,want", [
    (4096, 4096, BF16, 2 * 4096 * 4096), (1000, 4096, BF16, 2 * 1024 * 4096), (9, 128, BF16, 2 * 32 * 128),
    (8, 4096, BF16, 0), (1, 4096, BF16, 0), (4096, 4096, 0, 0), (0, 4096, BF16, 0), (64, 100, BF16, 0),
    (64, 4096, 7, 0)])
def test_w4a16_workspace_bytes(L, M, K, dt, want):
    """The prefill's copy of X: bf16 X with more than 8 tokens, 2 round_up(M, 32) K bytes; no
    workspace for the decode, fp32 X or invalid sizes."""
    assert L.awq_w4a16_workspace_bytes(M, K, dt) == want
