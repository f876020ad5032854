"""Python binding of libawq (argument marshalling only; every step runs in the HIP kernels).

Tensors are torch tensors on a ROCm device; the calls are queued on the device's current
torch stream.  Shapes follow PyTorch: X is [M, K] activations, W is a Linear weight [N, K].
Data errors that only the device can see come back as flag bits; with ``check=True`` (the
default) the call synchronises and raises ``ValueError`` for them, like the explainer page's
reference code rejects non-finite input ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §3).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libawq.so")

AWQ_DTYPE_F32 = 0
AWQ_DTYPE_BF16 = 1
FLAG_NONFINITE_X = 0x1
FLAG_NONFINITE_W = 0x2
FLAG_SCALE_RANGE = 0x4
FLAG_F16_RANGE = 0x8
FLAG_NONFINITE_LOSS = 0x10
STATIC_SCRATCH_BYTES = 128 * 1024 * 1024  # awq_search_static's workspace (AWQ_STATIC_SCRATCH_BYTES)
_FLAG_TEXT = {
    FLAG_NONFINITE_X: "activations must be finite",
    FLAG_NONFINITE_W: "weights (and weights times scales) must be finite",
    FLAG_SCALE_RANGE: "scales must be finite and positive (and clip thresholds finite and non-negative)",
    FLAG_F16_RANGE: "a group step does not fit fp16",
    FLAG_NONFINITE_LOSS: "a candidate loss is not finite (non-finite X or W)",
}
GROUP = 128
N_GRID = 20
N_CLIP = 10
ACT_GELU = 0
ACT_SILU = 1

_lib = None


class AwqError(RuntimeError):
    """A status other than AWQ_OK returned by the library."""

    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.awq_status_string(status).decode()} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libawq.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing; build it with "
                              "`python -m post_weight_quantization_mean_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.awq_abi_version.restype = ctypes.c_int
        L.awq_status_string.restype = ctypes.c_char_p
        L.awq_status_string.argtypes = [ctypes.c_int]
        L.awq_stats_workspace_bytes.restype = sz
        L.awq_stats_workspace_bytes.argtypes = [i64, i64]
        L.awq_stats.restype = ctypes.c_int
        L.awq_stats.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, sz, vp, vp]
        L.awq_search_workspace_bytes.restype = sz
        L.awq_search_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
        L.awq_search.restype = ctypes.c_int
        L.awq_search.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_int, i64, i64, vp,
                                 i32, i32, vp, vp, vp, vp, vp, sz, vp, vp]
        L.awq_search_timed.restype = ctypes.c_int
        L.awq_search_timed.argtypes = L.awq_search.argtypes + [vp, vp]
        L.awq_search_static.restype = ctypes.c_int
        L.awq_search_static.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_int, i64, i64, vp,
                                        i32, i32, vp, vp, vp, vp, vp, vp]
        L.awq_search_gram_workspace_bytes.restype = sz
        L.awq_search_gram_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
        L.awq_search_gram.restype = ctypes.c_int
        L.awq_search_gram.argtypes = L.awq_search.argtypes
        L.awq_search_multi_workspace_bytes.restype = sz
        L.awq_search_multi_workspace_bytes.argtypes = [i64, i64, vp, i32, i32, i32]
        L.awq_search_multi.restype = ctypes.c_int
        L.awq_search_multi.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_int, vp, vp, i32, vp,
                                       i32, i32, vp, vp, vp, vp, vp, sz, vp, vp]
        L.awq_pack.restype = ctypes.c_int
        L.awq_pack.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, vp, vp, vp, vp, vp]
        L.awq_pack_clipped.restype = ctypes.c_int
        L.awq_pack_clipped.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, i32, vp, vp, vp, vp, vp]
        L.awq_clip_workspace_bytes.restype = sz
        L.awq_clip_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
        L.awq_clip.restype = ctypes.c_int
        L.awq_clip.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_int, i64, i64, vp,
                               i32, i32, vp, vp, vp, vp, sz, vp, vp]
        for name in ("awq_fold_rows", "awq_scale_cols"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp]
        L.awq_scaled_act.restype = ctypes.c_int
        L.awq_scaled_act.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, vp, vp, vp]
        L.awq_w4a16.restype = ctypes.c_int
        L.awq_w4a16.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, i64, i32, vp, i64, vp]
        L.awq_w4a16_workspace_bytes.restype = sz
        L.awq_w4a16_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
        L.awq_w4a16_ws.restype = ctypes.c_int
        L.awq_w4a16_ws.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp, i64, i32, vp, i64, vp, sz, vp]
        if L.awq_abi_version() != 8:
            raise ImportError("libawq ABI version mismatch")
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return AWQ_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return AWQ_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _matrix(t: torch.Tensor, name: str) -> Tuple[int, int, int]:
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along K")
    return t.shape[0], t.shape[1], t.stride(0)


def _same_device(t: torch.Tensor, dev: torch.device, name: str) -> None:
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} must be on {dev}")


def _out(t: torch.Tensor, shape: Tuple[int, ...], dtype: torch.dtype, dev: torch.device, name: str) -> torch.Tensor:
    """A caller-supplied output buffer: the kernels write shape x dtype bytes through its pointer,
    so anything else (a smaller, strided or mistyped tensor, or one on another device) is refused."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)}")
    _same_device(t, dev, name)
    return t


def _workspace(t: Optional[torch.Tensor], need: int, dev: torch.device) -> Tuple[torch.Tensor, int]:
    """The workspace tensor and its size in bytes (the library refuses one below ``need``)."""
    if t is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev), max(need, 1)
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _same_device(t, dev, "workspace")
    return t, t.numel() * t.element_size()


def _flags(t: Optional[torch.Tensor], dev: torch.device) -> torch.Tensor:
    if t is None:
        return torch.zeros(1, dtype=torch.int32, device=dev)
    if t.dtype != torch.int32 or t.numel() < 1 or not t.is_contiguous():
        raise ValueError("flags must be a contiguous int32 tensor with at least one element")
    _same_device(t, dev, "flags")
    return t


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(status: int, what: str) -> None:
    if status != 0:
        raise AwqError(status, what)


def raise_for_flags(flags: torch.Tensor) -> None:
    """Synchronise on ``flags`` and raise ValueError naming every data error it carries."""
    f = int(flags.item())
    if f:
        msgs = [txt for bit, txt in _FLAG_TEXT.items() if f & bit]
        raise ValueError("; ".join(msgs) + f" (flags 0x{f:x})")


def stats_workspace_bytes(M: int, K: int) -> int:
    return int(lib().awq_stats_workspace_bytes(M, K))


def search_workspace_bytes(M: int, K: int, N, group: int = GROUP, n_grid: int = N_GRID, gram: bool = False) -> int:
    """N: the weight's rows, or a sequence of several weights' rows (awq_search_multi)."""
    if gram:
        return int(lib().awq_search_gram_workspace_bytes(M, K, N, group, n_grid))
    if isinstance(N, (list, tuple)):
        ns = (ctypes.c_int64 * len(N))(*N)
        return int(lib().awq_search_multi_workspace_bytes(M, K, ns, len(N), group, n_grid))
    return int(lib().awq_search_workspace_bytes(M, K, N, group, n_grid))


def stats(X: torch.Tensor, *, out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
          flags: Optional[torch.Tensor] = None, check: bool = True) -> torch.Tensor:
    """a[j] = mean_m |X[m, j]| as fp32 [K]."""
    M, K, ldx = _matrix(X, "X")
    dev = X.device
    a = _out(out, (K,), torch.float32, dev, "out") if out is not None else \
        torch.empty(K, dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(workspace, stats_workspace_bytes(M, K), dev)
    fl = _flags(flags, dev)
    st = lib().awq_stats(X.data_ptr(), _dtype_code(X), M, K, ldx, a.data_ptr(), ws.data_ptr(),
                         ws_bytes, fl.data_ptr(), _stream(dev))
    _check(st, "awq_stats")
    if check:
        raise_for_flags(fl)
    return a


@dataclasses.dataclass
class SearchResult:
    losses: torch.Tensor       # fp64 [n_grid] (device)
    best: torch.Tensor         # int32 [1] (device)
    s_best: torch.Tensor       # fp32 [K] (device)
    s_table: Optional[torch.Tensor]  # fp32 [n_grid, K] (device) when requested
    flags: torch.Tensor        # int32 [1] (device)

    @property
    def best_index(self) -> int:
        return int(self.best.item())


def search(X: torch.Tensor, W, a: torch.Tensor, group_size: int = GROUP, n_grid: int = N_GRID,
           *, return_table: bool = False, workspace: Optional[torch.Tensor] = None,
           flags: Optional[torch.Tensor] = None, check: bool = True, gram: bool = False,
           fused_events: Optional[Tuple[torch.cuda.Event, torch.cuda.Event]] = None,
           no_alloc: bool = False) -> SearchResult:
    """The candidate scale search over alpha = i / n_grid for one layer.  ``W`` is one weight
    [N, K], or a list of weights [N_w, K] of projections that read X and share the scales
    (query/key/value, gate/up): searched as one layer without concatenating them
    (awq_search_multi), all of one dtype.

    ``gram``: evaluate the losses in the Gram form sum_n E[n] (X^T X) E[n]^T (awq_search_gram;
    bf16 X and a single bf16 W): cheaper when M > K + 512, equal up to rounding.

    ``fused_events``: two timing events that the library records right before and after the
    fused candidate kernel (awq_search_timed), so that ``e0.elapsed_time(e1)`` is that
    kernel's time alone; single weight only.

    ``no_alloc``: run awq_search_static, whose workspace is the library's static device array
    (STATIC_SCRATCH_BYTES per GPU) instead of ``workspace``; single weight, direct form.  Calls
    that overlap on one GPU race on that array."""
    M, K, ldx = _matrix(X, "X")
    Ws = list(W) if isinstance(W, (list, tuple)) else None
    if Ws is not None:
        if not Ws:
            raise ValueError("W is an empty list")
        if any(w.dtype != Ws[0].dtype for w in Ws):
            raise ValueError("the weights of one search share a dtype")
        shapes = [_matrix(w, f"W[{i}]") for i, w in enumerate(Ws)]
        for i, w in enumerate(Ws):
            _same_device(w, X.device, f"W[{i}]")
        if any(kw != K for _, kw, _ in shapes):
            raise ValueError("X and W disagree on K")
        if fused_events is not None or gram:
            raise ValueError("fused_events and the Gram form take a single weight")
        N = [n for n, _, _ in shapes]
    else:
        N, Kw, ldw = _matrix(W, "W")
        if Kw != K:
            raise ValueError("X and W disagree on K")
        _same_device(W, X.device, "W")
    if a.shape != (K,) or a.dtype != torch.float32 or not a.is_cuda or not a.is_contiguous():
        raise ValueError("a must be a contiguous fp32 device vector of length K")
    dev = X.device
    _same_device(a, dev, "a")
    losses = torch.empty(n_grid, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    s_table = torch.empty((n_grid, K), dtype=torch.float32, device=dev) if return_table else None
    if gram and fused_events is not None:
        raise ValueError("fused_events times the direct form")
    if no_alloc:
        if Ws is not None or gram or fused_events is not None or workspace is not None:
            raise ValueError("no_alloc runs a single weight in the direct form, without workspace or events")
        fl = _flags(flags, dev)
        st = lib().awq_search_static(X.data_ptr(), _dtype_code(X), M, K, ldx, W.data_ptr(), _dtype_code(W), N, ldw,
                                     a.data_ptr(), group_size, n_grid, losses.data_ptr(), best.data_ptr(),
                                     s_best.data_ptr(), s_table.data_ptr() if s_table is not None else None,
                                     fl.data_ptr(), _stream(dev))
        _check(st, "awq_search_static")
        if check:
            raise_for_flags(fl)
        return SearchResult(losses, best, s_best, s_table, fl)
    ws, ws_bytes = _workspace(workspace, search_workspace_bytes(M, K, N, group_size, n_grid, gram=gram), dev)
    fl = _flags(flags, dev)
    outs = (a.data_ptr(), group_size, n_grid, losses.data_ptr(), best.data_ptr(), s_best.data_ptr(),
            s_table.data_ptr() if s_table is not None else None, ws.data_ptr(), ws_bytes, fl.data_ptr(),
            _stream(dev))
    if Ws is not None:
        ptrs = (ctypes.c_void_p * len(Ws))(*[w.data_ptr() for w in Ws])
        ns = (ctypes.c_int64 * len(Ws))(*N)
        lds = (ctypes.c_int64 * len(Ws))(*[ld for _, _, ld in shapes])
        st = lib().awq_search_multi(X.data_ptr(), _dtype_code(X), M, K, ldx, ptrs, _dtype_code(Ws[0]), ns, lds,
                                    len(Ws), *outs)
        _check(st, "awq_search_multi")
        if check:
            raise_for_flags(fl)
        return SearchResult(losses, best, s_best, s_table, fl)
    args = (X.data_ptr(), _dtype_code(X), M, K, ldx, W.data_ptr(), _dtype_code(W), N, ldw) + outs
    if gram:
        st = lib().awq_search_gram(*args)
    elif fused_events is None:
        st = lib().awq_search(*args)
    else:
        evs = []
        for e in fused_events:
            if not e.cuda_event:  # torch creates the HIP event lazily, on its first record
                e.record(torch.cuda.current_stream(dev))
            evs.append(e.cuda_event)
        st = lib().awq_search_timed(*args, *evs)
    _check(st, "awq_search")
    if check:
        raise_for_flags(fl)
    return SearchResult(losses, best, s_best, s_table, fl)


def pack(W: torch.Tensor, s: torch.Tensor, group_size: int = GROUP, *, max_val: Optional[torch.Tensor] = None,
         flags: Optional[torch.Tensor] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
         check: bool = True) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Quantize S W exactly and pack: qweight int32 [N, K/8], scales fp16 [N, K/128] (Delta),
    zeros fp16 [N, K/128] (integer zero points).  ``max_val`` (fp32 [N, K/128], normally
    ``clip(...).max_val``) clamps S W to [-max_val, max_val] per (row, group) first."""
    N, K, ldw = _matrix(W, "W")
    if s.shape != (K,) or s.dtype != torch.float32 or not s.is_cuda or not s.is_contiguous():
        raise ValueError("s must be a contiguous fp32 device vector of length K")
    if max_val is not None and (max_val.shape != (N, K // group_size) or max_val.dtype != torch.float32
                                or not max_val.is_cuda or not max_val.is_contiguous()):
        raise ValueError("max_val must be a contiguous fp32 device tensor [N, K/group]")
    dev = W.device
    _same_device(s, dev, "s")
    if max_val is not None:
        _same_device(max_val, dev, "max_val")
    G = K // group_size if group_size > 0 else 0
    if out is None:
        qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
        scales = torch.empty((N, G), dtype=torch.float16, device=dev)
        zeros = torch.empty_like(scales)
    else:
        qweight, scales, zeros = out
        _out(qweight, (N, K // 8), torch.int32, dev, "qweight")
        _out(scales, (N, G), torch.float16, dev, "scales")
        _out(zeros, (N, G), torch.float16, dev, "zeros")
    fl = _flags(flags, dev)
    if max_val is None:
        st = lib().awq_pack(W.data_ptr(), _dtype_code(W), N, K, ldw, s.data_ptr(), group_size,
                            qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), fl.data_ptr(), _stream(dev))
    else:
        st = lib().awq_pack_clipped(W.data_ptr(), _dtype_code(W), N, K, ldw, s.data_ptr(), max_val.data_ptr(),
                                    group_size, qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(),
                                    fl.data_ptr(), _stream(dev))
    _check(st, "awq_pack")
    if check:
        raise_for_flags(fl)
    return qweight, scales, zeros


# Linear modules that the clipping search leaves alone, by name ("AWQ：为什么 4-bit 权重量化要先观察
# Activation", §5): the query and key projections (and a fused QKV weight) keep the full range
# of their scaled groups.
CLIP_SKIP_NAME_PARTS = ("q_", "k_", "query", "key", "Wqkv")


def clip_skipped(module_name: str) -> bool:
    """True when a Linear module of this name takes no clipping search (its name contains one of
    CLIP_SKIP_NAME_PARTS, case-sensitive substrings); pack such a layer with ``max_val=None``."""
    return any(part in module_name for part in CLIP_SKIP_NAME_PARTS)


def clip_workspace_bytes(M: int, K: int, N: int, group: int = GROUP, n_clip: int = N_CLIP) -> int:
    return int(lib().awq_clip_workspace_bytes(M, K, N, group, n_clip))


@dataclasses.dataclass
class ClipResult:
    max_val: torch.Tensor             # fp32 [N, K/128]: the chosen thresholds (device)
    best: torch.Tensor                # int32 [N, K/128]: the chosen candidate (device)
    err: Optional[torch.Tensor]       # fp64 [n_clip, N, K/128] when requested (device)
    flags: torch.Tensor               # int32 [1] (device)


def clip(X: torch.Tensor, W: torch.Tensor, s: torch.Tensor, group_size: int = GROUP, n_clip: int = N_CLIP,
         *, return_err: bool = False, workspace: Optional[torch.Tensor] = None,
         flags: Optional[torch.Tensor] = None, check: bool = True) -> ClipResult:
    """The clipping search after the scales s: per (output channel, group) the first of the
    thresholds absmax * (1 - i/20), i < n_clip, with the least mean squared partial-output
    error over the tokens of X (pass the sampled calibration tokens; a strided view such as
    ``X[::8]`` works without a copy)."""
    M, K, ldx = _matrix(X, "X")
    N, Kw, ldw = _matrix(W, "W")
    if Kw != K:
        raise ValueError("X and W disagree on K")
    if s.shape != (K,) or s.dtype != torch.float32 or not s.is_cuda or not s.is_contiguous():
        raise ValueError("s must be a contiguous fp32 device vector of length K")
    dev = X.device
    _same_device(W, dev, "W")
    _same_device(s, dev, "s")
    G = K // group_size if group_size > 0 else 0
    max_val = torch.empty((N, G), dtype=torch.float32, device=dev)
    best = torch.empty((N, G), dtype=torch.int32, device=dev)
    err = torch.empty((n_clip, N, G), dtype=torch.float64, device=dev) if return_err else None
    ws, ws_bytes = _workspace(workspace, clip_workspace_bytes(M, K, N, group_size, n_clip), dev)
    fl = _flags(flags, dev)
    st = lib().awq_clip(X.data_ptr(), _dtype_code(X), M, K, ldx, W.data_ptr(), _dtype_code(W), N, ldw,
                        s.data_ptr(), group_size, n_clip, max_val.data_ptr(), best.data_ptr(),
                        err.data_ptr() if err is not None else None, ws.data_ptr(), ws_bytes,
                        fl.data_ptr(), _stream(dev))
    _check(st, "awq_clip")
    if check:
        raise_for_flags(fl)
    return ClipResult(max_val, best, err, fl)


def _rows2d(t: torch.Tensor, name: str) -> Tuple[int, int, int]:
    """[rows, cols] view of a 1-D or 2-D device tensor with unit stride along its last axis."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() == 1:
        if t.stride(0) != 1:
            raise ValueError(f"{name} must be contiguous")
        return t.shape[0], 1, 1
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 1-D or 2-D with unit stride along its last axis")
    return t.shape[0], t.shape[1], t.stride(0)


def _scales_vec(s: torch.Tensor, n: int) -> None:
    if s.shape != (n,) or s.dtype != torch.float32 or not s.is_cuda or not s.is_contiguous():
        raise ValueError(f"s must be a contiguous fp32 device vector of length {n}")


def fold_rows(A: torch.Tensor, s: torch.Tensor, *, flags: Optional[torch.Tensor] = None,
              check: bool = True) -> torch.Tensor:
    """In place: row k of A divided by s[k] -- a norm's gamma or beta ([K]) or a preceding
    Linear's weight [K, K_in] and bias [K] absorb the inverse scaling.  Returns A."""
    rows, cols, ld = _rows2d(A, "A")
    _scales_vec(s, rows)
    _same_device(s, A.device, "s")
    fl = _flags(flags, A.device)
    _check(lib().awq_fold_rows(A.data_ptr(), _dtype_code(A), rows, cols, ld, s.data_ptr(), fl.data_ptr(),
                               _stream(A.device)), "awq_fold_rows")
    if check:
        raise_for_flags(fl)
    return A


def scale_cols(W: torch.Tensor, s: torch.Tensor, *, flags: Optional[torch.Tensor] = None,
               check: bool = True) -> torch.Tensor:
    """In place: column k of a consuming Linear weight W [N, K] multiplied by s[k].  Returns W."""
    N, K, ld = _matrix(W, "W")
    _scales_vec(s, K)
    _same_device(s, W.device, "s")
    fl = _flags(flags, W.device)
    _check(lib().awq_scale_cols(W.data_ptr(), _dtype_code(W), N, K, ld, s.data_ptr(), fl.data_ptr(),
                                _stream(W.device)), "awq_scale_cols")
    if check:
        raise_for_flags(fl)
    return W


def scaled_act(X: torch.Tensor, s: torch.Tensor, act: str = "gelu", *, out: Optional[torch.Tensor] = None,
               flags: Optional[torch.Tensor] = None, check: bool = True) -> torch.Tensor:
    """act(X) / s per input channel (``act`` "gelu" (exact) or "silu"); ``out`` may be X."""
    M, K, ld = _matrix(X, "X")
    _scales_vec(s, K)
    code = {"gelu": ACT_GELU, "silu": ACT_SILU}[act]
    Y = out if out is not None else torch.empty_strided(X.shape, X.stride(), dtype=X.dtype, device=X.device)
    if Y.shape != X.shape or Y.stride() != X.stride() or Y.dtype != X.dtype:
        raise ValueError("out must match X in shape, strides and dtype")
    _same_device(Y, X.device, "out")
    _same_device(s, X.device, "s")
    fl = _flags(flags, X.device)
    _check(lib().awq_scaled_act(X.data_ptr(), Y.data_ptr(), _dtype_code(X), M, K, ld, code, s.data_ptr(),
                                fl.data_ptr(), _stream(X.device)), "awq_scaled_act")
    if check:
        raise_for_flags(fl)
    return Y


def w4a16_workspace_bytes(M: int, K: int, dtype: torch.dtype = torch.bfloat16) -> int:
    """Bytes of the prefill's copy of X in matrix-core operand order (0 when none is used)."""
    return int(lib().awq_w4a16_workspace_bytes(M, K, 0 if dtype == torch.float32 else 1))


def w4a16(X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
          group_size: int = GROUP, *, out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, staged: bool = False) -> torch.Tensor:
    """Y = X' W_hat^T (fp32 [M, N]) for activations X' [M, K] that already carry S^-1 and the
    artefact (qweight int32 [N, K/8], scales and zeros fp16 [N, K/128]) of ``pack``.
    The prefill (bf16 X, more than 8 tokens) reads X from a copy in matrix-core operand order
    in ``workspace`` (allocated here when not given; ``w4a16_workspace_bytes``); ``staged``
    runs it without the copy (X staged on chip), with the same result bit for bit."""
    M, K, ldx = _matrix(X, "X")
    N = qweight.shape[0]
    if qweight.shape != (N, K // 8) or qweight.dtype != torch.int32 or not qweight.is_contiguous():
        raise ValueError("qweight must be a contiguous int32 [N, K/8] tensor")
    for t, name in ((scales, "scales"), (zeros, "zeros")):
        if t.shape != (N, K // group_size) or t.dtype != torch.float16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous fp16 [N, K/group] tensor")
    for t, name in ((qweight, "qweight"), (scales, "scales"), (zeros, "zeros")):
        _same_device(t, X.device, name)
    Y = out if out is not None else torch.empty((M, N), dtype=torch.float32, device=X.device)
    if Y.shape != (M, N) or Y.dtype != torch.float32 or Y.stride(1) != 1:
        raise ValueError("out must be fp32 [M, N] with unit stride along N")
    _same_device(Y, X.device, "out")
    need = 0 if staged else w4a16_workspace_bytes(M, K, X.dtype)
    if need > 0:
        ws, ws_bytes = _workspace(workspace, need, X.device)
        ws_ptr = ws.data_ptr()
    else:
        ws_ptr, ws_bytes = None, 0
    _check(lib().awq_w4a16_ws(X.data_ptr(), _dtype_code(X), M, K, ldx, qweight.data_ptr(), scales.data_ptr(),
                              zeros.data_ptr(), N, group_size, Y.data_ptr(), Y.stride(0), ws_ptr, ws_bytes,
                              _stream(X.device)),
           "awq_w4a16_ws")
    return Y
