"""AWQ per-layer hot path on MI355X (gfx950): Python binding of libawq.so.

This module only marshals arguments: torch tensors are checked for device,
dtype and layout, their device pointers and the current HIP stream are handed
to the C ABI declared in ``include/awq.h``, and errors come back as
``AwqError``.  Every step of the computation runs in the library's HIP
kernels; there is no CPU fallback.  The library must have been built
(``python -m post_weight_quantization_awq_amd.build``); the first call without
it raises ImportError.

Entry points (same names as the C ABI):

* ``act_stats``           per-input-channel mean |x|        ("AWQ scaling", konic.io)
* ``candidate_scales``    s_k = clamp(x^(k/n), s_min) / sqrt(max*min)   ("The scale search as code", aicassindra.com)
* ``search_scales``       alpha grid search, weight or output score, optional clip search
* ``quantize_pack``       INT4 codes + fp16 scales in the AutoAWQ GEMM layout
* ``unpack_dequant``      inverse of quantize_pack
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libawq.so")

AWQ_OK, AWQ_EINVAL, AWQ_ESHAPE, AWQ_EDTYPE, AWQ_EWORKSPACE, AWQ_EALIGN, AWQ_EHIP = range(7)
AWQ_F16, AWQ_BF16, AWQ_F32 = 0, 1, 2
AWQ_SCORE_WEIGHT, AWQ_SCORE_OUTPUT = 0, 1
AWQ_FLAG_DUO = 1
AWQ_FLAG_ASYM = 2
AWQ_FLAG_OUT_DIRECT = 4
AWQ_FLAG_OUT_GRAM = 8
_OUT_FORM = {"auto": 0, "direct": AWQ_FLAG_OUT_DIRECT, "gram": AWQ_FLAG_OUT_GRAM}
STATUS_NAMES = {0: "AWQ_OK", 1: "AWQ_EINVAL", 2: "AWQ_ESHAPE", 3: "AWQ_EDTYPE",
                4: "AWQ_EWORKSPACE", 5: "AWQ_EALIGN", 6: "AWQ_EHIP"}

EXPORTED = ("awq_act_stats_workspace", "awq_act_stats", "awq_candidate_scales_workspace", "awq_candidate_scales",
            "awq_search_workspace", "awq_search_output_form", "awq_search_scales", "awq_quantize_pack", "awq_quantize_pack_asym",
            "awq_unpack_dequant", "awq_norm_group_fold", "awq_weight_channel_mean_workspace",
            "awq_weight_channel_mean", "awq_candidate_scales_duo_workspace", "awq_candidate_scales_duo",
            "awq_w4a16_workspace", "awq_w4a16_matmul", "awq_search_scales_noalloc",
            "awq_last_error", "awq_abi_version", "awq_set_timing_events")


class AwqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class SearchCfg(ctypes.Structure):
    _fields_ = [("group_size", ctypes.c_int32), ("n_grid", ctypes.c_int32),
                ("score", ctypes.c_int32), ("n_clip", ctypes.c_int32),
                ("s_min", ctypes.c_double), ("clip_lo", ctypes.c_float),
                ("flags", ctypes.c_int32)]


class WGroup(ctypes.Structure):
    _fields_ = [("n_parts", ctypes.c_int32), ("w", ctypes.POINTER(ctypes.c_void_p)),
                ("rows", ctypes.POINTER(ctypes.c_int64))]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m post_weight_quantization_awq_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32, F64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "awq_act_stats_workspace": [I64, I64, PSZ],
        "awq_act_stats": [P, I32, I64, I64, I64, F32, I32, P, P, SZ, P],
        "awq_candidate_scales_workspace": [I64, I32, PSZ],
        "awq_candidate_scales": [P, I64, I32, F64, P, P, SZ, P],
        "awq_search_workspace": [ctypes.POINTER(SearchCfg), I64, I64, I64, PSZ],
        "awq_search_output_form": [ctypes.POINTER(SearchCfg), I64, I64, I64, ctypes.POINTER(I32)],
        "awq_search_scales": [ctypes.POINTER(SearchCfg), ctypes.POINTER(WGroup), I64, P, P, I32, I64, I64,
                              P, P, P, P, P, P, SZ, P],
        "awq_quantize_pack": [P, I64, I64, I32, P, P, P, P, P, P],
        "awq_quantize_pack_asym": [P, I64, I64, I32, P, P, P, P, P, P],
        "awq_unpack_dequant": [P, P, P, I64, I64, I32, P, P, I32, P],
        "awq_norm_group_fold": [ctypes.POINTER(ctypes.c_void_p), I32, I64, P, I32, P, P, P],
        "awq_weight_channel_mean_workspace": [I64, I64, PSZ],
        "awq_weight_channel_mean": [ctypes.POINTER(WGroup), I64, P, P, SZ, P],
        "awq_candidate_scales_duo_workspace": [I64, I32, PSZ],
        "awq_candidate_scales_duo": [P, P, I64, I32, F64, P, P, SZ, P],
        "awq_w4a16_workspace": [I64, I64, I64, PSZ],
        "awq_w4a16_matmul": [P, I64, I64, P, P, P, I64, I64, I32, P, I64, I32, P, SZ, P],
        "awq_set_timing_events": [P, P],
        "awq_search_scales_noalloc": [ctypes.POINTER(SearchCfg), ctypes.POINTER(WGroup), I64, P, P, P, P, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int32
    lib.awq_last_error.argtypes = []
    lib.awq_last_error.restype = ctypes.c_char_p
    lib.awq_abi_version.argtypes = []
    lib.awq_abi_version.restype = ctypes.c_int32
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libawq.so (loaded on first use; ImportError if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def _check(st: int) -> None:
    if st != AWQ_OK:
        raise AwqError(st, lib().awq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _tensor(t: Optional[torch.Tensor], name: str, dtype, shape=None, *, contiguous: bool = True,
            unit_col_stride: bool = False, min_numel: Optional[int] = None, like: Optional[torch.Tensor] = None,
            optional: bool = False) -> None:
    """Checks a tensor the library will read or write before anything is launched:
    dtype, shape (a tuple, entries None = any), layout (contiguous, or 2-D with
    unit column stride), size, and that it lives where `like` does.  That the
    tensors are on the device is checked once all of them passed (_dev).
    Raises ValueError."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and g != w for g, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            raise ValueError(f"{name} must have shape {want}, got {list(t.shape)}")
    if unit_col_stride:
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
            raise ValueError(f"{name} must be 2-D with unit column stride and rows at least a row apart")
    elif contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    if like is not None and t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, not on {like.device}")


def _x_dtype(X: torch.Tensor) -> int:
    if X.dtype == torch.bfloat16:
        return AWQ_BF16
    if X.dtype == torch.float16:
        return AWQ_F16
    raise ValueError(f"activations must be bf16 or fp16, got {X.dtype}")


def _rows_view(X: torch.Tensor, name: str):
    if X.dim() != 2 or (X.shape[1] > 1 and X.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    # a tensor of at most one row may report any row stride; its rows are never stepped over
    ld = X.stride(0) if X.shape[0] > 1 else max(X.stride(0), X.shape[1])
    return X.shape[0], X.shape[1], ld


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------
# Prepared calls: the ctypes argument tuple is built once; run() is one call
# into the library (no allocation, no size queries), so repeated use costs a
# few microseconds of host time.
# ---------------------------------------------------------------------------
class _Prepared:
    _fn = ""

    def _bind(self, *args) -> None:
        self._f = getattr(lib(), self._fn)
        self._args = args

    def launch(self) -> None:
        _check(self._f(*self._args))


def act_stats_workspace_bytes(T: int, d_in: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().awq_act_stats_workspace(T, d_in, ctypes.byref(n)))
    return n.value


class ActStatsPlan(_Prepared):
    """x_mean[i] (+)= inv_count * sum_t |X[t, i]| (inv_count defaults to 1/T)."""
    _fn = "awq_act_stats"

    def __init__(self, X: torch.Tensor, x_mean: Optional[torch.Tensor] = None, inv_count: Optional[float] = None,
                 accumulate: bool = False, ws: Optional[torch.Tensor] = None, stream=None):
        _tensor(X, "X", (torch.bfloat16, torch.float16), (None, None), unit_col_stride=True)
        T, d_in, ld = _rows_view(X, "X")
        _tensor(x_mean, "x_mean", torch.float32, (d_in,), like=X, optional=True)
        _tensor(ws, "ws", torch.uint8, (None,), like=X, optional=True)
        _dev(X, "X")
        self.x_mean = torch.empty(d_in, dtype=torch.float32, device=X.device) if x_mean is None else x_mean
        if inv_count is None:
            inv_count = 1.0 / T if T > 0 else 0.0
        need = act_stats_workspace_bytes(T, d_in)
        self.ws = workspace(need, X.device) if (ws is None or ws.numel() < need) else ws
        self._keep = (X,)
        self._bind(_ptr(X), _x_dtype(X), T, d_in, ld, inv_count, int(accumulate), _ptr(self.x_mean),
                   _ptr(self.ws), self.ws.numel(), _stream(stream))

    def run(self) -> torch.Tensor:
        self.launch()
        return self.x_mean


def act_stats(X: torch.Tensor, x_mean: Optional[torch.Tensor] = None, inv_count: Optional[float] = None,
              accumulate: bool = False, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """x_mean[i] (+)= inv_count * sum_t |X[t, i]| (inv_count defaults to 1/T)."""
    return ActStatsPlan(X, x_mean, inv_count, accumulate, ws, stream).run()


def candidate_scales(x_mean: torch.Tensor, n_grid: int = 20, s_min: float = 1e-4, stream=None) -> torch.Tensor:
    _tensor(x_mean, "x_mean", torch.float32, (None,))
    _dev(x_mean, "x_mean")
    d_in = x_mean.numel()
    S = torch.empty((n_grid, d_in), dtype=torch.float32, device=x_mean.device)
    n = ctypes.c_size_t()
    _check(lib().awq_candidate_scales_workspace(d_in, n_grid, ctypes.byref(n)))
    ws = workspace(n.value, x_mean.device)
    _check(lib().awq_candidate_scales(_ptr(x_mean), d_in, n_grid, s_min, _ptr(S), _ptr(ws), ws.numel(),
                                      _stream(stream)))
    return S


def _wgroup(parts):
    ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    rows = (ctypes.c_int64 * len(parts))(*[p.shape[0] for p in parts])
    return WGroup(len(parts), ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)),
                  ctypes.cast(rows, ctypes.POINTER(ctypes.c_int64))), (ptrs, rows)


def weight_channel_mean(W_parts: Sequence[torch.Tensor], stream=None) -> torch.Tensor:
    """Duo scaling's w_mean: row-normalised mean |w| per input channel of the
    group's concatenated rows (fp32 [d_in])."""
    parts = list(W_parts)
    for p in parts:
        _dev(p, "W")
        if p.dtype != torch.float16 or p.dim() != 2 or not p.is_contiguous() or p.shape[1] != parts[0].shape[1]:
            raise ValueError("weights must be contiguous fp16 [rows, d_in] with one d_in")
    d_in, dev = parts[0].shape[1], parts[0].device
    d_out = sum(p.shape[0] for p in parts)
    n = ctypes.c_size_t()
    _check(lib().awq_weight_channel_mean_workspace(d_out, d_in, ctypes.byref(n)))
    ws = workspace(n.value, dev)
    out = torch.empty(d_in, dtype=torch.float32, device=dev)
    grp, keep = _wgroup(parts)
    _check(lib().awq_weight_channel_mean(ctypes.byref(grp), d_in, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def candidate_scales_duo(x_mean: torch.Tensor, w_mean: torch.Tensor, n_grid: int = 20, s_min: float = 1e-4,
                         stream=None) -> torch.Tensor:
    """Duo-scaling candidate table S [n_grid, d_in]."""
    _tensor(x_mean, "x_mean", torch.float32, (None,))
    _tensor(w_mean, "w_mean", torch.float32, (x_mean.numel(),), like=x_mean)
    _dev(x_mean, "x_mean")
    d_in = x_mean.numel()
    S = torch.empty((n_grid, d_in), dtype=torch.float32, device=x_mean.device)
    n = ctypes.c_size_t()
    _check(lib().awq_candidate_scales_duo_workspace(d_in, n_grid, ctypes.byref(n)))
    ws = workspace(n.value, x_mean.device)
    _check(lib().awq_candidate_scales_duo(_ptr(x_mean), _ptr(w_mean), d_in, n_grid, s_min, _ptr(S), _ptr(ws),
                                          ws.numel(), _stream(stream)))
    return S


@dataclasses.dataclass
class SearchResult:
    err: torch.Tensor                 # fp32 [n_grid]
    best_idx: torch.Tensor            # int32 [1]
    best_s: torch.Tensor              # fp32 [d_in]
    clip: Optional[torch.Tensor]      # fp32 [d_out] or None
    clip_err: Optional[torch.Tensor]  # fp32 [d_out, n_clip] or None


def _cfg(group_size, n_grid, score, n_clip, clip_lo, s_min, duo=False, asym=False, out_form="auto") -> SearchCfg:
    sc = {"weight": AWQ_SCORE_WEIGHT, "output": AWQ_SCORE_OUTPUT}[score] if isinstance(score, str) else score
    if out_form not in _OUT_FORM:
        raise ValueError(f"out_form {out_form!r} not in {sorted(_OUT_FORM)}")
    flags = (AWQ_FLAG_DUO if duo else 0) | (AWQ_FLAG_ASYM if asym else 0) | _OUT_FORM[out_form]
    return SearchCfg(group_size, n_grid, sc, n_clip, s_min, clip_lo, flags)


def search_workspace_bytes(d_out: int, d_in: int, T: int = 0, *, group_size: int = 128, n_grid: int = 20,
                           score="weight", n_clip: int = 0, clip_lo: float = 0.5, s_min: float = 1e-4,
                           duo: bool = False, asym: bool = False, out_form: str = "auto") -> int:
    cfg = _cfg(group_size, n_grid, score, n_clip, clip_lo, s_min, duo, asym, out_form)
    n = ctypes.c_size_t()
    _check(lib().awq_search_workspace(ctypes.byref(cfg), d_out, d_in, T, ctypes.byref(n)))
    return n.value


def search_output_form(d_out: int, d_in: int, T: int, *, group_size: int = 128, n_grid: int = 20, n_clip: int = 0,
                       clip_lo: float = 0.5, s_min: float = 1e-4, duo: bool = False, asym: bool = False,
                       out_form: str = "auto") -> str:
    """The form the output-score alpha search takes for these arguments: "direct" or "gram"."""
    return search_output_forms(d_out, d_in, T, group_size=group_size, n_grid=n_grid, n_clip=n_clip,
                               clip_lo=clip_lo, s_min=s_min, duo=duo, asym=asym, out_form=out_form)[0]


def search_output_forms(d_out: int, d_in: int, T: int, *, group_size: int = 128, n_grid: int = 20, n_clip: int = 0,
                        clip_lo: float = 0.5, s_min: float = 1e-4, duo: bool = False, asym: bool = False,
                        out_form: str = "auto"):
    """(alpha search form, clip search form or None): "direct" or "gram" each."""
    cfg = _cfg(group_size, n_grid, "output", n_clip, clip_lo, s_min, duo, asym, out_form)
    f = ctypes.c_int32()
    _check(lib().awq_search_output_form(ctypes.byref(cfg), d_out, d_in, T, ctypes.byref(f)))
    return ("gram" if f.value & 1 else "direct",
            ("gram" if f.value & 2 else "direct") if n_clip >= 2 else None)


class SearchPlan(_Prepared):
    """Grid search of alpha for one group of linears sharing an input (rows concatenated).
    out_form (output score): "auto" (the library picks), "direct" (X times each candidate's
    dW) or "gram" (the second-moment form dW H dW^T with H = X^T X)."""
    _fn = "awq_search_scales"

    def __init__(self, W_parts: Sequence[torch.Tensor], x_mean: torch.Tensor, *, group_size: int = 128,
                 n_grid: int = 20, score="weight", X: Optional[torch.Tensor] = None, n_clip: int = 0,
                 clip_lo: float = 0.5, s_min: float = 1e-4, want_clip_err: bool = False,
                 ws: Optional[torch.Tensor] = None, out: Optional[SearchResult] = None, stream=None,
                 duo: bool = False, asym: bool = False, out_form: str = "auto"):
        parts: List[torch.Tensor] = list(W_parts)
        if not parts:
            raise ValueError("empty weight group")
        d_in = parts[0].shape[1]
        for p in parts:
            if p.dtype != torch.float16 or p.dim() != 2 or not p.is_contiguous() or p.shape[1] != d_in:
                raise ValueError("weights must be contiguous fp16 [rows, d_in] with one d_in")
        dev = parts[0].device
        for p in parts[1:]:
            if p.device != dev:
                raise ValueError("the parts of a group must live on one device")
        d_out = sum(p.shape[0] for p in parts)
        _tensor(x_mean, "x_mean", torch.float32, (d_in,), like=parts[0])
        self.cfg = _cfg(group_size, n_grid, score, n_clip, clip_lo, s_min, duo, asym, out_form)
        T, ld, xdt = 0, 0, AWQ_BF16
        if X is not None:
            _tensor(X, "X", (torch.bfloat16, torch.float16), (None, d_in), unit_col_stride=True, like=parts[0])
            T, dx, ld = _rows_view(X, "X")
            xdt = _x_dtype(X)
        if out is not None:
            _tensor(out.err, "out.err", torch.float32, (n_grid,), like=parts[0])
            _tensor(out.best_idx, "out.best_idx", torch.int32, (1,), like=parts[0])
            _tensor(out.best_s, "out.best_s", torch.float32, (d_in,), like=parts[0])
            _tensor(out.clip, "out.clip", torch.float32, (d_out,), like=parts[0], optional=not n_clip)
            _tensor(out.clip_err, "out.clip_err", torch.float32, (d_out, n_clip), like=parts[0], optional=True)
        _tensor(ws, "ws", torch.uint8, (None,), like=parts[0], optional=True)
        _dev(parts[0], "W")
        n = ctypes.c_size_t()
        _check(lib().awq_search_workspace(ctypes.byref(self.cfg), d_out, d_in, max(T, 1), ctypes.byref(n)))
        self.ws = workspace(n.value, dev) if (ws is None or ws.numel() < n.value) else ws
        if out is None:
            out = SearchResult(
                err=torch.empty(n_grid, dtype=torch.float32, device=dev),
                best_idx=torch.empty(1, dtype=torch.int32, device=dev),
                best_s=torch.empty(d_in, dtype=torch.float32, device=dev),
                clip=torch.empty(d_out, dtype=torch.float32, device=dev) if n_clip else None,
                clip_err=torch.empty((d_out, n_clip), dtype=torch.float32, device=dev)
                if (n_clip and want_clip_err) else None)
        self.out = out
        self._wptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
        self._rows = (ctypes.c_int64 * len(parts))(*[p.shape[0] for p in parts])
        self.grp = WGroup(len(parts), ctypes.cast(self._wptrs, ctypes.POINTER(ctypes.c_void_p)),
                          ctypes.cast(self._rows, ctypes.POINTER(ctypes.c_int64)))
        self._keep = (parts, x_mean, X)
        self._bind(ctypes.byref(self.cfg), ctypes.byref(self.grp), d_in, _ptr(x_mean), _ptr(X), xdt, T, ld,
                   _ptr(out.err), _ptr(out.best_idx), _ptr(out.best_s), _ptr(out.clip), _ptr(out.clip_err),
                   _ptr(self.ws), self.ws.numel(), _stream(stream))

    def run(self) -> SearchResult:
        self.launch()
        return self.out


def search_scales_noalloc(W_parts: Sequence[torch.Tensor], x_mean: torch.Tensor, out: SearchResult, *,
                          group_size: int = 128, n_grid: int = 20, s_min: float = 1e-4, duo: bool = False,
                          asym: bool = False, stream=None) -> SearchResult:
    """Weight-score search through awq_search_scales_noalloc: the library's own
    per-GPU scratch, no workspace, nothing allocated (the caller passes `out`).
    Calls that overlap on one GPU share that scratch and must not run concurrently."""
    parts: List[torch.Tensor] = list(W_parts)
    if not parts:
        raise ValueError("empty weight group")
    d_in = parts[0].shape[1]
    for p in parts:
        if p.dtype != torch.float16 or p.dim() != 2 or not p.is_contiguous() or p.shape[1] != d_in:
            raise ValueError("weights must be contiguous fp16 [rows, d_in] with one d_in")
        if p.device != parts[0].device:
            raise ValueError("the parts of a group must live on one device")
    _tensor(x_mean, "x_mean", torch.float32, (d_in,), like=parts[0])
    _tensor(out.err, "out.err", torch.float32, (n_grid,), like=parts[0])
    _tensor(out.best_idx, "out.best_idx", torch.int32, (1,), like=parts[0])
    _tensor(out.best_s, "out.best_s", torch.float32, (d_in,), like=parts[0])
    _dev(parts[0], "W")
    cfg = _cfg(group_size, n_grid, "weight", 0, 0.5, s_min, duo, asym)
    grp, keep = _wgroup(parts)
    _check(lib().awq_search_scales_noalloc(ctypes.byref(cfg), ctypes.byref(grp), d_in, _ptr(x_mean), _ptr(out.err),
                                           _ptr(out.best_idx), _ptr(out.best_s), _stream(stream)))
    return out


def search_scales(W_parts: Sequence[torch.Tensor], x_mean: torch.Tensor, **kw) -> SearchResult:
    """Grid search of alpha for one group of linears sharing an input (rows concatenated)."""
    return SearchPlan(W_parts, x_mean, **kw).run()


class PackPlan(_Prepared):
    """INT4 quantize + pack of W*s: qweight int32 [d_in, d_out/8], scales fp16 [d_in/G, d_out],
    qzeros int32 [d_in/G, d_out/8] (or None; always written for the asymmetric grid)."""
    _fn = "awq_quantize_pack"

    def __init__(self, W: torch.Tensor, group_size: int = 128, s: Optional[torch.Tensor] = None,
                 clip: Optional[torch.Tensor] = None, with_zeros: bool = True, out=None, stream=None,
                 asym: bool = False):
        if asym:
            self._fn = "awq_quantize_pack_asym"
            with_zeros = True
        _tensor(W, "W", torch.float16, (None, None))
        d_out, d_in = W.shape
        if group_size not in (32, 64, 128) or d_in % group_size or d_out % 8:
            raise ValueError(f"W [{d_out}, {d_in}]: need d_out % 8 == 0 and d_in a multiple of "
                             f"group_size in {{32, 64, 128}}, got {group_size}")
        _tensor(s, "s", torch.float32, (d_in,), like=W, optional=True)
        _tensor(clip, "clip", torch.float32, (d_out,), like=W, optional=True)
        if out is not None:
            qweight, scales, qzeros = out
            _tensor(qweight, "qweight", torch.int32, (d_in, d_out // 8), like=W)
            _tensor(scales, "scales", torch.float16, (d_in // group_size, d_out), like=W)
            _tensor(qzeros, "qzeros", torch.int32, (d_in // group_size, d_out // 8), like=W, optional=not asym)
        _dev(W, "W")
        if out is None:
            qweight = torch.empty((d_in, d_out // 8), dtype=torch.int32, device=W.device)
            scales = torch.empty((d_in // group_size, d_out), dtype=torch.float16, device=W.device)
            qzeros = torch.empty((d_in // group_size, d_out // 8), dtype=torch.int32, device=W.device) \
                if with_zeros else None
            out = (qweight, scales, qzeros)
        self.out = out
        self._keep = (W, s, clip)
        qweight, scales, qzeros = out
        self._bind(_ptr(W), d_out, d_in, group_size, _ptr(s), _ptr(clip), _ptr(qweight), _ptr(scales),
                   _ptr(qzeros), _stream(stream))

    def run(self):
        self.launch()
        return self.out


def quantize_pack(W: torch.Tensor, group_size: int = 128, s: Optional[torch.Tensor] = None,
                  clip: Optional[torch.Tensor] = None, with_zeros: bool = True, out=None, stream=None,
                  asym: bool = False):
    """Returns (qweight int32 [d_in, d_out/8], scales fp16 [d_in/G, d_out], qzeros int32 [d_in/G, d_out/8]);
    asym = True: the asymmetric grid with data zero points."""
    return PackPlan(W, group_size, s, clip, with_zeros, out, stream, asym).run()


class W4A16Plan(_Prepared):
    """Y [M, d_out] = X [M, d_in] (fp16, carrying the folded 1/s) times the
    dequantized packed weights, transposed (the decode GEMV)."""
    _fn = "awq_w4a16_matmul"

    def __init__(self, X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor,
                 qzeros: Optional[torch.Tensor], d_out: int, group_size: int = 128, out_dtype=torch.float16,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
        _tensor(X, "X", torch.float16, (None, None), unit_col_stride=True)
        M, d_in, ld = _rows_view(X, "X")
        if group_size not in (32, 64, 128) or d_in % group_size or d_out % 8:
            raise ValueError(f"need d_out % 8 == 0 and d_in ({d_in}) a multiple of group_size in "
                             f"{{32, 64, 128}}, got d_out {d_out}, group_size {group_size}")
        _tensor(qweight, "qweight", torch.int32, (d_in, d_out // 8), like=X)
        _tensor(scales, "scales", torch.float16, (d_in // group_size, d_out), like=X)
        _tensor(qzeros, "qzeros", torch.int32, (d_in // group_size, d_out // 8), like=X, optional=True)
        if out is not None:
            _tensor(out, "out", (torch.float16, torch.float32), (M, d_out), unit_col_stride=True, like=X)
        _tensor(ws, "ws", torch.uint8, (None,), like=X, optional=True)
        _dev(X, "X")
        n = ctypes.c_size_t()
        _check(lib().awq_w4a16_workspace(M, d_out, d_in, ctypes.byref(n)))
        self.ws = workspace(n.value, X.device) if (ws is None or ws.numel() < n.value) else ws
        self.out = torch.empty((M, d_out), dtype=out_dtype, device=X.device) if out is None else out
        ydt = {torch.float32: AWQ_F32, torch.float16: AWQ_F16}[self.out.dtype]
        self._keep = (X, qweight, scales, qzeros)
        self._bind(_ptr(X), M, ld, _ptr(qweight), _ptr(scales), _ptr(qzeros), d_out, d_in, group_size,
                   _ptr(self.out), self.out.stride(0), ydt, _ptr(self.ws), self.ws.numel(), _stream(stream))

    def run(self) -> torch.Tensor:
        self.launch()
        return self.out


def w4a16_matmul(X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, qzeros: Optional[torch.Tensor],
                 d_out: int, group_size: int = 128, out_dtype=torch.float16, stream=None) -> torch.Tensor:
    """Y = X W_hat^T on the packed layout (W_hat = (u - z) * scale in the stored domain)."""
    return W4A16Plan(X, qweight, scales, qzeros, d_out, group_size, out_dtype, stream=stream).run()


def unpack_dequant(qweight: torch.Tensor, scales: torch.Tensor, qzeros: Optional[torch.Tensor], d_out: int,
                   group_size: int = 128, s: Optional[torch.Tensor] = None, out_dtype=torch.float32,
                   stream=None) -> torch.Tensor:
    _tensor(qweight, "qweight", torch.int32, (None, d_out // 8))
    d_in = qweight.shape[0]
    if group_size not in (32, 64, 128) or d_in % group_size or d_out % 8:
        raise ValueError(f"need d_out % 8 == 0 and d_in ({d_in}) a multiple of group_size in "
                         f"{{32, 64, 128}}, got d_out {d_out}, group_size {group_size}")
    _tensor(scales, "scales", torch.float16, (d_in // group_size, d_out), like=qweight)
    _tensor(qzeros, "qzeros", torch.int32, (d_in // group_size, d_out // 8), like=qweight, optional=True)
    _tensor(s, "s", torch.float32, (d_in,), like=qweight, optional=True)
    _dev(qweight, "qweight")
    out = torch.empty((d_out, d_in), dtype=out_dtype, device=qweight.device)
    odt = {torch.float32: AWQ_F32, torch.float16: AWQ_F16}[out_dtype]
    _check(lib().awq_unpack_dequant(_ptr(qweight), _ptr(scales), _ptr(qzeros), d_out, d_in, group_size, _ptr(s),
                                    _ptr(out), odt, _stream(stream)))
    return out


class FoldPlan(_Prepared):
    """Shared scale of a norm group (per-channel geometric mean of the members'
    scales) and the norm folded with it (norm / s_shared in the norm's dtype)."""
    _fn = "awq_norm_group_fold"

    def __init__(self, s_members: Sequence[torch.Tensor], norm: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, s_shared: Optional[torch.Tensor] = None, stream=None):
        members = list(s_members)
        if not members:
            raise ValueError("no member scales")
        d_in = members[0].numel()
        for t in members:
            _dev(t, "s")
            if t.dtype != torch.float32 or t.numel() != d_in or not t.is_contiguous():
                raise ValueError("member scales must be contiguous fp32 [d_in] with one d_in")
        dev = members[0].device
        ndt = 0
        if norm is not None:
            _dev(norm, "norm")
            if norm.numel() != d_in or not norm.is_contiguous():
                raise ValueError("norm must be contiguous [d_in]")
            ndt = {torch.float16: AWQ_F16, torch.bfloat16: AWQ_BF16, torch.float32: AWQ_F32}[norm.dtype]
            if out is None:
                out = torch.empty_like(norm)
        self.s_shared = torch.empty(d_in, dtype=torch.float32, device=dev) if s_shared is None else s_shared
        self.norm_out = out
        self._sptrs = (ctypes.c_void_p * len(members))(*[t.data_ptr() for t in members])
        self._keep = (members, norm)
        self._bind(ctypes.cast(self._sptrs, ctypes.POINTER(ctypes.c_void_p)), len(members), d_in, _ptr(norm), ndt,
                   _ptr(out), _ptr(self.s_shared), _stream(stream))

    def run(self):
        self.launch()
        return self.s_shared, self.norm_out


def norm_group_fold(s_members: Sequence[torch.Tensor], norm: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, s_shared: Optional[torch.Tensor] = None, stream=None):
    """Returns (s_shared fp32 [d_in], norm_out or None): the geometric mean of the
    member scales and norm / s_shared (out may be norm itself, in place)."""
    return FoldPlan(s_members, norm, out, s_shared, stream).run()


def set_timing_events(before: Optional[int], after: Optional[int]) -> None:
    """Record raw hipEvent_t handles around the main kernel of every later call (None clears)."""
    _check(lib().awq_set_timing_events(before, after))


__all__ = ["set_timing_events", "ActStatsPlan", "SearchPlan", "search_scales_noalloc", "PackPlan", "FoldPlan", "norm_group_fold",
           "weight_channel_mean", "candidate_scales_duo", "W4A16Plan", "w4a16_matmul", "AwqError", "act_stats", "candidate_scales", "search_scales", "quantize_pack", "unpack_dequant",
           "search_workspace_bytes", "act_stats_workspace_bytes", "SearchResult", "lib", "LIB_PATH"]
