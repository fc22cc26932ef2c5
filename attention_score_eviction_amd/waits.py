"""Python binding of libwaits.so (include/waits.h): argument marshalling only.

Every step of the path runs in the HIP library; this module turns torch
tensors into pointers, strides and the caller's current HIP stream, and
raises ``WaitsError`` on a nonzero status.  There is no fallback: if the
library is not built, every call raises.

Calls that take a ``workspace`` allocate one of the size the matching
``*_workspace_bytes`` query returns when none is given; a caller's workspace
is passed as it is, and the library rejects one that is too small
(``WaitsError`` with status WAITS_EWORKSPACE), so a call with its workspace
makes no separate size query.

Layouts (token-major packed batch, positions restart per sequence):
  q [T, Hq, d], k / v [T, Hkv, d]  (any strides with d contiguous)
  lse [Hq, T] fp32, scores [Hkv, T] fp32
  idx [B, Hkv, budget] int32, k_out / v_out [B, Hkv, budget, d]
Decode over the compacted cache (dense):
  q [B, Hq, d], k_cache / v_cache [B, Hkv, capacity, d], lens [B] int32,
  out [B, Hq, d] fp32, lse [B, Hq] fp32
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from typing import Optional, Sequence, Union

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwaits.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "waits.h")

WAITS_OK, WAITS_EINVAL, WAITS_EUNSUPPORTED, WAITS_EWORKSPACE, WAITS_EDEVICE, WAITS_ESCRATCH = range(6)
STATIC_SCRATCH_BYTES = 16 << 20  # WAITS_STATIC_SCRATCH_BYTES
WAITS_BF16, WAITS_F32 = 0, 1
WAITS_PASS2_AUTO, WAITS_PASS2_KEY_BLOCKS = 0, 1
_PASS2 = {"auto": WAITS_PASS2_AUTO, "key_blocks": WAITS_PASS2_KEY_BLOCKS}


class WaitsError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {strerror(code)} (status {code})")
        self.code = code


class WaitsShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("cu_seqlens", ctypes.POINTER(ctypes.c_int64)),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("kv_stride_tok", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("pass2", ctypes.c_int32),
    ]


class WaitsDecodeShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


_lib = None
_P = ctypes.c_void_p
_SP = ctypes.POINTER(WaitsShape)
_DSP = ctypes.POINTER(WaitsDecodeShape)
_FP = ctypes.POINTER(ctypes.c_float)
_IP = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "waits_first_rows": [_SP, _FP, _IP, _IP],
    "waits_lse_workspace_bytes": [_SP, _FP, _IP, ctypes.POINTER(ctypes.c_size_t)],
    "waits_score_workspace_bytes": [_SP, _FP, _IP, ctypes.POINTER(ctypes.c_size_t)],
    "waits_lse": [_SP, _P, _P, _FP, _IP, _P, _P, ctypes.c_size_t, _P],
    "waits_colsum_workspace_bytes": [_SP, _FP, _IP, ctypes.POINTER(ctypes.c_size_t)],
    "waits_colsum": [_SP, _P, _P, _P, _FP, _IP, _P, _P, ctypes.c_size_t, _P],
    "waits_score": [_SP, _P, _P, _FP, _IP, _P, _P, ctypes.c_size_t, _P],
    "waits_select": [_SP, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P],
    "waits_select_workspace_bytes": [_SP, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "waits_compact": [_SP, _P, _P, _P, ctypes.c_int32, _P, _P, _P],
    "waits_select_compact": [_SP, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "waits_select_compact_noalloc": [_SP, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P],
    "waits_attention": [_SP, _P, _P, _P, _P, _P, _P],
    "waits_decode_workspace_bytes": [_DSP, ctypes.POINTER(ctypes.c_size_t)],
    "waits_decode": [_DSP, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m attention_score_eviction_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        handle.waits_strerror.argtypes = [ctypes.c_int]
        handle.waits_strerror.restype = ctypes.c_char_p
        _lib = handle
    return _lib


def header_symbols() -> list:
    """Entry points declared in include/waits.h."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(waits_\w+)\s*\(", text, re.M)))


def strerror(code: int) -> str:
    return lib().waits_strerror(int(code)).decode()


def _check(fn: str, rc: int) -> None:
    if rc != WAITS_OK:
        raise WaitsError(fn, rc)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


class _Marshal:
    """Host-side argument block for one call (keeps the host arrays alive)."""

    def __init__(self, cu_seqlens, q: Optional[torch.Tensor], kv: torch.Tensor,
                 scale: Optional[float], a=None, b=None, n_q_heads: Optional[int] = None,
                 pass2: str = "auto"):
        self.cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        batch = len(self.cu) - 1
        if kv.dtype == torch.bfloat16:
            dt = WAITS_BF16
        elif kv.dtype == torch.float32:
            dt = WAITS_F32
        else:
            raise TypeError(f"K/V must be bfloat16 or float32, got {kv.dtype}")
        if q is not None and q.dtype != kv.dtype:
            raise TypeError("Q and K must share a dtype")
        d = kv.shape[-1]
        self.shape = WaitsShape()
        self.shape.batch = batch
        self.shape.cu_seqlens = self.cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        self.shape.n_kv_heads = kv.shape[1]
        self.shape.n_q_heads = q.shape[1] if q is not None else (n_q_heads or kv.shape[1])
        self.shape.head_dim = d
        self.shape.dtype = dt
        self.shape.kv_stride_tok, self.shape.kv_stride_head = kv.stride(0), kv.stride(1)
        if q is not None:
            self.shape.q_stride_tok, self.shape.q_stride_head = q.stride(0), q.stride(1)
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        self.shape.scale = float(scale)
        if pass2 not in _PASS2:
            raise ValueError(f"pass2 must be one of {sorted(_PASS2)}, got {pass2!r}")
        self.shape.pass2 = _PASS2[pass2]
        self.a = self.b = None
        if a is not None:
            self.a = _per_seq(a, np.float32, batch)
            self.b = _per_seq(b, np.int32, batch)

    @property
    def sp(self):
        return ctypes.byref(self.shape)

    @property
    def ap(self):
        return self.a.ctypes.data_as(_FP)

    @property
    def bp(self):
        return self.b.ctypes.data_as(_IP)


def _per_seq(x, dtype, batch: int) -> np.ndarray:
    """One value per sequence, from a scalar or a length-batch sequence."""
    arr = np.asarray(x, dtype)
    if arr.ndim == 0:
        return np.full(batch, arr, dtype)
    return np.ascontiguousarray(np.broadcast_to(arr, (batch,)))


def _size_query(fn: str, *args) -> int:
    out = ctypes.c_size_t(0)
    _check(fn, getattr(lib(), fn)(*args, ctypes.byref(out)))
    return out.value


def _ws_args(ws: Optional[torch.Tensor]):
    """Pointer and byte size of a workspace tensor (the library checks the
    size against what the call needs and returns WAITS_EWORKSPACE if short)."""
    if ws is None:
        return ctypes.c_void_p(0), ctypes.c_size_t(0)
    return ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size())


def _last_dim_contiguous(*ts):
    for t in ts:
        if t is not None and t.stride(-1) != 1:
            raise ValueError("the head_dim axis must be contiguous")


def first_rows(cu_seqlens, a, b) -> np.ndarray:
    """First processed query row of every sequence (host-only query)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    nb = len(cu) - 1
    shape = WaitsShape()
    shape.batch = nb
    shape.cu_seqlens = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    a32 = np.ascontiguousarray(np.broadcast_to(np.asarray(a, np.float32), (nb,)))
    b32 = np.ascontiguousarray(np.broadcast_to(np.asarray(b, np.int32), (nb,)))
    out = np.zeros(nb, dtype=np.int32)
    _check("waits_first_rows", lib().waits_first_rows(
        ctypes.byref(shape), a32.ctypes.data_as(_FP), b32.ctypes.data_as(_IP),
        out.ctypes.data_as(_IP)))
    return out


def lse_workspace_bytes(q, k, cu_seqlens, a, b, scale=None, pass2: str = "auto") -> int:
    m = _Marshal(cu_seqlens, q, k, scale, a, b, pass2=pass2)
    return _size_query("waits_lse_workspace_bytes", m.sp, m.ap, m.bp)


def colsum_workspace_bytes(q, k, cu_seqlens, a, b, scale=None, pass2: str = "auto") -> int:
    m = _Marshal(cu_seqlens, q, k, scale, a, b, pass2=pass2)
    return _size_query("waits_colsum_workspace_bytes", m.sp, m.ap, m.bp)


def score_workspace_bytes(q, k, cu_seqlens, a, b, scale=None, pass2: str = "auto") -> int:
    m = _Marshal(cu_seqlens, q, k, scale, a, b, pass2=pass2)
    return _size_query("waits_score_workspace_bytes", m.sp, m.ap, m.bp)


def _workspace(query, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    """The caller's workspace as given (the library checks its size), or, if
    there is none, a new one of the size ``query()`` returns (None if 0)."""
    if workspace is not None:
        return workspace
    nbytes = query()
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def lse(q: torch.Tensor, k: torch.Tensor, cu_seqlens, a, b, scale=None,
        out: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Pass 1: per-row natural-log normaliser, [Hq, T] fp32 (processed rows)."""
    _last_dim_contiguous(q, k)
    m = _Marshal(cu_seqlens, q, k, scale, a, b)
    if out is None:
        out = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    ws = _workspace(lambda: _size_query("waits_lse_workspace_bytes", m.sp, m.ap, m.bp), q.device, workspace)
    _check("waits_lse", lib().waits_lse(
        m.sp, _ptr(q), _ptr(k), m.ap, m.bp, _ptr(out), *_ws_args(ws), _stream(q)))
    return out


def colsum(q: torch.Tensor, k: torch.Tensor, lse_rows: torch.Tensor, cu_seqlens, a, b,
           scale=None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, pass2: str = "auto") -> torch.Tensor:
    """Pass 2: WAITS key scores [Hkv, T] fp32 from the pass-1 normalisers.
    ``pass2`` picks the plan of long sequences: "auto" or "key_blocks"."""
    _last_dim_contiguous(q, k)
    m = _Marshal(cu_seqlens, q, k, scale, a, b, pass2=pass2)
    if out is None:
        out = torch.empty((k.shape[1], k.shape[0]), dtype=torch.float32, device=k.device)
    ws = _workspace(lambda: _size_query("waits_colsum_workspace_bytes", m.sp, m.ap, m.bp), q.device,
                    workspace)
    _check("waits_colsum", lib().waits_colsum(
        m.sp, _ptr(q), _ptr(k), _ptr(lse_rows), m.ap, m.bp, _ptr(out), *_ws_args(ws), _stream(q)))
    return out


def score(q: torch.Tensor, k: torch.Tensor, cu_seqlens, a, b, scale=None,
          out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None, pass2: str = "auto") -> torch.Tensor:
    """Both passes: WAITS key scores [Hkv, T] fp32 (``pass2`` as in colsum)."""
    _last_dim_contiguous(q, k)
    m = _Marshal(cu_seqlens, q, k, scale, a, b, pass2=pass2)
    if out is None:
        out = torch.empty((k.shape[1], k.shape[0]), dtype=torch.float32, device=k.device)
    ws = _workspace(lambda: _size_query("waits_score_workspace_bytes", m.sp, m.ap, m.bp), q.device,
                    workspace)
    _check("waits_score", lib().waits_score(
        m.sp, _ptr(q), _ptr(k), m.ap, m.bp, _ptr(out), *_ws_args(ws), _stream(q)))
    return out


def _select_shape(cu_seqlens, hkv: int):
    cu_c = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    shape = WaitsShape()
    shape.batch = len(cu_c) - 1
    shape.cu_seqlens = cu_c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    shape.n_kv_heads = hkv
    shape.n_q_heads = hkv
    return shape, cu_c


def select_workspace_bytes(cu_seqlens, hkv: int, budget: int) -> int:
    shape, _keep = _select_shape(cu_seqlens, hkv)
    return _size_query("waits_select_workspace_bytes", ctypes.byref(shape), int(budget))


def select(scores: torch.Tensor, cu_seqlens, budget: int,
           out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-``budget`` key positions per (sequence, KV head), ascending, -1 padded."""
    hkv = scores.shape[0]
    shape, cu_c = _select_shape(cu_seqlens, hkv)
    if out is None:
        out = torch.empty((len(cu_c) - 1, hkv, int(budget)), dtype=torch.int32,
                          device=scores.device)
    ws = _workspace(lambda: _size_query("waits_select_workspace_bytes", ctypes.byref(shape), int(budget)),
                    scores.device, workspace)
    _check("waits_select", lib().waits_select(
        ctypes.byref(shape), _ptr(scores), int(budget), _ptr(out), *_ws_args(ws), _stream(scores)))
    return out


def compact(k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, cu_seqlens, budget: int,
            k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None):
    """Gather the selected K/V rows into [B, Hkv, budget, d] (bit-exact)."""
    _last_dim_contiguous(k, v)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    m = _Marshal(cu_seqlens, None, k, 1.0)
    nb, hkv, d = len(m.cu) - 1, k.shape[1], k.shape[2]
    if k_out is None:
        k_out = torch.empty((nb, hkv, int(budget), d), dtype=k.dtype, device=k.device)
    if v_out is None:
        v_out = torch.empty((nb, hkv, int(budget), d), dtype=v.dtype, device=v.device)
    _check("waits_compact", lib().waits_compact(
        m.sp, _ptr(k), _ptr(v), _ptr(idx), int(budget), _ptr(k_out), _ptr(v_out), _stream(k)))
    return k_out, v_out


def select_compact(scores: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens,
                   budget: int, idx: Optional[torch.Tensor] = None,
                   k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None):
    """select() then compact() in one launch: (idx, k_out, v_out)."""
    _last_dim_contiguous(k, v)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    m = _Marshal(cu_seqlens, None, k, 1.0)
    nb, hkv, d = len(m.cu) - 1, k.shape[1], k.shape[2]
    if scores.shape[0] != hkv:
        raise ValueError("scores must be [n_kv_heads, T]")
    if idx is None:
        idx = torch.empty((nb, hkv, int(budget)), dtype=torch.int32, device=k.device)
    if k_out is None:
        k_out = torch.empty((nb, hkv, int(budget), d), dtype=k.dtype, device=k.device)
    if v_out is None:
        v_out = torch.empty((nb, hkv, int(budget), d), dtype=v.dtype, device=v.device)
    ws = _workspace(lambda: _size_query("waits_select_workspace_bytes", m.sp, int(budget)), k.device,
                    workspace)
    _check("waits_select_compact", lib().waits_select_compact(
        m.sp, _ptr(scores), _ptr(k), _ptr(v), int(budget), _ptr(idx), _ptr(k_out), _ptr(v_out),
        *_ws_args(ws), _stream(k)))
    return idx, k_out, v_out


def select_compact_noalloc(scores: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens,
                           budget: int, idx: torch.Tensor, k_out: torch.Tensor, v_out: torch.Tensor):
    """select_compact() with no workspace: the library's static per-GPU
    scratch serves the select of long heads (calls on one GPU must not
    overlap).  The outputs are the caller's; nothing is allocated."""
    _last_dim_contiguous(k, v)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    m = _Marshal(cu_seqlens, None, k, 1.0)
    if scores.shape[0] != k.shape[1]:
        raise ValueError("scores must be [n_kv_heads, T]")
    _check("waits_select_compact_noalloc", lib().waits_select_compact_noalloc(
        m.sp, _ptr(scores), _ptr(k), _ptr(v), int(budget), _ptr(idx), _ptr(k_out), _ptr(v_out),
        _stream(k)))
    return idx, k_out, v_out


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens, scale=None,
              out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
              want_lse: bool = True):
    """Causal prefill attention with the row log-sum-exp: (out, lse).

    q [T, Hq, d], k / v [T, Hkv, d] bf16 (K and V share strides); out bf16
    [T, Hq, d] dense; lse fp32 [Hq, T], the same values lse() writes."""
    _last_dim_contiguous(q, k, v)
    if k.stride() != v.stride():
        raise ValueError("K and V must share strides")
    m = _Marshal(cu_seqlens, q, k, scale)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be a dense tensor shaped and typed like q")
    if lse is None and want_lse:
        lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
    _check("waits_attention", lib().waits_attention(
        m.sp, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def score_select_compact(q, k, v, cu_seqlens, a, b, budget, scale=None, pass2: str = "auto"):
    """The whole path: scores, kept positions and the compacted K/V."""
    s = score(q, k, cu_seqlens, a, b, scale, pass2=pass2)
    idx, kc, vc = select_compact(s, k, v, cu_seqlens, budget)
    return s, idx, kc, vc


def _decode_shape(q: torch.Tensor, k_cache: torch.Tensor, scale=None) -> WaitsDecodeShape:
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B, Hq, d] and the caches [B, Hkv, capacity, d]")
    if k_cache.dtype == torch.bfloat16:
        dt = WAITS_BF16
    elif k_cache.dtype == torch.float32:
        dt = WAITS_F32
    else:
        raise TypeError(f"caches must be bfloat16 or float32, got {k_cache.dtype}")
    if q.dtype != k_cache.dtype:
        raise TypeError("q and the caches must share a dtype")
    if q.shape[0] != k_cache.shape[0] or q.shape[2] != k_cache.shape[3]:
        raise ValueError("q and the caches disagree on batch or head_dim")
    sh = WaitsDecodeShape()
    sh.batch, sh.n_q_heads, sh.head_dim = q.shape[0], q.shape[1], q.shape[2]
    sh.n_kv_heads, sh.capacity = k_cache.shape[1], k_cache.shape[2]
    sh.dtype = dt
    sh.scale = 1.0 / math.sqrt(q.shape[2]) if scale is None else float(scale)
    return sh


def decode_workspace_bytes(q: torch.Tensor, k_cache: torch.Tensor, scale=None) -> int:
    """Device workspace bytes decode() needs for these shapes."""
    sh = _decode_shape(q, k_cache, scale)
    n = ctypes.c_size_t(0)
    _check("waits_decode_workspace_bytes", lib().waits_decode_workspace_bytes(ctypes.byref(sh), ctypes.byref(n)))
    return int(n.value)


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, lens: torch.Tensor,
           scale=None, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, want_lse: bool = True):
    """One decoding step's attention over the (compacted) cache: (out, lse).

    q [B, Hq, d]; k_cache / v_cache [B, Hkv, capacity, d] dense (the layout
    compact() returns); lens int32 [B] on the device (rows attended per
    sequence).  out fp32 [B, Hq, d]; lse fp32 [B, Hq] (None if not wanted)."""
    for t in (q, k_cache, v_cache):
        if not t.is_contiguous():
            raise ValueError("q and the caches must be dense (contiguous)")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("k_cache and v_cache must share shape and dtype")
    if lens.dtype != torch.int32 or lens.shape != (q.shape[0],) or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 tensor of shape [B]")
    sh = _decode_shape(q, k_cache, scale)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], q.shape[2]), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    ws = _workspace(lambda: _size_query("waits_decode_workspace_bytes", ctypes.byref(sh)), q.device, workspace)
    _check("waits_decode", lib().waits_decode(
        ctypes.byref(sh), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), _ptr(out), _ptr(lse),
        *_ws_args(ws), _stream(q)))
    return out, lse
