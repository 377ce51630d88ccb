"""Thin ctypes binding of libfa_varlen.so (argument marshalling only).

Every step of the backward runs in the library's HIP kernels; this module
only turns torch tensors (device memory) and host sequences into the C
structs of include/fa_varlen.h and passes the current HIP stream.  If the
library is missing, every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# FA_VARLEN_LIB may name another build of the same library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("FA_VARLEN_LIB") or os.path.join(_PKG, "lib", "libfa_varlen.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_NULLPTR, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_RUNTIME = 0, 1, 2, 3, 4
FA_MASK_NONE, FA_MASK_CAUSAL, FA_MASK_BAND = 0, 1, 2
FA_ITEMS_KEY_BLOCKS, FA_ITEMS_QUERY_BLOCKS = 0, 1

_DTYPE_CODE = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}


class FaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("tokens", ctypes.c_int64),
                ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64), ("stride_t", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class FaSeqlens(ctypes.Structure):
    _fields_ = [("cu", ctypes.POINTER(ctypes.c_int64)), ("batch", ctypes.c_int64)]


class FaMask(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("stride_q", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class FaWorkItem(ctypes.Structure):
    _fields_ = [("q_start", ctypes.c_int32), ("kv_start", ctypes.c_int32), ("len_q", ctypes.c_int32),
                ("len_kv", ctypes.c_int32), ("block", ctypes.c_int32), ("tile_begin", ctypes.c_int32),
                ("tile_end", ctypes.c_int32), ("seq", ctypes.c_int32), ("drop_base", ctypes.c_int64)]


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"fa_varlen status {status}: {message}")
        self.status = status


_lib = None

EXPORTS = ("fa_varlen_bwd", "fa_varlen_bwd_noalloc", "fa_varlen_bwd_masked", "fa_varlen_fwd", "fa_varlen_fwd_masked", "fa_last_error",
           "fa_release", "fa_varlen_worklist", "fa_profile_enable", "fa_profile_read")
KERNEL_NAMES = ("preprocess", "bwd_main", "unused", "bwd_dq", "fwd")


def load(path: Optional[str] = None):
    """Load (once) and return the ctypes handle of libfa_varlen.so; raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run `python -m variable_length_flashattention_fa_amd.csrc.build`")
    lib = ctypes.CDLL(p)
    T = ctypes.POINTER(FaTensor)
    S = ctypes.POINTER(FaSeqlens)
    lib.fa_varlen_bwd.argtypes = [T, T, T, T, T, ctypes.c_void_p, ctypes.c_void_p, S, S, ctypes.c_int32,
                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p,
                                  ctypes.c_double, ctypes.c_int64, T, T, T, ctypes.c_void_p]
    lib.fa_varlen_bwd.restype = ctypes.c_int
    lib.fa_varlen_bwd_noalloc.argtypes = lib.fa_varlen_bwd.argtypes
    lib.fa_varlen_bwd_noalloc.restype = ctypes.c_int
    lib.fa_varlen_fwd.argtypes = [T, T, T, S, S, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                  ctypes.c_void_p, ctypes.c_double, ctypes.c_int64, T, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_varlen_fwd.restype = ctypes.c_int
    M = ctypes.POINTER(FaMask)
    lib.fa_varlen_bwd_masked.argtypes = [T, T, T, T, T, ctypes.c_void_p, ctypes.c_void_p, S, S, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, M,
                                         ctypes.c_double, ctypes.c_int64, T, T, T, ctypes.c_void_p]
    lib.fa_varlen_bwd_masked.restype = ctypes.c_int
    lib.fa_varlen_fwd_masked.argtypes = [T, T, T, S, S, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_double, ctypes.c_void_p, M, ctypes.c_double, ctypes.c_int64, T,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.fa_varlen_fwd_masked.restype = ctypes.c_int
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_release.argtypes = []
    lib.fa_release.restype = None
    lib.fa_varlen_worklist.argtypes = [S, S, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(FaWorkItem),
                                       ctypes.c_int64]
    lib.fa_varlen_worklist.restype = ctypes.c_int64
    lib.fa_profile_enable.argtypes = [ctypes.c_int]
    lib.fa_profile_enable.restype = None
    lib.fa_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
    lib.fa_profile_read.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def last_error() -> str:
    return load().fa_last_error().decode()


def release() -> None:
    load().fa_release()


def tensor_desc(t: Optional[torch.Tensor]) -> Optional[FaTensor]:
    """TND view of a torch tensor (None -> None, so the library reports a null pointer)."""
    if t is None:
        return None
    if t.dim() != 3:
        raise ValueError("TND tensors must be 3-D")
    if t.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    if t.numel() and t.stride(2) != 1:
        raise ValueError("the head-dim stride must be 1")
    return FaTensor(ctypes.c_void_p(t.data_ptr() if t.numel() else 0), _DTYPE_CODE[t.dtype], t.shape[0],
                    t.shape[1], t.shape[2], t.stride(0), t.stride(1))


def mask_desc(m: Optional[torch.Tensor]) -> Optional[FaMask]:
    """fa_mask_t view of an explicit mask tensor (uint8 / bool, nonzero = excluded) of shape
    [B, N, Sq, Skv], [B, 1, Sq, Skv], [1, 1, Sq, Skv] or [Sq, Skv]; size-1 axes get stride 0."""
    if m is None:
        return None
    if m.dtype not in (torch.uint8, torch.bool):
        raise ValueError("atten_mask must be uint8 or bool")
    if m.dim() == 2:
        sb, sn, sq = 0, 0, m.stride(0)
    elif m.dim() == 4:
        sb = m.stride(0) if m.shape[0] > 1 else 0
        sn = m.stride(1) if m.shape[1] > 1 else 0
        sq = m.stride(2)
    else:
        raise ValueError("atten_mask must be 2-D [Sq, Skv] or 4-D [B|1, N|1, Sq, Skv]")
    if m.numel() and m.stride(-1) != 1:
        raise ValueError("the key stride of atten_mask must be 1")
    return FaMask(ctypes.c_void_p(m.data_ptr() if m.numel() else 0), sb, sn, sq, m.shape[-2], m.shape[-1])


def _seqlens(cu: Sequence[int]):
    arr = np.ascontiguousarray(np.asarray(cu, dtype=np.int64))
    return FaSeqlens(arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), arr.size - 1), arr


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_args(q, tensors: dict, stats: dict, cu_q, cu_kv, keep_prob, drop_mask, atten_mask) -> None:
    """Checks what the C ABI cannot see behind its raw pointers: every tensor lives on q's device,
    the statistics are [N, Tq, 8] fp32 and contiguous, the dropout mask holds enough bits and an
    explicit mask's batch and head axes are 1 or full.  Raises ValueError."""
    if q is None:
        return  # the library reports the null pointer
    for name, t in dict(tensors, **stats, drop_mask=drop_mask, atten_mask=atten_mask).items():
        if t is not None and (not t.is_cuda or t.device != q.device):
            raise ValueError(f"{name} must be a device tensor on {q.device}")
    heads, tq = q.shape[1], q.shape[0]
    for name, t in stats.items():
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (heads, tq, 8) or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 [N, Tq, 8] = [{heads}, {tq}, 8] tensor")
    lq = np.diff(np.asarray(cu_q, dtype=np.int64))
    lk = np.diff(np.asarray(cu_kv, dtype=np.int64))
    if drop_mask is not None and keep_prob < 1.0 and lq.size == lk.size:
        need = (int(np.sum(heads * lq * lk)) + 7) // 8
        if drop_mask.dtype != torch.uint8 or drop_mask.numel() < need:
            raise ValueError(f"drop_mask must be uint8 with at least {need} bytes")
    if atten_mask is not None and atten_mask.dim() == 4:
        if atten_mask.shape[0] not in (1, lq.size) or atten_mask.shape[1] not in (1, heads):
            raise ValueError("atten_mask axes must be [B or 1, N or 1, Sq, Skv]")


def _bwd(entry: str, q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
         pre_tokens, next_tokens, keep_prob, drop_mask, scale, head_num, dq, dk, dv, stream) -> None:
    lib = load()
    _check_args(q, dict(k=k, v=v, dy=dy, y=y, dq=dq, dk=dk, dv=dv), dict(softmax_max=softmax_max,
                softmax_sum=softmax_sum), cu_seqlens_q, cu_seqlens_kv, keep_prob, drop_mask, None)
    tq, tk, tv, tdy, ty = (tensor_desc(x) for x in (q, k, v, dy, y))
    tdq, tdk, tdv = (tensor_desc(x) for x in (dq, dk, dv))
    sq, aq = _seqlens(cu_seqlens_q)
    sk, ak = _seqlens(cu_seqlens_kv)
    for st in (softmax_max, softmax_sum):
        if st is not None and not st.is_contiguous():
            raise ValueError("softmax statistics must be contiguous [N, T, 8] fp32")
    stream = _stream(q, stream)

    def ref(x):
        return None if x is None else ctypes.byref(x)

    status = getattr(lib, entry)(ref(tq), ref(tk), ref(tv), ref(tdy), ref(ty), _ptr(softmax_max),
                                 _ptr(softmax_sum), ctypes.byref(sq), ctypes.byref(sk), int(atten_mode),
                                 int(pre_tokens), int(next_tokens), float(keep_prob), _ptr(drop_mask),
                                 float(scale), int(head_num), ref(tdq), ref(tdk), ref(tdv),
                                 ctypes.c_void_p(int(stream)))
    del aq, ak
    if status != FA_OK:
        raise FaError(status, last_error())


def fa_varlen_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dy: torch.Tensor, y: torch.Tensor,
                  softmax_max: torch.Tensor, softmax_sum: torch.Tensor, cu_seqlens_q, cu_seqlens_kv,
                  atten_mode: int, pre_tokens: int, next_tokens: int, keep_prob: float,
                  drop_mask: Optional[torch.Tensor], scale: float, head_num: int, dq: torch.Tensor,
                  dk: torch.Tensor, dv: torch.Tensor, stream=None) -> None:
    """Same arguments as the C entry point; tensors are device tensors, cu_seqlens host sequences.

    Enqueues the backward on `stream` (default: torch's current stream) and
    raises FaError on a non-OK status.
    """
    _bwd("fa_varlen_bwd", q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
         pre_tokens, next_tokens, keep_prob, drop_mask, scale, head_num, dq, dk, dv, stream)


def fa_varlen_bwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dy: torch.Tensor,
                          y: torch.Tensor, softmax_max: torch.Tensor, softmax_sum: torch.Tensor, cu_seqlens_q,
                          cu_seqlens_kv, atten_mode: int, pre_tokens: int, next_tokens: int, keep_prob: float,
                          drop_mask: Optional[torch.Tensor], scale: float, head_num: int, dq: torch.Tensor,
                          dk: torch.Tensor, dv: torch.Tensor, stream=None) -> None:
    """The C entry point of the same name (no device allocation); conventions of fa_varlen_bwd."""
    _bwd("fa_varlen_bwd_noalloc", q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv,
         atten_mode, pre_tokens, next_tokens, keep_prob, drop_mask, scale, head_num, dq, dk, dv, stream)


def fa_varlen_bwd_masked(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv,
                         atten_mode: int, pre_tokens: int, next_tokens: int, keep_prob: float,
                         drop_mask: Optional[torch.Tensor], atten_mask: Optional[torch.Tensor], scale: float,
                         head_num: int, dq, dk, dv, stream=None) -> None:
    """fa_varlen_bwd with an explicit mask tensor (see mask_desc); same conventions."""
    lib = load()
    _check_args(q, dict(k=k, v=v, dy=dy, y=y, dq=dq, dk=dk, dv=dv), dict(softmax_max=softmax_max,
                softmax_sum=softmax_sum), cu_seqlens_q, cu_seqlens_kv, keep_prob, drop_mask, atten_mask)
    tq, tk, tv, tdy, ty = (tensor_desc(x) for x in (q, k, v, dy, y))
    tdq, tdk, tdv = (tensor_desc(x) for x in (dq, dk, dv))
    tm = mask_desc(atten_mask)
    sq, aq = _seqlens(cu_seqlens_q)
    sk, ak = _seqlens(cu_seqlens_kv)
    for st in (softmax_max, softmax_sum):
        if st is not None and not st.is_contiguous():
            raise ValueError("softmax statistics must be contiguous [N, T, 8] fp32")
    stream = _stream(q, stream)

    def ref(x):
        return None if x is None else ctypes.byref(x)

    status = lib.fa_varlen_bwd_masked(ref(tq), ref(tk), ref(tv), ref(tdy), ref(ty), _ptr(softmax_max),
                                      _ptr(softmax_sum), ctypes.byref(sq), ctypes.byref(sk), int(atten_mode),
                                      int(pre_tokens), int(next_tokens), float(keep_prob), _ptr(drop_mask), ref(tm),
                                      float(scale), int(head_num), ref(tdq), ref(tdk), ref(tdv),
                                      ctypes.c_void_p(int(stream)))
    del aq, ak
    if status != FA_OK:
        raise FaError(status, last_error())


def _stream(q, stream):
    if stream is None:
        return torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def varlen_bwd(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, *,
               atten_mode: int = FA_MASK_NONE, pre_tokens: int = 0, next_tokens: int = 0,
               keep_prob: float = 1.0, drop_mask=None, scale: Optional[float] = None, head_num=None,
               atten_mask=None):
    """Convenience wrapper: allocates dq, dk, dv like q, k, v and returns them."""
    if scale is None:
        scale = 1.0 / float(q.shape[2]) ** 0.5
    if head_num is None:
        head_num = q.shape[1]
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if atten_mask is None:
        fa_varlen_bwd(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
                      pre_tokens, next_tokens, keep_prob, drop_mask, scale, head_num, dq, dk, dv)
    else:
        fa_varlen_bwd_masked(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
                             pre_tokens, next_tokens, keep_prob, drop_mask, atten_mask, scale, head_num, dq, dk, dv)
    return dq, dk, dv


def fa_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q, cu_seqlens_kv,
                  atten_mode: int, pre_tokens: int, next_tokens: int, keep_prob: float,
                  drop_mask: Optional[torch.Tensor], scale: float, head_num: int, y: torch.Tensor,
                  softmax_max: torch.Tensor, softmax_sum: torch.Tensor, stream=None) -> None:
    """Same arguments as the C entry point; tensors are device tensors, cu_seqlens host sequences.

    Enqueues the forward on `stream` (default: torch's current stream) and raises FaError on a
    non-OK status.
    """
    lib = load()
    _check_args(q, dict(k=k, v=v, y=y), dict(softmax_max=softmax_max, softmax_sum=softmax_sum), cu_seqlens_q,
                cu_seqlens_kv, keep_prob, drop_mask, None)
    tq, tk, tv, ty = (tensor_desc(x) for x in (q, k, v, y))
    sq, aq = _seqlens(cu_seqlens_q)
    sk, ak = _seqlens(cu_seqlens_kv)
    for st in (softmax_max, softmax_sum):
        if st is not None and not st.is_contiguous():
            raise ValueError("softmax statistics must be contiguous [N, T, 8] fp32")
    stream = _stream(q, stream)

    def ref(x):
        return None if x is None else ctypes.byref(x)

    status = lib.fa_varlen_fwd(ref(tq), ref(tk), ref(tv), ctypes.byref(sq), ctypes.byref(sk), int(atten_mode),
                               int(pre_tokens), int(next_tokens), float(keep_prob), _ptr(drop_mask), float(scale),
                               int(head_num), ref(ty), _ptr(softmax_max), _ptr(softmax_sum),
                               ctypes.c_void_p(int(stream)))
    del aq, ak
    if status != FA_OK:
        raise FaError(status, last_error())


def fa_varlen_fwd_masked(q, k, v, cu_seqlens_q, cu_seqlens_kv, atten_mode: int, pre_tokens: int,
                         next_tokens: int, keep_prob: float, drop_mask: Optional[torch.Tensor],
                         atten_mask: Optional[torch.Tensor], scale: float, head_num: int, y, softmax_max,
                         softmax_sum, stream=None) -> None:
    """fa_varlen_fwd with an explicit mask tensor (see mask_desc); same conventions."""
    lib = load()
    _check_args(q, dict(k=k, v=v, y=y), dict(softmax_max=softmax_max, softmax_sum=softmax_sum), cu_seqlens_q,
                cu_seqlens_kv, keep_prob, drop_mask, atten_mask)
    tq, tk, tv, ty = (tensor_desc(x) for x in (q, k, v, y))
    tm = mask_desc(atten_mask)
    sq, aq = _seqlens(cu_seqlens_q)
    sk, ak = _seqlens(cu_seqlens_kv)
    for st in (softmax_max, softmax_sum):
        if st is not None and not st.is_contiguous():
            raise ValueError("softmax statistics must be contiguous [N, T, 8] fp32")
    stream = _stream(q, stream)

    def ref(x):
        return None if x is None else ctypes.byref(x)

    status = lib.fa_varlen_fwd_masked(ref(tq), ref(tk), ref(tv), ctypes.byref(sq), ctypes.byref(sk),
                                      int(atten_mode), int(pre_tokens), int(next_tokens), float(keep_prob),
                                      _ptr(drop_mask), ref(tm), float(scale), int(head_num), ref(ty),
                                      _ptr(softmax_max), _ptr(softmax_sum), ctypes.c_void_p(int(stream)))
    del aq, ak
    if status != FA_OK:
        raise FaError(status, last_error())


def varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_kv, *, atten_mode: int = FA_MASK_NONE, pre_tokens: int = 0,
               next_tokens: int = 0, keep_prob: float = 1.0, drop_mask=None, scale: Optional[float] = None,
               head_num=None, atten_mask=None):
    """Convenience wrapper: allocates y like q and the [N, T, 8] statistics; returns (y, max, sum)."""
    if scale is None:
        scale = 1.0 / float(q.shape[2]) ** 0.5
    if head_num is None:
        head_num = q.shape[1]
    y = torch.empty(q.shape[0], q.shape[1], v.shape[2], dtype=q.dtype, device=q.device)
    smax = torch.empty(q.shape[1], q.shape[0], 8, dtype=torch.float32, device=q.device)
    ssum = torch.empty_like(smax)
    if atten_mask is None:
        fa_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_kv, atten_mode, pre_tokens, next_tokens, keep_prob,
                      drop_mask, scale, head_num, y, smax, ssum)
    else:
        fa_varlen_fwd_masked(q, k, v, cu_seqlens_q, cu_seqlens_kv, atten_mode, pre_tokens, next_tokens, keep_prob,
                             drop_mask, atten_mask, scale, head_num, y, smax, ssum)
    return y, smax, ssum


def worklist(cu_seqlens_q, cu_seqlens_kv, atten_mode: int, pre_tokens: int, next_tokens: int, heads: int,
             kind: int, block_rows: int, tile_rows: int):
    """A host work list (FA_ITEMS_KEY_BLOCKS or FA_ITEMS_QUERY_BLOCKS) as a list of dicts."""
    lib = load()
    sq, aq = _seqlens(cu_seqlens_q)
    sk, ak = _seqlens(cu_seqlens_kv)
    args = (ctypes.byref(sq), ctypes.byref(sk), int(atten_mode), int(pre_tokens), int(next_tokens), int(heads),
            int(kind), int(block_rows), int(tile_rows))
    n = lib.fa_varlen_worklist(*args, None, 0)
    if n < 0:
        raise FaError(-n, last_error())
    buf = (FaWorkItem * max(n, 1))()
    lib.fa_varlen_worklist(*args, buf, n)
    del aq, ak
    return [{f: getattr(buf[i], f) for f, _ in FaWorkItem._fields_} for i in range(n)]


def profile_enable(on: bool = True) -> None:
    """Record HIP events around each library kernel on the call's stream."""
    load().fa_profile_enable(1 if on else 0)


def profile_read() -> dict:
    """{kernel name: (summed ms, launches)} since the last read; clears the record."""
    k = len(KERNEL_NAMES)
    ms = (ctypes.c_double * k)()
    cnt = (ctypes.c_int64 * k)()
    n = load().fa_profile_read(ms, cnt, k)
    if n < 0:
        raise FaError(-n, last_error())
    return {KERNEL_NAMES[i]: (ms[i], cnt[i]) for i in range(min(n, k))}

