"""C ABI checks that need no GPU: exported symbols and every validation path.

All validation returns before any device work, so these calls run on the CPU
with fake (never dereferenced) device addresses.
"""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

from variable_length_flashattention_fa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16-byte aligned, never dereferenced


def _header_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                             text, flags=re.M):
            names.add(m.group(1))
    return names


def test_library_exports_every_header_function():
    lib = B.load()
    names = _header_functions()
    assert {"fa_varlen_bwd", "fa_varlen_bwd_masked", "fa_varlen_fwd", "fa_varlen_fwd_masked", "fa_last_error",
            "fa_release", "fa_varlen_worklist"} <= names
    for n in names:
        assert hasattr(lib, n), n


def _t(tokens, heads=2, dim=64, dtype=B.FA_BF16, data=FAKE):
    return B.FaTensor(ctypes.c_void_p(data), dtype, tokens, heads, dim, heads * dim, dim)


def _call(q=None, k=None, v=None, dy=None, y=None, smax=FAKE, ssum=FAKE, cu_q=(0, 10), cu_kv=(0, 10),
          mode=0, pre=0, nxt=0, kp=1.0, drop=None, scale=0.125, head_num=2, dq=None, dk=None, dv=None,
          entry="fa_varlen_bwd"):
    tq = cu_q[-1]
    tk = cu_kv[-1]
    q = q if q is not None else _t(tq)
    k = k if k is not None else _t(tk)
    v = v if v is not None else _t(tk)
    dy = dy if dy is not None else _t(tq)
    y = y if y is not None else _t(tq)
    dq = dq if dq is not None else _t(tq)
    dk = dk if dk is not None else _t(tk)
    dv = dv if dv is not None else _t(tk)
    aq = np.asarray(cu_q, dtype=np.int64)
    ak = np.asarray(cu_kv, dtype=np.int64)
    sq = B.FaSeqlens(aq.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), aq.size - 1)
    sk = B.FaSeqlens(ak.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ak.size - 1)
    lib = B.load()
    ref = lambda x: None if x is None else ctypes.byref(x)  # noqa: E731
    st = getattr(lib, entry)(ref(q), ref(k), ref(v), ref(dy), ref(y),
                           None if smax is None else ctypes.c_void_p(smax),
                           None if ssum is None else ctypes.c_void_p(ssum), ctypes.byref(sq), ctypes.byref(sk),
                           mode, pre, nxt, kp, None if drop is None else ctypes.c_void_p(drop), scale,
                           head_num, ref(dq), ref(dk), ref(dv), None)
    return st, lib.fa_last_error().decode()


def test_null_pointers():
    lib = B.load()
    st = lib.fa_varlen_bwd(None, None, None, None, None, None, None, None, None, 0, 0, 0, 1.0, None, 1.0, 1,
                           None, None, None, None)
    assert st == B.FA_ERR_NULLPTR
    assert _call(q=_t(10, data=0))[0] == B.FA_ERR_NULLPTR
    assert _call(dv=_t(10, data=0))[0] == B.FA_ERR_NULLPTR
    assert _call(smax=None)[0] == B.FA_ERR_NULLPTR
    st, msg = _call(kp=0.9, drop=None)
    assert st == B.FA_ERR_NULLPTR and "drop_mask" in msg


@pytest.mark.parametrize("kwargs", [
    dict(kp=0.0), dict(kp=1.5), dict(kp=float("nan")),
    dict(head_num=3),
    dict(dq=_t(10, dtype=B.FA_F16)),
    dict(q=_t(10, dtype=7)),
    dict(q=_t(10, heads=300), k=_t(10, heads=300), v=_t(10, heads=300), dy=_t(10, heads=300),
         y=_t(10, heads=300), dq=_t(10, heads=300), dk=_t(10, heads=300), dv=_t(10, heads=300), head_num=300),
    dict(cu_q=(0, 1 << 21), cu_kv=(0, 10)),
    dict(cu_q=(1, 10)), dict(cu_q=(0, 6, 4, 10), cu_kv=(0, 3, 7, 10)),
    dict(cu_q=(0, 9), q=_t(10), dy=_t(10), y=_t(10), dq=_t(10)),
    dict(cu_q=(0, 4, 10), cu_kv=(0, 10)),
    dict(mode=3), dict(mode=-1),
    dict(q=_t(10, dim=128)),
    dict(k=_t(12)),
    dict(scale=float("inf")),
])
def test_invalid_arguments(kwargs):
    st, msg = _call(**kwargs)
    assert st == B.FA_ERR_INVALID, (kwargs, st, msg)
    assert msg


def test_batch_limits():
    cu = tuple(range(0, 2050))  # 2049 sequences of one token
    st, _ = _call(cu_q=cu, cu_kv=cu, q=_t(2049), k=_t(2049), v=_t(2049), dy=_t(2049), y=_t(2049),
                  dq=_t(2049), dk=_t(2049), dv=_t(2049))
    assert st == B.FA_ERR_INVALID
    assert _call(cu_q=(0,), cu_kv=(0,))[0] == B.FA_ERR_INVALID


def test_unsupported_variants():
    # head dims outside {64, 128}
    args = {n: _t(10, dim=96) for n in ("q", "k", "v", "dy", "y", "dq", "dk", "dv")}
    assert _call(**args)[0] == B.FA_ERR_UNSUPPORTED
    # v head dim smaller than k's, in a pair no kernel is built for: (64, 32)
    assert _call(v=_t(10, dim=32), dv=_t(10, dim=32), dy=_t(10, dim=32), y=_t(10, dim=32))[0] == B.FA_ERR_UNSUPPORTED
    # (128, 32) likewise
    args = {n: _t(10, dim=128) for n in ("q", "k", "dq", "dk")}
    args.update({n: _t(10, dim=32) for n in ("v", "dv", "dy", "y")})
    assert _call(**args)[0] == B.FA_ERR_UNSUPPORTED
    # misaligned base address
    assert _call(q=_t(10, data=FAKE + 2))[0] == B.FA_ERR_UNSUPPORTED


def test_grouped_heads_validation():
    # 4 query heads over 3 key/value heads: not a multiple
    args = {n: _t(10, heads=4) for n in ("q", "dy", "y", "dq")}
    args.update({n: _t(10, heads=3) for n in ("k", "v", "dk", "dv")})
    assert _call(head_num=4, **args)[0] == B.FA_ERR_INVALID
    # dk / dv must have the key/value head count
    args = {n: _t(10, heads=4) for n in ("q", "dy", "y", "dq", "dk")}
    args.update({n: _t(10, heads=2) for n in ("k", "v", "dv")})
    assert _call(head_num=4, **args)[0] == B.FA_ERR_INVALID
    # a valid grouped layout with no query tokens passes validation and returns before device work
    args = {n: _t(0, heads=4, data=0) for n in ("q", "dy", "y", "dq")}
    args.update({n: _t(0, heads=2, data=0) for n in ("k", "v", "dk", "dv")})
    st, msg = _call(head_num=4, cu_q=(0, 0), cu_kv=(0, 0), **args)
    assert st == B.FA_OK, msg


def test_narrow_v_validation():
    # dy and y take v's head dim; dv must match v
    args = {n: _t(10, dim=128) for n in ("q", "k", "dq", "dk")}
    args.update({n: _t(10, dim=64) for n in ("v", "dv", "y")})
    assert _call(dy=_t(10, dim=128), **args)[0] == B.FA_ERR_INVALID
    args = {n: _t(10, dim=128) for n in ("q", "k", "dq", "dk", "dv")}
    args.update({n: _t(10, dim=64) for n in ("v", "dy", "y")})
    assert _call(**args)[0] == B.FA_ERR_INVALID
    # v wider than k is outside the page's constraints
    args = {n: _t(10, dim=64) for n in ("q", "k", "dq", "dk")}
    args.update({n: _t(10, dim=128) for n in ("v", "dv", "dy", "y")})
    assert _call(**args)[0] == B.FA_ERR_INVALID
    # (128, 64) with no query tokens: validated, then no device work
    args = {n: _t(0, dim=128, data=0) for n in ("q", "k", "dq", "dk")}
    args.update({n: _t(0, dim=64, data=0) for n in ("v", "dv", "dy", "y")})
    st, msg = _call(cu_q=(0, 0), cu_kv=(0, 0), **args)
    assert st == B.FA_OK, msg


def _mcall(mask, **kw):
    """fa_varlen_bwd_masked with the default valid arguments of _call and the given mask view."""
    cu_q, cu_kv = kw.pop("cu_q", (0, 10)), kw.pop("cu_kv", (0, 10))
    tq, tk = cu_q[-1], cu_kv[-1]
    t = {n: kw.pop(n, _t(tq if n in ("q", "dy", "y", "dq") else tk)) for n in ("q", "k", "v", "dy", "y", "dq", "dk", "dv")}
    aq = np.asarray(cu_q, dtype=np.int64)
    ak = np.asarray(cu_kv, dtype=np.int64)
    sq = B.FaSeqlens(aq.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), aq.size - 1)
    sk = B.FaSeqlens(ak.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ak.size - 1)
    lib = B.load()
    r = ctypes.byref
    st = lib.fa_varlen_bwd_masked(r(t["q"]), r(t["k"]), r(t["v"]), r(t["dy"]), r(t["y"]), ctypes.c_void_p(FAKE),
                                  ctypes.c_void_p(FAKE), r(sq), r(sk), 0, 0, 0, 1.0, None,
                                  None if mask is None else r(mask), 0.125, 2, r(t["dq"]), r(t["dk"]), r(t["dv"]),
                                  None)
    return st, lib.fa_last_error().decode()


def _mask(data=FAKE, sb=0, sn=0, sq=16, rows=10, cols=10):
    return B.FaMask(ctypes.c_void_p(data), sb, sn, sq, rows, cols)


def test_explicit_mask_validation():
    assert _mcall(_mask(data=0))[0] == B.FA_ERR_NULLPTR
    assert _mcall(_mask(rows=9))[0] == B.FA_ERR_INVALID          # rows < Lq
    assert _mcall(_mask(cols=9, sq=9))[0] == B.FA_ERR_INVALID    # cols < Lkv
    assert _mcall(_mask(sq=8))[0] == B.FA_ERR_INVALID            # stride_q < cols
    assert _mcall(_mask(sb=-1))[0] == B.FA_ERR_INVALID
    assert _mcall(_mask(sq=1 << 28))[0] == B.FA_ERR_UNSUPPORTED  # a block spans >= 2^31 bytes
    st, msg = _mcall(_mask(data=0), cu_q=(0, 0), cu_kv=(0, 0), **{n: _t(0, data=0) for n in
                                                                    ("q", "k", "v", "dy", "y", "dq", "dk", "dv")})
    assert st == B.FA_OK, msg


def test_explicit_mask_forward_validation():
    lib = B.load()
    aq = np.asarray((0, 10), dtype=np.int64)
    sq = B.FaSeqlens(aq.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1)
    r = ctypes.byref
    q, k, v, y = _t(10), _t(10), _t(10), _t(10)

    def call(m):
        return lib.fa_varlen_fwd_masked(r(q), r(k), r(v), r(sq), r(sq), 0, 0, 0, 1.0, None, r(m), 0.125, 2, r(y),
                                        ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None)

    assert call(_mask(data=0)) == B.FA_ERR_NULLPTR
    assert call(_mask(rows=3)) == B.FA_ERR_INVALID
    assert call(_mask(sq=1 << 28)) == B.FA_ERR_UNSUPPORTED


def test_mask_desc_strides():
    import torch
    m = torch.zeros(3, 4, 20, 30, dtype=torch.uint8)
    d = B.mask_desc(m)
    assert (d.stride_b, d.stride_n, d.stride_q, d.rows, d.cols) == (2400, 600, 30, 20, 30)
    d = B.mask_desc(m[:, :1])
    assert (d.stride_b, d.stride_n) == (2400, 0)
    d = B.mask_desc(torch.zeros(20, 30, dtype=torch.bool))
    assert (d.stride_b, d.stride_n, d.stride_q) == (0, 0, 30)
    with pytest.raises(ValueError):
        B.mask_desc(torch.zeros(20, 30, dtype=torch.float32))


def test_empty_query_returns_ok_without_device_work():
    # T == 0: validated, then returned before any HIP call (runs on a GPU-less host)
    st, msg = _call(cu_q=(0, 0), cu_kv=(0, 0), q=_t(0, data=0), k=_t(0, data=0), v=_t(0, data=0),
                    dy=_t(0, data=0), y=_t(0, data=0), dq=_t(0, data=0), dk=_t(0, data=0), dv=_t(0, data=0))
    assert st == B.FA_OK, msg


def _no_gpu():
    # counting devices does not initialise the GPU on this image
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu(), reason="needs a host without a GPU: the HIP runtime must fail")
@pytest.mark.parametrize("entry", ["fa_varlen_bwd", "fa_varlen_bwd_noalloc"])
def test_hip_failure_is_reported_as_runtime_error(entry):
    # a valid call on a host where the HIP runtime has no device: the first HIP call fails, and the
    # status is FA_ERR_RUNTIME with the runtime's message (nothing can have been launched)
    st, msg = _call(entry=entry)
    assert st == B.FA_ERR_RUNTIME, (st, msg)
    assert msg and "hipGetDevice" in msg, msg
    st, msg = _fwd()
    assert st == B.FA_ERR_RUNTIME, (st, msg)
    assert msg


def test_noalloc_rejects_inputs_beyond_its_fixed_space():
    # 2^20 tokens x 7 heads needs 56 MiB of row statistics, more than the fixed 48 MiB: refused
    # before any device work, with a message naming the limit
    t = 1 << 20
    st, msg = _call(q=_t(t, heads=7), k=_t(t, heads=7), v=_t(t, heads=7), dy=_t(t, heads=7), y=_t(t, heads=7),
                    dq=_t(t, heads=7), dk=_t(t, heads=7), dv=_t(t, heads=7), cu_q=(0, t), cu_kv=(0, t),
                    head_num=7, entry="fa_varlen_bwd_noalloc")
    assert st == B.FA_ERR_UNSUPPORTED, (st, msg)
    assert "6291456" in msg, msg
    # and the same validation as fa_varlen_bwd
    assert _call(q=_t(10, data=0), entry="fa_varlen_bwd_noalloc")[0] == B.FA_ERR_NULLPTR
    assert _call(kp=1.5, entry="fa_varlen_bwd_noalloc")[0] == B.FA_ERR_INVALID


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        B.load(str(tmp_path / "libfa_varlen.so"))


def _fwd(q=None, k=None, v=None, y=None, smax=FAKE, ssum=FAKE, cu_q=(0, 10), cu_kv=(0, 10), mode=0, pre=0,
         nxt=0, kp=1.0, drop=None, scale=0.125, head_num=2):
    tq, tk = cu_q[-1], cu_kv[-1]
    q = q if q is not None else _t(tq)
    k = k if k is not None else _t(tk)
    v = v if v is not None else _t(tk)
    y = y if y is not None else _t(tq)
    aq = np.asarray(cu_q, dtype=np.int64)
    ak = np.asarray(cu_kv, dtype=np.int64)
    sq = B.FaSeqlens(aq.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), aq.size - 1)
    sk = B.FaSeqlens(ak.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ak.size - 1)
    lib = B.load()
    ref = lambda x: None if x is None else ctypes.byref(x)  # noqa: E731
    st = lib.fa_varlen_fwd(ref(q), ref(k), ref(v), ctypes.byref(sq), ctypes.byref(sk), mode, pre, nxt, kp,
                           None if drop is None else ctypes.c_void_p(drop), scale, head_num, ref(y),
                           None if smax is None else ctypes.c_void_p(smax),
                           None if ssum is None else ctypes.c_void_p(ssum), None)
    return st, lib.fa_last_error().decode()


def test_forward_null_pointers():
    lib = B.load()
    assert lib.fa_varlen_fwd(None, None, None, None, None, 0, 0, 0, 1.0, None, 1.0, 1, None, None, None,
                             None) == B.FA_ERR_NULLPTR
    assert _fwd(y=_t(10, data=0))[0] == B.FA_ERR_NULLPTR
    assert _fwd(smax=None)[0] == B.FA_ERR_NULLPTR
    assert _fwd(kp=0.9, drop=None)[0] == B.FA_ERR_NULLPTR


@pytest.mark.parametrize("kwargs,status", [
    (dict(kp=0.0), B.FA_ERR_INVALID),
    (dict(kp=1.5), B.FA_ERR_INVALID),
    (dict(mode=3), B.FA_ERR_INVALID),
    (dict(scale=float("inf")), B.FA_ERR_INVALID),
    (dict(head_num=3), B.FA_ERR_INVALID),
    (dict(y=_t(10, dtype=B.FA_F16)), B.FA_ERR_INVALID),
    (dict(y=_t(11)), B.FA_ERR_INVALID),
    (dict(cu_q=(0, 4, 10), cu_kv=(0, 10)), B.FA_ERR_INVALID),
    (dict(cu_q=(0, 12, 10), cu_kv=(0, 5, 10)), B.FA_ERR_INVALID),
    (dict(k=_t(10, heads=3), v=_t(10, heads=3)), B.FA_ERR_INVALID),
    (dict(k=_t(10, heads=1), v=_t(10, heads=2)), B.FA_ERR_INVALID),
    (dict(q=_t(10, dim=96), k=_t(10, dim=96), v=_t(10, dim=96), y=_t(10, dim=96)), B.FA_ERR_UNSUPPORTED),
    (dict(smax=FAKE + 4), B.FA_ERR_UNSUPPORTED),
])
def test_forward_invalid_arguments(kwargs, status):
    st, msg = _fwd(**kwargs)
    assert st == status, msg
    assert msg


def test_forward_narrow_v():
    # y takes v's head dim
    q, k = _t(10, dim=128), _t(10, dim=128)
    assert _fwd(q=q, k=k, v=_t(10, dim=64), y=_t(10, dim=128))[0] == B.FA_ERR_INVALID
    assert _fwd(q=q, k=k, v=_t(10, dim=32), y=_t(10, dim=32))[0] == B.FA_ERR_UNSUPPORTED
    st, msg = _fwd(q=_t(0, dim=128), k=k, v=_t(10, dim=64), y=_t(0, dim=64), cu_q=(0, 0), smax=None, ssum=None)
    assert st == B.FA_OK, msg


def test_forward_empty_input_is_ok():
    assert _fwd(q=_t(0), y=_t(0), cu_q=(0, 0), cu_kv=(0, 10), smax=None, ssum=None)[0] == B.FA_OK


# --- the Python binding's checks of what the raw pointers hide -------------------------------

def _cpu_args(dtype=None):
    import torch
    dt = dtype or torch.bfloat16
    q = torch.zeros(10, 2, 64, dtype=dt)
    st = torch.zeros(2, 10, 8, dtype=torch.float32)
    return q, st


def test_binding_rejects_host_tensors():
    q, st = _cpu_args()
    with pytest.raises(ValueError, match="device tensor"):
        B.fa_varlen_bwd(q, q, q, q, q, st, st, (0, 10), (0, 10), 0, 0, 0, 1.0, None, 0.125, 2, q, q, q)
    with pytest.raises(ValueError, match="device tensor"):
        B.fa_varlen_fwd(q, q, q, (0, 10), (0, 10), 0, 0, 0, 1.0, None, 0.125, 2, q, st, st)


def test_binding_checks_shapes_and_mask_sizes(monkeypatch):
    import torch
    # stand-in device placement so the shape checks can run without a GPU
    q, st = _cpu_args()
    monkeypatch.setattr(torch.Tensor, "is_cuda", property(lambda self: True))
    with pytest.raises(ValueError, match=r"\[N, Tq, 8\]"):
        B._check_args(q, {}, dict(softmax_max=st[:, :9]), (0, 10), (0, 10), 1.0, None, None)
    with pytest.raises(ValueError, match=r"\[N, Tq, 8\]"):
        B._check_args(q, {}, dict(softmax_max=st.double()), (0, 10), (0, 10), 1.0, None, None)
    drop = torch.zeros(24, dtype=torch.uint8)  # 2 heads * 10 * 10 bits need 25 bytes
    with pytest.raises(ValueError, match="25 bytes"):
        B._check_args(q, {}, {}, (0, 10), (0, 10), 0.9, drop, None)
    B._check_args(q, {}, {}, (0, 10), (0, 10), 0.9, torch.zeros(25, dtype=torch.uint8), None)
    with pytest.raises(ValueError, match="atten_mask axes"):
        B._check_args(q, {}, {}, (0, 10), (0, 10), 1.0, None, torch.zeros(2, 2, 10, 10, dtype=torch.uint8))
    B._check_args(q, {}, {}, (0, 10), (0, 10), 1.0, None, torch.zeros(1, 2, 10, 10, dtype=torch.uint8))
