"""Plain fp64 CPU oracle for the varlen FlashAttention backward (TND layout).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP library.

Source: the CANN ops-transformer page "FlashAttention梯度V2"
(aclnnFlashAttentionUnpaddingScoreGradV2).  Its 计算公式 (formulas) section
defines the forward

    S = Mask(scale * Q K^T, atten_mask)
    P = Dropout(Softmax(S), keep_prob)
    Y = P V

and the backward dV = P^T dY, dQ = dS K * scale, dK = dS^T Q * scale.
The page gives no formula for dS; the softmax Jacobian step used here is
dP = dY V^T and dS = P o (dP - rowsum(dY o Y)) (reading R1 below).

Readings of points the page leaves open (each one is listed in the design doc):
  R1  dS uses the pre-dropout softmax Ps; dP carries the dropout factor Z/kp;
      the row term Delta_i = sum_d dY_i,d * Y_i,d uses the *given* Y.
  R2  scaleValue replaces 1/sqrt(d) everywhere (参数说明 table, scaleValue).
  R4  inverted dropout: bit 1 keeps, kept values are scaled by 1/keep_prob;
      at keep_prob == 1 the mask is not read.
  R5  dropMask is one flat little-endian bit stream: for each sequence b in
      order, a row-major [N, Lq_b, Lkv_b] block with no padding (the same
      per-sequence flattening the page's 约束说明 gives for PSE in TND).
  R6  softmaxMax / softmaxSum are [N, T, 8] fp32 with the value replicated
      over the last axis; element 0 is read.
  R7  m is the row max of the scaled, masked scores and l the sum of
      exp(S - m) over admitted keys; P = exp(S - m) / l.
  R8  causal is aligned lower-right: admit(i, j) <=> j <= i + (Lkv - Lq).
  R9  band: admit(i, j) <=> i + off - pre <= j <= i + off + next, off = Lkv - Lq.
  R10 a row with no admitted key has P == 0 exactly (dQ row 0, no dK/dV
      contribution); its stats are never read.
  R11 cu_seqlens are prefix sums with a leading 0 (B + 1 entries).
  R15 grouped heads (N query heads over Nkv key/value heads, N a multiple of
      Nkv, 约束说明): query head n reads key/value head n // (N / Nkv), so
      each key/value head serves a contiguous group of query heads; its dK and
      dV are the sums of the group's per-head contributions.  The dropout mask
      is indexed by the query head.
  R16 Dv < Dk (参数说明: V may have a smaller head dim than Q and K): Y, dY
      and dV have V's head dim, dQ and dK have Q's; nothing else changes.
  R17 explicit atten_mask (参数说明: attenMaskOptional, 1 = the position takes
      no part, shapes [B,N,Sq,Skv], [B,1,Sq,Skv], [1,1,Sq,Skv] or [Sq,Skv]):
      element (b, n, i, j) with sequence-relative i, j and the query head n,
      size-1 axes broadcast; a pair is admitted when the mode's window admits
      it and its mask element is 0 (the window and the mask intersect; with
      no window the mask alone decides).

Every function below computes the plain definition (one library matmul per
contraction, no blocking beyond splitting query rows into chunks, which only
changes which rows are held in memory at a time).
"""
from __future__ import annotations

import os
from typing import Optional, Sequence

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BAND = 2

_ROW_CHUNK = 1024


# ---------------------------------------------------------------------------
# mask, dropout bits, sequence bookkeeping
# ---------------------------------------------------------------------------

def admit_mask(lq: int, lkv: int, mode: int, pre: int = 0, nxt: int = 0,
               rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Boolean [len(rows), lkv] matrix: True where query i may attend key j.

    The page's atten_mask marks excluded positions with 1 (参数说明 table,
    attenMaskOptional); this returns its complement.  Causal follows R8,
    band follows R9 (preTokens/nextTokens are the left/right window bounds
    in the 参数说明 table).
    """
    if rows is None:
        rows = np.arange(lq, dtype=np.int64)
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(lkv, dtype=np.int64)[None, :]
    off = lkv - lq
    if mode == MASK_NONE:
        return np.ones((i.shape[0], lkv), dtype=bool)
    if mode == MASK_CAUSAL:
        return j <= i + off
    if mode == MASK_BAND:
        return (j >= i + off - int(pre)) & (j <= i + off + int(nxt))
    raise ValueError(f"unknown mask mode {mode}")


def explicit_mask_block(atten_mask, b: int, n: int, lq: int, lkv: int):
    """Excluded positions (bool [lq, lkv]) of sequence b, query head n, from an explicit mask
    (R17), or None without one."""
    if atten_mask is None:
        return None
    m = np.asarray(atten_mask)
    if m.ndim == 4:
        m = m[b if m.shape[0] > 1 else 0, n if m.shape[1] > 1 else 0]
    elif m.ndim != 2:
        raise ValueError("atten_mask must be [B|1, N|1, Sq, Skv] or [Sq, Skv]")
    return m[:lq, :lkv] != 0


def seq_lengths(cu: Sequence[int]) -> np.ndarray:
    cu = np.asarray(cu, dtype=np.int64)
    return cu[1:] - cu[:-1]


def dropout_bit_bases(cu_q: Sequence[int], cu_kv: Sequence[int], heads: int) -> np.ndarray:
    """Bit offset of each sequence's [N, Lq_b, Lkv_b] block in the flat mask (R5)."""
    lq = seq_lengths(cu_q)
    lkv = seq_lengths(cu_kv)
    sizes = heads * lq * lkv
    return np.concatenate([[0], np.cumsum(sizes)[:-1]]).astype(np.int64)


def dropout_keep(drop_mask: np.ndarray, bit0: int, rows: np.ndarray, lkv: int) -> np.ndarray:
    """Keep bits Z[i, j] (0/1 as float64) for the given rows of one (b, n) block.

    bit0 is the bit index of element (0, 0) of the block; element (i, j) is
    bit bit0 + i * lkv + j of the stream, least significant bit first within
    each byte (R5).
    """
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, lkv), dtype=np.float64)
    for r, i in enumerate(rows):
        first = bit0 + int(i) * lkv
        last = first + lkv
        b0, b1 = first >> 3, (last + 7) >> 3
        bits = np.unpackbits(np.asarray(drop_mask[b0:b1], dtype=np.uint8), bitorder="little")
        s = first - (b0 << 3)
        out[r] = bits[s:s + lkv]
    return out


def kv_head(n: int, head_num: int, kv_heads: int) -> int:
    """Key/value head read by query head n (R15): contiguous groups of head_num // kv_heads."""
    return n // (head_num // kv_heads)


# ---------------------------------------------------------------------------
# forward (used only to produce consistent Y and statistics for tests)
# ---------------------------------------------------------------------------

def forward_unit(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 mode: int, pre: int, nxt: int, keep_prob: float,
                 drop_mask: Optional[np.ndarray], bit0: int, xmask=None):
    """Forward of one (sequence, head): returns Y [Lq, D], m [Lq], l [Lq] in fp64.

    S = scale * Q K^T; m_i = max over admitted j; l_i = sum_j exp(S_ij - m_i);
    Ps = exp(S - m) / l on admitted entries, 0 elsewhere; Y = (Ps o Z / kp) V.
    An empty row gets m = -inf, l = 0, Y = 0 (R10).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lq = q.shape[0]
    y = np.zeros((lq, v.shape[1]), dtype=np.float64)
    m = np.full(lq, -np.inf, dtype=np.float64)
    l = np.zeros(lq, dtype=np.float64)
    for c0 in range(0, lq, _ROW_CHUNK):
        rows = np.arange(c0, min(lq, c0 + _ROW_CHUNK))
        y[rows], m[rows], l[rows] = _forward_rows(q[rows], k, v, lq, rows, scale, mode, pre, nxt,
                                                  keep_prob, drop_mask, bit0, xmask)
    return y, m, l


def _admitted(lq, lkv, mode, pre, nxt, rows, xmask):
    """Admitted pairs of the given rows: the mode's window without the explicitly masked ones."""
    a = admit_mask(lq, lkv, mode, pre, nxt, rows)
    if xmask is not None:
        a = a & ~xmask[np.asarray(rows, dtype=np.int64)]
    return a


def _forward_rows(qr, k, v, lq: int, rows, scale, mode, pre, nxt, keep_prob, drop_mask, bit0, xmask=None):
    """Y, m, l of the given query rows (sequence-relative), with qr their Q rows (fp64)."""
    lkv = k.shape[0]
    s = scale * (qr @ k.T)
    a = _admitted(lq, lkv, mode, pre, nxt, rows, xmask)
    has = a.any(axis=1)
    sm = np.where(a, s, -np.inf)
    mc = sm.max(axis=1, initial=-np.inf)
    e = np.exp(np.where(a, s - np.where(has, mc, 0.0)[:, None], -np.inf))
    lc = e.sum(axis=1)
    ps = np.where(has[:, None], e / np.where(has, lc, 1.0)[:, None], 0.0)
    if keep_prob < 1.0:
        ps = ps * dropout_keep(drop_mask, bit0, rows, lkv) / keep_prob
    return ps @ v, mc, lc


def forward_rows(q, k, v, cu_q, cu_kv, b: int, n: int, rows, *, mode: int = MASK_NONE, pre: int = 0,
                 nxt: int = 0, keep_prob: float = 1.0, drop_mask=None, scale: float, head_num: int,
                 atten_mask=None):
    """Forward of selected query rows (sequence-relative) of one (b, n): Y [len(rows), D], m, l.

    The same definition as forward_unit restricted to those rows (each row needs only its own
    row of S).
    """
    q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
    k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
    bit0 = int(dropout_bit_bases(cu_q, cu_kv, head_num)[b]) + n * (q1 - q0) * (k1 - k0)
    rows = np.asarray(rows, dtype=np.int64)
    hk = kv_head(n, head_num, k.shape[1])
    qr = np.asarray(q[q0:q1, n], dtype=np.float64)[rows]
    ks = np.asarray(k[k0:k1, hk], dtype=np.float64)
    vs = np.asarray(v[k0:k1, hk], dtype=np.float64)
    xm = explicit_mask_block(atten_mask, b, n, q1 - q0, k1 - k0)
    return _forward_rows(qr, ks, vs, q1 - q0, rows, scale, mode, pre, nxt, keep_prob, drop_mask, bit0, xm)


def _forward_pool_unit(job):
    b, n = job
    st = _POOL_STATE
    q, k, cu_q, cu_kv, head_num = st["q"], st["k"], st["cu_q"], st["cu_kv"], st["head_num"]
    q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
    k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
    bit0 = int(st["bases"][b]) + n * (q1 - q0) * (k1 - k0)
    hk = kv_head(n, head_num, k.shape[1])
    return (b, n) + forward_unit(q[q0:q1, n], k[k0:k1, hk], st["v"][k0:k1, hk], st["scale"], st["mode"],
                                 st["pre"], st["nxt"], st["keep_prob"], st["drop_mask"], bit0,
                                 explicit_mask_block(st["atten_mask"], b, n, q1 - q0, k1 - k0))


def forward(q, k, v, cu_q, cu_kv, *, mode: int = MASK_NONE, pre: int = 0, nxt: int = 0,
            keep_prob: float = 1.0, drop_mask=None, scale: float, head_num: int, atten_mask=None,
            workers: int = 1):
    """Varlen forward over TND tensors; returns Y [T, N, Dv], m [N, T], l [N, T] (fp64).

    q is [Tq, N, Dk]; k and v are [Tkv, Nkv, Dk] and [Tkv, Nkv, Dv] with N a multiple of Nkv (R15).
    With workers > 1 the (sequence, head) units run in a fork-based process pool, each computed
    exactly as with workers == 1.
    """
    tq = q.shape[0]
    y = np.zeros((tq, head_num, v.shape[2]), dtype=np.float64)
    m = np.full((head_num, tq), -np.inf, dtype=np.float64)
    l = np.zeros((head_num, tq), dtype=np.float64)
    bases = dropout_bit_bases(cu_q, cu_kv, head_num)
    units = [(b, n) for b in range(len(cu_q) - 1) for n in range(head_num) if cu_q[b + 1] > cu_q[b]]

    def put(b, n, yb, mb, lb):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        y[q0:q1, n] = yb
        m[n, q0:q1] = mb
        l[n, q0:q1] = lb

    if workers <= 1 or len(units) <= 1:
        for b, n in units:
            q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
            k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
            bit0 = int(bases[b]) + n * (q1 - q0) * (k1 - k0)
            hk = kv_head(n, head_num, k.shape[1])
            put(b, n, *forward_unit(q[q0:q1, n], k[k0:k1, hk], v[k0:k1, hk], scale,
                                    mode, pre, nxt, keep_prob, drop_mask, bit0,
                                    explicit_mask_block(atten_mask, b, n, q1 - q0, k1 - k0)))
        return y, m, l
    state = dict(q=q, k=k, v=v, cu_q=np.asarray(cu_q, dtype=np.int64), cu_kv=np.asarray(cu_kv, dtype=np.int64),
                 bases=bases, scale=scale, mode=mode, pre=pre, nxt=nxt, keep_prob=keep_prob,
                 drop_mask=drop_mask, atten_mask=atten_mask, head_num=head_num)
    for b, n, yb, mb, lb in _pool_map(_forward_pool_unit, units, state, workers):
        put(b, n, yb, mb, lb)
    return y, m, l


def stats_to_page_layout(m: np.ndarray, l: np.ndarray):
    """[N, T] fp64 stats -> the page's [N, T, 8] fp32 arrays (R6), rounded to nearest."""
    mm = np.repeat(m.astype(np.float32)[:, :, None], 8, axis=2)
    ll = np.repeat(l.astype(np.float32)[:, :, None], 8, axis=2)
    return mm, ll


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------

def _probs(s, a, m, l):
    """Pre-dropout softmax Ps = exp(S - m) / l on admitted entries, exact 0 elsewhere (R7, R10)."""
    has = a.any(axis=1)
    mm = np.where(has, m, 0.0)[:, None]
    ll = np.where(has, l, 1.0)[:, None]
    return np.exp(np.where(a, s - mm, -np.inf)) / ll


def backward_unit(q, k, v, dy, y, m, l, scale: float, mode: int, pre: int, nxt: int,
                  keep_prob: float, drop_mask, bit0: int, want_ds: bool = False, xmask=None):
    """Backward of one (sequence, head) in fp64.

    Inputs are the [L, D] slices of Q, dY, Y and the [Lkv, D] slices of K, V,
    plus the row statistics m, l [L].  Steps (formulas section of the page,
    with reading R1 for dS):
        S   = scale * Q K^T
        Ps  = exp(S - m) / l          (admitted entries only)
        Pd  = Ps o Z / kp
        dV  = Pd^T dY
        dPd = dY V^T
        D_i = sum_d dY_i,d Y_i,d
        dS  = Ps o (dPd o Z / kp - D)
        dQ  = scale * dS K
        dK  = scale * dS^T Q
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    lq, lkv = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros((lkv, v.shape[1]), dtype=np.float64)
    ds_all = np.zeros((lq, lkv), dtype=np.float64) if want_ds else None
    delta = np.sum(dy * y, axis=1)
    for c0 in range(0, lq, _ROW_CHUNK):
        rows = np.arange(c0, min(lq, c0 + _ROW_CHUNK))
        s = scale * (q[rows] @ k.T)
        a = _admitted(lq, lkv, mode, pre, nxt, rows, xmask)
        ps = _probs(s, a, m[rows], l[rows])
        if keep_prob < 1.0:
            zk = dropout_keep(drop_mask, bit0, rows, lkv) / keep_prob
        else:
            zk = 1.0
        pd = ps * zk
        dv += pd.T @ dy[rows]
        dpd = dy[rows] @ v.T
        ds = ps * (dpd * zk - delta[rows][:, None])
        dq[rows] = scale * (ds @ k)
        dk += scale * (ds.T @ q[rows])
        if want_ds:
            ds_all[rows] = ds
    if want_ds:
        return dq, dk, dv, ds_all
    return dq, dk, dv


def _stat0(stat):
    """Element 0 of the page's [N, T, 8] statistics, or an [N, T] array as is (R6)."""
    stat = np.asarray(stat)
    return stat[..., 0] if stat.ndim == 3 else stat


def _unit_args(b, n, q, k, v, dy, y, mstat, lstat, cu_q, cu_kv, bases, atten_mask=None):
    """Slices of query head n of sequence b, with the key/value head it reads (R15) and the
    unit's explicitly masked positions (R17, or None)."""
    q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
    k0, k1 = int(cu_kv[b]), int(cu_kv[b + 1])
    bit0 = int(bases[b]) + n * (q1 - q0) * (k1 - k0)
    hk = kv_head(n, q.shape[1], k.shape[1])
    return (q[q0:q1, n], k[k0:k1, hk], v[k0:k1, hk], dy[q0:q1, n], y[q0:q1, n],
            mstat[n, q0:q1], lstat[n, q0:q1], bit0,
            explicit_mask_block(atten_mask, b, n, q1 - q0, k1 - k0))


_POOL_STATE = {}


def _pool_init(state):
    _POOL_STATE.clear()
    _POOL_STATE.update(state)


def _pool_unit(job):
    b, n = job
    st = _POOL_STATE
    qs, ks, vs, dys, ys, ms, ls, bit0, xm = _unit_args(
        b, n, st["q"], st["k"], st["v"], st["dy"], st["y"], st["m"], st["l"],
        st["cu_q"], st["cu_kv"], st["bases"], st["atten_mask"])
    return (b, n) + backward_unit(qs, ks, vs, dys, ys, ms, ls, st["scale"], st["mode"],
                                  st["pre"], st["nxt"], st["keep_prob"], st["drop_mask"], bit0, xmask=xm)


def backward(q, k, v, dy, y, softmax_max, softmax_sum, cu_q, cu_kv, *, mode: int = MASK_NONE,
             pre: int = 0, nxt: int = 0, keep_prob: float = 1.0, drop_mask=None,
             scale: float, head_num: int, workers: int = 1, units=None, atten_mask=None):
    """Varlen backward over TND tensors; returns dQ [Tq, N, Dk], dK [Tkv, Nkv, Dk], dV [Tkv, Nkv, Dv] in fp64.

    Rows or keys that no admitted pair touches stay exactly 0.  `units` may
    restrict the work to a list of (b, n) pairs of sequence and query head
    (their contributions are written, the rest stays 0).  A key/value head
    shared by several query heads receives the sum of their dK and dV (R15).  With workers > 1 the (b, n) units run in a fork-based
    process pool, each unit computed exactly as with workers == 1.
    """
    mstat, lstat = _stat0(softmax_max), _stat0(softmax_sum)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    nb = len(cu_q) - 1
    bases = dropout_bit_bases(cu_q, cu_kv, head_num)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    if units is None:
        units = [(b, n) for b in range(nb) for n in range(head_num)
                 if cu_q[b + 1] > cu_q[b] and cu_kv[b + 1] > cu_kv[b]]

    def put(b, n, dqs, dks, dvs):
        hk = kv_head(n, head_num, k.shape[1])
        dq[cu_q[b]:cu_q[b + 1], n] = dqs
        dk[cu_kv[b]:cu_kv[b + 1], hk] += dks
        dv[cu_kv[b]:cu_kv[b + 1], hk] += dvs

    if workers <= 1 or len(units) <= 1:
        for b, n in units:
            qs, ks, vs, dys, ys, ms, ls, bit0, xm = _unit_args(b, n, q, k, v, dy, y, mstat, lstat,
                                                               cu_q, cu_kv, bases, atten_mask)
            put(b, n, *backward_unit(qs, ks, vs, dys, ys, ms, ls, scale, mode, pre, nxt,
                                     keep_prob, drop_mask, bit0, xmask=xm))
        return dq, dk, dv

    state = dict(q=q, k=k, v=v, dy=dy, y=y, m=mstat, l=lstat, cu_q=cu_q, cu_kv=cu_kv,
                 bases=bases, scale=scale, mode=mode, pre=pre, nxt=nxt,
                 keep_prob=keep_prob, drop_mask=drop_mask, atten_mask=atten_mask)
    for b, n, dqs, dks, dvs in _pool_map(_pool_unit, units, state, workers):
        put(b, n, dqs, dks, dvs)
    return dq, dk, dv


def _pool_map(fn, jobs, state, workers):
    """fn over jobs in a fork-based process pool whose workers see `state`; results in job order."""
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    # one BLAS thread per worker: the pool supplies the parallelism
    old = {key: os.environ.get(key) for key in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for key in old:
        os.environ[key] = "1"
    try:
        with ctx.Pool(processes=workers, initializer=_pool_init, initargs=(state,)) as pool:
            for r in pool.imap(fn, jobs):
                yield r
    finally:
        for key, val in old.items():
            if val is None:
                os.environ.pop(key, None)
            else:
                os.environ[key] = val


# ---------------------------------------------------------------------------
# sampled outputs (for checks at sizes where the full backward is too slow)
# ---------------------------------------------------------------------------

def backward_dq_rows(q, k, v, dy, y, softmax_max, softmax_sum, cu_q, cu_kv, b: int, n: int,
                     rows, *, mode: int = MASK_NONE, pre: int = 0, nxt: int = 0,
                     keep_prob: float = 1.0, drop_mask=None, scale: float, head_num: int, atten_mask=None):
    """dQ for selected query rows (sequence-relative) of one (b, n): [len(rows), D] fp64.

    The same definition as backward_unit restricted to those rows: each needs
    only its own row of S, Ps, dPd and its own Delta.
    """
    mstat, lstat = _stat0(softmax_max), _stat0(softmax_sum)
    bases = dropout_bit_bases(cu_q, cu_kv, head_num)
    qs, ks, vs, dys, ys, ms, ls, bit0, xm = _unit_args(b, n, q, k, v, dy, y, mstat, lstat,
                                                       np.asarray(cu_q), np.asarray(cu_kv), bases, atten_mask)
    rows = np.asarray(rows, dtype=np.int64)
    qs = np.asarray(qs, dtype=np.float64)[rows]
    ks = np.asarray(ks, dtype=np.float64)
    vs = np.asarray(vs, dtype=np.float64)
    dys = np.asarray(dys, dtype=np.float64)[rows]
    ys = np.asarray(ys, dtype=np.float64)[rows]
    ms = np.asarray(ms, dtype=np.float64)[rows]
    ls = np.asarray(ls, dtype=np.float64)[rows]
    lq = int(cu_q[b + 1] - cu_q[b])
    s = scale * (qs @ ks.T)
    a = _admitted(lq, ks.shape[0], mode, pre, nxt, rows, xm)
    ps = _probs(s, a, ms, ls)
    zk = dropout_keep(drop_mask, bit0, rows, ks.shape[0]) / keep_prob if keep_prob < 1.0 else 1.0
    delta = np.sum(dys * ys, axis=1)
    ds = ps * ((dys @ vs.T) * zk - delta[:, None])
    return scale * (ds @ ks)


def backward_dkdv_cols(q, k, v, dy, y, softmax_max, softmax_sum, cu_q, cu_kv, b: int, n: int,
                       cols, *, mode: int = MASK_NONE, pre: int = 0, nxt: int = 0,
                       keep_prob: float = 1.0, drop_mask=None, scale: float, head_num: int, atten_mask=None):
    """dK and dV for selected keys (sequence-relative) of key/value head n of sequence b.

    Returns two [len(cols), Dk] and [len(cols), Dv] fp64 arrays: the sums over the query heads
    that read head n (R15) of the same definition as backward_unit restricted to those keys.
    Each needs its column of S, Ps, dPd over all query rows, with every row's Delta.
    """
    group = head_num // k.shape[1]
    cols = np.asarray(cols, dtype=np.int64)
    dk = np.zeros((cols.size, k.shape[2]), dtype=np.float64)
    dv = np.zeros((cols.size, v.shape[2]), dtype=np.float64)
    for nq in range(n * group, (n + 1) * group):
        a, c = _dkdv_cols_one_head(q, k, v, dy, y, softmax_max, softmax_sum, cu_q, cu_kv, b, nq, cols,
                                   mode, pre, nxt, keep_prob, drop_mask, scale, head_num, atten_mask)
        dk += a
        dv += c
    return dk, dv


def _dkdv_cols_one_head(q, k, v, dy, y, softmax_max, softmax_sum, cu_q, cu_kv, b, n, cols, mode, pre, nxt,
                        keep_prob, drop_mask, scale, head_num, atten_mask=None):
    """Contribution of query head n to dK and dV of the selected keys of its key/value head."""
    mstat, lstat = _stat0(softmax_max), _stat0(softmax_sum)
    bases = dropout_bit_bases(cu_q, cu_kv, head_num)
    qs, ks, vs, dys, ys, ms, ls, bit0, xm = _unit_args(b, n, q, k, v, dy, y, mstat, lstat,
                                                       np.asarray(cu_q), np.asarray(cu_kv), bases, atten_mask)
    lq, lkv = qs.shape[0], ks.shape[0]
    qs = np.asarray(qs, dtype=np.float64)
    kc = np.asarray(ks, dtype=np.float64)[cols]
    vc = np.asarray(vs, dtype=np.float64)[cols]
    dk = np.zeros((cols.size, kc.shape[1]), dtype=np.float64)
    dv = np.zeros((cols.size, vc.shape[1]), dtype=np.float64)
    for c0 in range(0, lq, _ROW_CHUNK):
        rows = np.arange(c0, min(lq, c0 + _ROW_CHUNK))
        qr = qs[rows]
        dyr = np.asarray(dys[rows], dtype=np.float64)
        yr = np.asarray(ys[rows], dtype=np.float64)
        s = scale * (qr @ kc.T)
        a_full = _admitted(lq, lkv, mode, pre, nxt, rows, xm)
        ps = _probs_cols(s, a_full[:, cols], np.asarray(ms[rows], dtype=np.float64),
                         np.asarray(ls[rows], dtype=np.float64), a_full.any(axis=1))
        if keep_prob < 1.0:
            zk = dropout_keep(drop_mask, bit0, rows, lkv)[:, cols] / keep_prob
        else:
            zk = 1.0
        delta = np.sum(dyr * yr, axis=1)
        dv += (ps * zk).T @ dyr
        ds = ps * ((dyr @ vc.T) * zk - delta[:, None])
        dk += scale * (ds.T @ qr)
    return dk, dv


def _probs_cols(s, a, m, l, row_has_any):
    """Ps on a column subset; rows with no admitted key anywhere are 0 (R10)."""
    mm = np.where(row_has_any, m, 0.0)[:, None]
    ll = np.where(row_has_any, l, 1.0)[:, None]
    return np.exp(np.where(a, s - mm, -np.inf)) / ll


def admitted_pairs(cu_q, cu_kv, mode: int, pre: int = 0, nxt: int = 0) -> int:
    """Number of admitted (query, key) pairs per head, counted by brute force over rows."""
    total = 0
    lq, lkv = seq_lengths(cu_q), seq_lengths(cu_kv)
    for a, c in zip(lq.tolist(), lkv.tolist()):
        for r0 in range(0, a, 4096):
            total += int(admit_mask(a, c, mode, pre, nxt, np.arange(r0, min(a, r0 + 4096))).sum())
    return total
