"""Helpers shared by the GPU test modules (not a test module itself)."""
import sys

import numpy as np
import torch

from oracle import fa_oracle as O
from variable_length_flashattention_fa_amd import binding as B
from variable_length_flashattention_fa_amd import synth

DEV = "cuda:0"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def tol_for(dtype):
    return 1e-5 if dtype == torch.float32 else 1e-2


def assert_close(name, g, o, dtype, zero_bound=0.0):
    """The parity criterion on one output tensor: relative Frobenius error <= 1e-5 (fp32) or 1e-2
    (bf16 / fp16) and max |gpu - oracle| <= 5e-2 * max |oracle|.

    For an all-zero oracle tensor the relative criterion is undefined: every GPU value must then
    lie within `zero_bound` of zero (0: exact zeros; see cancellation_bound for the one case where
    the oracle's zero is an exact cancellation the GPU reproduces only up to fp32 rounding)."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values (unwritten or overflowed elements)"
    ref = np.linalg.norm(o)
    err = np.linalg.norm(g - o)
    mx = np.max(np.abs(o)) if o.size else 0.0
    if ref == 0.0:
        got = np.max(np.abs(g)) if g.size else 0.0
        assert got <= zero_bound, f"{name}: expected zeros (bound {zero_bound:.3e}), max |gpu| = {got:.3e}"
        return
    rel = err / ref
    log(f"  {name}: relative Frobenius error {rel:.3e}, max abs error {np.max(np.abs(g - o)):.3e} "
        f"(max |ref| {mx:.3e})")
    assert rel <= tol_for(dtype), f"{name}: relative Frobenius error {rel:.3e}"
    assert np.max(np.abs(g - o)) <= 5e-2 * mx, f"{name}: max abs error {np.max(np.abs(g - o)):.3e} vs {mx:.3e}"


def cancellation_bound(inp, scale, rows_per_key=1):
    """Bound on |dQ| and |dK| where the oracle's dS is exactly zero because dP_ij = D_i.

    That happens when a row's admitted keys all carry the same V row as Y (e.g. one-token
    sequences: P = 1, Y = V_j).  The GPU forms dP_ij = dY_i . V_j with the matrix cores and D_i =
    dY_i . Y_i in its row pass: two fp32 sums of the same Dv products in different orders, each
    within gamma = Dv * 2^-24 * sum_d |dY_id V_jd| <= gamma * ||dY_i|| ||V_j|| of the exact value,
    so |dP - D| <= 2 gamma ||dY_i|| ||V_j||.  Then |dQ_i| = |scale| |sum_j P_ij (dP - D)_ij K_j|
    <= |scale| max |dP - D| max |K| (the P_ij sum to 1), and |dK_j| <= |scale| rows_per_key
    max |dP - D| max |Q| (rows_per_key bounds sum_i P_ij).  Returned as (dq_bound, dk_bound)."""
    f = lambda t: synth.as_float_array(t)  # noqa: E731
    q, k, v, dy = f(inp.q), f(inp.k), f(inp.v), f(inp.dy)
    dv_dim = v.shape[2]
    gamma = dv_dim * 2.0 ** -24
    r = 2.0 * gamma * np.max(np.linalg.norm(dy, axis=2)) * np.max(np.linalg.norm(v, axis=2))
    return abs(scale) * r * np.max(np.abs(k)), abs(scale) * rows_per_key * r * np.max(np.abs(q))


def oracle_forward(inp, mode, pre, nxt, kp, scale, atten_mask=None):
    q, k, v = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v))
    y, m, l = O.forward(q, k, v, inp.cu_q, inp.cu_kv, mode=mode, pre=pre, nxt=nxt, keep_prob=kp,
                        drop_mask=inp.drop_mask, scale=scale, head_num=inp.q.shape[1], atten_mask=atten_mask)
    yt = torch.from_numpy(y).to(inp.q.dtype)
    smax, ssum = O.stats_to_page_layout(m, l)
    return yt, smax, ssum


def oracle_backward(inp, yt, smax, ssum, mode, pre, nxt, kp, scale, workers=4, atten_mask=None):
    q, k, v, dy = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v, inp.dy))
    y = synth.as_float_array(yt)
    return O.backward(q, k, v, dy, y, smax, ssum, inp.cu_q, inp.cu_kv, mode=mode, pre=pre, nxt=nxt,
                      keep_prob=kp, drop_mask=inp.drop_mask, scale=scale, head_num=inp.q.shape[1],
                      workers=workers, atten_mask=atten_mask)


def gpu_backward(inp, yt, smax, ssum, mode, pre, nxt, kp, scale, views=None, atten_mask=None):
    dev = torch.device(DEV)
    q, k, v, dy, y = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dy, yt))
    smax_d = torch.as_tensor(np.ascontiguousarray(smax)).to(dev)
    ssum_d = torch.as_tensor(np.ascontiguousarray(ssum)).to(dev)
    drop = torch.from_numpy(inp.drop_mask).to(dev) if inp.drop_mask is not None else None
    if views is not None:
        q, k, v, dy, y = (views(x) for x in (q, k, v, dy, y))
        dq, dk, dv = views(torch.empty_like(q)), views(torch.empty_like(k)), views(torch.empty_like(v))
    else:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # poison the outputs: every element must be written by the library
    for t in (dq, dk, dv):
        t.fill_(float("nan"))
    if atten_mask is None:
        B.fa_varlen_bwd(q, k, v, dy, y, smax_d, ssum_d, inp.cu_q, inp.cu_kv, mode, pre, nxt, kp, drop, scale,
                        q.shape[1], dq, dk, dv)
    else:
        am = torch.from_numpy(np.ascontiguousarray(atten_mask)).to(dev)
        B.fa_varlen_bwd_masked(q, k, v, dy, y, smax_d, ssum_d, inp.cu_q, inp.cu_kv, mode, pre, nxt, kp, drop, am,
                               scale, q.shape[1], dq, dk, dv)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def run_small(inp, mode, pre=0, nxt=0, kp=1.0, scale=None, poison_empty=False, views=None, atten_mask=None):
    scale = scale if scale is not None else 1.0 / np.sqrt(inp.q.shape[2])
    log(f"case T={inp.q.shape[0]} N={inp.q.shape[1]} D={inp.q.shape[2]} {inp.q.dtype} mode={mode} "
        f"pre={pre} nxt={nxt} kp={kp} lens={np.diff(inp.cu_q).tolist()[:12]} "
        f"mask={None if atten_mask is None else atten_mask.shape}")
    yt, smax, ssum = oracle_forward(inp, mode, pre, nxt, kp, scale, atten_mask=atten_mask)
    if poison_empty:
        empty = ~np.isfinite(smax[:, :, 0]) | (ssum[:, :, 0] == 0)
        assert empty.any()
        smax = smax.copy(); ssum = ssum.copy()
        smax[empty] = np.nan
        ssum[empty] = np.nan
    ref = oracle_backward(inp, yt, smax, ssum, mode, pre, nxt, kp, scale, atten_mask=atten_mask)
    got = gpu_backward(inp, yt, smax, ssum, mode, pre, nxt, kp, scale, views=views, atten_mask=atten_mask)
    bq, bk = cancellation_bound(inp, scale, rows_per_key=int(np.max(np.diff(inp.cu_q))))
    for name, g, o, zb in zip(("dq", "dk", "dv"), got, ref, (bq, bk, 0.0)):
        assert_close(name, g.double().numpy(), o, inp.q.dtype, zero_bound=zb)
    return got, ref, (yt, smax, ssum)


def make(lens, heads, dim, dtype, mode=0, pre=0, nxt=0, kp=1.0, seed=0, kv_lens=None, dy_scale=0.1,
         kv_heads=None, dim_v=None):
    """Seeded inputs for an edge case (lengths, heads, head dims as given)."""
    wl = synth.Workload("edge", dtype, tuple(lens), heads, dim, mode, pre, nxt, kp, dy_scale, seed,
                        kv_lengths=None if kv_lens is None else tuple(kv_lens), kv_heads=kv_heads,
                        head_dim_v=dim_v)
    return synth.make(wl)
