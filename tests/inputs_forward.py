"""Forward output Y and softmax statistics for large synthetic workloads.

The backward consumes the forward's output Y and its row max / row sum.  For
workloads where the fp64 CPU forward would take too long, this module produces
them on the GPU with plain torch fp32 matmuls, one sequence and a chunk of
query rows at a time.  It is input preparation for the tests' full-size checks and
for bench.py, outside any timed region; the library never calls it.

Definitions (formulas section of the "FlashAttention梯度V2" page):
S = scale * Q K^T restricted to admitted keys, m = row max, l = sum exp(S - m),
P = exp(S - m) / l, Y = (P o Z / keep_prob) V; rows with no admitted key get
m = -inf, l = 0, Y = 0.  Y is rounded to the input dtype, m and l to fp32 and
replicated into the [N, T, 8] layout the backward reads.
"""
from __future__ import annotations

import numpy as np
import torch

MASK_NONE, MASK_CAUSAL, MASK_BAND = 0, 1, 2


def _admit(rows: torch.Tensor, lkv: int, lq: int, mode: int, pre: int, nxt: int) -> torch.Tensor:
    j = torch.arange(lkv, device=rows.device, dtype=torch.int64)[None, :]
    i = rows[:, None]
    off = lkv - lq
    if mode == MASK_NONE:
        return torch.ones(rows.numel(), lkv, dtype=torch.bool, device=rows.device)
    if mode == MASK_CAUSAL:
        return j <= i + off
    return (j >= i + off - pre) & (j <= i + off + nxt)


@torch.no_grad()
def forward_stats(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_q, cu_kv, *, mode: int, pre: int = 0,
                  nxt: int = 0, keep_prob: float = 1.0, drop_mask: torch.Tensor | None = None, scale: float,
                  row_chunk: int = 2048):
    """Returns (y [T, N, Dv] in q.dtype, softmax_max [N, T, 8] fp32, softmax_sum [N, T, 8] fp32).

    k and v may hold fewer heads than q (a divisor of N): query head n reads key/value head
    n // (N / Nkv).  v may have a smaller head dim than q and k.
    """
    dev = q.device
    tq, heads, d = q.shape
    group = heads // k.shape[1]
    y = torch.zeros(tq, heads, v.shape[2], dtype=q.dtype, device=dev)
    mx = torch.full((heads, tq), float("-inf"), dtype=torch.float32, device=dev)
    sm = torch.zeros((heads, tq), dtype=torch.float32, device=dev)
    cu_q = [int(x) for x in cu_q]
    cu_kv = [int(x) for x in cu_kv]
    bit_base = 0
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_kv[b], cu_kv[b + 1]
        lq, lkv = q1 - q0, k1 - k0
        if lq == 0 or lkv == 0:
            bit_base += heads * lq * lkv
            continue
        qb = q[q0:q1].float().permute(1, 0, 2).contiguous()            # [N, Lq, D]
        kt = k[k0:k1].float().permute(1, 2, 0)                          # [Nkv, D, Lkv]
        vb = v[k0:k1].float().permute(1, 0, 2)                          # [Nkv, Lkv, Dv]
        if group > 1:
            kt = kt.repeat_interleave(group, dim=0)                     # [N, D, Lkv]
            vb = vb.repeat_interleave(group, dim=0)
        kt, vb = kt.contiguous(), vb.contiguous()
        for r0 in range(0, lq, row_chunk):
            r1 = min(lq, r0 + row_chunk)
            rows = torch.arange(r0, r1, device=dev, dtype=torch.int64)
            s = torch.matmul(qb[:, r0:r1].contiguous(), kt) * scale     # [N, rc, Lkv]
            adm = _admit(rows, lkv, lq, mode, pre, nxt)[None]
            s = s.masked_fill(~adm, float("-inf"))
            m = s.amax(dim=-1)                                           # -inf on empty rows
            m_safe = torch.where(torch.isfinite(m), m, torch.zeros_like(m))
            e = torch.exp(s - m_safe[..., None])
            del s
            l = e.sum(dim=-1)
            p = e / torch.where(l > 0, l, torch.ones_like(l))[..., None]
            del e
            if keep_prob < 1.0:
                hn = torch.arange(heads, device=dev, dtype=torch.int64)[:, None, None]
                bit = (bit_base + (hn * lq + rows[None, :, None]) * lkv
                       + torch.arange(lkv, device=dev, dtype=torch.int64)[None, None, :])
                z = (drop_mask[bit >> 3].to(torch.int32) >> (bit & 7).to(torch.int32)) & 1
                del bit
                p = p * (z.float() / keep_prob)
                del z
            yb = torch.matmul(p, vb)                                     # [N, rc, Dv]
            del p
            y[q0 + r0:q0 + r1] = yb.permute(1, 0, 2).to(q.dtype)
            mx[:, q0 + r0:q0 + r1] = m
            sm[:, q0 + r0:q0 + r1] = l
        bit_base += heads * lq * lkv
    smax = mx[:, :, None].expand(heads, tq, 8).contiguous()
    ssum = sm[:, :, None].expand(heads, tq, 8).contiguous()
    return y, smax, ssum


def pair_count(cu_q, cu_kv, mode: int, pre: int = 0, nxt: int = 0) -> int:
    """Admitted (query, key) pairs per head, in closed form per sequence."""
    total = 0
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_kv = np.asarray(cu_kv, dtype=np.int64)
    for lq, lkv in zip(np.diff(cu_q).tolist(), np.diff(cu_kv).tolist()):
        if lq == 0 or lkv == 0:
            continue
        off = lkv - lq
        if mode == MASK_NONE:
            total += lq * lkv
            continue
        lo_off, hi_off = (-(1 << 40), 0) if mode == MASK_CAUSAL else (-int(pre), int(nxt))
        # row i admits keys j in [i + off + lo_off, i + off + hi_off] clipped to [0, lkv - 1]
        i = np.arange(lq, dtype=np.int64)
        lo = np.maximum(i + off + lo_off, 0)
        hi = np.minimum(i + off + hi_off, lkv - 1)
        total += int(np.maximum(hi - lo + 1, 0).sum())
    return total
