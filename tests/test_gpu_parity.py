"""GPU parity: the HIP library against the fp64 oracle, element by element.

Tolerances (per output tensor, over every element compared):
  relative Frobenius error <= 1e-5 for fp32 inputs, <= 1e-2 for bf16 / fp16;
  max |gpu - oracle| <= 5e-2 * max |oracle|.
Inputs come from the seeded generator; Y and the statistics from the oracle's
forward (small cases, and workloads 2 and 5 at their exact shapes, compared over
whole tensors) or from a plain torch forward on the device (workloads 3 and 4,
compared on two complete (sequence, head) units plus sampled rows and keys of
every head).  Outputs are NaN-poisoned before each call, so an element the
library does not write fails.
"""
import os
import time

import numpy as np
import pytest
import torch

from gpu_common import assert_close, gpu_backward, log, make, oracle_backward, run_small
from progress import progress
from oracle import fa_oracle as O
from variable_length_flashattention_fa_amd import binding as B
from variable_length_flashattention_fa_amd import synth
from inputs_forward import forward_stats

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


# --- the five workloads at oracle-sized shapes ---------------------------------------------

def test_workload1_tiny_fp32_exact_shape():
    wl = synth.workload(1)
    run_small(synth.make(wl), wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)


@pytest.mark.parametrize("number,max_len,seqs,heads", [(2, 700, 4, 2), (3, 1000, 2, 2), (4, 2600, 2, 1),
                                                       (5, 600, 6, 3)])
def test_workloads_shrunk(number, max_len, seqs, heads):
    wl = synth.shrunk(synth.workload(number), max_len, seqs, heads)
    run_small(synth.make(wl), wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)


# --- edge cases -------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("dim", [64, 128])
def test_ragged_lengths_causal(dtype, dim):
    lens = (1, 2, 63, 64, 65, 127, 129, 0, 200)
    inp = make(lens, 2, dim, dtype, mode=O.MASK_CAUSAL, seed=7)
    run_small(inp, O.MASK_CAUSAL)


@pytest.mark.parametrize("mode,pre,nxt", [(O.MASK_NONE, 0, 0), (O.MASK_CAUSAL, 0, 0), (O.MASK_BAND, 37, 5),
                                          (O.MASK_BAND, -3, 10), (O.MASK_BAND, 200, 150)])
def test_unequal_q_kv_lengths(mode, pre, nxt):
    lq, lk = (100, 300, 0, 50, 130), (300, 100, 40, 0, 129)
    inp = make(lq, 2, 128, "bf16", mode=mode, pre=pre, nxt=nxt, seed=8, kv_lens=lk)
    run_small(inp, mode, pre, nxt)


def test_empty_rows_with_poisoned_stats():
    # Lq > Lkv under bottom-right causal: the first Lq - Lkv rows see no key
    lq, lk = (200, 90), (70, 90)
    inp = make(lq, 2, 128, "bf16", mode=O.MASK_CAUSAL, seed=9, kv_lens=lk)
    (dq, _, _), _, _ = run_small(inp, O.MASK_CAUSAL, poison_empty=True)
    assert torch.all(dq[:130] == 0)


def test_dropout_fp16_and_bf16():
    for dtype in ("fp16", "bf16"):
        inp = make((333, 64, 129, 1), 3, 128, dtype, mode=O.MASK_CAUSAL, kp=0.8, seed=10)
        run_small(inp, O.MASK_CAUSAL, kp=0.8)


def test_dropout_band_unaligned_bits():
    inp = make((77, 191, 5), 2, 64, "fp16", mode=O.MASK_BAND, pre=40, nxt=9, kp=0.7, seed=11, kv_lens=(81, 150, 13))
    run_small(inp, O.MASK_BAND, 40, 9, kp=0.7)


@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("fp16", 64)])
def test_dropout_mask_ends_inside_tile_records(dtype, dim):
    # The last sequence has 70 queries and 5 keys, so its rows sit 5 bits apart at the very end of the
    # mask: the keep-bit records of both of its query tiles reach past the mask's last byte (the
    # kernel then loads them byte by byte), one tile right after the other.
    inp = make((100, 70), 2, dim, dtype, mode=O.MASK_NONE, kp=0.7, seed=14, kv_lens=(90, 5))
    run_small(inp, O.MASK_NONE, kp=0.7)


def test_dropout_bits_at_masked_positions_are_ignored():
    lens = (150, 70)
    kp = 0.75
    inp = make(lens, 2, 128, "bf16", mode=O.MASK_CAUSAL, kp=kp, seed=12)
    got, ref, (yt, smax, ssum) = run_small(inp, O.MASK_CAUSAL, kp=kp)
    bits = np.unpackbits(inp.drop_mask, bitorder="little")
    pos = 0
    for L in lens:
        a = O.admit_mask(L, L, O.MASK_CAUSAL)
        for _ in range(2):
            blk = bits[pos:pos + L * L].reshape(L, L)
            blk[~a] ^= 1
            pos += L * L
    inp.drop_mask = np.packbits(bits, bitorder="little")
    got2 = gpu_backward(inp, yt, smax, ssum, O.MASK_CAUSAL, 0, 0, kp, 1.0 / np.sqrt(128))
    assert torch.equal(got2[1], got[1]) and torch.equal(got2[2], got[2])  # dK, dV: no atomics
    assert_close("dq", got2[0].double().numpy(), ref[0], torch.bfloat16)


def test_non_contiguous_views():
    inp = make((90, 130), 2, 64, "bf16", mode=O.MASK_CAUSAL, seed=13)

    def views(x):
        # a [T, N, D] view into a [T, N, 2D] buffer (head and token strides not packed)
        big = torch.zeros(x.shape[0], x.shape[1], 2 * x.shape[2], dtype=x.dtype, device=x.device)
        big[:, :, 32:32 + x.shape[2]] = x
        return big[:, :, 32:32 + x.shape[2]]

    run_small(inp, O.MASK_CAUSAL, views=views)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_negative_scale(dtype):
    inp = make((130, 77, 300), 2, 64, dtype, mode=O.MASK_BAND, pre=60, nxt=5, seed=17)
    run_small(inp, O.MASK_BAND, 60, 5, scale=-0.09)


def test_single_token_sequences():
    # P = 1, so dV = dY and dQ = dK = 0 up to rounding: the kernels form P = exp2(S * scale *
    # log2(e) - beta) with the scale folded into the K (or Q) operand before its bf16 rounding, so
    # P is 1 only to within that rounding (about 2^-9 * |S * scale * log2(e)| in the exponent)
    # (each product Q_d K_d c moves by at most 2^-8 of itself, so |log2 P| <= 2^-8 c sum_d |Q_d K_d|),
    # and dV is rounded to bf16 once more (2^-8 relative)
    inp = make((1, 1, 1, 1), 2, 128, "bf16", mode=O.MASK_CAUSAL, seed=14)
    (dq, dk, dv), _, _ = run_small(inp, O.MASK_CAUSAL)
    q, k, dy = (x.double() for x in (inp.q, inp.k, inp.dy))
    c = (1.0 / np.sqrt(128)) * np.log2(np.e)
    p_dev = torch.exp2(2.0 ** -8 * c * (q * k).abs().sum(-1, keepdim=True)) - 1.0  # per token and head
    bound = (p_dev + 2.0 ** -8 * (1 + p_dev)) * dy.abs()
    assert torch.all((dv.double() - dy).abs() <= bound)


def test_page_example_closed_form():
    # the page's call example: all-ones fp32 inputs, stats 3.0, T = 256, N = 1, D = 128
    dev = torch.device(DEV)
    ones = torch.ones(256, 1, 128, dtype=torch.float32, device=dev)
    smax = torch.full((1, 256, 8), 3.0, device=dev)
    ssum = torch.full((1, 256, 8), 3.0, device=dev)
    dq, dk, dv = (torch.empty_like(ones) for _ in range(3))
    B.fa_varlen_bwd(ones, ones, ones, ones, ones, smax, ssum, [0, 256], [0, 256], O.MASK_BAND, 65536, 65536, 1.0,
                    None, 0.088388, 1, dq, dk, dv)
    torch.cuda.synchronize()
    expect = 256 * np.exp(0.088388 * 128 - 3) / 3
    assert torch.all(dq == 0) and torch.all(dk == 0)
    assert np.allclose(dv.cpu().numpy(), expect, rtol=1e-5)


@pytest.mark.parametrize("dtype,kv_heads,dim_v,kp", [("bf16", 2, 128, 1.0), ("fp16", 1, 64, 0.8),
                                                      ("fp32", 2, 128, 0.8), ("fp32", 4, 64, 1.0)])
def test_repeated_calls_are_bitwise_identical(dtype, kv_heads, dim_v, kp):
    # deterministic on every path: no atomics, one owner per output row, fixed summation order
    # (grouped heads sum their group in a fixed order inside one workgroup)
    inp = make((400, 257, 3), 4, 128, dtype, mode=O.MASK_CAUSAL, kp=kp, seed=15, kv_heads=kv_heads, dim_v=dim_v)
    got, ref, (yt, smax, ssum) = run_small(inp, O.MASK_CAUSAL, kp=kp)
    for _ in range(3):
        again = gpu_backward(inp, yt, smax, ssum, O.MASK_CAUSAL, 0, 0, kp, 1.0 / np.sqrt(128))
        for a, b in zip(again, got):
            assert torch.equal(a, b)


def test_packed_equals_per_sequence():
    lens = (300, 45, 190)
    inp = make(lens, 2, 128, "bf16", mode=O.MASK_CAUSAL, seed=16)
    got, ref, (yt, smax, ssum) = run_small(inp, O.MASK_CAUSAL)
    for b in range(3):
        s = slice(int(inp.cu_q[b]), int(inp.cu_q[b + 1]))
        sub = synth.Inputs(inp.wl, inp.q[s], inp.k[s], inp.v[s], inp.dy[s], np.array([0, lens[b]]),
                           np.array([0, lens[b]]))
        g = gpu_backward(sub, yt[s], smax[:, s], ssum[:, s], O.MASK_CAUSAL, 0, 0, 1.0, 1.0 / np.sqrt(128))
        assert torch.equal(g[1], got[1][s]) and torch.equal(g[2], got[2][s])
        assert_close("dq", g[0].double().numpy(), ref[0][s], torch.bfloat16)


# --- full-size workloads ---------------------------------------------------------------------

def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


@pytest.mark.parametrize("number", [2, 5])
def test_full_size_whole_tensors(number):
    """Workloads 2 and 5 at their exact shapes: Y and the statistics from the oracle forward, then
    dQ, dK and dV compared with the oracle over every element (relative Frobenius error and max
    abs error per tensor, the stated criterion)."""
    t0 = time.time()
    wl = synth.workload(number)
    inp = synth.make(wl)
    w = _workers()
    progress(f"full-size workload {number} ({wl.name}): T={inp.q.shape[0]} N={wl.heads}; oracle forward on {w} workers")
    q, k, v = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v))
    y, m, l = O.forward(q, k, v, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt, keep_prob=wl.keep_prob,
                        drop_mask=inp.drop_mask, scale=wl.scale, head_num=wl.heads, workers=w)
    yt = torch.from_numpy(y).to(wl.torch_dtype)
    smax, ssum = O.stats_to_page_layout(m, l)
    del y, m, l
    progress(f"  forward done {time.time() - t0:.1f}s; GPU backward (outputs NaN-poisoned)")
    got = gpu_backward(inp, yt, smax, ssum, wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)
    progress(f"  GPU done {time.time() - t0:.1f}s; oracle backward on {w} workers")
    # The oracle runs in chunks of (sequence, head) units, longest first, so that a line appears
    # every few tens of seconds.  Each call fills only its units (zeros elsewhere) and adds the
    # grouped heads' dK / dV, so the chunks' results sum to the whole.
    lens_q, lens_k = np.diff(inp.cu_q), np.diff(inp.cu_kv)
    units = sorted(((b, n) for b in range(len(lens_q)) for n in range(wl.heads) if lens_q[b] > 0 and lens_k[b] > 0),
                   key=lambda u: -int(lens_q[u[0]]) * int(lens_k[u[0]]))
    cost = np.cumsum([int(lens_q[b]) * int(lens_k[b]) for b, _ in units])
    chunks = np.searchsorted(cost, cost[-1] * np.arange(1, 8) / 8, side="left")
    bounds = [0] + sorted(set(int(c) + 1 for c in chunks if c + 1 < len(units))) + [len(units)]
    y64 = synth.as_float_array(yt)
    q64, k64, v64, dy64 = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v, inp.dy))
    ref = None
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        part = O.backward(q64, k64, v64, dy64, y64, smax, ssum, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre,
                          nxt=wl.nxt, keep_prob=wl.keep_prob, drop_mask=inp.drop_mask, scale=wl.scale,
                          head_num=wl.heads, workers=w, units=units[c0:c1])
        ref = part if ref is None else tuple(r + s for r, s in zip(ref, part))
        progress(f"  oracle units {c1} of {len(units)} done {time.time() - t0:.1f}s")
    for name, g, o in zip(("dq", "dk", "dv"), got, ref):
        assert_close(name, g.double().numpy(), o, wl.torch_dtype)
    progress(f"  workload {number} whole-tensor parity ok ({time.time() - t0:.1f}s)")


@pytest.mark.parametrize("number", [3, 4])
def test_full_size_complete_units_and_every_head(number):
    """Workloads 3 and 4 at their exact shapes (Y and statistics from a torch fp32 forward on the
    device).  Compared with the oracle: two complete (sequence, head) units, every row of dQ and
    every key of dK / dV; and, for every head, sampled rows and keys, including the shortest items
    of both work lists (the first query blocks and the last key blocks of each sequence, which the
    work-list order runs last within each sequence) and the tile and block edges."""
    t0 = time.time()
    wl = synth.workload(number)
    progress(f"full-size workload {number} ({wl.name}): generating inputs")
    inp = synth.make(wl)
    dev = torch.device(DEV)
    q, k, v, dy = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dy))
    drop = torch.from_numpy(inp.drop_mask).to(dev) if inp.drop_mask is not None else None
    progress(f"  inputs ready {time.time() - t0:.1f}s; device forward for Y and statistics")
    y, smax, ssum = forward_stats(q, k, v, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt,
                                  keep_prob=wl.keep_prob, drop_mask=drop, scale=wl.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for t in (dq, dk, dv):
        t.fill_(float("nan"))  # every element must be written
    B.fa_varlen_bwd(q, k, v, dy, y, smax, ssum, inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt, wl.keep_prob, drop,
                    wl.scale, wl.heads, dq, dk, dv)
    torch.cuda.synchronize()
    progress(f"  backward done {time.time() - t0:.1f}s; comparing with the oracle")
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(t.float()).all(), f"{name}: unwritten or non-finite elements"
    yh, smh, ssh = synth.as_float_array(y.cpu()), smax.cpu().numpy(), ssum.cpu().numpy()
    qh, kh, vh, dyh = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v, inp.dy))
    del q, k, v, dy, y, smax, ssum
    lens = np.diff(inp.cu_q)
    nb = len(lens)
    kw = dict(mode=wl.mode, pre=wl.pre, nxt=wl.nxt, keep_prob=wl.keep_prob, drop_mask=inp.drop_mask,
              scale=wl.scale, head_num=wl.heads)
    # two complete units
    units = [(0, 0), (nb - 1, wl.heads - 1)]
    ref = O.backward(qh, kh, vh, dyh, yh, smh, ssh, inp.cu_q, inp.cu_kv, units=units, workers=len(units), **kw)
    for b, n in units:
        sq = slice(int(inp.cu_q[b]), int(inp.cu_q[b + 1]))
        sk = slice(int(inp.cu_kv[b]), int(inp.cu_kv[b + 1]))
        log(f"  complete unit (sequence {b}, head {n}), {lens[b]} rows and keys")
        assert_close(f"dq[{b},{n}]", dq[sq, n].double().numpy(), ref[0][sq, n], wl.torch_dtype)
        assert_close(f"dk[{b},{n}]", dk[sk, n].double().numpy(), ref[1][sk, n], wl.torch_dtype)
        assert_close(f"dv[{b},{n}]", dv[sk, n].double().numpy(), ref[2][sk, n], wl.torch_dtype)
    del ref
    progress(f"  complete units ok {time.time() - t0:.1f}s; sampled rows and keys of every head")
    rng = np.random.default_rng(1000 + number)
    gq, oq, gk, ok_, gv, ov = [], [], [], [], [], []
    for n in range(wl.heads):
        b = int(rng.integers(nb))
        L = int(lens[b])
        edges = [0, 1, 2, 3, 63, 64, 127, 128, 255, 256, L // 2, L - 129, L - 128, L - 65, L - 64, L - 4, L - 3,
                 L - 2, L - 1]
        if wl.mode == O.MASK_BAND:
            edges += [wl.pre - 1, wl.pre, wl.pre + 1, wl.pre + 64, L - wl.pre - 1, L - wl.pre]
        idx = np.unique(np.clip(np.concatenate([edges, rng.integers(0, L, 6)]), 0, L - 1))
        oq.append(O.backward_dq_rows(qh, kh, vh, dyh, yh, smh, ssh, inp.cu_q, inp.cu_kv, b, n, idx, **kw))
        gq.append(dq[inp.cu_q[b] + idx, n].double().numpy())
        a, c = O.backward_dkdv_cols(qh, kh, vh, dyh, yh, smh, ssh, inp.cu_q, inp.cu_kv, b, n, idx, **kw)
        ok_.append(a)
        ov.append(c)
        gk.append(dk[inp.cu_kv[b] + idx, n].double().numpy())
        gv.append(dv[inp.cu_kv[b] + idx, n].double().numpy())
        if n % 8 == 7:
            progress(f"  sampled heads {n + 1} of {wl.heads} done {time.time() - t0:.1f}s")
    for name, g, o in (("dq", gq, oq), ("dk", gk, ok_), ("dv", gv, ov)):
        assert_close(f"{name} (every head, sampled)", np.concatenate(g), np.concatenate(o), wl.torch_dtype)
    progress(f"  workload {number} full-size parity ok ({time.time() - t0:.1f}s)")
