"""GPU parity of the varlen forward (Y, softmaxMax, softmaxSum) against the fp64 oracle.

Y is held to the backward's bar: relative Frobenius error <= 1e-5 (fp32) or 1e-2 (bf16 / fp16)
and max-abs error <= 5e-2 max|ref|.  The statistics: max within 1e-4 (absolute, natural units)
and sum within a relative 1e-5 (fp32) or 1e-3 (bf16 / fp16); rows without an admitted key must
give exactly max = -inf, sum = 0 and Y = 0.
"""
import numpy as np
import pytest
import torch

from gpu_common import assert_close, log, make
from oracle import fa_oracle as O
from variable_length_flashattention_fa_amd import binding as B
from variable_length_flashattention_fa_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_forward(inp, mode, pre, nxt, kp, scale, views=None, atten_mask=None):
    dev = torch.device(DEV)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    drop = torch.from_numpy(inp.drop_mask).to(dev) if inp.drop_mask is not None else None
    y = torch.empty(q.shape[0], q.shape[1], v.shape[2], dtype=q.dtype, device=dev)  # v's head dim
    if views is not None:
        q, k, v, y = (views(x) for x in (q, k, v, y))
    smax = torch.empty(q.shape[1], q.shape[0], 8, dtype=torch.float32, device=dev)
    ssum = torch.empty_like(smax)
    for t in (y, smax, ssum):
        t.fill_(float("nan"))  # every element must be written
    if atten_mask is None:
        B.fa_varlen_fwd(q, k, v, inp.cu_q, inp.cu_kv, mode, pre, nxt, kp, drop, scale, q.shape[1], y, smax, ssum)
    else:
        am = torch.from_numpy(np.ascontiguousarray(atten_mask)).to(dev)
        B.fa_varlen_fwd_masked(q, k, v, inp.cu_q, inp.cu_kv, mode, pre, nxt, kp, drop, am, scale, q.shape[1], y,
                               smax, ssum)
    torch.cuda.synchronize()
    return y.cpu(), smax.cpu().numpy(), ssum.cpu().numpy()


def check_stats(gm, gl, m, l, dtype):
    """gm, gl: [N, T, 8] from the GPU; m, l: [N, T] (or rows) from the oracle."""
    assert np.all(gm == gm[..., :1]) and np.all(gl == gl[..., :1]), "statistics not repeated over the last axis"
    gm, gl = gm[..., 0].astype(np.float64), gl[..., 0].astype(np.float64)
    empty = ~np.isfinite(m)
    assert np.array_equal(empty, ~np.isfinite(gm)), "rows without keys differ"
    assert np.all(gm[empty] == -np.inf) and np.all(gl[empty] == 0.0)
    np.testing.assert_allclose(gm[~empty], m[~empty], rtol=0, atol=1e-4)
    np.testing.assert_allclose(gl[~empty], l[~empty], rtol=1e-5 if dtype == torch.float32 else 1e-3, atol=0)


def run_fwd(inp, mode, pre=0, nxt=0, kp=1.0, scale=None, views=None, atten_mask=None):
    scale = scale if scale is not None else 1.0 / np.sqrt(inp.q.shape[2])
    log(f"forward T={inp.q.shape[0]} N={inp.q.shape[1]} D={inp.q.shape[2]} {inp.q.dtype} mode={mode} "
        f"pre={pre} nxt={nxt} kp={kp} lens={np.diff(inp.cu_q).tolist()[:12]}")
    q, k, v = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v))
    y, m, l = O.forward(q, k, v, inp.cu_q, inp.cu_kv, mode=mode, pre=pre, nxt=nxt, keep_prob=kp,
                        drop_mask=inp.drop_mask, scale=scale, head_num=inp.q.shape[1], atten_mask=atten_mask)
    gy, gm, gl = gpu_forward(inp, mode, pre, nxt, kp, scale, views=views, atten_mask=atten_mask)
    assert_close("y", gy.double().numpy(), y, inp.q.dtype)
    check_stats(gm, gl, m, l, inp.q.dtype)
    empty = ~np.isfinite(m)  # [N, T]
    if empty.any():
        ys = gy.double().numpy().transpose(1, 0, 2)[empty]
        assert np.all(ys == 0.0), "rows without keys must give Y = 0"
    return gy, gm, gl


def test_forward_workload1_tiny_fp32():
    wl = synth.workload(1)
    run_fwd(synth.make(wl), wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)


@pytest.mark.parametrize("number,max_len,seqs,heads", [(2, 700, 4, 2), (3, 1000, 2, 2), (4, 2600, 2, 1),
                                                       (5, 600, 6, 3)])
def test_forward_workloads_shrunk(number, max_len, seqs, heads):
    wl = synth.shrunk(synth.workload(number), max_len, seqs, heads)
    run_fwd(synth.make(wl), wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("dim", [64, 128])
def test_forward_ragged_lengths_causal(dtype, dim):
    inp = make((1, 2, 63, 64, 65, 127, 129, 0, 200), 2, dim, dtype, mode=O.MASK_CAUSAL, seed=7)
    run_fwd(inp, O.MASK_CAUSAL)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode,pre,nxt", [(O.MASK_NONE, 0, 0), (O.MASK_CAUSAL, 0, 0), (O.MASK_BAND, 37, 5),
                                          (O.MASK_BAND, -3, 10), (O.MASK_BAND, 200, 150)])
def test_forward_unequal_q_kv_lengths(dtype, mode, pre, nxt):
    # causal with Lq > Lkv and the narrow band leave rows without keys
    inp = make((300, 100, 70), 2, 128, dtype, mode=mode, pre=pre, nxt=nxt, seed=3, kv_lens=(100, 300, 33))
    run_fwd(inp, mode, pre, nxt)


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_forward_dropout(dtype):
    inp = make((130, 77, 300), 3, 128, dtype, mode=O.MASK_CAUSAL, kp=0.8, seed=11)
    run_fwd(inp, O.MASK_CAUSAL, kp=0.8)


@pytest.mark.parametrize("dtype,dim", [("bf16", 128), ("fp16", 64)])
def test_forward_dropout_mask_ends_inside_tile_records(dtype, dim):
    # The last sequence has 70 queries and 5 keys, so its rows sit 5 bits apart at the very end of the
    # mask: the keep-bit records of its rows reach past the mask's last byte (the kernel then loads
    # them byte by byte), in several waves of the workgroup at once.
    inp = make((100, 70), 2, dim, dtype, mode=O.MASK_NONE, kp=0.7, seed=15, kv_lens=(90, 5))
    run_fwd(inp, O.MASK_NONE, kp=0.7)


def test_forward_dropout_band_unaligned_bits():
    inp = make((93, 45, 257), 2, 64, "bf16", mode=O.MASK_BAND, pre=40, nxt=7, kp=0.7, seed=12,
               kv_lens=(101, 38, 255))
    run_fwd(inp, O.MASK_BAND, 40, 7, kp=0.7)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("scale", [-0.07, 0.0])
def test_forward_negative_and_zero_scale(dtype, scale):
    # a negative scale turns the row max into the row min of the raw scores; a zero scale makes
    # every admitted key equally likely
    inp = make((100, 257, 1, 64), 2, 128, dtype, mode=O.MASK_CAUSAL, seed=13)
    run_fwd(inp, O.MASK_CAUSAL, scale=scale)


def test_forward_non_contiguous_views():
    inp = make((90, 200), 2, 128, "bf16", mode=O.MASK_CAUSAL, seed=5)

    def views(t):  # the same values with a head stride of 2 * D and a token stride of 4 * D
        big = torch.zeros(t.shape[0], t.shape[1] * 2, t.shape[2], dtype=t.dtype, device=t.device)
        big[:, ::2] = t
        return big[:, ::2]

    run_fwd(inp, O.MASK_CAUSAL, views=views)


def test_forward_then_backward_matches_oracle():
    """Our forward's Y and statistics feed our backward; the result matches the oracle end to end."""
    wl = synth.shrunk(synth.workload(5), 500, 4, 2)
    inp = synth.make(wl)
    gy, gm, gl = gpu_forward(inp, wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)
    dev = torch.device(DEV)
    q, k, v, dy = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dy))
    drop = torch.from_numpy(inp.drop_mask).to(dev) if inp.drop_mask is not None else None
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B.fa_varlen_bwd(q, k, v, dy, gy.to(dev), torch.from_numpy(gm).to(dev), torch.from_numpy(gl).to(dev),
                    inp.cu_q, inp.cu_kv, wl.mode, wl.pre, wl.nxt, wl.keep_prob, drop, wl.scale, q.shape[1],
                    dq, dk, dv)
    torch.cuda.synchronize()
    qf, kf, vf, dyf = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v, inp.dy))
    y, m, l = O.forward(qf, kf, vf, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt,
                        keep_prob=wl.keep_prob, drop_mask=inp.drop_mask, scale=wl.scale, head_num=q.shape[1])
    ref = O.backward(qf, kf, vf, dyf, y, m, l, inp.cu_q, inp.cu_kv, mode=wl.mode, pre=wl.pre, nxt=wl.nxt,
                     keep_prob=wl.keep_prob, drop_mask=inp.drop_mask, scale=wl.scale, head_num=q.shape[1])
    for name, g, o in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert_close(name, g.cpu().double().numpy(), o, inp.q.dtype)


@pytest.mark.parametrize("number", [2, 3, 4, 5])
def test_forward_full_size_sampled(number):
    """The full workload on the GPU; the oracle checks sampled rows of a few (sequence, head) units."""
    wl = synth.workload(number)
    inp = synth.make(wl)
    gy, gm, gl = gpu_forward(inp, wl.mode, wl.pre, wl.nxt, wl.keep_prob, wl.scale)
    q, k, v = (synth.as_float_array(x) for x in (inp.q, inp.k, inp.v))
    rng = np.random.default_rng(100 + number)
    nb = len(inp.cu_q) - 1
    for b in sorted(set([0, nb - 1, int(rng.integers(nb))])):
        lq = int(inp.cu_q[b + 1] - inp.cu_q[b])
        for n in sorted(set([0, wl.heads - 1])):
            rows = np.unique(np.concatenate([[0, lq - 1], rng.integers(0, lq, 6)]))
            y, m, l = O.forward_rows(q, k, v, inp.cu_q, inp.cu_kv, b, n, rows, mode=wl.mode, pre=wl.pre,
                                     nxt=wl.nxt, keep_prob=wl.keep_prob, drop_mask=inp.drop_mask, scale=wl.scale,
                                     head_num=wl.heads)
            t = inp.cu_q[b] + rows
            assert_close(f"y[b={b},n={n}]", gy[t, n].double().numpy(), y, inp.q.dtype)
            check_stats(gm[n, t][None], gl[n, t][None], m[None], l[None], inp.q.dtype)
