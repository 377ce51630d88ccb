"""GPU parity for the explicit attention mask (uint8, 1 = excluded) against the fp64 oracle.

The mask intersects the window of the mask mode. Shapes [B, N, Sq, Skv], [B, 1, Sq, Skv],
[1, 1, Sq, Skv] and [Sq, Skv], with Sq / Skv larger than every sequence. Rows the mask empties
get zero gradients; their statistics are NaN-poisoned where the test says so. Same bar as the
other parity tests.
"""
import numpy as np
import pytest
import torch

from gpu_common import DEV, assert_close, gpu_backward, log, make, oracle_backward, oracle_forward, run_small
from oracle import fa_oracle as O
from test_gpu_forward import run_fwd
from variable_length_flashattention_fa_amd import binding as B
from variable_length_flashattention_fa_amd import synth

pytestmark = pytest.mark.gpu

LENS = (1, 63, 64, 65, 0, 129, 300)


def _shape(kind, batch, heads, sq, sk):
    return {"bnqk": (batch, heads, sq, sk), "b1qk": (batch, 1, sq, sk), "11qk": (1, 1, sq, sk),
            "qk": (sq, sk)}[kind]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("kind", ["bnqk", "qk"])
def test_explicit_mask_backward_no_window(dtype, kind):
    inp = make(LENS, 2, 128, dtype, seed=51)
    am = synth.explicit_mask(151, _shape(kind, len(LENS), 2, 310, 305), 0.3, empty_rows=(2,))
    run_small(inp, O.MASK_NONE, atten_mask=am)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode,pre,nxt", [(O.MASK_CAUSAL, 0, 0), (O.MASK_BAND, 40, 3)])
def test_explicit_mask_backward_with_window_dropout(dtype, mode, pre, nxt):
    inp = make((150, 77, 260), 4, 128, dtype, mode=mode, pre=pre, nxt=nxt, kp=0.8, seed=52, kv_heads=2,
               kv_lens=(170, 60, 255))
    am = synth.explicit_mask(152, _shape("b1qk", 3, 4, 270, 256), 0.2, empty_rows=(5,))
    run_small(inp, mode, pre, nxt, kp=0.8, atten_mask=am, poison_empty=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_explicit_mask_backward_head_dims(dtype):
    # D = 64 and the narrower V (128, 64)
    for dim, dim_v in ((64, 64), (128, 64)):
        inp = make((200, 33, 97), 2, dim, dtype, mode=O.MASK_CAUSAL, seed=53, dim_v=dim_v)
        am = synth.explicit_mask(153, _shape("11qk", 3, 2, 200, 200), 0.4)
        run_small(inp, O.MASK_CAUSAL, atten_mask=am)


def test_explicit_mask_backward_several_tiles():
    inp = make((1100, 700), 2, 128, "bf16", seed=54)
    am = synth.explicit_mask(154, _shape("bnqk", 2, 2, 1100, 1100), 0.1)
    run_small(inp, O.MASK_NONE, atten_mask=am)


def test_explicit_causal_pattern_matches_the_causal_mode():
    # the causal window written out as an explicit mask gives the causal mode's gradients: both
    # within the parity bar of the same oracle result (the two kernel variants round differently:
    # without a mask the softmax scale is folded into the K / Q operand before its rounding)
    lens = (300, 129, 64)
    inp = make(lens, 2, 128, "bf16", mode=O.MASK_CAUSAL, seed=55)
    sq = max(lens)
    am = np.ones((len(lens), 1, sq, sq), dtype=np.uint8)
    for b, L in enumerate(lens):
        am[b, 0, :L, :L] = ~O.admit_mask(L, L, O.MASK_CAUSAL)
    got_x, ref, (yt, smax, ssum) = run_small(inp, O.MASK_NONE, atten_mask=am)
    got_c = gpu_backward(inp, yt, smax, ssum, O.MASK_CAUSAL, 0, 0, 1.0, 1.0 / np.sqrt(128))
    for name, c, o in zip(("dq", "dk", "dv"), got_c, ref):
        assert_close(name, c.double().numpy(), o, torch.bfloat16)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("kind", ["bnqk", "b1qk", "qk"])
def test_explicit_mask_forward(dtype, kind):
    inp = make(LENS, 4, 128, dtype, mode=O.MASK_CAUSAL, seed=56, kv_heads=2)
    am = synth.explicit_mask(156, _shape(kind, len(LENS), 4, 300, 320), 0.3, empty_rows=(3,))
    run_fwd(inp, O.MASK_CAUSAL, atten_mask=am)


def test_explicit_mask_forward_dropout_band_narrow_v():
    inp = make((93, 210), 2, 128, "fp16", mode=O.MASK_BAND, pre=50, nxt=9, kp=0.75, seed=57, dim_v=64,
               kv_lens=(130, 180))
    am = synth.explicit_mask(157, (2, 2, 210, 180), 0.25)
    run_fwd(inp, O.MASK_BAND, 50, 9, kp=0.75, atten_mask=am)


def test_explicit_mask_forward_then_backward():
    inp = make((300, 520), 4, 128, "bf16", mode=O.MASK_CAUSAL, kp=0.9, seed=58, kv_heads=2)
    am_np = synth.explicit_mask(158, (2, 4, 520, 520), 0.2, empty_rows=(7,))
    scale = 1.0 / np.sqrt(128)
    dev = torch.device(DEV)
    q, k, v, dy = (x.to(dev) for x in (inp.q, inp.k, inp.v, inp.dy))
    drop = torch.from_numpy(inp.drop_mask).to(dev)
    am = torch.from_numpy(am_np).to(dev)
    log("explicit mask forward -> backward")
    y, smax, ssum = B.varlen_fwd(q, k, v, inp.cu_q, inp.cu_kv, atten_mode=O.MASK_CAUSAL, keep_prob=0.9,
                                 drop_mask=drop, scale=scale, atten_mask=am)
    dq, dk, dv = B.varlen_bwd(q, k, v, dy, y, smax, ssum, inp.cu_q, inp.cu_kv, atten_mode=O.MASK_CAUSAL,
                              keep_prob=0.9, drop_mask=drop, scale=scale, atten_mask=am)
    torch.cuda.synchronize()
    # the oracle's own chain: its forward's Y and statistics, then its backward
    yo, mo, lo = oracle_forward(inp, O.MASK_CAUSAL, 0, 0, 0.9, scale, atten_mask=am_np)
    ref = oracle_backward(inp, yo, mo, lo, O.MASK_CAUSAL, 0, 0, 0.9, scale, atten_mask=am_np)
    for name, g, o in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        assert_close(name, g.double().cpu().numpy(), o, torch.bfloat16)
