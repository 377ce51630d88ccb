"""Helpers shared by the GPU test modules (not a test module itself)."""
import sys

import numpy as np
import torch

from variable_length_flashattention_fa_amd import synth


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def tol_for(dtype):
    return 1e-5 if dtype == torch.float32 else 1e-2


def assert_close(name, g, o, dtype):
    """Relative Frobenius error within tol_for(dtype) and max-abs error within 5e-2 max|ref|."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    ref = np.linalg.norm(o)
    if ref == 0.0:
        assert np.max(np.abs(g)) <= 1e-5, f"{name}: expected zeros, max |gpu| = {np.max(np.abs(g)):.3e}"
        return
    rel = np.linalg.norm(g - o) / ref
    mx = np.max(np.abs(o))
    assert rel <= tol_for(dtype), f"{name}: relative Frobenius error {rel:.3e}"
    assert np.max(np.abs(g - o)) <= 5e-2 * mx, f"{name}: max abs error {np.max(np.abs(g - o)):.3e} vs {mx:.3e}"


def make(lens, heads, dim, dtype, mode=0, pre=0, nxt=0, kp=1.0, seed=0, kv_lens=None, dy_scale=0.1):
    wl = synth.Workload("edge", dtype, tuple(lens), heads, dim, mode, pre, nxt, kp, dy_scale, seed,
                        kv_lengths=None if kv_lens is None else tuple(kv_lens))
    return synth.make(wl)
