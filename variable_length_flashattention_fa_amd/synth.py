"""Seeded synthetic workloads for the varlen attention backward.

This module only draws random numbers and lays them out: sequence lengths,
Q/K/V/dY values rounded to the working dtype, and the packed dropout keep
bits.  It holds none of the attention arithmetic, so the fp64 checker and the
HIP library can both consume its output without sharing any computation.

Recipe (seed = workload number unless given):
  1. lengths, drawn first from numpy.random.default_rng(seed);
  2. Q, K, V, each standard_normal((T, N, D)) in fp64 (K and V with the
     key/value head count and V with its own head dim when those differ);
  3. dY = standard_normal((T, N, Dv)) * dy_scale;
  4. with keep_prob < 1: for each sequence b, for each head n, a
     [Lq_b, Lkv_b] block of random() < keep_prob, concatenated in that order
     and packed least-significant-bit first into uint8;
  5. every fp64 draw is rounded to the dtype (round to nearest even).
Sequence lengths are equal for queries and keys (cu_q == cu_kv).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np
import torch

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_BAND = 2

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                 # "fp32" | "bf16" | "fp16"
    lengths: tuple             # per-sequence lengths (queries == keys)
    heads: int
    head_dim: int
    mode: int = MASK_NONE
    pre: int = 0
    nxt: int = 0
    keep_prob: float = 1.0
    dy_scale: float = 0.1
    seed: int = 0
    kv_lengths: Optional[tuple] = None   # only for edge cases with Lq != Lkv
    length_draw: Optional[tuple] = None  # how the lengths were drawn (first draw of the seed)
    kv_heads: Optional[int] = None       # key/value heads (grouped heads); None = heads
    head_dim_v: Optional[int] = None     # V head dim; None = head_dim

    @property
    def n_kv(self) -> int:
        return self.heads if self.kv_heads is None else self.kv_heads

    @property
    def dv(self) -> int:
        return self.head_dim if self.head_dim_v is None else self.head_dim_v

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        return _DTYPES[self.dtype]

    @property
    def tokens(self) -> int:
        return int(sum(self.lengths))

    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)

    def cu_kv(self) -> np.ndarray:
        lk = self.lengths if self.kv_lengths is None else self.kv_lengths
        return np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)


def _draw_lengths(rng, spec) -> tuple:
    kind = spec[0]
    if kind == "uniform":
        _, lo, hi, count = spec
        return tuple(int(x) for x in rng.integers(lo, hi, count, endpoint=True))
    if kind == "lognormal":
        _, mu, sigma, count, lo, hi = spec
        return tuple(int(x) for x in np.clip(np.rint(rng.lognormal(mu, sigma, count)), lo, hi))
    raise ValueError(spec)


def workload(number: int) -> Workload:
    """The five benchmark workloads, numbered 1..5 (lengths drawn from seed = number)."""
    rng = np.random.default_rng(number)
    uni = ("uniform", 256, 4096, 16)
    logn = ("lognormal", 7.0, 0.8, 32, 64, 8192)
    if number == 1:
        return Workload("tiny_fp32_2seq_none", "fp32", (37, 91), 2, 64, MASK_NONE,
                        dy_scale=1.0, seed=1)
    if number == 2:
        return Workload("bf16_causal_16seq_u256_4096", "bf16", _draw_lengths(rng, uni),
                        32, 128, MASK_CAUSAL, seed=2, length_draw=uni)
    if number == 3:
        return Workload("bf16_causal_4x16384", "bf16", (16384,) * 4, 16, 128, MASK_CAUSAL, seed=3)
    if number == 4:
        return Workload("bf16_band_8x8192_pre2048", "bf16", (8192,) * 8, 32, 128, MASK_BAND,
                        pre=2048, nxt=0, seed=4)
    if number == 5:
        return Workload("fp16_causal_dropout_32seq_lognormal", "fp16",
                        _draw_lengths(rng, logn), 24, 128, MASK_CAUSAL,
                        keep_prob=0.9, seed=5, length_draw=logn)
    raise ValueError(f"no workload {number}")


def shrunk(wl: Workload, max_len: int, max_seqs: int, heads: int) -> Workload:
    """A smaller workload of the same kind: the first sequences, lengths capped."""
    lens = tuple(min(int(x), max_len) for x in wl.lengths[:max_seqs])
    return replace(wl, name=wl.name + f"_shrunk{max_len}", lengths=lens, heads=heads)


@dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor            # [T, N, D] in the workload dtype (CPU)
    k: torch.Tensor
    v: torch.Tensor
    dy: torch.Tensor
    cu_q: np.ndarray           # int64 [B + 1]
    cu_kv: np.ndarray
    drop_mask: Optional[np.ndarray] = None   # uint8 packed bits, or None at keep_prob == 1
    extra: dict = field(default_factory=dict)


def _normal(rng, shape, dtype, mult=1.0):
    x = rng.standard_normal(shape)
    if mult != 1.0:
        x *= mult
    return torch.from_numpy(x).to(dtype)


def keep_bits(rng, lq: List[int], lkv: List[int], heads: int, keep_prob: float) -> np.ndarray:
    """Packed keep bits: per sequence, per head, a [Lq_b, Lkv_b] Bernoulli(keep_prob) block."""
    chunks = []
    carry = np.zeros(0, dtype=np.uint8)
    for a, c in zip(lq, lkv):
        for _ in range(heads):
            bits = (rng.random((a, c)) < keep_prob).astype(np.uint8).ravel()
            if carry.size:
                bits = np.concatenate([carry, bits])
            whole = (bits.size // 8) * 8
            chunks.append(np.packbits(bits[:whole], bitorder="little"))
            carry = bits[whole:]
    if carry.size:
        chunks.append(np.packbits(carry, bitorder="little"))
    if not chunks:
        return np.zeros(1, dtype=np.uint8)
    out = np.concatenate(chunks)
    return out if out.size else np.zeros(1, dtype=np.uint8)


def explicit_mask(seed: int, shape, frac: float, empty_rows=()) -> np.ndarray:
    """A seeded uint8 attention mask (1 = excluded) of the given shape: each element is 1 with
    probability frac; the rows listed in empty_rows (last-but-one axis) are excluded entirely."""
    rng = np.random.default_rng(seed)
    m = (rng.random(shape) < frac).astype(np.uint8)
    for r in empty_rows:
        m[..., r, :] = 1
    return m


def make(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the inputs of a workload on the CPU, following the recipe in the module docstring."""
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    if wl.length_draw is not None:
        _draw_lengths(rng, wl.length_draw)   # the lengths were this stream's first draw
    t = wl.tokens
    cu_q, cu_kv = wl.cu_q(), wl.cu_kv()
    tk = int(cu_kv[-1])
    dt = wl.torch_dtype
    q = _normal(rng, (t, wl.heads, wl.head_dim), dt)
    k = _normal(rng, (tk, wl.n_kv, wl.head_dim), dt)
    v = _normal(rng, (tk, wl.n_kv, wl.dv), dt)
    dy = _normal(rng, (t, wl.heads, wl.dv), dt, wl.dy_scale)
    drop = None
    if wl.keep_prob < 1.0:
        lq = np.diff(cu_q).tolist()
        lk = np.diff(cu_kv).tolist()
        drop = keep_bits(rng, lq, lk, wl.heads, wl.keep_prob)
    return Inputs(wl, q, k, v, dy, cu_q, cu_kv, drop)


def as_float_array(t: torch.Tensor) -> np.ndarray:
    """A float32/float64 numpy view of a CPU tensor (bf16/fp16 widen exactly to fp32)."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.float().numpy()
    return t.numpy()
