"""The host work list against brute-force enumeration of admitted pairs.

The admitted set comes from the oracle's mask (an independent implementation
of the causal / band windows); the work list comes from the C library.
"""
import numpy as np
import pytest

from oracle import fa_oracle as O
from variable_length_flashattention_fa_amd import binding as B
from variable_length_flashattention_fa_amd.inputs_forward import pair_count

BKV = B.FA_BLOCK_KV


def _check(lq, lkv, mode, pre, nxt, heads, block_q):
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lkv)]).astype(np.int64)
    items = B.worklist(cu_q, cu_k, mode, pre, nxt, heads, block_q)
    # one item per key block of every sequence with keys
    expect_blocks = {(b, jb) for b in range(len(lq)) for jb in range((lkv[b] + BKV - 1) // BKV)}
    got_blocks = [(it["seq"], it["kv_block"]) for it in items]
    assert len(got_blocks) == len(set(got_blocks))
    assert set(got_blocks) == expect_blocks
    # longest first
    spans = [it["tile_end"] - it["tile_begin"] for it in items]
    assert spans == sorted(spans, reverse=True)
    bases = O.dropout_bit_bases(cu_q, cu_k, heads)
    by_block = {(it["seq"], it["kv_block"]): it for it in items}
    for b in range(len(lq)):
        a = O.admit_mask(lq[b], lkv[b], mode, pre, nxt) if lq[b] and lkv[b] else np.zeros((lq[b], lkv[b]), bool)
        for jb in range((lkv[b] + BKV - 1) // BKV):
            it = by_block[(b, jb)]
            assert it["q_start"] == cu_q[b] and it["kv_start"] == cu_k[b]
            assert it["len_q"] == lq[b] and it["len_kv"] == lkv[b]
            assert it["drop_base"] == bases[b]
            blk = a[:, jb * BKV:(jb + 1) * BKV]
            rows = np.where(blk.any(axis=1))[0]
            tiles = set((rows // block_q).tolist())
            got = set(range(it["tile_begin"], it["tile_end"]))
            # exactly the tiles that hold an admitted pair: every pair covered, no dead tile
            assert got == tiles, (b, jb, sorted(got), sorted(tiles))


CASES = [
    ((37, 91), (37, 91), O.MASK_NONE, 0, 0),
    ((1, 2, 63, 64, 65, 127, 129, 300), None, O.MASK_CAUSAL, 0, 0),
    ((0, 200, 0, 5), (3, 200, 0, 0), O.MASK_CAUSAL, 0, 0),
    ((300, 100), (100, 300), O.MASK_CAUSAL, 0, 0),
    ((700, 257), None, O.MASK_BAND, 100, 0),
    ((700, 257), (500, 400), O.MASK_BAND, 64, 30),
    ((600,), None, O.MASK_BAND, 65536, 65536),
    ((600,), None, O.MASK_BAND, -5, 20),
    ((600,), None, O.MASK_BAND, -10, 3),
    ((400, 129), (129, 400), O.MASK_NONE, 0, 0),
]


@pytest.mark.parametrize("lq,lkv,mode,pre,nxt", CASES)
@pytest.mark.parametrize("block_q", [32, 64])
def test_worklist_covers_exactly_admitted_tiles(lq, lkv, mode, pre, nxt, block_q):
    _check(list(lq), list(lkv if lkv is not None else lq), mode, pre, nxt, heads=3, block_q=block_q)


def test_worklist_random_cases():
    rng = np.random.default_rng(0)
    for _ in range(30):
        b = int(rng.integers(1, 6))
        lq = rng.integers(0, 400, b).tolist()
        lkv = lq if rng.random() < 0.5 else rng.integers(0, 400, b).tolist()
        mode = int(rng.integers(0, 3))
        pre, nxt = int(rng.integers(-20, 300)), int(rng.integers(-20, 300))
        _check(lq, lkv, mode, pre, nxt, heads=2, block_q=int(rng.choice([32, 64])))


def test_worklist_rejects_bad_input():
    with pytest.raises(B.FaError):
        B.worklist([0, 5, 3], [0, 5, 3], 0, 0, 0, 1, 64)
    with pytest.raises(B.FaError):
        B.worklist([0, 5], [0, 5, 6], 0, 0, 0, 1, 64)


@pytest.mark.parametrize("lq,lkv,mode,pre,nxt", CASES)
def test_pair_count_closed_form(lq, lkv, mode, pre, nxt):
    lkv = lq if lkv is None else lkv
    cu_q = np.concatenate([[0], np.cumsum(lq)])
    cu_k = np.concatenate([[0], np.cumsum(lkv)])
    assert pair_count(cu_q, cu_k, mode, pre, nxt) == O.admitted_pairs(cu_q, cu_k, mode, pre, nxt)


def test_pair_count_of_workloads():
    from variable_length_flashattention_fa_amd import synth
    expect = {1: 9650, 2: 47953195, 3: 536903680, 4: 117497856, 5: 35371200}
    for i, n in expect.items():
        wl = synth.workload(i)
        assert pair_count(wl.cu_q(), wl.cu_kv(), wl.mode, wl.pre, wl.nxt) == n
