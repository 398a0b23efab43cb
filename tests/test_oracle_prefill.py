"""Pins of the oracle's prefill-shaped rows (CPU only).

Row r of query tile i sees the keys below row_ends[r] of request
tile_requests[i] (page "flashinfer.sdsa.indexer_threshold_select",
Parameters: row_ends, tile_requests); its score is the logits formula of page
"flashinfer.attn_scores".  Each pin would catch a plausible slip in the
prefill indexing: the tile's request taken as the tile index (the permutation
and shared-request pins), the end of the tile used for every row (the prefix
and brute-force pins), the rows of a tile mixed up (the decode reduction).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import paged_mqa_logits, prefill_logits, prefill_tolerance, row_ends, row_tolerance

from test_oracle_logits import _e4m3, _fraction_e4m3, _pack, _tiny


def _pool(seed, lens, H=4, D=8, bs=4):
    """Random pages for requests of the given key counts; block table rows in order."""
    g = np.random.default_rng(seed)
    nb = sum(math.ceil(L / bs) for L in lens) + 1
    vals = _e4m3(g.normal(size=(nb, bs, D)) * 2)
    scales = g.uniform(0.5, 2.0, size=(nb, bs)).astype(np.float32)
    perm = g.permutation(nb - 1).astype(np.int32)
    width = max(math.ceil(L / bs) for L in lens)
    bt = np.full((len(lens), width), nb - 1, dtype=np.int32)
    off = 0
    for b, L in enumerate(lens):
        n = math.ceil(L / bs)
        bt[b, :n] = perm[off:off + n]
        off += n
    return _pack(vals, scales), bt, g


@pytest.mark.parametrize("seed", [0, 1])
def test_decode_rows_are_a_special_case(seed):
    """tile_rows = next_n, tile i on request i, row ends from seq_lens: the
    decode definition, row for row."""
    q, kv, w, bt, seq, bs = _tiny(seed, B=3, nn=2, seq=(5, 9, 1))
    B, nn, H, D = q.shape
    ends = row_ends(seq, nn)
    got = prefill_logits(q.reshape(B * nn, H, D), kv, w, bt, np.arange(B, dtype=np.int32), ends, nn, bs, max(seq))
    want = paged_mqa_logits(q, kv, w, bt, seq, bs, max(seq))
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_array_equal(got[~np.isnan(got)], want[~np.isnan(want)])
    np.testing.assert_array_equal(
        prefill_tolerance(q.reshape(B * nn, H, D), kv, w, bt, np.arange(B, dtype=np.int32), ends, nn, bs),
        row_tolerance(q, kv, w, bt, seq, bs))


def test_causal_prefix_consistency():
    """Rows with the same q and weights on one request: each row's scores are
    the first row_ends[r] scores of the longest row; different tiles on the
    same request see the same keys."""
    kv, bt, g = _pool(3, [23])
    H, D, bs = 4, 8, 4
    ends = np.array([1, 2, 3, 4, 17, 18, 0, 23], np.int32)  # two tiles of 4 rows
    q1 = _e4m3(g.normal(size=(H, D)) * 2)
    q = np.broadcast_to(q1, (8, H, D)).copy()
    w = np.broadcast_to(g.uniform(-1, 1, size=H).astype(np.float32), (8, H)).copy()
    got = prefill_logits(q, kv, w, bt, np.array([0, 0], np.int32), ends, 4, bs, 23)
    longest = got[7]
    for r, e in enumerate(ends):
        np.testing.assert_array_equal(got[r, :e], longest[:e])
        assert np.all(np.isnan(got[r, e:]))


def test_request_permutation_invariance():
    """Permuting the block table's rows and remapping tile_requests the same
    way changes nothing."""
    kv, bt, g = _pool(4, [9, 14, 6])
    H, D, bs = 4, 8, 4
    tiles, T = 5, 2
    treq = np.array([2, 0, 1, 1, 0], np.int32)
    lens = np.array([9, 14, 6])
    ends = np.array([g.integers(0, lens[treq[i // T]] + 1) for i in range(tiles * T)], np.int32)
    q = _e4m3(g.normal(size=(tiles * T, H, D)) * 2)
    w = g.uniform(-1, 1, size=(tiles * T, H)).astype(np.float32)
    base = prefill_logits(q, kv, w, bt, treq, ends, T, bs, 14)
    perm = np.array([1, 2, 0])        # new row j holds old row perm[j]
    inv = np.argsort(perm)
    permuted = prefill_logits(q, kv, w, bt[perm], inv[treq].astype(np.int32), ends, T, bs, 14)
    np.testing.assert_array_equal(np.isnan(base), np.isnan(permuted))
    np.testing.assert_array_equal(base[~np.isnan(base)], permuted[~np.isnan(permuted)])


def _brute(q, kv, w, bt, treq, ends, T, bs):
    out = {}
    R, H, D = q.shape
    for r in range(R):
        b = int(treq[r // T])
        for p in range(int(ends[r])):
            blk = kv[bt[b, p // bs]]
            slot = p % bs
            kp = blk[slot * D:(slot + 1) * D]
            sp = Fraction(float(blk[bs * D + 4 * slot: bs * D + 4 * slot + 4].view("<f4")[0]))
            acc = Fraction(0)
            for h in range(H):
                dot = sum(_fraction_e4m3(q[r, h, d]) * _fraction_e4m3(kp[d]) for d in range(D))
                acc += Fraction(float(w[r, h])) * max(dot, Fraction(0))
            out[(r, p)] = sp * acc
    return out


@pytest.mark.parametrize("seed", [5, 6])
def test_fraction_brute_force(seed):
    """Three tiles of 2 rows: two on request 1 (rows of unequal ends, one row
    with none), one on request 0."""
    kv, bt, g = _pool(seed, [7, 11])
    H, D, bs = 4, 8, 4
    treq = np.array([1, 0, 1], np.int32)
    ends = np.array([11, 3, 0, 7, 10, 0], np.int32)
    q = _e4m3(g.normal(size=(6, H, D)) * 2)
    w = g.uniform(-1, 1, size=(6, H)).astype(np.float32)
    got = prefill_logits(q, kv, w, bt, treq, ends, 2, bs, 11)
    ref = _brute(q, kv, w, bt, treq, ends, 2, bs)
    for (r, p), v in ref.items():
        assert abs(got[r, p] - float(v)) <= 1e-15 * max(1.0, abs(float(v)))
    for r, e in enumerate(ends):
        assert np.all(np.isnan(got[r, e:])) and not np.any(np.isnan(got[r, :e]))


def test_mistaken_request_lookup_fails_a_pin():
    """A copy that reads tile i's pages from block-table row i (ignoring
    tile_requests) disagrees with the brute force."""
    kv, bt, g = _pool(5, [7, 11])
    H, D, bs = 4, 8, 4
    treq = np.array([1, 0, 1], np.int32)
    ends = np.array([11, 3, 0, 7, 10, 0], np.int32)
    q = _e4m3(g.normal(size=(6, H, D)) * 2)
    w = g.uniform(-1, 1, size=(6, H)).astype(np.float32)
    ref = _brute(q, kv, w, bt, treq, ends, 2, bs)
    bt_wrong = np.stack([bt[min(i, 1)] for i in range(3)])  # row i for tile i
    try:
        wrong = prefill_logits(q, kv, w, bt_wrong, np.arange(3, dtype=np.int32), ends, 2, bs, 11)
    except IndexError:
        return
    assert any(abs(wrong[r, p] - float(v)) > 1e-9 for (r, p), v in ref.items() if not np.isnan(wrong[r, p]))
