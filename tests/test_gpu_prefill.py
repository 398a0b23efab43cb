"""GPU parity of pmqa_prefill_select (prefill-shaped rows: query tiles of
tile_rows rows of one request each, explicit row ends) against the float64
oracle, every row checked against the select contract, and bit for bit
against pmqa_fused_logits_select where the two describe the same rows."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_mqa_amd as pm
import workloads as W
from gpu_util import GOLDEN, SENTINEL_I32, SelectBuffers, dev, slot_sets
from oracle.checker import check_row
from report import GAP_STATS

pytestmark = pytest.mark.gpu


def _dev(wl):
    return {
        "q": torch.from_numpy(wl.q).cuda(),
        "kv": torch.from_numpy(wl.kv_fused).cuda().view(wl.num_blocks, wl.block_size, 1, 132),
        "w": torch.from_numpy(wl.weights).cuda(),
        "bt": torch.from_numpy(wl.block_tables).cuda(),
        "treq": torch.from_numpy(wl.tile_requests).cuda(),
        "re": torch.from_numpy(wl.row_ends).cuda(),
    }


def _oracle(wl, rows=None):
    s64 = oracle.prefill_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.tile_requests, wl.row_ends,
                                wl.tile_rows, wl.block_size, wl.max_context, rows=rows)
    tau = oracle.prefill_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.tile_requests, wl.row_ends,
                                   wl.tile_rows, wl.block_size, rows=rows)
    return s64, tau


def _thresholds(wl, s64, mode, seed=0):
    g = np.random.default_rng(seed)
    thr = np.zeros(wl.rows, np.float32)
    for r, e in enumerate(wl.row_ends):
        if e <= 0:
            continue
        srt = np.sort(s64[r, :e])[::-1]
        k = min(int(e), wl.top_k)
        m = mode if mode != "mixed" else ["kth", "inf", "low", "high"][r % 4]
        thr[r] = {"kth": srt[k - 1] - 1e-3, "inf": np.inf, "low": srt[-1] - 1,
                  "high": srt[max(0, k // 8 - 1)]}[m]
    return thr


def run_prefill(wl, d, thr, capacity=None, arrivals=True):
    cap = wl.capacity if capacity is None else capacity
    sb = SelectBuffers(wl.rows, wl.tiles, wl.top_k, cap, thr, arrivals=arrivals, which="fused",
                       max_context=wl.max_context)
    pm.prefill_select(d["q"], d["kv"], d["w"], d["bt"], d["treq"], d["re"], wl.tile_rows, wl.max_context,
                      **sb.kwargs())
    return sb.host()


def _check(wl, res, s64, tau, rows=None, capacity=None):
    cap = wl.capacity if capacity is None else capacity
    errs = []
    for r in (range(wl.rows) if rows is None else rows):
        errs += check_row(r, e_r=int(wl.row_ends[r]), top_k=wl.top_k, capacity=cap, threshold_in=res["thr_in"][r],
                          threshold_out=res["thr"][r], counters=res["counters"][r], cand_row=res["cand"][r],
                          rng=None if res["ranges"] is None else res["ranges"][:, r],
                          topk_row=None if res["topk"] is None else res["topk"][r], repair=res["ranges"] is not None,
                          scores64=s64[r], tau=float(tau[r]), untouched_slots=SENTINEL_I32, stats=GAP_STATS)
    if res["arrivals"] is not None:
        assert np.all(res["arrivals"] == 0), "arrivals not left zeroed"
    assert not errs, "\n".join(errs[:20])


CASES = [
    # seed, prompts (prefix, new), tile_rows, block_size, top_k, capacity
    (1, [(300, 9), (0, 5), (2000, 3)], 4, 64, 64, 128),
    (2, [(1000, 40)], 4, 32, 256, 255),
    (3, [(5000, 6), (64, 64)], 3, 128, 512, 1024),
    (4, [(100, 12), (4096, 2)], 2, 64, 32, 31),
    (5, [(700, 5), (0, 1)], 1, 64, 128, 256),
]


@pytest.mark.parametrize("seed,prompts,T,bs,top_k,cap", CASES)
@pytest.mark.parametrize("mode", ["kth", "mixed"])
def test_prefill_vs_oracle(seed, prompts, T, bs, top_k, cap, mode):
    wl = W.prefill_random(seed, prompts, T, bs, top_k, cap)
    s64, tau = _oracle(wl)
    thr = _thresholds(wl, s64, mode, seed)
    res = run_prefill(wl, _dev(wl), thr)
    _check(wl, res, s64, tau)


def test_prefill_without_finish_stage():
    """No arrivals: the single-pass select alone, counts and slots against the oracle."""
    wl = W.prefill_random(7, [(900, 10), (50, 7)], 4, 64, 64, 4096)
    s64, tau = _oracle(wl)
    thr = _thresholds(wl, s64, "mixed", 7)
    res = run_prefill(wl, _dev(wl), thr, arrivals=False)
    _check(wl, res, s64, tau)


def test_prefill_tile_with_no_keys():
    """A tile whose rows all see nothing next to tiles that see keys: its rows
    keep zero counters and untouched slots, and its arrival counter is reset."""
    wl = W.prefill_random(8, [(0, 0), (600, 6)], 4, 64, 64, 128, shuffle_tiles=False)
    wl.row_ends[:4] = 0   # the first tile: every row empty
    s64, tau = _oracle(wl)
    thr = _thresholds(wl, s64, "kth", 8)
    res = run_prefill(wl, _dev(wl), thr)
    _check(wl, res, s64, tau)
    assert np.all(res["counters"][:4] == 0)


@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_decode_rows_through_prefill_equal_fused(next_n):
    """Decode rows given as prefill rows (tile i on request i, row ends from the
    lengths) give the fused select's outputs bit for bit."""
    from gpu_util import run_fused
    wl = W.small_random(60 + next_n, [3000, 77, 0, 5000], next_n, 64, top_k=128, capacity=256)
    ends = oracle.row_ends(wl.seq_lens, next_n).astype(np.int32)
    ref = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                                  wl.max_seq_len)
    thr = np.zeros(wl.rows, np.float32)
    for r, e in enumerate(ends):
        if e:
            thr[r] = [np.inf, np.sort(ref[r, :e])[::-1][min(e, 128) - 1] - 1e-3][r % 2]
    fused = run_fused(wl, dev(wl), thr)
    pw = W.PrefillWorkload(name="decode_as_prefill", q=wl.q.reshape(wl.rows, 64, 128), kv_fused=wl.kv_fused,
                           weights=wl.weights, block_tables=wl.block_tables, seq_lens=wl.seq_lens,
                           tile_requests=np.arange(wl.batch, dtype=np.int32), row_ends=ends,
                           max_context=wl.max_seq_len, block_size=wl.block_size, tile_rows=next_n, top_k=wl.top_k,
                           capacity=wl.capacity, description="")
    pre = run_prefill(pw, _dev(pw), thr)
    assert np.array_equal(fused["thr"].view(np.int32), pre["thr"].view(np.int32))
    assert np.array_equal(fused["counters"], pre["counters"])
    assert np.array_equal(fused["ranges"], pre["ranges"])
    for r in range(wl.rows):
        assert slot_sets(fused, r, wl.top_k, wl.capacity) == slot_sets(pre, r, wl.top_k, wl.capacity), r
        assert sorted(fused["topk"][r].tolist()) == sorted(pre["topk"][r].tolist()), r


def test_prefill_chunk_all_rows():
    """The benchmark's prefill chunk (two requests, 512 new tokens each, 256
    tiles in random order) at its stored thresholds, in the launch
    configuration the benchmark times: every row against the float64 oracle."""
    wl = W.prefill_chunk()
    gold = json.load(open(os.path.join(GOLDEN, "thresholds_prefill_chunk.json")))
    assert gold["fingerprint"] == W.prefill_fingerprint(wl), "input generator drifted from the golden thresholds"
    thr = np.array(gold["threshold_bits"], np.int32).view(np.float32)
    res = run_prefill(wl, _dev(wl), thr)
    s64, tau = _oracle(wl)
    _check(wl, res, s64, tau)
