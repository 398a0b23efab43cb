"""pmqa_fused_logits_select_noalloc (the library's static scratch as the
finish-stage workspace) against pmqa_fused_logits_select with a workspace of
the caller's: the same kernels on the same inputs, so counters, thresholds,
ranges and the slot and Top-k sets agree bit for bit.  Two calls in a row, the
second smaller and laid out for another next_n, then the first again; every
row needs the repair in one of its forms (too few candidates, too many, or a
radix select of the k-th score)."""
import numpy as np
import pytest
import torch

import oracle
import paged_fp8_mqa_amd as pm
import workloads as W
from gpu_util import SENTINEL_I32, SelectBuffers, dev, slot_sets
from oracle.checker import check_row

pytestmark = pytest.mark.gpu


def _thresholds(wl, ref):
    """Per row, in turn: +inf (no candidate), below every score (all keys are
    candidates), the score of rank k/8 (too many), the k-th score (about
    fits), from the oracle's float64 scores."""
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = np.zeros(wl.rows, np.float32)
    for r, e in enumerate(ends):
        if e == 0:
            continue
        s = np.sort(ref[r, :e])[::-1]
        k = min(int(e), wl.top_k)
        thr[r] = [np.inf, s[-1] - 1, s[max(0, k // 8 - 1)], s[k - 1]][r % 4]
    return thr


def _run(wl, d, thr, noalloc):
    sb = SelectBuffers(wl.rows, wl.batch, wl.top_k, wl.capacity, thr, max_context=wl.max_seq_len,
                       workspace=None if not noalloc else torch.empty(0, dtype=torch.uint8, device="cuda"))
    kw = sb.kwargs()
    if noalloc:
        kw.pop("workspace")
        pm.fused_logits_select_noalloc(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, **kw)
    else:
        pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, **kw)
    return sb.host()


def _same(wl, a, b):
    assert np.array_equal(a["thr"].view(np.int32), b["thr"].view(np.int32)), "thresholds differ"
    assert np.array_equal(a["counters"], b["counters"]), "counters differ"
    assert np.array_equal(a["ranges"], b["ranges"]), "ranges differ"
    assert np.all(a["arrivals"] == 0) and np.all(b["arrivals"] == 0), "arrivals not left zeroed"
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    for r in range(wl.rows):
        assert slot_sets(a, r, wl.top_k, wl.capacity) == slot_sets(b, r, wl.top_k, wl.capacity), f"row {r}: slots"
        ta = sorted(a["topk"][r].tolist())
        tb = sorted(b["topk"][r].tolist())
        assert ta == tb, f"row {r}: Top-k sets differ"
        k = min(int(ends[r]), wl.top_k)
        assert SENTINEL_I32 not in ta and ta.count(-1) == wl.top_k - k, f"row {r}: Top-k not written"


def test_noalloc_matches_workspace_entry_point():
    big = W.small_random(61, [9000, 20000, 0, 12000], 2, 64, top_k=512, capacity=1024)
    small = W.small_random(62, [3000, 700, 5000], 3, 64, top_k=256, capacity=255)
    for wl in (big, small, big):
        assert pm.workspace_bytes("fused", wl.batch, wl.next_n, wl.max_seq_len) <= pm.NOALLOC_SCRATCH_BYTES
        d = dev(wl)
        s64 = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens,
                                      wl.block_size, wl.max_seq_len)
        tau = oracle.row_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size)
        thr = _thresholds(wl, s64)
        ref = _run(wl, d, thr, noalloc=False)
        got = _run(wl, d, thr, noalloc=True)
        _same(wl, ref, got)
        ends = oracle.row_ends(wl.seq_lens, wl.next_n)
        errs = []
        for r in range(wl.rows):
            errs += check_row(r, e_r=int(ends[r]), top_k=wl.top_k, capacity=wl.capacity, threshold_in=thr[r],
                              threshold_out=got["thr"][r], counters=got["counters"][r], cand_row=got["cand"][r],
                              rng=got["ranges"][:, r], topk_row=got["topk"][r], repair=True,
                              scores64=s64[r], tau=float(tau[r]), untouched_slots=SENTINEL_I32)
        assert not errs, "\n".join(errs[:20])
        assert np.sum(got["thr"].view(np.int32) != thr.view(np.int32)) >= wl.rows // 2, "repair did not run"


def test_noalloc_rejects_a_call_past_the_scratch():
    """64 requests of next_n 4 over 65536 keys need about 128 MiB: refused with
    PMQA_ERR_SCRATCH before anything runs (the buffers are small; every
    length is 10, so even a launch would stay inside them)."""
    B, nn, mc, bs, top_k, cap = 64, 4, 65536, 64, 16, 16
    assert pm.workspace_bytes("fused", B, nn, mc) > pm.NOALLOC_SCRATCH_BYTES
    g = torch.Generator().manual_seed(5)
    q = torch.randint(0, 0x70, (B, nn, 64, 128), generator=g, dtype=torch.uint8).cuda()
    kv = torch.zeros(4, bs, 1, 132, dtype=torch.uint8, device="cuda")
    w = torch.zeros(B * nn, 64, dtype=torch.float32, device="cuda")
    bt = torch.zeros(B, mc // bs, dtype=torch.int32, device="cuda")
    sl = torch.full((B,), 10, dtype=torch.int32, device="cuda")
    sb = SelectBuffers(B * nn, B, top_k, cap, np.full(B * nn, np.inf, np.float32),
                       workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    kw = sb.kwargs()
    kw.pop("workspace")
    with pytest.raises(pm.PmqaError) as e:
        pm.fused_logits_select_noalloc(q, kv, w, bt, sl, mc, **kw)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert np.all(sb.cand.cpu().numpy() == SENTINEL_I32), "written despite the error"
