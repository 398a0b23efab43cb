"""HIP-graph capture and replay of the fused select: each replay, with the
program's own eager calls and synchronisations between replays, gives the
eager call's results, bit for bit; replays with new seq_lens and thresholds
written into the captured buffers follow the new inputs."""
import numpy as np
import pytest
import torch

import oracle
import paged_fp8_mqa_amd as pm
import workloads as W
from gpu_util import SENTINEL_I32, dev, slot_sets

pytestmark = pytest.mark.gpu


def _buffers(wl, thr, ws):
    R = wl.rows
    return dict(
        thr_in=torch.as_tensor(thr).cuda(), thr=torch.empty(R, dtype=torch.float32, device="cuda"),
        counters=torch.zeros(R, 2, dtype=torch.int32, device="cuda"),
        cand=torch.full((R, wl.top_k + wl.capacity, 2), SENTINEL_I32, dtype=torch.int32, device="cuda"),
        arrivals=torch.zeros(wl.batch, dtype=torch.int32, device="cuda"),
        ranges=torch.zeros(2, R, dtype=torch.int32, device="cuda"),
        topk=torch.zeros(R, wl.top_k, dtype=torch.int32, device="cuda"), ws=ws)


def _call(wl, d, b, sl=None):
    # the resets are kernels (a fill and an add), so that a captured graph
    # holds no memset node
    b["counters"].zero_()
    torch.add(b["thr_in"], 0.0, out=b["thr"])
    pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"] if sl is None else sl, wl.max_seq_len,
                           b["thr"], b["counters"], b["cand"], wl.capacity, wl.top_k, arrivals=b["arrivals"],
                           ranges=b["ranges"], topk_idx=b["topk"], workspace=b["ws"])


def _host(b):
    torch.cuda.synchronize()
    return {k: b[k].cpu().numpy() for k in ("thr", "counters", "cand", "arrivals", "ranges", "topk")}


def _same(wl, a, b, seq_lens=None):
    assert np.array_equal(a["thr"].view(np.int32), b["thr"].view(np.int32)), "thresholds differ"
    assert np.array_equal(a["counters"], b["counters"]), "counters differ"
    assert np.array_equal(a["ranges"], b["ranges"]), "ranges differ"
    assert np.all(b["arrivals"] == 0), "arrivals not left zeroed"
    ends = oracle.row_ends(wl.seq_lens if seq_lens is None else seq_lens, wl.next_n)
    for r in range(wl.rows):
        ra = {"counters": a["counters"], "cand": a["cand"]}
        rb = {"counters": b["counters"], "cand": b["cand"]}
        assert slot_sets(ra, r, wl.top_k, wl.capacity) == slot_sets(rb, r, wl.top_k, wl.capacity), f"row {r} slots"
        k = min(int(ends[r]), wl.top_k)
        assert set(a["topk"][r, :k].tolist()) == set(b["topk"][r, :k].tolist()), f"row {r} top-k"


def _thresholds(wl, seq_lens, mode, rng):
    """Per-row thresholds from the oracle's scores at these lengths: "inf" repairs
    every row, "mixed" repairs the even rows and puts the odd ones at their k-th
    score, "jitter" moves each k-th score by a random amount (some rows fit,
    some do not)."""
    ref = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, seq_lens, wl.block_size,
                                  wl.max_seq_len)
    ends = oracle.row_ends(seq_lens, wl.next_n)
    thr = np.zeros(wl.rows, np.float32)
    for r, e in enumerate(ends):
        if e:
            s = np.sort(ref[r, :e].astype(np.float32))[::-1]
            k = min(int(e), wl.top_k)
            if mode == "inf" or (mode == "mixed" and r % 2 == 0):
                thr[r] = np.inf
            elif mode == "mixed":
                thr[r] = s[k - 1]
            else:
                thr[r] = s[min(int(e) - 1, max(0, k - 1 + int(rng.integers(-20, 20))))]
    return ref, thr


def _check_oracle(wl, got, ref, seq_lens):
    from oracle.checker import check_row
    tau = oracle.row_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, seq_lens, wl.block_size)
    ends = oracle.row_ends(seq_lens, wl.next_n)
    errs = []
    for r in range(wl.rows):
        errs += check_row(r, e_r=int(ends[r]), top_k=wl.top_k, capacity=wl.capacity, threshold_in=got["thr_in"][r],
                          threshold_out=got["thr"][r], counters=got["counters"][r], cand_row=got["cand"][r],
                          rng=got["ranges"][:, r], topk_row=got["topk"][r], repair=True, scores64=ref[r],
                          tau=float(tau[r]))
    assert not errs, "\n".join(errs[:10])


@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_fused_graph_replays_with_changed_inputs(next_n):
    """One capture, replayed with new seq_lens and new thresholds written into the
    captured buffers between replays (the grid's split of the batch is made on
    the device from seq_lens at each replay): every replay equals an eager call
    on the same inputs and passes the oracle's checks, and arrivals stays
    zeroed."""
    base = [3000, 700, 0, 5000]
    wl = W.small_random(62 + next_n, base, next_n, 64, top_k=128, capacity=256)
    d = dev(wl)
    rng = np.random.default_rng(next_n)
    ws = pm.make_workspace("fused", wl.batch, wl.next_n, wl.max_seq_len)
    sl_g = torch.from_numpy(wl.seq_lens.copy()).cuda()
    graphed = _buffers(wl, np.zeros(wl.rows, np.float32), ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _call(wl, d, graphed, sl=sl_g)
    torch.cuda.synchronize()
    # each variant keeps every length within the request's own pages
    variants = [(base, "mixed"), ([2500, 1, 0, 4990], "inf"), ([3000, 0, 0, 64], "jitter"),
                ([1, 700, 0, 5000], "jitter"), (base, "inf")]
    for lens, mode in variants:
        lens = np.array(lens, np.int32)
        ref, thr = _thresholds(wl, lens, mode, rng)
        sl_g.copy_(torch.from_numpy(lens))
        graphed["thr_in"].copy_(torch.from_numpy(thr))
        graphed["cand"].fill_(SENTINEL_I32)
        graphed["topk"].fill_(SENTINEL_I32)
        torch.cuda.synchronize()
        g.replay()
        got = _host(graphed)
        got["thr_in"] = thr
        eager = _buffers(wl, thr, ws)
        _call(wl, d, eager, sl=torch.from_numpy(lens).cuda())
        want = _host(eager)
        _same(wl, want, got, seq_lens=lens)
        _check_oracle(wl, got, ref, lens)


@pytest.mark.parametrize("next_n", [1, 2])
@pytest.mark.parametrize("mode", ["inf", "mixed"])
def test_fused_graph_replays_match_eager(mode, next_n):
    """Every row repaired, or the even rows repaired and the odd ones fitting:
    the swept rows' repair scores their keys again from the KV pages inside the
    captured launch, replay after replay."""
    wl = W.small_random(61, [3000, 700, 0, 5000], next_n, 64, top_k=128, capacity=256)
    d = dev(wl)
    ref = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                                  wl.max_seq_len)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = np.zeros(wl.rows, np.float32)
    for r, e in enumerate(ends):
        if e:
            s = np.sort(ref[r, :e].astype(np.float32))[::-1]
            k = min(int(e), wl.top_k)
            # "inf": every row repaired; "mixed": even rows repaired, odd rows fit
            thr[r] = np.inf if (mode == "inf" or r % 2 == 0) else s[k - 1]
    ws = pm.make_workspace("fused", wl.batch, wl.next_n, wl.max_seq_len)
    eager = _buffers(wl, thr, ws)
    _call(wl, d, eager)
    want = _host(eager)

    graphed = _buffers(wl, thr, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _call(wl, d, graphed)
    torch.cuda.synchronize()
    for rep in range(4):
        graphed["cand"].fill_(SENTINEL_I32)
        graphed["topk"].fill_(SENTINEL_I32)
        g.replay()
        got = _host(graphed)
        _same(wl, want, got)
        # the program's own work between replays, on the same workspace
        _call(wl, d, eager)
        _same(wl, want, _host(eager))


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fn()
    torch.cuda.synchronize()
    return g


def test_prefill_graph_replays_match_eager():
    """pmqa_prefill_select captured once and replayed with new thresholds
    written into the captured buffer: each replay equals an eager call and
    passes the oracle's checks."""
    from test_gpu_prefill import _check as pcheck, _dev as pdev, _oracle as poracle, _thresholds as pthr
    wl = W.prefill_random(71, [(900, 10), (50, 7)], 4, 64, 64, 128)
    d = pdev(wl)
    s64, tau = poracle(wl)
    ws = pm.make_workspace("fused", wl.tiles, wl.tile_rows, wl.max_context)

    def bufs():
        R = wl.rows
        return dict(thr_in=torch.zeros(R, dtype=torch.float32, device="cuda"),
                    thr=torch.empty(R, dtype=torch.float32, device="cuda"),
                    counters=torch.zeros(R, 2, dtype=torch.int32, device="cuda"),
                    cand=torch.full((R, wl.top_k + wl.capacity, 2), SENTINEL_I32, dtype=torch.int32, device="cuda"),
                    arrivals=torch.zeros(wl.tiles, dtype=torch.int32, device="cuda"),
                    ranges=torch.zeros(2, R, dtype=torch.int32, device="cuda"),
                    topk=torch.zeros(R, wl.top_k, dtype=torch.int32, device="cuda"), ws=ws)

    def call(b):
        b["counters"].zero_()
        torch.add(b["thr_in"], 0.0, out=b["thr"])
        pm.prefill_select(d["q"], d["kv"], d["w"], d["bt"], d["treq"], d["re"], wl.tile_rows, wl.max_context,
                          b["thr"], b["counters"], b["cand"], wl.capacity, wl.top_k, b["arrivals"], b["ranges"],
                          b["topk"], workspace=b["ws"])

    graphed = bufs()
    g = _capture(lambda: call(graphed))
    for seed, mode in [(1, "kth"), (2, "mixed"), (3, "inf")]:
        thr = pthr(wl, s64, mode, seed)
        graphed["thr_in"].copy_(torch.from_numpy(thr))
        graphed["cand"].fill_(SENTINEL_I32)
        torch.cuda.synchronize()
        g.replay()
        got = _host(graphed)
        eager = bufs()
        eager["thr_in"].copy_(torch.from_numpy(thr))
        call(eager)
        want = _host(eager)
        assert np.array_equal(want["thr"].view(np.int32), got["thr"].view(np.int32))
        assert np.array_equal(want["counters"], got["counters"]) and np.array_equal(want["ranges"], got["ranges"])
        assert np.all(got["arrivals"] == 0)
        for r in range(wl.rows):
            assert slot_sets(want, r, wl.top_k, wl.capacity) == slot_sets(got, r, wl.top_k, wl.capacity), r
            assert sorted(want["topk"][r].tolist()) == sorted(got["topk"][r].tolist()), r
        got["thr_in"] = thr
        pcheck(wl, got, s64, tau)


@pytest.mark.parametrize("which", ["typed", "fp4"])
def test_logits_graph_replays_match_eager(which):
    """The float16-option and the MXFP4 logits captured once and replayed with
    new seq_lens: each replay equals an eager call, bit for bit."""
    if which == "typed":
        wl = W.small_random(72, [3000, 700, 0, 5000], 3, 64, top_k=1, capacity=1)
        d = dev(wl)
        kw = dict(output_dtype=torch.float16, epi_dtype=torch.float16, acc_dtype=torch.float32)
        dt = torch.float16
        run = lambda sl, out: pm.mqa_logits(d["q"], d["kv"], d["w"], d["bt"], sl, wl.max_seq_len, out=out, **kw)
    else:
        wl = W.fp4_random(73, [3000, 700, 0, 5000], 2, 64)
        d = {"q": torch.from_numpy(wl.q).cuda(), "qsf": torch.from_numpy(wl.q_sf).cuda(),
             "kv": torch.from_numpy(wl.kv_fused).cuda().view(wl.num_blocks, wl.block_size, 1, 68),
             "w": torch.from_numpy(wl.weights).cuda(), "bt": torch.from_numpy(wl.block_tables).cuda()}
        dt = torch.bfloat16
        run = lambda sl, out: pm.fp4_mqa_logits(d["q"], d["qsf"], d["kv"], d["w"], d["bt"], sl, wl.max_seq_len,
                                                out=out)
    cols = pm.padded_seq_len(wl.max_seq_len)
    sl_g = torch.from_numpy(wl.seq_lens.copy()).cuda()
    out_g = torch.zeros(wl.rows, cols, dtype=dt, device="cuda")
    g = _capture(lambda: run(sl_g, out_g))
    for lens in ([3000, 700, 0, 5000], [2500, 1, 0, 4990], [64, 700, 0, 100]):
        lens = np.array(lens, np.int32)
        sl_g.copy_(torch.from_numpy(lens))
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = torch.zeros_like(out_g)
        run(torch.from_numpy(lens).cuda(), eager)
        torch.cuda.synchronize()
        ends = oracle.row_ends(lens, wl.next_n)
        for r, e in enumerate(ends):
            assert torch.equal(out_g[r, :e].view(torch.int16), eager[r, :e].view(torch.int16)), (which, r)
