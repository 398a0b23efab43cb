"""GPU parity of the select paths: pmqa_indexer_topk (exact, against the
oracle's select on the same float32 scores), pmqa_fused_logits_select (against
the float64 oracle within tau, and bit for bit against the unfused pair)."""
import numpy as np
import pytest
import torch

import oracle
import paged_fp8_mqa_amd as pm
import workloads as W
from gpu_util import SENTINEL_I32, dev, golden_thresholds, run_fused, run_logits, run_select, slot_sets
from oracle.checker import check_row

pytestmark = pytest.mark.gpu


from report import GAP_STATS


def _check(wl, res, repair, scores32=None, scores64=None, tau=None, rows=None, capacity=None, untouched=True,
           stats=None):
    """Every row (or the given rows) against the select contract, and against the
    oracle's scores when given: exact float32 scores (the unfused select reads
    them) or float64 ones within tau_r.  With fresh sentinel-filled slots
    (untouched), slots outside the ranges of rows that were not repaired must
    still hold the sentinel."""
    cap = wl.capacity if capacity is None else capacity
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    errs = []
    for r in (range(wl.rows) if rows is None else rows):
        errs += check_row(
            r, e_r=int(ends[r]), top_k=wl.top_k, capacity=cap, threshold_in=res["thr_in"][r],
            threshold_out=res["thr"][r], counters=res["counters"][r], cand_row=res["cand"][r],
            rng=None if res["ranges"] is None else res["ranges"][:, r],
            topk_row=None if res["topk"] is None else res["topk"][r], repair=repair,
            scores32=None if scores32 is None else scores32[r],
            scores64=None if scores64 is None else scores64[r], tau=0.0 if tau is None else float(tau[r]),
            untouched_slots=SENTINEL_I32 if untouched else None,
            stats=GAP_STATS if stats is None else stats)
    if res["arrivals"] is not None:
        assert np.all(res["arrivals"] == 0), "arrivals not left zeroed"
    assert not errs, "\n".join(errs[:20])


def _synthetic_logits(seed, R, cols, ends, tie_frac=0.3):
    """Seeded float32 scores with many exact repeats (ties), NaN past each row's end."""
    g = np.random.default_rng(seed)
    x = g.normal(size=(R, cols)).astype(np.float32) * 4
    pool = g.normal(size=8).astype(np.float32) * 4
    rep = g.random((R, cols)) < tie_frac
    x[rep] = pool[g.integers(0, 8, size=int(rep.sum()))]
    for r in range(R):
        x[r, ends[r]:] = np.nan
    return x


SEL_CASES = [
    # seed, seq_lens, next_n, top_k, capacity, threshold mode
    (1, [5000, 20, 0, 9000], 2, 64, 128, "sigma"),
    (2, [5000, 20, 0, 9000], 2, 64, 63, "inf"),
    (3, [3000, 8000], 3, 512, 1024, "low"),
    (4, [100, 4096, 4097, 1], 4, 256, 255, "sigma"),
    (5, [17000], 1, 2048, 4096, "mixed"),
    (6, [300, 300, 300], 1, 1024, 2048, "low"),   # row_end < top_k
]


def _thresholds(mode, scores, ends, top_k, seed):
    g = np.random.default_rng(seed)
    thr = np.zeros(len(ends), np.float32)
    for r, e in enumerate(ends):
        if e == 0:
            continue
        s = np.sort(scores[r, :e])[::-1]
        k = min(e, top_k)
        m = mode if mode != "mixed" else ["sigma", "inf", "low", "high"][r % 4]
        thr[r] = {"sigma": s[k - 1], "inf": np.inf, "low": -np.inf,
                  "high": s[max(0, k // 8 - 1)]}[m] if m != "low" else s[-1] - 1
    return thr


@pytest.mark.parametrize("seed,seq_lens,next_n,top_k,cap,mode", SEL_CASES)
def test_indexer_topk_exact(seed, seq_lens, next_n, top_k, cap, mode):
    B = len(seq_lens)
    R = B * next_n
    ends = oracle.row_ends(np.array(seq_lens), next_n)
    cols = max(max(seq_lens), 1)
    x = _synthetic_logits(seed, R, cols + 7, ends)
    thr = _thresholds(mode, x, ends, top_k, seed)
    wl = W.Workload(name="syn", q=None, kv_fused=np.zeros((1, 1), np.uint8), weights=None, block_tables=None,
                    seq_lens=np.array(seq_lens, np.int32), max_seq_len=cols, block_size=64, next_n=next_n,
                    top_k=top_k, capacity=cap, threshold_recipe="", description="")
    logits = torch.from_numpy(x).to("cuda")
    res = run_select(wl, logits, thr)
    _check(wl, res, True, scores32=x)
    # without arrivals: a single pass, no repair
    res2 = run_select(wl, logits, thr, arrivals=False)
    _check(wl, res2, False, scores32=x)


@pytest.mark.parametrize("tied", [False, True])
def test_indexer_topk_few_extra_candidates(tied):
    """Rows that fit with 1, 2 or 3 candidates more than k (the Top-k leaves the
    smallest out), with the smallest candidates tied at the k-th value or not,
    and rows with 0 and 4 extra (the copy and the radix paths beside them)."""
    top_k, cap, n = 256, 512, 5000
    extras = [1, 2, 3, 0, 4, 1, 2, 3]
    R = len(extras)
    g = np.random.default_rng(77 + tied)
    x = (g.normal(size=(R, n + 3)) * 4).astype(np.float32)
    thr = np.zeros(R, np.float32)
    for r, d in enumerate(extras):
        order = np.argsort(-x[r, :n], kind="stable")
        if tied:
            # the last few candidates (and one key that stays a candidate) share the k-th value
            x[r, order[top_k - 2:top_k + d]] = x[r, order[top_k - 2]]
        v_in, v_out = np.float32(x[r, order[top_k + d - 1]]), np.float32(x[r, order[top_k + d]])
        assert v_out < v_in
        thr[r] = np.float32((np.float64(v_in) + np.float64(v_out)) / 2)
        assert int(np.sum(x[r, :n] > thr[r])) == top_k + d
    wl = W.Workload(name="syn", q=None, kv_fused=np.zeros((1, 1), np.uint8), weights=None, block_tables=None,
                    seq_lens=np.full(R, n, np.int32), max_seq_len=n, block_size=64, next_n=1,
                    top_k=top_k, capacity=cap, threshold_recipe="", description="")
    res = run_select(wl, torch.from_numpy(x).to("cuda"), thr)
    _check(wl, res, True, scores32=x)
    assert np.array_equal(res["counters"][:, 0], top_k + np.array(extras))


@pytest.mark.parametrize("mode", ["low", "inf"])
def test_indexer_topk_repair_heavy_ties(mode):
    """Repaired rows whose k-th largest score is shared by thousands of keys (more
    than a final in-LDS select holds), so that the repair needs every key bit
    before it selects the row again; rows aligned and not (odd row stride)."""
    top_k, cap, n = 2048, 4096, 20000
    R = 3
    g = np.random.default_rng(91)
    x = (g.normal(size=(R, n + 1)) * 4).astype(np.float32)
    for r in range(R):
        order = np.argsort(-x[r, :n], kind="stable")
        tie = order[1500:1500 + 6000]          # the k-th position falls inside this block
        x[r, tie] = x[r, order[1500]]
    x[:, n] = np.nan
    thr = np.full(R, -np.inf if mode == "low" else np.inf, np.float32)
    wl = W.Workload(name="syn", q=None, kv_fused=np.zeros((1, 1), np.uint8), weights=None, block_tables=None,
                    seq_lens=np.full(R, n, np.int32), max_seq_len=n, block_size=64, next_n=1,
                    top_k=top_k, capacity=cap, threshold_recipe="", description="")
    res = run_select(wl, torch.from_numpy(x).to("cuda"), thr)
    _check(wl, res, True, scores32=x)
    assert np.all(res["counters"][:, 1] >= 6000 - 1)


@pytest.mark.parametrize("mode", ["low", "inf", "sigma"])
def test_indexer_topk_repair_large_k(mode):
    """Repaired rows with k above 2048 (the candidates above the final digit
    stored raw, then re-encoded, instead of kept in LDS), on aligned and
    unaligned rows, with and without ties at the k-th score."""
    top_k, cap, n = 3000, 6000, 12000
    R = 4
    g = np.random.default_rng(123)
    x = (g.normal(size=(R, n + 3)) * 4).astype(np.float32)
    for r in (1, 3):
        order = np.argsort(-x[r, :n], kind="stable")
        x[r, order[2900:3100]] = x[r, order[2900]]   # ties across the k-th position
    x[:, n:] = np.nan
    ends = oracle.row_ends(np.full(R, n), 1)
    thr = _thresholds(mode, x, ends, top_k, 5) if mode == "sigma" else \
        np.full(R, -np.inf if mode == "low" else np.inf, np.float32)
    wl = W.Workload(name="syn", q=None, kv_fused=np.zeros((1, 1), np.uint8), weights=None, block_tables=None,
                    seq_lens=np.full(R, n, np.int32), max_seq_len=n, block_size=64, next_n=1,
                    top_k=top_k, capacity=cap, threshold_recipe="", description="")
    res = run_select(wl, torch.from_numpy(x).to("cuda"), thr)
    _check(wl, res, True, scores32=x)


def _oracle_rows(wl, rows):
    ref = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                                  wl.max_seq_len, rows=rows)
    tau = oracle.row_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                               rows=rows)
    return ref, tau


def _sigma_thresholds(ref, ends, top_k, mode):
    thr = np.zeros(len(ends), np.float32)
    for r, e in enumerate(ends):
        if e == 0:
            continue
        k = min(int(e), top_k)
        s = np.sort(ref[r, :e])[::-1]
        thr[r] = np.float32(np.inf) if mode == "inf" else np.float32(s[k - 1])
    return thr


@pytest.mark.parametrize("cfg,mode", [(1, "inf"), (1, "sigma"), (2, "inf"), (2, "sigma")])
def test_fused_small_configs_vs_oracle(cfg, mode):
    wl = W.make(cfg)
    ref, tau = _oracle_rows(wl, None)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = _sigma_thresholds(ref, ends, wl.top_k, mode)
    d = dev(wl)
    res = run_fused(wl, d, thr)
    _check(wl, res, True, scores64=ref, tau=tau)


FUSED_EDGE = [
    (31, [1, 17, 64, 65, 200], 1, 32, 16, 32),
    (32, [0, 2, 3, 130, 1000], 3, 64, 64, 63),
    (33, [127, 128, 129, 0, 4096], 2, 128, 100, 200),
    (34, [5, 63, 64, 2049, 3], 4, 64, 512, 511),
    (35, [0, 0], 2, 64, 8, 8),
]


@pytest.mark.parametrize("seed,seq_lens,next_n,bs,top_k,cap", FUSED_EDGE)
@pytest.mark.parametrize("mode", ["inf", "sigma"])
def test_fused_edge_vs_oracle_and_unfused(seed, seq_lens, next_n, bs, top_k, cap, mode):
    wl = W.small_random(seed, seq_lens, next_n, bs, top_k=top_k, capacity=cap)
    ref, tau = _oracle_rows(wl, None)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = _sigma_thresholds(ref, ends, wl.top_k, mode)
    d = dev(wl)
    fused = run_fused(wl, d, thr)
    _check(wl, fused, True, scores64=ref, tau=tau)
    # the unfused pair on the same inputs gives the same bits
    out, _ = run_logits(wl, d)
    unf = run_select(wl, out, thr, max_context=wl.max_seq_len)
    _same(wl, fused, unf)


def _same(wl, a, b, capacity=None):
    cap = wl.capacity if capacity is None else capacity
    assert np.array_equal(a["thr"].view(np.int32), b["thr"].view(np.int32)), "thresholds differ"
    assert np.array_equal(a["counters"], b["counters"]), "counters differ"
    if a["ranges"] is not None:
        assert np.array_equal(a["ranges"], b["ranges"]), "ranges differ"
    for r in range(wl.rows):
        ca, ta = slot_sets(a, r, wl.top_k, cap)
        cb, tb = slot_sets(b, r, wl.top_k, cap)
        if int(a["counters"][r, 0]) <= cap:
            assert ca == cb, f"row {r}: candidate slots differ"
        if int(a["counters"][r, 1]) <= wl.top_k:
            assert ta == tb, f"row {r}: tie slots differ"


def test_swept_rows_of_a_very_long_request():
    """A 600000-key request beside a short one, next_n 2, every row swept
    (threshold +inf): the long rows are scored again in repair items of the
    largest size (32768 keys, the limit of an item's packed 16-bit histogram
    counts); every row against the float64 oracle."""
    wl = W.small_random(81, [600000, 3000], 2, 64, top_k=2048, capacity=4096)
    d = dev(wl)
    ref, tau = _oracle_rows(wl, None)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = _sigma_thresholds(ref, ends, wl.top_k, "inf")
    res = run_fused(wl, d, thr)
    _check(wl, res, True, scores64=ref, tau=tau)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_fused_large_configs(cfg):
    """Every row of the large workloads against the float64 oracle (contract,
    counts within tau, candidate scores, repaired thresholds, the Top-k set
    rule), in the launch configuration the benchmark times."""
    wl = W.make(cfg)
    gold, thr = golden_thresholds(cfg)
    assert gold["fingerprint"] == W.fingerprint(wl), "input generator drifted from the golden thresholds"
    d = dev(wl)
    ref, tau = _oracle_rows(wl, None)
    res = run_fused(wl, d, thr)
    _check(wl, res, True, scores64=ref, tau=tau)
    if cfg == 5:
        assert np.sum(res["thr"].view(np.int32) != thr.view(np.int32)) >= 7   # the too-high rows repaired
        res2 = run_fused(wl, d, thr, capacity=wl.top_k - 1)
        _check(wl, res2, True, scores64=ref, tau=tau, capacity=wl.top_k - 1)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_unfused_large_configs(cfg):
    """mqa_logits then indexer_topk on the large workloads: the select exactly
    against the oracle's select over the GPU's own float32 logits, every row
    against the float64 oracle within tau, and bit for bit equal to the fused
    path."""
    wl = W.make(cfg)
    gold, thr = golden_thresholds(cfg)
    d = dev(wl)
    out, _ = run_logits(wl, d)
    logits = out.cpu().numpy()
    unf = run_select(wl, out, thr)
    _check(wl, unf, True, scores32=logits)
    ref, tau = _oracle_rows(wl, None)
    _check(wl, unf, True, scores64=ref, tau=tau)
    fused = run_fused(wl, d, thr)
    _same(wl, fused, unf)


def test_fused_large_batch_grid():
    """More than 1024 requests (batch x chunks grid), fused against unfused bit for bit."""
    rng = np.random.default_rng(6)
    seq = [int(x) for x in rng.integers(0, 2000, size=1100)]
    wl = W.small_random(42, seq, 1, 64, top_k=32, capacity=64)
    thr = np.full(wl.rows, np.inf, np.float32)
    d = dev(wl)
    fused = run_fused(wl, d, thr)
    _check(wl, fused, True)
    out, _ = run_logits(wl, d)
    unf = run_select(wl, out, thr, max_context=wl.max_seq_len)
    _same(wl, fused, unf)
    rows = [0, 1, 500, wl.rows - 1]
    ref, tau = _oracle_rows(wl, rows)
    _check(wl, fused, True, scores64=ref, tau=tau, rows=rows)


def test_fused_large_batch_fitting_rows():
    """1100 requests, more tiles than the launch can place with the located
    grid (a fixed number of CTAs per request instead), thresholds at each
    row's k-th score: most rows fit (their Top-k from the main pass's slots, or
    with a few extra candidates left out), and every row matches the oracle and
    the select over a logits matrix."""
    rng = np.random.default_rng(8)
    seq = [int(x) for x in rng.integers(0, 1500, size=1100)]
    wl = W.small_random(43, seq, 1, 64, top_k=32, capacity=64)
    ref, tau = _oracle_rows(wl, None)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = _sigma_thresholds(ref, ends, wl.top_k, "kth")
    d = dev(wl)
    fused = run_fused(wl, d, thr)
    _check(wl, fused, True, scores64=ref, tau=tau)
    assert np.sum(fused["thr"].view(np.int32) == thr.view(np.int32)) > wl.rows // 2  # most rows fit
    out, _ = run_logits(wl, d)
    unf = run_select(wl, out, thr, max_context=wl.max_seq_len)
    _same(wl, fused, unf)


def test_fused_repeated_calls_reuse_arrivals():
    wl = W.small_random(41, [3000, 5000], 2, 64, top_k=128, capacity=256)
    ref, tau = _oracle_rows(wl, None)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = _sigma_thresholds(ref, ends, wl.top_k, "inf")
    d = dev(wl)
    import gpu_util
    sb = gpu_util.SelectBuffers(wl.rows, wl.batch, wl.top_k, wl.capacity, thr, max_context=wl.max_seq_len)
    first = None
    for it in range(3):
        sb.counters.zero_()
        sb.thr.copy_(sb.thr_in)
        pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, **sb.kwargs())
        h = sb.host()
        _check(wl, h, True, scores64=ref, tau=tau, untouched=False)
        if first is None:
            first = h
        else:
            _same(wl, first, h)


@pytest.mark.gpu
def test_workspace_reused_across_batch_sizes():
    """One workspace, sized for the largest call, serves calls of different
    batch sizes and next_n in turn, every row repaired each time (the finish
    stage keeps state in the workspace between calls, laid out by each call's
    batch and next_n, and the fused repair's score buffer sits right after that
    state, so each layout's scores cover another layout's state words)."""
    wa = W.small_random(51, [3000, 5000], 2, 64, top_k=128, capacity=256)
    wb = W.small_random(52, [900, 4000, 0, 2500, 7000], 2, 64, top_k=128, capacity=256)
    wc = W.small_random(53, [6000, 2100, 4500], 1, 64, top_k=128, capacity=256)
    wls = (wa, wb, wc)
    ws = torch.zeros(max(pm.workspace_bytes("fused", w.batch, w.next_n, w.max_seq_len) for w in wls),
                     dtype=torch.uint8, device="cuda")
    import gpu_util
    for wl in (wa, wb, wa, wc, wb, wc, wa):
        ref, tau = _oracle_rows(wl, None)
        ends = oracle.row_ends(wl.seq_lens, wl.next_n)
        thr = _sigma_thresholds(ref, ends, wl.top_k, "inf")
        d = dev(wl)
        sb = gpu_util.SelectBuffers(wl.rows, wl.batch, wl.top_k, wl.capacity, thr, workspace=ws)
        pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, **sb.kwargs())
        _check(wl, sb.host(), True, scores64=ref, tau=tau, untouched=False)


@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
def test_repair_rescore_bits_equal_logits_kernel(next_n):
    """The fused select's score buffer holds the logits kernel's bits: for
    next_n = 1 the repair scores a repaired request again and keeps its scores
    there, for next_n >= 2 the main pass writes every row's scores there (q and
    weights from LDS for next_n >= 3)."""
    wl = W.small_random(71 + next_n, [3000, 5000, 700, 1], next_n, 64, top_k=128, capacity=256)
    d = dev(wl)
    out, _ = run_logits(wl, d)
    logits = out.cpu().numpy()
    ws = pm.make_workspace("fused", wl.batch, wl.next_n, wl.max_seq_len)
    import gpu_util
    thr = np.full(wl.rows, np.inf, np.float32)  # every row with keys is repaired
    sb = gpu_util.SelectBuffers(wl.rows, wl.batch, wl.top_k, wl.capacity, thr, workspace=ws)
    pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, **sb.kwargs())
    sb.host()
    stride = -(-wl.max_seq_len // 64) * 64
    state = ws.numel() - wl.rows * stride * 4
    assert state == pm.workspace_bytes("indexer_topk", wl.batch, wl.next_n, wl.max_seq_len)
    scores = ws[state:].view(torch.float32).view(wl.rows, stride).cpu().numpy()
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    for r, e in enumerate(ends):
        a, b = scores[r, :e].view(np.int32), logits[r, :e].view(np.int32)
        assert np.array_equal(a, b), f"row {r}: {int(np.sum(a != b))} of {e} scores differ in their bits"


@pytest.mark.parametrize("next_n", [1, 2, 4])
def test_fused_writes_no_scores_when_rows_fit(next_n):
    """No score matrix in the fused path: with every row fitting (each
    threshold below the row's k-th score by more than the logits error, and
    room for every key above it), the score buffer at the end of the fused
    workspace keeps a sentinel in every byte, and no row is repaired."""
    wl = W.small_random(70 + next_n, [5000, 9000, 0, 3000], next_n, 64, top_k=256, capacity=1024)
    ref, tau = _oracle_rows(wl, None)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    thr = np.full(wl.rows, np.inf, np.float32)
    for r, e in enumerate(ends):
        if e == 0:
            continue
        s = np.sort(ref[r, :e])[::-1]
        k = min(int(e), wl.top_k)
        thr[r] = np.float32(s[k - 1] - 3 * tau[r])
        assert np.sum(ref[r, :e] > thr[r] - tau[r]) <= wl.capacity, "test input: too many keys near the threshold"
    import gpu_util
    nbytes = pm.workspace_bytes("fused", wl.batch, wl.next_n, wl.max_seq_len)
    score_bytes = wl.rows * (-(-wl.max_seq_len // 64) * 64) * 4
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ws[nbytes - score_bytes:] = 0xA5
    sb = gpu_util.SelectBuffers(wl.rows, wl.batch, wl.top_k, wl.capacity, thr, workspace=ws)
    d = dev(wl)
    pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, **sb.kwargs())
    res = sb.host()
    _check(wl, res, False, scores64=ref, tau=tau)
    tail = ws[nbytes - score_bytes:].cpu().numpy()
    assert np.all(tail == 0xA5), f"{int(np.sum(tail != 0xA5))} score-buffer bytes written"


def _duplicated_keys(seed, nn):
    """Two requests whose keys 128..255 (request 0) and 64..191 (request 1) are
    copies of one key (values and scale): 64-key groups in which every key
    scores the same for each row."""
    wl = W.small_random(seed, [1500, 900], nn, 64, top_k=256, capacity=512)
    kv = wl.kv_fused.copy()
    bs, D = wl.block_size, 128

    def tok(b, p):
        return int(wl.block_tables[b, p // bs]), p % bs

    for b, (src, lo, hi) in enumerate([(127, 128, 256), (63, 64, 192)]):
        ps, ss = tok(b, src)
        for p in range(lo, hi):
            pg, sl = tok(b, p)
            kv[pg, sl * D:(sl + 1) * D] = kv[ps, ss * D:(ss + 1) * D]
            kv[pg, bs * D + 4 * sl:bs * D + 4 * sl + 4] = kv[ps, bs * D + 4 * ss:bs * D + 4 * ss + 4]
    wl.kv_fused = kv
    return wl, [128, 64]


@pytest.mark.parametrize("nn", [1, 3, 4])
@pytest.mark.parametrize("path", ["fused", "unfused"])
def test_groups_full_of_near_band_keys(nn, path):
    """Thresholds just above the duplicated keys' common score put 64 near-band
    keys of every row in each of their groups, more than half a wave's list: the
    list is flushed before such a group, and every row still matches the
    oracle (a tie list of 32 entries for next_n 3 and 4 used to take them and
    write past its end)."""
    wl, first = _duplicated_keys(40 + nn, nn)
    s64 = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                                  wl.max_seq_len)
    tau = oracle.row_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size)
    thr = np.zeros(wl.rows, np.float32)
    for r in range(wl.rows):
        S = float(s64[r, first[r // nn]])
        thr[r] = np.float32(S * (1 + 2.0 ** -10) if S > 0 else S * (1 - 2.0 ** -10))
    d = dev(wl)
    if path == "fused":
        res = run_fused(wl, d, thr)
    else:
        _, view = run_logits(wl, d)
        res = run_select(wl, view, thr)
    _check(wl, res, True, scores64=s64, tau=tau)
