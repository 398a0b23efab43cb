"""Pins of the oracle's select semantics and mutation tests of the contract
checker (CPU only)."""
import numpy as np
import pytest

from oracle import select as S
from oracle.checker import check_row, check_set_rule
from select_sim import simulate, f32_bits

F32 = np.float32


def test_kth_largest_brute_force():
    g = np.random.default_rng(0)
    for trial in range(200):
        n = int(g.integers(1, 40))
        x = g.choice(np.array([-2, -1, -0.0, 0.0, 0.5, 1, 1, 3, np.nan], np.float32), size=n)
        k = int(g.integers(1, n + 1))
        # brute force: NaN lowest, -0 == +0, k-th in descending order
        key = lambda v: (0, 0.0) if np.isnan(v) else (1, float(v))
        want = sorted(x.tolist(), key=key, reverse=True)[k - 1]
        got = S.kth_largest(x, k)
        if np.isnan(want):
            assert np.isnan(got)
        else:
            assert got == want
            if want == 0:
                assert np.signbit(got) == False  # noqa: E712  (canonical +0)


def test_radix_key_order():
    vals = np.array([-np.inf, -3.5, -1e-30, -0.0, 0.0, 1e-30, 2.0, np.inf], np.float32)
    k = S.radix_key(vals)
    assert k[3] == k[4]
    assert np.all(np.diff(k[[0, 1, 2, 4, 5, 6, 7]].astype(np.int64)) > 0)
    assert S.radix_key(np.array([np.nan, -np.nan], np.float32)).tolist() == [0, 0]
    assert k.min() > 0


def test_topk_equals_sort_prefix():
    g = np.random.default_rng(1)
    x = g.normal(size=500)
    idx, sk, sk1 = S.topk_indices(x, 37)
    ref = sorted(range(500), key=lambda i: -x[i])[:37]
    assert list(idx) == ref and sk == x[ref[-1]] and sk1 < sk


def test_classify_ties_and_nan():
    s = np.array([1.0, 2.0, np.nan, 2.0, -0.0, 3.0], np.float32)
    c, t = S.classify(s, F32(2.0))
    assert c.tolist() == [False, False, False, False, False, True]
    assert t.tolist() == [False, True, True, True, False, False]
    c0, t0 = S.classify(np.array([0.0, -0.0], np.float32), F32(-0.0))
    assert t0.tolist() == [True, True]


def test_threshold_select_counts_brute_force():
    g = np.random.default_rng(2)
    for _ in range(100):
        n = int(g.integers(0, 60))
        x = g.choice(np.arange(-4, 5).astype(np.float32), size=n)
        t = F32(g.integers(-4, 5))
        e = int(g.integers(0, n + 1))
        top_k, cap = int(g.integers(1, 10)), int(g.integers(0, 12))
        res = S.threshold_select(x, e, t, top_k, cap)
        nc = sum(1 for v in x[:e] if v > t)
        nt = sum(1 for v in x[:e] if v == t)
        assert (res["n_cand"], res["n_tie"]) == (nc, nt)
        k = min(e, top_k)
        assert res["fit"] == (nc <= cap and nc + min(nt, top_k) >= k)
        if res["fit"]:
            # the exact Top-k (by value) lies among candidates + stored ties
            order = sorted(range(e), key=lambda i: -x[i])[:k]
            kth = x[order[-1]] if k else None
            assert all(x[i] >= t for i in order) or k == 0


@pytest.mark.parametrize("cap_mode", ["topk_minus_1", "double"])
def test_repair_always_fits(cap_mode):
    g = np.random.default_rng(3)
    for _ in range(200):
        n = int(g.integers(1, 80))
        x = (g.integers(-5, 6, size=n) * 0.5).astype(np.float32)
        top_k = int(g.integers(1, 12))
        cap = top_k - 1 if cap_mode == "topk_minus_1" else 2 * top_k
        e = int(g.integers(0, n + 1))
        t = F32(g.choice([-10, -1, 0, 0.5, 2, 10, np.inf]))
        res = S.select_with_repair(x, e, t, top_k, cap)
        assert res["fit"]
        k = min(e, top_k)
        if res["repaired"]:
            assert res["threshold"] == S.kth_largest(x[:e], k)
        must, maybe, need = res["topk"]
        chosen = set(must.tolist()) | set(maybe[:need].tolist())
        assert len(chosen) == k
        ref_vals = sorted(x[:e].tolist(), reverse=True)[:k]
        assert sorted((x[i] for i in chosen), reverse=True) == ref_vals


def test_encoding_roundtrip_and_order():
    g = np.random.default_rng(4)
    for t in [F32(1.5), F32(-2.0), F32(0.0), F32(1e-30), F32(3e38), F32(0.001)]:
        s = np.sort(np.concatenate([
            np.nextafter(t, np.float32(np.inf)) + np.abs(g.normal(size=50)).astype(np.float32) * abs(t if t else 1),
            np.array([np.nextafter(t, np.float32(np.inf)), F32(2) * t if t > 0 else F32(1), np.float32(np.inf)], np.float32)]).astype(np.float32))
        s = s[s > t]
        enc = np.array([S.encode_candidate(v, t) for v in s], np.float32)
        dec = np.array([S.decode_slot(v, t, False) for v in enc], np.float32)
        assert np.array_equal(dec.view(np.int32), s.view(np.int32))
        assert np.all(enc[1:] >= enc[:-1])      # order kept
        if t > 0:
            near = s[s <= F32(2) * t]
            assert np.all(np.array([S.encode_candidate(v, t) for v in near]) == near - t)
    assert S.encode_tie(F32(2.0), F32(2.0)) == 0 and np.isnan(S.encode_tie(F32(np.nan), F32(2.0)))
    assert S.decode_slot(F32(0.0), F32(2.0), True) == 2.0


# ---------------------------------------------------------------- checker mutations

def _setup(seed=5, R=4, n=300, top_k=16, cap=32, repair=True):
    g = np.random.default_rng(seed)
    scores = [np.round(g.normal(size=n) * 8).astype(np.float32) / 4 for _ in range(R)]  # many exact ties
    ends = [n, n - 1, 10, 0][:R]
    thr = [F32(np.sort(scores[0])[::-1][top_k - 1]), F32(100.0), F32(-100.0), F32(0.0)][:R]
    out = simulate(scores, ends, thr, top_k, cap, repair=repair, seed=seed)
    return scores, ends, thr, out, top_k, cap


def _errs(scores, ends, thr, out, top_k, cap, repair=True, exact=True):
    errs = []
    for r in range(len(ends)):
        errs += check_row(r, e_r=ends[r], top_k=top_k, capacity=cap, threshold_in=thr[r],
                          threshold_out=out["thresholds"][r], counters=out["counters"][r],
                          cand_row=out["candidates"][r], rng=out["ranges"][:, r] if repair else None,
                          topk_row=out["topk"][r] if repair else None, repair=repair,
                          scores32=scores[r] if exact else None,
                          scores64=None if exact else scores[r].astype(np.float64), tau=1e-6)
    return errs


@pytest.mark.parametrize("exact", [True, False])
def test_checker_accepts_correct_output(exact):
    a = _setup()
    assert _errs(*a, exact=exact) == []
    b = _setup(seed=6, repair=False)
    assert _errs(*b, repair=False, exact=exact) == []


def _mutate_and_expect(mut, exact=True, seed=5):
    scores, ends, thr, out, top_k, cap = _setup(seed=seed)
    mut(out, top_k, cap, ends, scores)
    e = _errs(scores, ends, thr, out, top_k, cap, exact=exact)
    assert e, "checker missed a planted flaw"
    return e


@pytest.mark.parametrize("exact", [True, False])
def test_mutation_candidate_not_above(exact):
    def m(out, top_k, cap, ends, scores):
        r = 0
        t = out["thresholds"][r]
        out["candidates"][r, top_k, 1] = f32_bits(np.float32(-1e9))
    _mutate_and_expect(m, exact)


@pytest.mark.parametrize("exact", [True, False])
def test_mutation_tie_in_wrong_slot(exact):
    def m(out, top_k, cap, ends, scores):
        r = 0
        nt = int(out["counters"][r, 1])
        assert nt >= 1
        # move the first tie into the first unused candidate slot and drop the tie count
        nc = int(out["counters"][r, 0])
        out["candidates"][r, top_k + nc] = out["candidates"][r, top_k - 1]
        out["counters"][r] = (nc + 1, nt - 1)
    _mutate_and_expect(m, exact)


@pytest.mark.parametrize("exact", [True, False])
def test_mutation_wrong_range(exact):
    def m(out, top_k, cap, ends, scores):
        out["ranges"][1, 1] += 1
    _mutate_and_expect(m, exact)


@pytest.mark.parametrize("exact", [True, False])
def test_mutation_non_fitting_row_reported(exact):
    def m(out, top_k, cap, ends, scores):
        out["counters"][0] = (cap + 1, 0)
    _mutate_and_expect(m, exact)


@pytest.mark.parametrize("exact", [True, False])
def test_mutation_index_past_row_end(exact):
    def m(out, top_k, cap, ends, scores):
        out["candidates"][2, top_k, 0] = ends[2]
        out["counters"][2, 0] = max(1, out["counters"][2, 0])
    _mutate_and_expect(m, exact)


@pytest.mark.parametrize("exact", [True, False])
def test_mutation_duplicate_index(exact):
    def m(out, top_k, cap, ends, scores):
        nc = int(out["counters"][0, 0])
        assert nc >= 2
        out["candidates"][0, top_k + 1, 0] = out["candidates"][0, top_k, 0]
    _mutate_and_expect(m, exact)


def test_mutation_wrong_threshold_exact():
    def m(out, top_k, cap, ends, scores):
        out["thresholds"][1] = np.nextafter(out["thresholds"][1], np.float32(np.inf))
    _mutate_and_expect(m, True)


def test_mutation_wrong_topk():
    def m(out, top_k, cap, ends, scores):
        r = 1
        s = scores[r][:ends[r]]
        worst = int(np.argmin(s))
        out["topk"][r, 0] = worst
    _mutate_and_expect(m, True)
    _mutate_and_expect(m, False)


def test_mutation_counter_off_by_one():
    def m(out, top_k, cap, ends, scores):
        out["counters"][1, 0] += 1
    _mutate_and_expect(m, True)


def test_set_rule():
    s = np.array([5.0, 4.0, 3.0, 2.0, 2.0, 1.0])
    assert check_set_rule(0, [0, 1, 2], s, 3, 0.0) == []
    assert check_set_rule(0, [0, 1, 3], s, 3, 0.0) != []
    assert check_set_rule(0, [0, 1, 2, 3], s, 4, 0.0) == []
    assert check_set_rule(0, [0, 1, 2, 4], s, 4, 0.0) == []   # equal scores: either tie member
    assert check_set_rule(0, [0, 1, 3, 4], s, 4, 0.6) == []   # within 2 tau of sigma_k


def test_decode_slots_matches_scalar_decode():
    g = np.random.default_rng(12)
    vals = np.concatenate([g.normal(size=200).astype(np.float32) * 5,
                           np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3e38, 1e-38], np.float32)])
    for t in [F32(1.5), F32(-2.0), F32(0.0), F32(3e38), F32(np.inf), F32(-np.inf)]:
        for tie in (False, True):
            want = np.array([S.decode_slot(v, t, tie) for v in vals], np.float32)
            got = S.decode_slots(vals, t, tie)
            assert np.array_equal(want.view(np.int32), got.view(np.int32)), (t, tie)


def test_mutation_stray_slot_write():
    """A write into a slot outside a row's ranges (rows not repaired, or empty)
    is reported when the slots' prior contents are known."""
    SENT = -0x21524111
    scores, ends, thr, out, top_k, cap = _setup(seed=6, repair=False)
    for r in range(len(ends)):
        lo = top_k - min(int(out["counters"][r, 1]), top_k)
        hi = top_k + min(int(out["counters"][r, 0]), cap)
        out["candidates"][r, :lo] = SENT
        out["candidates"][r, hi:] = SENT

    def errs(o):
        e = []
        for r in range(len(ends)):
            e += check_row(r, e_r=ends[r], top_k=top_k, capacity=cap, threshold_in=thr[r],
                           threshold_out=o["thresholds"][r], counters=o["counters"][r],
                           cand_row=o["candidates"][r], rng=None, topk_row=None, repair=False,
                           scores32=scores[r], untouched_slots=SENT)
        return e
    assert errs(out) == []
    for r in (0, 3):   # a row with slots in use, and the empty one
        bad = {k: v.copy() for k, v in out.items()}
        bad["candidates"][r, -1] = (0, 0)
        assert errs(bad), f"stray write in row {r} not reported"


def test_gap_stats_bands():
    from oracle.checker import gap_stats, exact_set_when_gapped
    s = np.array([9.0, 8.0, 5.0, 4.99, 1.0])
    st = {}
    gap_stats(st, [0, 1], s, 2, 1.0)        # gap 3 > 2 tau: exact
    gap_stats(st, [0, 2, 1], s, 3, 0.004)   # gap 0.01 > 2 tau
    gap_stats(st, [0, 1, 3], s, 3, 0.008)   # tau < gap 0.01 <= 2 tau, swapped: not exact
    gap_stats(st, [0, 1, 2], s, 3, 0.02)    # gap <= tau
    gap_stats(st, [0, 1, 2, 3, 4], s, 5, 0.1)
    assert st == {"gap>2tau": [2, 2], "tau<gap<=2tau": [1, 0], "gap<=tau": [1, 1], "all": [1, 1]}
    assert exact_set_when_gapped([0, 1], s, 2, 1.0) is True
    assert exact_set_when_gapped([0, 2], s, 2, 1.0) is False
    assert exact_set_when_gapped([0, 1, 3], s, 3, 0.008) is None
