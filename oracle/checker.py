"""Checker of a GPU select's outputs against the select contract and the oracle.

Page "flashinfer.sdsa.indexer_threshold_select" fixes what a correct output
holds (parameters counters, candidates, thresholds, arrivals, ranges and the
fit rule); the checker tests exactly those facts, on the raw int32 buffers a
call wrote.  Two modes:

* exact: the scores the GPU selected over are known bit for bit (the unfused
  indexer_topk reads them from a logits buffer the test supplied), so counts,
  index sets, repaired thresholds and ranges must match the oracle exactly;
* tolerant: only the float64 oracle scores are known (the fused path computes
  its own), so each check allows the per-row logits tolerance tau_r.

Pinned by: mutation tests that plant one flaw each in a correct output and
expect a complaint.
"""
import numpy as np

from .select import classify, decode_slots, fits, kth_largest, radix_key, select_with_repair

F32 = np.float32


def _bits_to_f32(b):
    return np.array([b], dtype=np.int32).view(np.float32)[0]


def read_slots(cand_row: np.ndarray, top_k: int, capacity: int, n_cand: int, n_tie: int):
    """(candidate pairs, tie pairs) actually stored in one row's slot buffer
    cand_row int32 [top_k + capacity, 2]."""
    nc = min(n_cand, capacity)
    nt = min(n_tie, top_k)
    cands = cand_row[top_k:top_k + nc]
    ties = cand_row[top_k - nt:top_k][::-1]
    return cands, ties


def check_row(r, *, e_r, top_k, capacity, threshold_in, threshold_out, counters, cand_row,
              rng, topk_row, repair, scores32=None, scores64=None, tau=0.0, untouched_slots=None,
              stats=None):
    """Violations (a list of strings, empty when the row is correct).

    untouched_slots: the int32 value every slot word held before the call; a
    row whose threshold did not change (or that sees no key) must then hold it
    in every slot outside its ranges (nothing else is written there).
    stats: a dict that collects, over the rows checked against float64 scores,
    how the k-th/(k+1)-th gap compares with tau (see exact_set_when_gapped).
    """
    errs = []
    n_cand, n_tie = int(counters[0]), int(counters[1])
    if n_cand < 0 or n_tie < 0:
        return [f"row {r}: negative counters {counters}"]
    t_out = F32(threshold_out)
    k = min(e_r, top_k)
    fit = fits(n_cand, n_tie, e_r, top_k, capacity)
    if repair and not fit:
        errs.append(f"row {r}: does not fit after repair (n_cand={n_cand}, n_tie={n_tie}, k={k})")
    if not repair and F32(threshold_in).view(np.int32) != t_out.view(np.int32):
        errs.append(f"row {r}: threshold changed without repair")
    cands, ties = read_slots(cand_row, top_k, capacity, n_cand, n_tie)
    idx = np.concatenate([cands[:, 0], ties[:, 0]]) if cands.size + ties.size else np.zeros(0, np.int32)
    if idx.size and (idx.min() < 0 or idx.max() >= e_r):
        errs.append(f"row {r}: slot index outside [0, {e_r})")
        return errs
    if np.unique(idx).size != idx.size:
        errs.append(f"row {r}: duplicate slot index")
    dec_c = decode_slots(np.ascontiguousarray(cands[:, 1]).view(np.float32), t_out, False)
    dec_t = decode_slots(np.ascontiguousarray(ties[:, 1]).view(np.float32), t_out, True)
    if dec_c.size and not np.all(dec_c > t_out):
        errs.append(f"row {r}: stored candidate not above threshold")
    if dec_t.size and not np.all((dec_t == t_out) | np.isnan(dec_t)):
        errs.append(f"row {r}: stored tie not equal to threshold")
    if rng is not None:
        exp = (top_k - min(n_tie, top_k), top_k + min(n_cand, capacity))
        if (int(rng[0]), int(rng[1])) != exp:
            errs.append(f"row {r}: ranges {tuple(int(x) for x in rng)} != {exp}")
    unchanged = F32(threshold_in).view(np.int32) == t_out.view(np.int32)
    if untouched_slots is not None and (unchanged or e_r == 0):
        lo, hi = top_k - min(n_tie, top_k), top_k + min(n_cand, capacity)
        outside = np.concatenate([cand_row[:lo].ravel(), cand_row[hi:].ravel()])
        if np.any(outside != np.int32(untouched_slots)):
            errs.append(f"row {r}: a slot outside [{lo},{hi}) was written")

    if scores32 is not None:
        s = np.asarray(scores32, dtype=np.float32)[:e_r]
        ref = select_with_repair(s, e_r, threshold_in, top_k, capacity) if repair else None
        if repair:
            if t_out.view(np.int32) != F32(ref["threshold"]).view(np.int32):
                errs.append(f"row {r}: threshold {t_out!r} != oracle {ref['threshold']!r}")
        cmask, tmask = classify(s, t_out)
        if n_cand != int(cmask.sum()) or n_tie != int(tmask.sum()):
            errs.append(f"row {r}: counters ({n_cand},{n_tie}) != ({int(cmask.sum())},{int(tmask.sum())})")
        if cands.size:
            if not np.all(cmask[cands[:, 0]]):
                errs.append(f"row {r}: stored candidate index is not a candidate")
            want = s[cands[:, 0]].astype(np.float32)
            if not np.array_equal(dec_c.view(np.int32), want.view(np.int32)):
                errs.append(f"row {r}: candidate score bits differ from the scores read")
        if ties.size and not np.all(tmask[ties[:, 0]]):
            errs.append(f"row {r}: stored tie index is not a tie")
        if n_cand <= capacity and cands.shape[0] == n_cand and set(cands[:, 0].tolist()) != set(np.nonzero(cmask)[0].tolist()):
            errs.append(f"row {r}: candidate set differs")
        if topk_row is not None and ref is not None and ref["topk"] is not None:
            must, maybe, need = ref["topk"]
            g = set(int(x) for x in np.asarray(topk_row)[:k])
            ms = set(must.tolist())
            if not ms <= g or not g <= ms | set(maybe.tolist()) or len(g) != k:
                errs.append(f"row {r}: topk differs from the oracle's Top-k")
    elif scores64 is not None:
        s = np.asarray(scores64, dtype=np.float64)[:e_r]
        t64 = np.float64(t_out)
        lo = int((s > t64 + tau).sum())
        hi = int((s > t64 - tau).sum())
        if not (lo <= n_cand <= hi):
            errs.append(f"row {r}: n_cand={n_cand} outside [{lo},{hi}] (tau={tau:.3g})")
        if cands.size:
            err = np.abs(dec_c.astype(np.float64) - s[cands[:, 0]])
            if err.max() > tau:
                errs.append(f"row {r}: candidate score off by {err.max():.3g} > tau {tau:.3g}")
        if ties.size:
            err = np.abs(s[ties[:, 0]] - t64)
            if err.max() > tau:
                errs.append(f"row {r}: tie score off the threshold by {err.max():.3g} > tau")
        if repair and k > 0 and F32(threshold_in).view(np.int32) != t_out.view(np.int32):
            sk = np.sort(s)[::-1][k - 1]
            if abs(np.float64(t_out) - sk) > tau:
                errs.append(f"row {r}: repaired threshold {t_out} not within tau of sigma_k={sk}")
    if topk_row is not None:
        errs += check_topk_against_slots(r, topk_row, cands, dec_c, ties, k, top_k, n_cand)
        if scores64 is not None and k > 0:
            s64 = np.asarray(scores64, dtype=np.float64)[:e_r]
            errs += check_set_rule(r, topk_row[:k], s64, k, tau)
            ex = exact_set_when_gapped(topk_row[:k], s64, k, tau)
            if ex is False:
                errs.append(f"row {r}: gap above 2 tau but the set is not the exact sort prefix")
            if stats is not None:
                gap_stats(stats, topk_row[:k], s64, k, tau)
    return errs


def check_topk_against_slots(r, topk_row, cands, dec_c, ties, k, top_k, n_cand):
    """The exact Top-k a fitting row's slots yield, compared as a set."""
    errs = []
    got = np.asarray(topk_row)
    if np.any(got[k:] != -1):
        errs.append(f"row {r}: topk entries past k={k} are not -1")
    g = got[:k]
    if np.any(g < 0) or np.unique(g).size != k:
        errs.append(f"row {r}: topk has {np.unique(g[g >= 0]).size} distinct valid entries, want {k}")
        return errs
    gs = set(g.tolist())
    cset = set(cands[:, 0].tolist())
    if n_cand <= k:
        if not cset <= gs:
            errs.append(f"row {r}: topk misses a candidate")
        tset = set(ties[:, 0].tolist())
        if not (gs - cset) <= tset:
            errs.append(f"row {r}: topk holds an index that is neither candidate nor tie")
    else:
        if not gs <= cset:
            errs.append(f"row {r}: topk holds a non-candidate")
        kth = kth_largest(dec_c, k)
        kk = radix_key(np.array([kth], dtype=np.float32))[0]
        keys = radix_key(dec_c)
        must = set(cands[keys > kk, 0].tolist())
        maybe = set(cands[keys == kk, 0].tolist())
        if not must <= gs or not gs <= (must | maybe):
            errs.append(f"row {r}: topk is not the k largest candidates")
    return errs


def check_set_rule(r, got, s64, k, tau):
    """Top-k set rule of the parity contract: the set has k members, holds every p with
    sigma_p > sigma_k + 2 tau and only p with sigma_p >= sigma_k - 2 tau
    (2 tau: each GPU score may be off by tau).  Exact when the k-th/(k+1)-th
    gap exceeds 2 tau."""
    errs = []
    srt = np.sort(s64)[::-1]
    sk = srt[k - 1]
    gs = set(int(x) for x in got)
    must = set(np.nonzero(s64 > sk + 2 * tau)[0].tolist())
    allowed = set(np.nonzero(s64 >= sk - 2 * tau)[0].tolist())
    if len(gs) != k:
        errs.append(f"row {r}: set size {len(gs)} != {k}")
    if not must <= gs:
        errs.append(f"row {r}: set misses {len(must - gs)} keys above sigma_k + 2 tau")
    if not gs <= allowed:
        errs.append(f"row {r}: set holds {len(gs - allowed)} keys below sigma_k - 2 tau")
    return errs


def gap_stats(stats, got, s64, k, tau):
    """Counts, per row, where the k-th/(k+1)-th gap lies against tau, and how
    often the set is the exact sort prefix in each band: "gap>2tau" (the sound
    form of the set rule; must be exact), "tau<gap<=2tau" (the literal
    form: exact unless the GPU's own rounding swapped the two), "gap<=tau"
    (tie membership only), "all" (k = row length: every key)."""
    if k >= s64.size:
        band = "all"
    else:
        srt = np.sort(s64)[::-1]
        gap = srt[k - 1] - srt[k]
        band = "gap>2tau" if gap > 2 * tau else ("tau<gap<=2tau" if gap > tau else "gap<=tau")
    ref = set(np.argsort(-s64, kind="stable")[:k].tolist())
    exact = set(int(x) for x in got) == ref
    d = stats.setdefault(band, [0, 0])
    d[0] += 1
    d[1] += int(exact)


def exact_set_when_gapped(got, s64, k, tau):
    """True when the k-th/(k+1)-th gap exceeds 2 tau and the set is then the exact
    sort prefix (the strict form of the set rule)."""
    srt = np.sort(s64)[::-1]
    if k >= s64.size or srt[k - 1] - srt[k] <= 2 * tau:
        return None
    ref = set(np.argsort(-s64, kind="stable")[:k].tolist())
    return set(int(x) for x in got) == ref
