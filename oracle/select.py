"""Threshold Top-k select with candidate and tie slots, fit test and repair.

Page "flashinfer.sdsa.indexer_threshold_select" (the description and the
parameters thresholds, counters, candidates, arrivals, ranges):

* A visible key (index below the row's end) whose score is above the row's
  threshold is a candidate; one that is neither above nor below it (equal, or
  NaN) is a tie.  Both are counted; the n-th candidate is stored in slot
  top_k + n if n < capacity, the n-th tie in slot top_k - 1 - n if n < top_k,
  each as (key index, score bits).
* A row fits when n_cand <= capacity and n_cand + min(n_tie, top_k) >=
  min(row_end, top_k).  Its exact Top-k is then among its slots.
* With arrivals, every row that does not fit is selected again at its
  min(row_end, top_k)-th largest score (radix-selected), which becomes its new
  threshold.  With capacity >= top_k - 1 every row then fits.
* ranges[0][r], ranges[1][r] bound the slots holding the row's ties and
  candidates.

Scores here are float32 values, compared exactly as float32 (the select works
on the scores the scoring step produced).  Radix order: -0.0 and +0.0 are the
same key, NaN ranks below everything.

Pinned by: brute force on tiny rows (Python sorted()), the page's fit rule
written as counts, and the checker's mutation tests.  The score encoding in
the slots follows a reading of a garbled sentence and is "parity unpinned"
(see encode_candidate).
"""
import numpy as np

F32 = np.float32


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def classify(scores, threshold):
    """(candidate mask, tie mask) of float32 scores against a float32 threshold."""
    s = _f32(scores)
    t = F32(threshold)
    cand = s > t
    tie = ~(s > t) & ~(s < t)
    return cand, tie


def fits(n_cand: int, n_tie: int, row_end: int, top_k: int, capacity: int) -> bool:
    return n_cand <= capacity and n_cand + min(n_tie, top_k) >= min(row_end, top_k)


def radix_key(scores) -> np.ndarray:
    """Order-preserving uint32 key: larger score -> larger key; +-0 share a key;
    NaN maps to 0, below every number."""
    s = _f32(scores).copy()
    s[s == 0] = F32(0.0)                  # -0.0 -> +0.0
    u = s.view(np.uint32).astype(np.uint64)
    key = np.where(u & 0x80000000, (~u) & 0xFFFFFFFF, u | 0x80000000).astype(np.uint32)
    key[np.isnan(s)] = 0
    return key


def kth_largest(scores, k: int):
    """The k-th largest float32 score in radix order (1-based k), returned as the
    float32 whose key it is (so a zero comes back as +0.0)."""
    assert k >= 1
    keys = np.sort(radix_key(scores))[::-1]
    kk = np.uint32(keys[k - 1])
    if kk == 0:
        return F32(np.nan)
    u = np.uint32(kk & 0x7FFFFFFF) if kk & 0x80000000 else np.uint32(~kk & 0xFFFFFFFF)
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def topk_indices(scores64, k: int):
    """Exact Top-k of a row by full sort (stable): (indices, sigma_k, sigma_{k+1})."""
    x = np.asarray(scores64, dtype=np.float64)
    order = np.argsort(-x, kind="stable")
    k = min(k, x.size)
    sk = x[order[k - 1]] if k > 0 else np.inf
    sk1 = x[order[k]] if k < x.size else -np.inf
    return order[:k], sk, sk1


def encode_candidate(score, threshold):
    """Stored value of a candidate.  The page's sentence on the stored score bits
    (indexer_threshold_select, description paragraph 2) is garbled; the reading
    taken: the difference s - t is stored where it is exact, i.e. when t > 0 and
    s <= 2t (exact by Sterbenz' lemma, since t < s <= 2t), else s itself.  The
    map is increasing in s, so it keeps the candidates' order.
    Parity unpinned: the pages give no value to check it against."""
    s = F32(score)
    t = F32(threshold)
    with np.errstate(over="ignore"):
        twice = F32(2.0) * t
    if t > 0 and s <= twice:
        return F32(s - t)
    return s


def encode_tie(score, threshold):
    """Stored value of a tie: s - t (a zero, or NaN for a NaN score)."""
    with np.errstate(invalid="ignore"):
        return F32(F32(score) - F32(threshold))


def decode_slot(value, threshold, is_tie: bool):
    """Inverse of the encodings: the score a stored value stands for."""
    v = F32(value)
    t = F32(threshold)
    if is_tie:
        return F32(np.nan) if np.isnan(v) else t
    if t > 0 and v <= t:
        return F32(v + t)
    return v


def decode_slots(values, threshold, is_tie: bool):
    """decode_slot over an array of stored float32 values (same arithmetic,
    element by element)."""
    v = np.asarray(values, dtype=np.float32)
    t = F32(threshold)
    if is_tie:
        return np.where(np.isnan(v), F32(np.nan), t).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        shifted = (v + t).astype(np.float32)
    return np.where((t > 0) & (v <= t), shifted, v).astype(np.float32)


def threshold_select(scores, row_end: int, threshold, top_k: int, capacity: int):
    """One row's single-pass select: counts and the full candidate / tie index
    sets over the visible keys (which of them land in slots when a class
    overflows its slots is unspecified)."""
    s = _f32(scores)[:row_end]
    cand, tie = classify(s, threshold)
    ci = np.nonzero(cand)[0]
    ti = np.nonzero(tie)[0]
    return {
        "n_cand": int(ci.size), "n_tie": int(ti.size), "cand": ci, "tie": ti,
        "fit": fits(int(ci.size), int(ti.size), row_end, top_k, capacity),
        "threshold": F32(threshold),
    }


def select_with_repair(scores, row_end: int, threshold, top_k: int, capacity: int):
    """Select, then (as with arrivals) repair a row that does not fit by selecting
    again at its min(row_end, top_k)-th largest score.  Returns the final
    select dict plus "repaired", "ranges" (half-open [lo, hi)) and "topk" (the
    set a finalize step extracts from the slots, when the row fits)."""
    res = threshold_select(scores, row_end, threshold, top_k, capacity)
    repaired = False
    if not res["fit"]:
        k = min(row_end, top_k)
        t2 = kth_largest(_f32(scores)[:row_end], k)
        res = threshold_select(scores, row_end, t2, top_k, capacity)
        repaired = True
    res["repaired"] = repaired
    nt = min(res["n_tie"], top_k)
    nc = min(res["n_cand"], capacity)
    res["ranges"] = (top_k - nt, top_k + nc)
    res["topk"] = finalize_from_sets(_f32(scores), res, row_end, top_k) if res["fit"] else None
    return res


def finalize_from_sets(scores32, res, row_end: int, top_k: int):
    """The k = min(row_end, top_k) indices a fitting row's slots yield: every
    candidate if there are at most k of them, topped up with ties; else the k
    largest candidates.  Returns (must, maybe, need): indices that must be in
    the set, indices of which exactly `need` more must be taken."""
    k = min(row_end, top_k)
    cand, tie = res["cand"], res["tie"]
    if cand.size <= k:
        return cand, tie, k - cand.size
    vals = scores32[cand]
    kth = kth_largest(vals, k)
    kk = radix_key(np.array([kth], dtype=np.float32))[0]
    keys = radix_key(vals)
    must = cand[keys > kk]
    maybe = cand[keys == kk]
    return must, maybe, k - must.size
