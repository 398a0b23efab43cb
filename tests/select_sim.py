"""Builds the buffers a correct select call writes, from the oracle's select
semantics, so the contract checker can be tested on known-good and
known-bad outputs.  Test helper; CPU only."""
import numpy as np

from oracle.select import encode_candidate, encode_tie, select_with_repair, threshold_select

SENTINEL = -0x21524111  # 0xDEADBEEF as int32


def f32_bits(x):
    return int(np.array([x], dtype=np.float32).view(np.int32)[0])


def simulate(scores32, ends, thresholds, top_k, capacity, repair=True, seed=0):
    """scores32: list of float32 rows (visible prefix at least); returns a dict of
    the output buffers (thresholds, counters, candidates, ranges, topk)."""
    rng = np.random.default_rng(seed)
    R = len(ends)
    thr = np.asarray(thresholds, dtype=np.float32).copy()
    counters = np.zeros((R, 2), np.int32)
    cand = np.full((R, top_k + capacity, 2), SENTINEL, np.int32)
    ranges = np.zeros((2, R), np.int32)
    topk = np.full((R, top_k), -1, np.int32)
    for r in range(R):
        e = int(ends[r])
        s = np.asarray(scores32[r], dtype=np.float32)[:e]
        res = select_with_repair(s, e, thr[r], top_k, capacity) if repair else threshold_select(s, e, thr[r], top_k, capacity)
        t = res["threshold"]
        thr[r] = t
        counters[r] = (res["n_cand"], res["n_tie"])
        ci = rng.permutation(res["cand"])[:capacity]
        ti = rng.permutation(res["tie"])[:top_k]
        for n, i in enumerate(ci):
            cand[r, top_k + n] = (i, f32_bits(encode_candidate(s[i], t)))
        for n, i in enumerate(ti):
            cand[r, top_k - 1 - n] = (i, f32_bits(encode_tie(s[i], t)))
        if repair:
            ranges[:, r] = res["ranges"]
            if res["topk"] is not None:
                must, maybe, need = res["topk"]
                chosen = list(must) + list(rng.permutation(maybe)[:need]) if need else list(must)
                if res["n_cand"] <= min(e, top_k):
                    # all candidates + the first `need` stored tie slots
                    chosen = list(res["cand"]) + [int(cand[r, top_k - 1 - n, 0]) for n in range(need)]
                topk[r, :len(chosen)] = chosen
    return {"thresholds": thr, "counters": counters, "candidates": cand, "ranges": ranges, "topk": topk}
