"""Writes the per-row thresholds of the large workloads, computed by the oracle.

Each large workload's select thresholds are defined from its exact row scores
(the k-th largest score, less 1e-3, or the 256-th largest for the rows meant
to be repaired).  This script computes them with the float64 oracle and
stores them, with sigma_k, sigma_{k+1} and the per-row tolerance, as JSON
beside it.  It imports only the oracle and the input generators.

    python tests/golden/make_thresholds.py 3 4 5 prefill

"prefill" is the prefill chunk (prefill-shaped rows): each row's threshold
is its min(row_end, 2048)-th largest score less 1e-3.
"""
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads as W  # noqa: E402


def row_stats(wl, k_main=2048, k_high=256):
    R = wl.rows
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    sig = {k: np.full(R, np.nan) for k in (k_high, k_main, k_main + 1)}
    tau = np.zeros(R)
    for b in range(wl.batch):
        L = int(wl.seq_lens[b])
        if L == 0:
            continue
        k, s = oracle.gather_request(wl.kv_fused, wl.block_tables[b], L, wl.block_size, 128)
        sc, hmax = oracle.request_scores(wl.q[b], k, s, wl.weights[b * wl.next_n:(b + 1) * wl.next_n],
                                         with_headmax=True)
        for t in range(wl.next_n):
            r = b * wl.next_n + t
            e = int(ends[r])
            if e == 0:
                continue
            srt = np.sort(sc[t, :e])[::-1]
            for kk in sig:
                if kk <= e:
                    sig[kk][r] = srt[kk - 1]
            tau[r] = 1e-4 * np.abs(wl.weights[r].astype(np.float64)).sum() * np.max(s[:e] * hmax[t, :e])
    return ends, sig, tau


def thresholds_for(cfg, wl, ends, sig):
    R = wl.rows
    thr = np.zeros(R, np.float32)
    for r in range(R):
        if ends[r] == 0:
            continue
        if cfg == 5 and r % wl.next_n == 0:
            thr[r] = np.float32(sig[256][r])
        else:
            thr[r] = np.float32(sig[2048][r] - 1e-3)
    return thr


def main(cfgs):
    for cfg in cfgs:
        t0 = time.time()
        wl = W.make(cfg)
        ends, sig, tau = row_stats(wl)
        thr = thresholds_for(cfg, wl, ends, sig)
        doc = {
            "_about": f"Oracle-computed select thresholds for workload {wl.name}; written by make_thresholds.py",
            "recipe": wl.threshold_recipe,
            "workload": wl.name,
            "fingerprint": W.fingerprint(wl),
            "threshold_bits": [int(x) for x in thr.view(np.int32)],
            "sigma_256": [None if np.isnan(x) else float(x) for x in sig[256]],
            "sigma_k": [None if np.isnan(x) else float(x) for x in sig[2048]],
            "sigma_k1": [None if np.isnan(x) else float(x) for x in sig[2049]],
            "tau": [float(x) for x in tau],
            "row_ends": [int(x) for x in ends],
        }
        with open(os.path.join(HERE, f"thresholds_cfg{cfg}.json"), "w") as f:
            json.dump(doc, f, indent=0)
        print(f"cfg{cfg}: {wl.rows} rows in {time.time() - t0:.1f}s", flush=True)


def prefill_main():
    t0 = time.time()
    wl = W.prefill_chunk()
    s64 = oracle.prefill_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.tile_requests, wl.row_ends,
                                wl.tile_rows, wl.block_size, wl.max_context)
    tau = oracle.prefill_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.tile_requests, wl.row_ends,
                                   wl.tile_rows, wl.block_size)
    thr = np.zeros(wl.rows, np.float32)
    sig_k = [None] * wl.rows
    sig_k1 = [None] * wl.rows
    for r, e in enumerate(wl.row_ends):
        if e <= 0:
            continue
        srt = np.sort(s64[r, :e])[::-1]
        k = min(int(e), wl.top_k)
        thr[r] = np.float32(srt[k - 1] - 1e-3)
        sig_k[r] = float(srt[k - 1])
        sig_k1[r] = float(srt[k]) if k < e else None
    doc = {
        "_about": f"Oracle-computed select thresholds for workload {wl.name}; written by make_thresholds.py",
        "recipe": "sigma_min(row_end,k)_minus_1e-3",
        "workload": wl.name,
        "fingerprint": W.prefill_fingerprint(wl),
        "threshold_bits": [int(x) for x in thr.view(np.int32)],
        "sigma_k": sig_k,
        "sigma_k1": sig_k1,
        "tau": [float(x) for x in tau],
        "row_ends": [int(x) for x in wl.row_ends],
    }
    with open(os.path.join(HERE, "thresholds_prefill_chunk.json"), "w") as f:
        json.dump(doc, f, indent=0)
    print(f"prefill chunk: {wl.rows} rows in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    args = sys.argv[1:] or ["3", "4", "5"]
    main([int(a) for a in args if a != "prefill"])
    if "prefill" in args:
        prefill_main()
