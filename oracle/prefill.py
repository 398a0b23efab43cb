"""Prefill-shaped rows in float64: explicit per-row key ends and a request per
query tile.

Page "flashinfer.sdsa.indexer_threshold_select", Parameters: row r sees the keys
below row_ends[r]; each query tile's request is tile_requests[tile], a row of
the block table.  Reading: a query tile is tile_rows consecutive rows (the
pages' tiles hold 128 rows; the rows of one tile all belong to its request),
row r = tile * tile_rows + t has its own q[r] and weights[r], and its score at
key p of its request is the logits formula of page "flashinfer.attn_scores"
(fp8_paged_mqa_logits: s_p * sum_h w[r, h] * relu(q[r, h, :] . k_p)).  The
select of a row is the same as for a decode row, with e_r = row_ends[r].

Pinned by: the decode case (tile_rows = next_n, tile_requests = 0..B-1,
row_ends from seq_lens) equal to paged_mqa_logits; prefix consistency (rows
with the same q and weights on one request: a shorter row's scores are the
prefix of a longer row's); Fraction brute force on a tiny shape with tiles
sharing a request and a row with no keys; invariance under a permutation of
the block table's rows applied through tile_requests.
"""
import numpy as np

from .layout import gather_request
from .logits import request_scores


def prefill_logits(q_rows: np.ndarray, kv_fused: np.ndarray, weights: np.ndarray, block_tables: np.ndarray,
                   tile_requests: np.ndarray, row_ends: np.ndarray, tile_rows: int, block_size: int,
                   max_context: int, rows=None):
    """Dense float64 scores [R, max_context] (R = len(row_ends)); NaN where a
    row sees no key.  q_rows: uint8 [R, H, D]; weights [R, H].
    rows: optional iterable of row indices to compute (others stay NaN)."""
    R = len(row_ends)
    Dd = q_rows.shape[2]
    out = np.full((R, max_context), np.nan, dtype=np.float64)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    for tile in range(R // tile_rows):
        rs = [tile * tile_rows + t for t in range(tile_rows)]
        if not any(r in want for r in rs):
            continue
        L = max(int(row_ends[r]) for r in rs)
        if L <= 0:
            continue
        b = int(tile_requests[tile])
        k, s = gather_request(kv_fused, block_tables[b], L, block_size, Dd)
        sc = request_scores(q_rows[rs[0]:rs[-1] + 1], k, s, weights[rs[0]:rs[-1] + 1])
        for t, r in enumerate(rs):
            e = int(row_ends[r])
            if r in want and e > 0:
                out[r, :e] = sc[t, :e]
    return out


def prefill_tolerance(q_rows: np.ndarray, kv_fused: np.ndarray, weights: np.ndarray, block_tables: np.ndarray,
                      tile_requests: np.ndarray, row_ends: np.ndarray, tile_rows: int, block_size: int,
                      rows=None, rel: float = 1e-4):
    """Per-row tolerance, the rule of row_tolerance with e_r = row_ends[r]:
    rel * sum_h |w_rh| * max_{p < e_r} s_p * max_h |q_rh . k_p|; rows seeing
    nothing get 0."""
    R = len(row_ends)
    Dd = q_rows.shape[2]
    tau = np.zeros(R, dtype=np.float64)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    for tile in range(R // tile_rows):
        rs = [tile * tile_rows + t for t in range(tile_rows)]
        if not any(r in want for r in rs):
            continue
        L = max(int(row_ends[r]) for r in rs)
        if L <= 0:
            continue
        b = int(tile_requests[tile])
        k, s = gather_request(kv_fused, block_tables[b], L, block_size, Dd)
        _, hmax = request_scores(q_rows[rs[0]:rs[-1] + 1], k, s, weights[rs[0]:rs[-1] + 1], with_headmax=True)
        for t, r in enumerate(rs):
            e = int(row_ends[r])
            if r in want and e > 0:
                tau[r] = rel * np.abs(weights[r].astype(np.float64)).sum() * np.max(s[:e] * hmax[t, :e])
    return tau
