"""Paged MQA logits in float64.

Page "flashinfer.attn_scores", fp8_paged_mqa_logits (the formula block and the
paragraph after it):

    logits[b*next_n + t, p] = s_p * sum_h w[b*next_n + t, h] * relu(q[b,t,h,:] . k_p)

with the ReLU applied to each head's dot product before the weighted head sum,
s_p the token's float32 scale from region 2 of its block, and row
b*next_n + t meaningful only for p in 0 .. seq_lens[b] - next_n + t (the Note
and Returns sections).  Requests with seq_lens[b] == 0 produce no output.

The dot products are exact in float64: an e4m3 x e4m3 product has at most 8
significant bits and is a multiple of 2^-18 below 2^18 in magnitude, so a
128-term sum needs at most 43 bits.  The only rounding is in the weighted head
sum and the scale multiply (about 1e-16 relative).

Pinned by: Fraction brute force on tiny shapes; per-head ReLU cases (dots +x
and -x with unit weights give x, not 0); negative weights giving negative
results; scale factoring (s_p = 2^j scales exactly; s_p = 1 reduces to the
unscaled formula); closed forms with all-ones inputs; block-table permutation
invariance; the per-slot visibility counts of the pages' Example.
"""
import numpy as np

from .e4m3 import decode_e4m3
from .layout import gather_request

CHUNK = 8192


def row_ends(seq_lens: np.ndarray, next_n: int) -> np.ndarray:
    """Visible key count of each row r = b*next_n + t: seq_lens[b] - next_n + t + 1,
    at least 0 (page "flashinfer.attn_scores", Note and Returns)."""
    L = np.repeat(np.asarray(seq_lens, dtype=np.int64), next_n)
    t = np.tile(np.arange(next_n, dtype=np.int64), len(seq_lens))
    return np.maximum(0, L - next_n + t + 1)


def request_scores(q_codes_b: np.ndarray, k: np.ndarray, s: np.ndarray, w_rows: np.ndarray,
                   with_headmax: bool = False):
    """Scores of one request's rows over all of its positions.

    q_codes_b: uint8 [next_n, H, D]; k: float64 [L, D]; s: float64 [L];
    w_rows: float32/64 [next_n, H].  Returns float64 [next_n, L] (and, if
    asked, max_h |q_h . k_p| as float64 [next_n, L]).
    """
    nn, Hh, Dd = q_codes_b.shape
    L = k.shape[0]
    q = decode_e4m3(q_codes_b)                       # [nn, H, D]
    w = np.asarray(w_rows, dtype=np.float64)          # [nn, H]
    out = np.empty((nn, L), dtype=np.float64)
    hmax = np.empty((nn, L), dtype=np.float64) if with_headmax else None
    for t in range(nn):
        for c0 in range(0, L, CHUNK):
            kc = k[c0:c0 + CHUNK]
            dots = q[t] @ kc.T                         # [H, chunk], exact
            out[t, c0:c0 + CHUNK] = s[c0:c0 + CHUNK] * (w[t] @ np.maximum(dots, 0.0))
            if with_headmax:
                hmax[t, c0:c0 + CHUNK] = np.abs(dots).max(axis=0)
    return (out, hmax) if with_headmax else out


def paged_mqa_logits(q: np.ndarray, kv_fused: np.ndarray, weights: np.ndarray,
                     block_tables: np.ndarray, seq_lens: np.ndarray, block_size: int,
                     max_seq_len: int, rows=None):
    """Dense float64 logits [B*next_n, max_seq_len]; NaN marks positions a row does
    not see and every position of a request with seq_lens[b] == 0.

    rows: optional iterable of row indices to compute (others stay NaN).
    """
    B, nn, Hh, Dd = q.shape
    R = B * nn
    out = np.full((R, max_seq_len), np.nan, dtype=np.float64)
    ends = row_ends(seq_lens, nn)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    for b in range(B):
        L = int(seq_lens[b])
        rs = [b * nn + t for t in range(nn)]
        if L == 0 or not any(r in want for r in rs):
            continue
        k, s = gather_request(kv_fused, block_tables[b], L, block_size, Dd)
        sc = request_scores(q[b], k, s, weights[b * nn:(b + 1) * nn])
        for t, r in enumerate(rs):
            if r in want:
                e = int(ends[r])
                out[r, :e] = sc[t, :e]
    return out


def row_tolerance(q: np.ndarray, kv_fused: np.ndarray, weights: np.ndarray,
                  block_tables: np.ndarray, seq_lens: np.ndarray, block_size: int, rows=None,
                  rel: float = 1e-4):
    """Per-row logits tolerance tau_r = rel * sum_h |w_rh| * max_{p visible} s_p * max_h |q_rh . k_p|.

    The stated bound scales with sum_h |w_h| * max_h |q_h . k|; the per-token
    scale multiplies every term of a row's score, so it enters the scale of
    the error as well.  Rows with nothing visible get 0.
    """
    B, nn, Hh, Dd = q.shape
    R = B * nn
    ends = row_ends(seq_lens, nn)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    tau = np.zeros(R, dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        rs = [b * nn + t for t in range(nn)]
        if L == 0 or not any(r in want for r in rs):
            continue
        k, s = gather_request(kv_fused, block_tables[b], L, block_size, Dd)
        _, hmax = request_scores(q[b], k, s, weights[b * nn:(b + 1) * nn], with_headmax=True)
        for t, r in enumerate(rs):
            e = int(ends[r])
            if r in want and e > 0:
                m = np.max(s[:e] * hmax[t, :e])
                tau[r] = rel * np.abs(weights[r].astype(np.float64)).sum() * m
    return tau
