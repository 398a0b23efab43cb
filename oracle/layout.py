"""Byte layout of the fused paged KV pool and the size helpers.

Page "flashinfer.attn_scores", fp8_paged_mqa_logits, parameter kv_fused (and
its byte-offset figure): each block is read as block_size*(head_dim+4) flat
bytes in two regions -- region 1 holds the e4m3 values token-major (token i at
byte i*head_dim), region 2 holds block_size little-endian float32 scales
(token i's at byte block_size*head_dim + 4*i).  It is not 132-byte per-token
rows.

Pinned by: the figure's offsets (region 2 at 4096, block end 4224, token i's
scale at 4096+4i for block_size=32, head_dim=128); a round trip through the
Example's torch.cat packing; and a negative test showing the per-token-row
misreading gives different values.
"""
import math

import numpy as np

from .e4m3 import decode_e4m3


def region2_offset(block_size: int, head_dim: int) -> int:
    return block_size * head_dim


def block_bytes(block_size: int, head_dim: int) -> int:
    return block_size * (head_dim + 4)


def parse_block(block: np.ndarray, block_size: int, head_dim: int):
    """One block's flat bytes -> (codes uint8 [bs, D], scales float64 [bs])."""
    flat = np.asarray(block, dtype=np.uint8).reshape(-1)
    assert flat.size == block_bytes(block_size, head_dim)
    r2 = region2_offset(block_size, head_dim)
    codes = flat[:r2].reshape(block_size, head_dim)
    scales = flat[r2:].view("<f4").astype(np.float64)
    return codes, scales


def gather_request(kv_fused: np.ndarray, block_table_row: np.ndarray, seq_len: int,
                   block_size: int, head_dim: int):
    """Keys and scales of one request's positions 0..seq_len-1, in logical order.

    Position p lives in physical block block_table_row[p // block_size], slot
    p % block_size (page "flashinfer.attn_scores", parameter block_tables).
    Only the first ceil(seq_len / block_size) table entries are read.
    Returns (k float64 [seq_len, D], s float64 [seq_len]).
    """
    n_pages = int(math.ceil(seq_len / block_size))
    ks, ss = [], []
    for j in range(n_pages):
        codes, scales = parse_block(kv_fused[int(block_table_row[j])], block_size, head_dim)
        ks.append(decode_e4m3(codes))
        ss.append(scales)
    if not ks:
        return np.zeros((0, head_dim)), np.zeros((0,))
    return np.concatenate(ks)[:seq_len], np.concatenate(ss)[:seq_len]


def min_block_table_width(seq_len: int, block_size: int) -> int:
    """ceil(seq_len / block_size): one table entry per block a request occupies
    (page "flashinfer.attn_scores", Example and parameter block_tables)."""
    return int(math.ceil(seq_len / block_size))


def padded_seq_len(max_seq_len: int) -> int:
    """Output column count.  The pages give one data point (8000 -> 8192, the
    Example's out= comment); the reading taken is rounding up to 256 columns."""
    return int(math.ceil(max_seq_len / 256)) * 256
