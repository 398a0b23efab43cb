"""Pins of the oracle's e4m3 decoding and kv_fused parsing (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import decode_e4m3, parse_block

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3_anchors():
    d = decode_e4m3(np.array([0x38, 0x7E, 0x01, 0x80, 0xFE, 0x7F, 0xFF, 0x08], dtype=np.uint8))
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -9
    assert d[3] == 0.0 and math.copysign(1, d[3]) < 0
    assert d[4] == -448.0 and np.isnan(d[5]) and np.isnan(d[6])
    assert d[7] == 2.0 ** -6        # smallest normal
    assert not np.any(np.isinf(decode_e4m3(np.arange(256, dtype=np.uint8))))


def test_printed_offsets():
    g = GOLD
    assert oracle.region2_offset(32, 128) == g["region2_offset"]["value"] == 4096
    assert oracle.block_bytes(32, 128) == g["block_bytes"]["value"] == 4224
    assert oracle.min_block_table_width(*g["min_block_table_width"]["args"]) == g["min_block_table_width"]["value"]
    assert oracle.padded_seq_len(*g["padded_seq_len"]["args"]) == g["padded_seq_len"]["value"]


def _torch_cat_block(values_u8, scales_f32):
    """The pages' Example packing recipe, for one or more blocks."""
    nb = values_u8.shape[0]
    return torch.cat([values_u8.reshape(nb, -1), scales_f32.view(torch.uint8).reshape(nb, -1)], dim=1)


def test_parse_block_roundtrip_and_scale_offsets():
    bs, D = 32, 128
    vals = torch.randint(0, 256, (1, bs, D), dtype=torch.uint8, generator=torch.Generator().manual_seed(1))
    vals[vals == 0x7F] = 0
    vals[vals == 0xFF] = 0
    scales = torch.arange(1, bs + 1, dtype=torch.float32).reshape(1, bs) * 0.25
    blk = _torch_cat_block(vals, scales)[0].numpy()
    assert blk.size == 4224
    codes, s = parse_block(blk, bs, D)
    assert np.array_equal(codes, vals[0].numpy())
    assert np.array_equal(s, scales[0].double().numpy())
    base, stride = GOLD["scale_offset"]["base"], GOLD["scale_offset"]["stride"]
    for i in (0, 1, 7, 31):
        raw = blk[base + stride * i: base + stride * i + 4].view("<f4")[0]
        assert raw == s[i]
        assert np.array_equal(blk[i * 128:(i + 1) * 128], codes[i])


def test_per_token_row_misreading_differs():
    """Reading the block as 32 rows of 132 bytes (values + scale per token) is the
    misreading the pages warn about; it must give different keys and scales."""
    bs, D = 32, 128
    g = torch.Generator().manual_seed(2)
    vals = torch.randn(1, bs, D, generator=g).to(torch.float8_e4m3fn).view(torch.uint8)
    scales = 0.5 + torch.rand(1, bs, generator=g)
    blk = _torch_cat_block(vals, scales)[0].numpy()
    rows = blk.reshape(bs, D + 4)
    wrong_codes = rows[:, :D]
    wrong_scales = rows[:, D:].copy().view("<f4")[:, 0]
    codes, s = parse_block(blk, bs, D)
    assert not np.array_equal(wrong_codes, codes)
    assert not np.allclose(wrong_scales, s, equal_nan=True)


def test_gather_follows_block_table():
    """Position p comes from block table[p // bs], slot p % bs: give every token a
    distinct scale and recover the positions from a permuted table."""
    bs, D, L = 32, 128, 100
    n = math.ceil(L / bs)
    perm = np.array([5, 2, 7, 0], dtype=np.int32)
    nb = 8
    vals = torch.zeros(nb, bs, D, dtype=torch.uint8)
    scales = torch.zeros(nb, bs)
    for j in range(n):
        for i in range(bs):
            scales[perm[j], i] = float(j * bs + i + 1)
            vals[perm[j], i, 0] = 0x38        # 1.0 at d=0
    kv = _torch_cat_block(vals, scales).numpy()
    table = np.concatenate([perm, np.full(4, 99, dtype=np.int32)])  # entries past ceil(L/bs) are never read
    k, s = oracle.gather_request(kv, table, L, bs, D)
    assert k.shape == (L, D)
    assert np.array_equal(s, np.arange(1, L + 1, dtype=np.float64))
    assert np.all(k[:, 0] == 1.0) and np.all(k[:, 1:] == 0.0)
