"""Pins of the oracle's paged MQA logits (CPU only)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import paged_mqa_logits, row_ends

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
ONE = 0x38  # e4m3 1.0


def _pack(vals_u8, scales):
    nb = vals_u8.shape[0]
    v = torch.as_tensor(vals_u8, dtype=torch.uint8).reshape(nb, -1)
    s = torch.as_tensor(scales, dtype=torch.float32).reshape(nb, -1).contiguous().view(torch.uint8)
    return torch.cat([v, s], dim=1).numpy()


def _e4m3(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _tiny(seed, B=2, nn=2, H=4, D=8, bs=4, seq=(5, 9), scale=True):
    g = np.random.default_rng(seed)
    nb = sum(math.ceil(L / bs) for L in seq) + 1
    vals = _e4m3(g.normal(size=(nb, bs, D)) * 2)
    scales = g.uniform(0.5, 2.0, size=(nb, bs)).astype(np.float32) if scale else np.ones((nb, bs), np.float32)
    q = _e4m3(g.normal(size=(B, nn, H, D)) * 2)
    w = g.uniform(-1, 1, size=(B * nn, H)).astype(np.float32)
    perm = g.permutation(nb - 1).astype(np.int32)
    width = max(math.ceil(L / bs) for L in seq)
    bt = np.full((B, width), nb - 1, dtype=np.int32)
    off = 0
    for b, L in enumerate(seq):
        n = math.ceil(L / bs)
        bt[b, :n] = perm[off:off + n]
        off += n
    return q, _pack(vals, scales), w, bt, np.array(seq, np.int32), bs


def _fraction_e4m3(code):
    code = int(code)
    sign = -1 if code & 0x80 else 1
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return sign * Fraction(m, 512)
    return sign * (8 + m) * Fraction(2) ** (e - 7) / 8


def _brute(q, kv, w, bt, seq, bs):
    """Exact rational arithmetic, one loop per index, straight from the formula."""
    B, nn, H, D = q.shape
    out = {}
    for b in range(B):
        for t in range(nn):
            r = b * nn + t
            e = int(seq[b]) - nn + t + 1
            for p in range(max(e, 0)):
                blk = kv[bt[b, p // bs]]
                slot = p % bs
                kp = blk[slot * D:(slot + 1) * D]
                sp = Fraction(float(blk[bs * D + 4 * slot: bs * D + 4 * slot + 4].view("<f4")[0]))
                acc = Fraction(0)
                for h in range(H):
                    dot = sum(_fraction_e4m3(q[b, t, h, d]) * _fraction_e4m3(kp[d]) for d in range(D))
                    acc += Fraction(float(w[r, h])) * max(dot, Fraction(0))
                out[(r, p)] = sp * acc
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fraction_brute_force(seed):
    q, kv, w, bt, seq, bs = _tiny(seed)
    ref = _brute(q, kv, w, bt, seq, bs)
    got = paged_mqa_logits(q, kv, w, bt, seq, bs, max(seq))
    for (r, p), v in ref.items():
        assert abs(got[r, p] - float(v)) <= 1e-15 * max(1.0, abs(float(v)))
    ends = row_ends(seq, q.shape[1])
    for r in range(got.shape[0]):
        assert np.all(np.isnan(got[r, ends[r]:])) and not np.any(np.isnan(got[r, :ends[r]]))


def _one_key_setup(q_rows, w_row, k_vec, s=1.0):
    """One request, next_n=1, H heads, one visible key (seq_len 1, bs 32)."""
    H, D = q_rows.shape
    bs = 32
    vals = np.zeros((1, bs, D), np.uint8)
    vals[0, 0] = k_vec
    sc = np.ones((1, bs), np.float32)
    sc[0, 0] = s
    kv = _pack(vals, sc)
    q = q_rows.reshape(1, 1, H, D).astype(np.uint8)
    return paged_mqa_logits(q, kv, np.asarray(w_row, np.float32).reshape(1, H), np.zeros((1, 1), np.int32),
                            np.array([1], np.int32), bs, 1)[0, 0]


def test_relu_per_head_not_of_sum():
    """Dots +x and -x with unit weights give x (ReLU of the sum would give 0)."""
    H, D = 64, 128
    k = np.zeros(D, np.uint8); k[0] = ONE
    q = np.zeros((H, D), np.uint8)
    q[0, 0] = _e4m3(3.0)
    q[1, 0] = _e4m3(-3.0)
    w = np.zeros(H, np.float32); w[0] = w[1] = 1.0
    assert _one_key_setup(q, w, k) == 3.0
    assert _one_key_setup(q, w, k, s=0.5) == 1.5


def test_negative_weights_give_negative_logits():
    wl = W.config1()
    wl.weights[:] = -np.abs(wl.weights) - 1e-3
    out = paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size, wl.max_seq_len)
    assert np.all(out[0] <= 0) and np.mean(out[0] < 0) > 0.99


def test_zero_weights_and_all_negative_dots():
    H, D = 64, 128
    k = np.zeros(D, np.uint8); k[:] = ONE
    q = np.full((H, D), _e4m3(-1.0), np.uint8)           # every dot is -128
    w = np.linspace(-1, 1, H).astype(np.float32)
    assert _one_key_setup(q, w, k) == 0.0
    q2 = np.full((H, D), ONE, np.uint8)
    assert _one_key_setup(q2, np.zeros(H, np.float32), k) == 0.0


def test_closed_form_all_ones():
    H, D = 64, 128
    k = np.full(D, ONE, np.uint8)
    q = np.full((H, D), ONE, np.uint8)
    w = np.arange(H, dtype=np.float32) / 64 - 0.25
    s = 1.75
    assert _one_key_setup(q, w, k, s) == s * 128.0 * float(np.sum(w.astype(np.float64)))


def test_scale_factoring_and_linearity():
    q, kv, w, bt, seq, bs = _tiny(5, H=64, D=128, bs=32, seq=(40, 70), scale=False)
    base = paged_mqa_logits(q, kv, w, bt, seq, bs, max(seq))
    # s_p = 2^j scales exactly (a power of two commutes with every rounding)
    kv2 = kv.copy()
    nb = kv.shape[0]
    for blk in range(nb):
        sc = kv2[blk, bs * 128:].view("<f4")
        sc[:] = 8.0
    scaled = paged_mqa_logits(q, kv2, w, bt, seq, bs, max(seq))
    ok = ~np.isnan(base)
    assert np.array_equal(scaled[ok], 8.0 * base[ok])
    # s_p = 1 reduces to the unscaled formula, recomputed head by head
    qd = oracle.decode_e4m3(q)
    for b in range(2):
        k, s = oracle.gather_request(kv, bt[b], int(seq[b]), bs, 128)
        assert np.all(s == 1.0)
        for t in range(2):
            r = b * 2 + t
            e = int(seq[b]) - 2 + t + 1
            ref = np.zeros(e)
            for h in range(64):
                ref += w[r, h].astype(np.float64) * np.maximum(k[:e] @ qd[b, t, h], 0)
            assert np.allclose(base[r, :e], ref, rtol=1e-12, atol=1e-12)
    # linear in the weights
    w2 = (np.random.default_rng(9).uniform(-1, 1, w.shape)).astype(np.float32)
    a = paged_mqa_logits(q, kv, w2, bt, seq, bs, max(seq))
    c = paged_mqa_logits(q, kv, (w.astype(np.float64) + w2).astype(np.float64), bt, seq, bs, max(seq))
    assert np.allclose(c[ok], base[ok] + a[ok], rtol=1e-12, atol=1e-9)


def test_block_table_permutation_invariance():
    q, kv, w, bt, seq, bs = _tiny(7, H=64, D=128, bs=32, seq=(33, 97))
    base = paged_mqa_logits(q, kv, w, bt, seq, bs, max(seq))
    g = np.random.default_rng(3)
    perm = g.permutation(kv.shape[0])
    inv = np.argsort(perm)
    kv2 = kv[perm]                       # physical block j of kv2 is old block perm[j]
    bt2 = inv[bt].astype(np.int32)
    got = paged_mqa_logits(q, kv2, w, bt2, seq, bs, max(seq))
    assert np.array_equal(np.isnan(base), np.isnan(got))
    ok = ~np.isnan(base)
    assert np.array_equal(base[ok], got[ok])
    # a wrong table changes the answer
    bt3 = bt.copy(); bt3[1, [0, 1]] = bt3[1, [1, 0]]
    bad = paged_mqa_logits(q, kv, w, bt3, seq, bs, max(seq))
    assert not np.allclose(bad[2:, :64], base[2:, :64], equal_nan=True)


def test_pages_example_visibility():
    g = GOLD["example_row_ends"]
    assert row_ends(np.array(g["seq_lens"]), g["next_n"]).tolist() == g["value"]
    wl = W.config2()
    out = paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                           wl.max_seq_len, rows=[0, 5])
    assert out.shape == tuple(GOLD["example_shapes"]["logits_view"])
    assert np.sum(~np.isnan(out[0])) == 2998 and np.sum(~np.isnan(out[5])) == 8000
    assert np.all(out[0][:2998] >= 0) and np.all(out[5] >= 0)  # weights U[0,1]


def test_empty_request_and_short_request():
    q, kv, w, bt, seq, bs = _tiny(11, B=3, nn=3, H=64, D=128, bs=32, seq=(0, 2, 40))
    out = paged_mqa_logits(q, kv, w, bt, seq, bs, 40)
    assert np.all(np.isnan(out[0:3]))                      # seq_len 0: no row written
    # seq_len 2 < next_n 3: rows see 0, 1, 2 positions
    assert [int(np.sum(~np.isnan(out[r]))) for r in (3, 4, 5)] == [0, 1, 2]
    assert [int(np.sum(~np.isnan(out[r]))) for r in (6, 7, 8)] == [38, 39, 40]
