"""Pins of the oracle's MXFP4 paged logits (CPU only).

Page "flashinfer.attn_scores", fp4_paged_mqa_logits: the formula block, the
parameters q, q_sf, kv_fused (the byte-offset figure and the nibble picture),
is_kv_sf_interleaved, and the Restrictions.  Each pin would catch a plausible
slip: a wrong E2M1 value or scale bias (the table and anchors), nibbles or
scale bytes in the wrong order (the figure's pictures and the brute force),
per-token rows instead of two regions (the misreading), the interleaved slot
rule inverted (the brute force over slots), a relu of the sum (the two-head
case), a double or missing rounding in the reduced precisions (the bfloat16
anchors and the simulations).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.fp4 import (E2M1_TABLE, decode_ue8m0, fp4_block_bytes, fp4_paged_mqa_logits, fp4_region2_offset,
                        parse_fp4_block, round_bf16, unpack_fp4)

# E2M1 codes of the OCP MX definition, by value (sign in bit 3)
CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


def _code(v):
    return CODE[abs(v)] | (8 if v < 0 else 0)


def _pack(vals):
    """float values [..., 2n] (E2M1 numbers) -> uint8 [..., n], element 2m in
    the low nibble of byte m (the page's nibble rule, written out here)."""
    v = np.asarray(vals, dtype=np.float64)
    codes = np.vectorize(_code)(v).astype(np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def _block(vals, scale_bytes, interleaved=False):
    """One block: vals [bs, 128] E2M1 numbers, scale_bytes uint8 [bs, 4] per
    token; the scale region in token order, or in the interleaved slot order
    (slot k holds token (k % 4) * (bs // 4) + k // 4), written out here."""
    bs = vals.shape[0]
    sb = np.asarray(scale_bytes, dtype=np.uint8)
    if interleaved:
        sb = np.stack([sb[(k % 4) * (bs // 4) + k // 4] for k in range(bs)])
    return np.concatenate([_pack(vals).reshape(-1), sb.reshape(-1)])


def test_e2m1_table_hand_values():
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    np.testing.assert_array_equal(E2M1_TABLE, want)
    assert np.signbit(E2M1_TABLE[8])
    assert E2M1_TABLE[:8].sum() == 18


def test_ue8m0_anchors():
    got = decode_ue8m0([127, 128, 120, 0, 254, 255])
    np.testing.assert_array_equal(got[:5], [1.0, 2.0, 2.0 ** -7, 2.0 ** -127, 2.0 ** 127])
    assert np.isnan(got[5])


def test_printed_offsets_and_scale_positions():
    assert fp4_region2_offset(32) == 2048 and fp4_block_bytes(32) == 2176
    g = np.random.default_rng(0)
    vals = g.choice(list(CODE), size=(32, 128)) * g.choice([-1, 1], size=(32, 128))
    sb = g.integers(120, 135, size=(32, 4)).astype(np.uint8)
    blk = _block(vals, sb)
    assert blk.size == 2176
    for i in range(32):
        assert list(blk[2048 + 4 * i: 2048 + 4 * i + 4]) == list(sb[i])
    deq, raw, sc = parse_fp4_block(blk, 32)
    np.testing.assert_array_equal(raw, vals)
    np.testing.assert_array_equal(sc, 2.0 ** (sb.astype(np.int64) - 127))
    np.testing.assert_array_equal(deq, vals * np.repeat(sc, 32, axis=1))


def test_nibble_rule_of_the_figure():
    # [e1|e0]: byte 0 holds e0 low, e1 high; e0 = 0.5 (code 1), e1 = -4 (code 0xE)
    row = np.zeros(64, np.uint8)
    row[0] = 0xE1
    row[63] = 0x72  # e126 = 1.0 (low), e127 = 6.0 (high)
    v = unpack_fp4(row)
    assert v[0] == 0.5 and v[1] == -4.0 and v[126] == 1.0 and v[127] == 6.0
    assert np.all(v[2:126] == 0)


def test_per_token_row_misreading_differs():
    """Reading a block as 68-byte per-token rows (values then scales of each
    token) gives other values: the layout is two regions."""
    g = np.random.default_rng(1)
    vals = g.choice(list(CODE), size=(32, 128))
    sb = g.integers(124, 130, size=(32, 4)).astype(np.uint8)
    blk = _block(vals, sb)
    rows = blk.reshape(32, 68)
    wrong = unpack_fp4(rows[:, :64]) * np.repeat(2.0 ** (rows[:, 64:].astype(np.int64) - 127), 32, axis=1)
    deq, _, _ = parse_fp4_block(blk, 32)
    assert not np.array_equal(wrong, deq)


def test_torch_cat_recipe_round_trip():
    """The fp8 Example's torch.cat recipe with the fp4 regions: values
    [nb, bs*64] then scales [nb, bs*4], per block."""
    g = np.random.default_rng(2)
    nb, bs = 3, 64
    vals = g.choice(list(CODE), size=(nb, bs, 128))
    sb = g.integers(120, 135, size=(nb, bs, 4)).astype(np.uint8)
    kv = torch.cat([torch.from_numpy(_pack(vals).reshape(nb, -1)), torch.from_numpy(sb.reshape(nb, -1))], 1).numpy()
    for j in range(nb):
        _, raw, sc = parse_fp4_block(kv[j], bs)
        np.testing.assert_array_equal(raw, vals[j])
        np.testing.assert_array_equal(sc, 2.0 ** (sb[j].astype(np.int64) - 127))


def test_interleaved_slot_rule():
    g = np.random.default_rng(3)
    bs = 128
    vals = g.choice(list(CODE), size=(bs, 128))
    sb = g.integers(100, 150, size=(bs, 4)).astype(np.uint8)
    inter = _block(vals, sb, interleaved=True)
    _, _, sc = parse_fp4_block(inter, bs, interleaved=True)
    np.testing.assert_array_equal(sc, 2.0 ** (sb.astype(np.int64) - 127))
    # brute force over slots: slot k of the region holds token (k % 4) * 32 + k // 4
    region = inter[bs * 64:].reshape(bs, 4)
    for k in range(bs):
        assert list(region[k]) == list(sb[(k % 4) * 32 + k // 4])
    # the token-order reading of an interleaved region is wrong
    _, _, wrong = parse_fp4_block(inter, bs, interleaved=False)
    assert not np.array_equal(wrong, sc)


def _tiny_fp4(seed, B=2, nn=2, H=2, bs=4, seq=(5, 9), interleaved=False):
    g = np.random.default_rng(seed)
    nblk = [-(-L // bs) for L in seq]
    nb = sum(nblk) + 1
    vals = g.choice(list(CODE), size=(nb, bs, 128)) * g.choice([-1, 1], size=(nb, bs, 128))
    sb = g.integers(124, 131, size=(nb, bs, 4)).astype(np.uint8)
    kv = np.stack([_block(vals[j], sb[j], interleaved) for j in range(nb)])
    qv = g.choice(list(CODE), size=(B, nn, H, 128)) * g.choice([-1, 1], size=(B, nn, H, 128))
    qsb = g.integers(124, 131, size=(B, nn, H, 4)).astype(np.uint8)
    q = _pack(qv)
    q_sf = qsb.view("<i4").reshape(B, nn, H)
    w = g.uniform(-1, 1, size=(B * nn, H)).astype(np.float32)
    perm = g.permutation(nb - 1)
    width = max(nblk)
    bt = np.full((B, width), nb - 1, np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    return dict(q=q, q_sf=q_sf, kv=kv, w=w, bt=bt, seq=np.array(seq, np.int32), bs=bs, vals=vals, sb=sb, qv=qv,
                qsb=qsb)


def _brute(d):
    """Exact rationals, one loop per index, from the formula; scale bytes read
    as (q_sf >> 8k) & 0xff here, independently of the oracle's decoding."""
    q, w, bt, seq, bs = d["qv"], d["w"], d["bt"], d["seq"], d["bs"]
    B, nn, H, D = q.shape
    out = {}
    for b in range(B):
        for t in range(nn):
            r = b * nn + t
            for p in range(max(int(seq[b]) - nn + t + 1, 0)):
                blk, slot = int(bt[b, p // bs]), p % bs
                acc = Fraction(0)
                for h in range(H):
                    sfw = int(d["q_sf"][b, t, h]) & 0xFFFFFFFF
                    dot = Fraction(0)
                    for i in range(D):
                        qs = Fraction(2) ** (((sfw >> (8 * (i // 32))) & 0xFF) - 127)
                        ks = Fraction(2) ** (int(d["sb"][blk, slot, i // 32]) - 127)
                        dot += Fraction(q[b, t, h, i]) * qs * Fraction(d["vals"][blk, slot, i]) * ks
                    acc += Fraction(float(w[r, h])) * max(dot, Fraction(0))
                out[(r, p)] = acc
    return out


@pytest.mark.parametrize("seed,interleaved,bs", [(0, False, 4), (1, False, 8), (2, True, 128)])
def test_fraction_brute_force(seed, interleaved, bs):
    seq = (5, 9) if bs < 128 else (130, 3)
    d = _tiny_fp4(seed, bs=bs, seq=seq, interleaved=interleaved)
    got = fp4_paged_mqa_logits(d["q"], d["q_sf"], d["kv"], d["w"], d["bt"], d["seq"], bs, max(seq),
                               output_dtype="f32", interleaved=interleaved)["value"]
    ref = _brute(d)
    for (r, p), v in ref.items():
        assert abs(got[r, p] - float(v)) <= 1e-15 * max(1.0, abs(float(v))), (r, p)
    ends = [max(int(d["seq"][r // 2]) - 2 + r % 2 + 1, 0) for r in range(4)]
    for r, e in enumerate(ends):
        assert np.all(np.isnan(got[r, e:])) and not np.any(np.isnan(got[r, :e]))


def test_relu_per_head_and_scale_factoring():
    d = _tiny_fp4(4, seq=(6, 6))
    base = fp4_paged_mqa_logits(d["q"], d["q_sf"], d["kv"], d["w"], d["bt"], d["seq"], 4, 6,
                                output_dtype="f32")["value"]
    # every group scale of every key raised by one: every logit doubles
    kv2 = d["kv"].copy()
    kv2[:, 4 * 64:] += 1
    dbl = fp4_paged_mqa_logits(d["q"], d["q_sf"], kv2, d["w"], d["bt"], d["seq"], 4, 6, output_dtype="f32")["value"]
    m = ~np.isnan(base)
    np.testing.assert_array_equal(dbl[m], 2 * base[m])
    # two heads with dots +x and -x and unit weights give x (relu per head)
    q = np.zeros((1, 1, 2, 64), np.uint8)
    q[0, 0, 0, 0] = 0x02   # head 0: element 0 = 1.0
    q[0, 0, 1, 0] = 0x0A   # head 1: element 0 = -1.0
    q_sf = np.full((1, 1, 2), 0x7F7F7F7F, np.int32)
    vals = np.zeros((4, 128))
    vals[0, 0] = 3.0
    kv = np.stack([_block(vals, np.full((4, 4), 127, np.uint8)), _block(vals, np.full((4, 4), 127, np.uint8))])
    r = fp4_paged_mqa_logits(q, q_sf, kv, np.ones((1, 2), np.float32), np.array([[0]], np.int32),
                             np.array([1], np.int32), 4, 1, output_dtype="f32")["value"]
    assert r[0, 0] == 3.0


def test_round_bf16_hand_values_and_torch():
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.4e38, 2.0 ** -134, 1.5 * 2.0 ** -133, -(1 + 2.0 ** -7), 0.1])
    want = np.array([1.0, 1 + 2.0 ** -6, np.inf, 0.0, 2.0 ** -132, -(1 + 2.0 ** -7), 0.10009765625])
    np.testing.assert_array_equal(round_bf16(x), want)
    g = np.random.default_rng(5)
    v = (g.normal(size=2000) * 10.0 ** g.integers(-30, 30, size=2000)).astype(np.float32)
    t = torch.from_numpy(v).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(round_bf16(v.astype(np.float64)), t)


def _simulate(d, epi, rng):
    """The reduced-precision epilogue with each product and sum rounded (torch
    float16 / bfloat16 scalars), heads in a random order."""
    from oracle.fp4 import dequant_q, gather_fp4_request
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[epi]
    qd = dequant_q(d["q"], d["q_sf"])
    B, nn, H, _ = d["q"].shape
    out = {}
    for b in range(B):
        L = int(d["seq"][b])
        k, _, _ = gather_fp4_request(d["kv"], d["bt"][b], L, d["bs"])
        for t in range(nn):
            r = b * nn + t
            for p in range(max(L - nn + t + 1, 0)):
                dots = torch.tensor(qd[b, t] @ k[p]).to(dt)
                c = torch.clamp(dots, min=0)
                w = torch.from_numpy(d["w"][r]).to(dt)
                acc = torch.zeros((), dtype=dt)
                for h in rng.permutation(H):
                    acc = acc + w[h] * c[h]
                out[(r, p)] = float(acc)
    return out


@pytest.mark.parametrize("epi", ["f16", "bf16"])
def test_reduced_epilogue_orders_stay_within_tol(epi):
    d = _tiny_fp4(6, H=64, seq=(7, 5))
    ref = fp4_paged_mqa_logits(d["q"], d["q_sf"], d["kv"], d["w"], d["bt"], d["seq"], 4, 7, output_dtype="f32",
                               epi_dtype=epi)
    rng = np.random.default_rng(7)
    worst = 0.0
    for _ in range(2):
        for (r, p), v in _simulate(d, epi, rng).items():
            err = abs(v - ref["value"][r, p])
            assert err <= ref["tol"][r, p], (r, p, v, ref["value"][r, p], ref["tol"][r, p])
            worst = max(worst, err)
    assert worst > 0
