"""Pins of the oracle's float16 options of the logits (CPU only).

Page "flashinfer.attn_scores", fp8_paged_mqa_logits: the formula block's three
precisions and the parameters output_dtype, epi_dtype, acc_dtype, weights.
Each pin would catch a plausible slip: a dot product not rounded (the 2049
pin), weights left unrounded in a float16 epilogue (the 0.1 pin and its
mutant), no overflow to infinity (the 2^17 pins), a bound too tight for some
summation order (the simulation pin).
"""
import numpy as np
import pytest

import oracle
from oracle.dtypes import F16, mqa_logits_dtypes, round_f16

from test_oracle_logits import _e4m3, _pack, _tiny

H, D, BS = 4, 8, 4


def _one_key(qv, kv_vals, w, s):
    """One request of one key, next_n = 1: q[0,0,h,:] = qv[h], key = kv_vals,
    weights w [H], scale s.  Values are exact e4m3 numbers."""
    q = _e4m3(np.array(qv, np.float32).reshape(1, 1, H, D))
    vals = np.zeros((2, BS, D), np.float32)
    vals[0, 0] = kv_vals
    kv = _pack(_e4m3(vals), np.full((2, BS), s, np.float32))
    bt = np.array([[0]], np.int32)
    return q, kv, np.array([w], np.float32), bt, np.array([1], np.int32)


def _vec(*pairs):
    v = np.zeros(D, np.float32)
    for i, x in pairs:
        v[i] = x
    return v


def _run(args, **kw):
    q, kv, w, bt, seq = args
    return mqa_logits_dtypes(q, kv, w, bt, seq, BS, 1, **kw)


def test_round_f16_hand_values():
    # (the subnormal spacing is 2^-24: 2.5 and 3.5 units are ties, to the even unit)
    x = np.array([2049, 2051, 0.1, 65504, 65519, 65520, 1e-8, -2049, 2.5 * 2 ** -24, 3.5 * 2 ** -24])
    want = np.array([2048, 2052, 0.0999755859375, 65504, 65504, np.inf, 0.0, -2048, 2 * 2.0 ** -24, 4 * 2.0 ** -24])
    np.testing.assert_array_equal(round_f16(x), want)


@pytest.mark.parametrize("seed", [0, 1])
def test_f32_options_reduce_to_the_definition(seed):
    q, kv, w, bt, seq, bs = _tiny(seed)
    got = mqa_logits_dtypes(q, kv, w, bt, seq, bs, int(seq.max()))
    ref = oracle.paged_mqa_logits(q, kv, w, bt, seq, bs, int(seq.max()))
    np.testing.assert_array_equal(np.isnan(got["value"]), np.isnan(ref))
    np.testing.assert_array_equal(got["value"][~np.isnan(ref)], ref[~np.isnan(ref)])
    tau = oracle.row_tolerance(q, kv, w, bt, seq, bs)
    ends = oracle.row_ends(seq, q.shape[1])
    for r, e in enumerate(ends):
        assert np.all(got["tol"][r, :e] == tau[r])
    assert not got["may_inf"].any()


def test_f16_accumulator_rounds_each_dot():
    # head 0: 256*8 + 1*1 = 2049, not a float16 number (12 significant bits)
    args = _one_key([_vec((0, 256), (1, 1)), _vec(), _vec(), _vec()], _vec((0, 8), (1, 1)), [1, 0, 0, 0], 1.0)
    assert _run(args)["value"][0, 0] == 2049
    assert _run(args, acc_dtype=F16)["value"][0, 0] == 2048
    assert _run(args, epi_dtype=F16)["value"][0, 0] == 2048
    assert _run(args, epi_dtype=F16, acc_dtype=F16)["value"][0, 0] == 2048
    # a float16 output rounds the float32 result: 2048 is within its tolerance
    r = _run(args, output_dtype=F16)
    assert r["value"][0, 0] == 2049 and abs(2048 - 2049) <= r["tol"][0, 0]


def test_f16_epilogue_rounds_the_weights_and_the_scale():
    args = _one_key([_vec((0, 1)), _vec(), _vec(), _vec()], _vec((0, 1)), [0.1, 0, 0, 0], 1.0)
    assert _run(args, epi_dtype=F16)["value"][0, 0] == 0.0999755859375
    assert _run(args)["value"][0, 0] == float(np.float32(0.1))
    args = _one_key([_vec((0, 1)), _vec(), _vec(), _vec()], _vec((0, 1)), [1, 0, 0, 0], 0.1)
    assert _run(args, epi_dtype=F16)["value"][0, 0] == 0.0999755859375


def test_unrounded_weights_fail_the_pin():
    """A copy of the float16 epilogue that forgets to round the weights misses
    the hand-computed value above."""
    w = np.float32(0.1)
    mutant = 1.0 * (float(w) * max(1.0, 0.0))  # s' * w * relu(S'), w unrounded
    assert mutant != 0.0999755859375


def test_overflow_to_infinity():
    # S = 256*8 = 2048 (a float16 number), s = 64: the result 2^17 is past 65504
    args = _one_key([_vec((0, 256)), _vec(), _vec(), _vec()], _vec((0, 8)), [1, 0, 0, 0], 64.0)
    r = _run(args, epi_dtype=F16)
    assert r["value"][0, 0] == 2.0 ** 17 and r["must_inf"][0, 0]
    r = _run(args, output_dtype=F16)
    assert r["must_inf"][0, 0]
    r = _run(args, acc_dtype=F16)
    assert r["value"][0, 0] == 2.0 ** 17 and not r["may_inf"][0, 0]
    # a dot product past the float16 range becomes infinite with a float16 accumulator
    args = _one_key([_vec((0, 256)), _vec(), _vec(), _vec()], _vec((0, 256)), [1, 0, 0, 0], 1.0)
    r = _run(args, acc_dtype=F16)
    assert r["value"][0, 0] == np.inf and r["may_inf"][0, 0]


def _simulate_f16(q, kv, w, bt, seq, bs, rng):
    """The float16 epilogue in numpy float16 arithmetic (each product and sum
    rounded), heads summed in a random order, then the scale multiply."""
    B, nn, Hh, Dd = q.shape
    out = {}
    ends = oracle.row_ends(seq, nn)
    for b in range(B):
        L = int(seq[b])
        if L == 0:
            continue
        k, s = oracle.gather_request(kv, bt[b], L, bs, Dd)
        qb = oracle.decode_e4m3(q[b])
        for t in range(nn):
            r = b * nn + t
            w16 = w[r].astype(np.float16)
            for p in range(int(ends[r])):
                dots = qb[t] @ k[p]
                c = np.maximum(dots.astype(np.float16), np.float16(0))
                terms = [np.float16(w16[h] * c[h]) for h in range(Hh)]
                acc = np.float16(0)
                for h in rng.permutation(Hh):
                    acc = np.float16(acc + terms[h])
                out[(r, p)] = float(np.float16(acc * np.float16(s[p])))
    return out


@pytest.mark.parametrize("seed", [0, 1])
def test_f16_summation_orders_stay_within_tol(seed):
    q, kv, w, bt, seq, bs = _tiny(seed, H=64, D=8, seq=(6, 9))
    q = _e4m3(oracle.decode_e4m3(q) * 4)  # larger dots, so float16 rounding shows
    rng = np.random.default_rng(seed)
    ref = mqa_logits_dtypes(q, kv, w, bt, seq, bs, int(seq.max()), epi_dtype=F16)
    worst = 0.0
    for _ in range(3):
        sim = _simulate_f16(q, kv, w, bt, seq, bs, rng)
        for (r, p), v in sim.items():
            err = abs(v - ref["value"][r, p])
            assert err <= ref["tol"][r, p], (r, p, v, ref["value"][r, p], ref["tol"][r, p])
            worst = max(worst, err)
    assert worst > 0  # the simulation does round


def test_bad_dtype_rejected():
    q, kv, w, bt, seq, bs = _tiny(0)
    with pytest.raises(ValueError):
        mqa_logits_dtypes(q, kv, w, bt, seq, bs, 9, output_dtype="bf16")
