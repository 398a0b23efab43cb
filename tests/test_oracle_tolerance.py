"""Pins of the oracle's per-row logits tolerance (CPU only).

The bound on a GPU logit's error is 1e-4 * sum_h |w_h| * max_h |q_h . k| per
row; the per-token scale multiplies every term of a score, so it enters the
scale (this reading of the tolerance includes s_p).  Each case below
is computed by hand from that rule on inputs where the dots are closed forms
(all-ones or constant e4m3 vectors), and each is chosen so that one plausible
mistake in the formula gives another value:

  * dropping s_p                      (the all-ones case with s = 1.5)
  * the max over invisible positions  (a huge scale just past a row's end)
  * max_h |w_h| instead of sum_h |w_h| (weights of unequal magnitude)
  * a wrong relative factor            (any case)
  * no |.| on the dots, or the max of s and of the dots taken apart
                                       (a negative head dot; scale and dot
                                        maxima at different positions)

The mutants at the end plant each mistake in a copy of the formula and check
that the pins reject it.
"""
import numpy as np
import pytest
import torch

import oracle

H, D = 64, 128
ONE, HALF_NEG, TWO, EIGHTH, NEG_ONE = 0x38, 0xB0, 0x40, 0x20, 0xB8  # e4m3 codes: 1, -0.5, 2, 0.125, -1


def _kv(values_u8, scales, bs):
    """Blocks of bs tokens from per-token value codes [n, D] and scales [n]."""
    n = values_u8.shape[0]
    nb = -(-n // bs)
    vals = np.zeros((nb * bs, D), np.uint8)
    vals[:n] = values_u8
    sc = np.ones(nb * bs, np.float32)
    sc[:n] = scales
    v = torch.from_numpy(vals.reshape(nb, -1))
    s = torch.from_numpy(sc.reshape(nb, bs)).contiguous().view(torch.uint8)
    return torch.cat([v, s], 1).numpy()


def _tau(q, kv, w, seq, bs, rel=1e-4):
    B = q.shape[0]
    width = max(1, max(-(-int(L) // bs) for L in seq))
    bt = np.arange(B * width, dtype=np.int32).reshape(B, width) % kv.shape[0]
    return oracle.row_tolerance(q, kv, w, bt, np.array(seq, np.int32), bs, rel=rel)


def case_all_ones():
    """One key, q = k = all ones: every head dot is 128, so tau = 1e-4 * sum|w| * s * 128."""
    q = np.full((1, 1, H, D), ONE, np.uint8)
    kv = _kv(np.full((1, D), ONE, np.uint8), np.array([1.5], np.float32), bs=4)
    w = np.where(np.arange(H) % 2 == 0, 0.5, -0.25).astype(np.float32).reshape(1, H)
    # sum |w| = 32 * 0.5 + 32 * 0.25 = 24
    return (q, kv, w, [1], 4), np.array([1e-4 * 24 * 1.5 * 128])


def case_visibility():
    """next_n = 2, three keys: row 0 sees keys 0-1, row 1 sees 0-2; key 2 has a
    huge scale that only row 1 may count."""
    q = np.full((1, 2, H, D), ONE, np.uint8)
    kv = _kv(np.full((3, D), ONE, np.uint8), np.array([1.0, 2.0, 1000.0], np.float32), bs=4)
    w = np.full((2, H), 1.0 / 64, np.float32)  # sum |w| = 1 (exact in binary)
    return (q, kv, w, [3], 4), np.array([1e-4 * 2.0 * 128, 1e-4 * 1000.0 * 128])


def case_abs_and_joint_max():
    """Head 0 of q is all -1, heads 1-63 all 0.125.  Key 0 = all 1 with s = 4:
    dots -128 and 16, so s * max_h |dot| = 512.  Key 1 = all 2 with s = 1: dots
    -256 and 32, so 256.  tau = 1e-4 * 64 * max(512, 256) with unit weights."""
    q = np.full((1, 1, H, D), EIGHTH, np.uint8)
    q[0, 0, 0, :] = NEG_ONE
    vals = np.stack([np.full(D, ONE, np.uint8), np.full(D, TWO, np.uint8)])
    kv = _kv(vals, np.array([4.0, 1.0], np.float32), bs=4)
    w = np.ones((1, H), np.float32)
    return (q, kv, w, [2], 4), np.array([1e-4 * 64 * 512])


def case_empty_rows():
    """A request with no keys and one shorter than next_n: their rows get 0."""
    q = np.full((2, 2, H, D), ONE, np.uint8)
    kv = _kv(np.full((1, D), ONE, np.uint8), np.array([3.0], np.float32), bs=4)
    w = np.full((4, H), 0.5, np.float32)
    # request 0: L = 0 (no rows); request 1: L = 1, row t=0 sees nothing, t=1 sees key 0
    return (q, kv, w, [0, 1], 4), np.array([0.0, 0.0, 0.0, 1e-4 * 32 * 3.0 * 128])


CASES = [case_all_ones, case_visibility, case_abs_and_joint_max, case_empty_rows]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.__name__)
def test_row_tolerance_hand_computed(case):
    args, want = case()
    got = _tau(*args)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)


def test_row_tolerance_rel_is_linear():
    args, want = case_all_ones()
    np.testing.assert_allclose(_tau(*args, rel=3e-4), 3 * want, rtol=1e-12)


# ---------------------------------------------------------------- mutants

def _mutant_tau(q, kv, w, seq, bs, mistake):
    """The tolerance with one planted mistake (same gather and dots as the oracle)."""
    B, nn = q.shape[:2]
    ends = oracle.row_ends(np.array(seq), nn)
    width = max(1, max(-(-int(L) // bs) for L in seq))
    bt = np.arange(B * width, dtype=np.int32).reshape(B, width) % kv.shape[0]
    tau = np.zeros(B * nn)
    for b in range(B):
        L = int(seq[b])
        if L == 0:
            continue
        k, s = oracle.gather_request(kv, bt[b], L, bs, D)
        qd = oracle.decode_e4m3(q[b]).astype(np.float64)
        for t in range(nn):
            r = b * nn + t
            e = int(ends[r])
            if e == 0:
                continue
            dots = qd[t] @ k.T                       # [H, L]
            hm = np.abs(dots).max(axis=0)
            wsum = np.abs(w[r].astype(np.float64)).sum()
            if mistake == "drop_scale":
                m = hm[:e].max()
            elif mistake == "invisible":
                m = (s[:L] * hm[:L]).max()
            elif mistake == "max_w":
                m = (s[:e] * hm[:e]).max()
                wsum = np.abs(w[r].astype(np.float64)).max()
            elif mistake == "no_abs":
                m = (s[:e] * dots[:, :e].max(axis=0)).max()
            elif mistake == "separate_max":
                m = s[:e].max() * hm[:e].max()
            else:
                m = (s[:e] * hm[:e]).max()
            rel = 1e-3 if mistake == "rel" else 1e-4
            tau[r] = rel * wsum * m
    return tau


MISTAKES = ["drop_scale", "invisible", "max_w", "rel", "no_abs", "separate_max"]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_each_mistake_fails_some_pin(mistake):
    caught = []
    for case in CASES:
        args, want = case()
        got = _mutant_tau(*args, mistake)
        caught.append(not np.allclose(got, want, rtol=1e-12, atol=0))
    assert any(caught), f"no pin rejects the mistake {mistake!r}"


def test_mutant_harness_without_mistake_passes_pins():
    for case in CASES:
        args, want = case()
        np.testing.assert_allclose(_mutant_tau(*args, None), want, rtol=1e-12, atol=0)
