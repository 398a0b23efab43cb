"""Paged MQA logits with the float16 options, in float64.

Page "flashinfer.attn_scores", fp8_paged_mqa_logits: the formula block with its
three precisions (accumulator, epilogue, stored output) and the parameters
output_dtype, epi_dtype, acc_dtype and weights.  Each head's dot product is
accumulated in acc_dtype; ReLU, the weight multiply, the head sum and the scale
multiply run in epi_dtype; the result is converted to output_dtype on store;
the weights are cast to float16 when the epilogue runs in float16, and float16
arithmetic overflows to infinity past 65504.

Readings (the pages name the precisions, not where each rounding happens):

* A float16 accumulator rounds each head's dot product once to float16
  (round to nearest even).  The FP8 matrix instruction of the hardware here
  accumulates in float32 only; one rounding at the end is at least as accurate
  as accumulating in float16.
* A float16 epilogue starts from the dot product rounded to float16 (the same
  rounding as a float16 accumulator, so acc_dtype makes no difference then),
  rounds the weights and the token scale to float16, and rounds every product
  and sum to float16 in an order the pages do not fix.
* A float16 output rounds the epilogue's result to float16.

So the oracle gives the exact value of the formula on the rounded operands,

    value = s' * sum_h w'_h * relu(S'_h)

(S'_h the dot product, rounded to float16 when either acc or epi is float16;
w', s' rounded to float16 when epi is), and a per-element bound `tol` on what
the unfixed order and the kernel's own float32 steps may add:

* float16 epilogue: gamma(H + 2) * s' * sum_h |w'_h| relu(S'_h), with
  gamma(n) = n u / (1 - n u), u = 2^-11: a term of the head sum goes through at
  most H - 1 additions, one fused product and the scale multiply, each a
  float16 rounding (the textbook bound for summation in any order), plus
  (H + 2) * 2^-25 * s' for the subnormal range;
* float32 epilogue: the row's float32 tolerance tau_r (row_tolerance);
* a float16 rounding of S_h: 2^-10 * s' * sum_h |w'_h| |S_h| more, because the
  kernel rounds its float32 dot product, which may fall on the other side of a
  float16 rounding boundary than the exact one (one unit in the last place of
  one head at most);
* float16 output: half a unit in the last place of the result, 2^-11 * (|value|
  + tol) + 2^-25.

Elements whose result may overflow float16 are flagged: `may_inf` where the sum
of the terms' magnitudes (or the value plus tol, for the output rounding)
reaches 65504, so an intermediate or final float16 value can round to
infinity; `must_inf` where |value| - tol already reaches 65520 (everything at
or above 65520 rounds to infinity), with the sign of the value.

Pinned by: the float32 options reducing to paged_mqa_logits; hand-computed
float16 roundings of a dot product (2049 -> 2048), of a weight (0.1 ->
0.0999755859375) and of the output; overflow to infinity of a 70000 result;
float16 simulations of the head sum in random orders all within tol; a copy
that forgets to round the weights failing a pin (tests/test_oracle_dtypes.py).
"""
import numpy as np

from .e4m3 import decode_e4m3
from .layout import gather_request
from .logits import CHUNK, row_ends, row_tolerance

F32, F16 = "f32", "f16"
U16 = 2.0 ** -11
F16_MAX = 65504.0
F16_OVERFLOW = 65520.0  # the smallest magnitude that rounds to infinity


def round_f16(x):
    """Round to float16 (nearest, ties to even; infinity past the range), back
    in float64."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def gamma(n: int, u: float = U16) -> float:
    return n * u / (1.0 - n * u)


def _check_dtype(name, value, allowed):
    if value not in allowed:
        raise ValueError(f"{name} must be one of {allowed}, got {value!r}")


def mqa_logits_dtypes(q: np.ndarray, kv_fused: np.ndarray, weights: np.ndarray, block_tables: np.ndarray,
                      seq_lens: np.ndarray, block_size: int, max_seq_len: int, *, output_dtype: str = F32,
                      epi_dtype: str = F32, acc_dtype: str = F32, rows=None):
    """Returns dict(value, tol, may_inf, must_inf), each [B*next_n, max_seq_len]:
    value float64 (NaN where a row sees nothing), tol float64, the two masks bool.

    rows: optional iterable of row indices to compute (others stay NaN / 0)."""
    for name, v in (("output_dtype", output_dtype), ("epi_dtype", epi_dtype), ("acc_dtype", acc_dtype)):
        _check_dtype(name, v, (F32, F16))
    B, nn, H, D = q.shape
    R = B * nn
    value = np.full((R, max_seq_len), np.nan)
    tol = np.zeros((R, max_seq_len))
    may_inf = np.zeros((R, max_seq_len), dtype=bool)
    must_inf = np.zeros((R, max_seq_len), dtype=bool)
    ends = row_ends(seq_lens, nn)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    epi16 = epi_dtype == F16
    round_dot = epi16 or acc_dtype == F16
    tau32 = None if epi16 else row_tolerance(q, kv_fused, weights, block_tables, seq_lens, block_size,
                                             rows=sorted(want))
    for b in range(B):
        L = int(seq_lens[b])
        rs = [b * nn + t for t in range(nn)]
        if L == 0 or not any(r in want for r in rs):
            continue
        k, s = gather_request(kv_fused, block_tables[b], L, block_size, D)
        qb = decode_e4m3(q[b])                                  # [nn, H, D]
        for t, r in enumerate(rs):
            e = int(ends[r])
            if r not in want or e == 0:
                continue
            w = weights[r].astype(np.float64)
            if epi16:
                w = round_f16(w)
            for c0 in range(0, e, CHUNK):
                c1 = min(e, c0 + CHUNK)
                dots = qb[t] @ k[c0:c1].T                       # [H, n], exact
                sc = s[c0:c1]
                if epi16:
                    sc = round_f16(sc)
                d = round_f16(dots) if round_dot else dots
                rel = np.maximum(d, 0.0)
                with np.errstate(invalid="ignore", over="ignore"):
                    v = sc * (w @ rel)
                    mag = sc * (np.abs(w) @ rel)
                t_ = np.zeros(c1 - c0)
                if epi16:
                    t_ += gamma(H + 2) * mag + (H + 2) * 2.0 ** -25 * sc
                else:
                    t_ += tau32[r]
                if round_dot:
                    with np.errstate(invalid="ignore", over="ignore"):
                        t_ += 2.0 ** -10 * sc * (np.abs(w) @ np.abs(dots))
                mi = (mag >= F16_MAX) if epi16 else np.zeros(c1 - c0, dtype=bool)
                if round_dot:
                    mi |= np.any(np.abs(dots) >= F16_MAX, axis=0)
                if output_dtype == F16:
                    with np.errstate(invalid="ignore", over="ignore"):
                        t_ += U16 * (np.abs(v) + t_) + 2.0 ** -25
                    mi |= np.abs(v) + t_ >= F16_MAX
                with np.errstate(invalid="ignore"):
                    mu = mi & (np.abs(v) - t_ >= F16_OVERFLOW)
                value[r, c0:c1] = v
                tol[r, c0:c1] = t_
                may_inf[r, c0:c1] = mi
                must_inf[r, c0:c1] = mu
    return {"value": value, "tol": tol, "may_inf": may_inf, "must_inf": must_inf}
