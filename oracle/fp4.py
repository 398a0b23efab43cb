"""MXFP4 paged MQA logits in float64.

Page "flashinfer.attn_scores", fp4_paged_mqa_logits: the formula block and the
paragraph after it, the parameters q, q_sf, kv_fused (with its byte-offset
figure and the nibble picture), weights, sf_vec_size, output_dtype, epi_dtype
and is_kv_sf_interleaved, and the Restrictions:

    logits[b*next_n + t, p] = sum_h w[b*next_n + t, h] * relu(q^[b,t,h,:] . k^[p,:])

q^ and k^ are the dequantised vectors: each of the 128 elements is an FP4
(E2M1) code times the UE8M0 scale of its group of 32 (sf_vec_size), the scale
2^(e - 127) of the raw exponent byte e (255 is NaN).  There is no per-token
scale.  ReLU is per head, before the weighted sum.  Row b*next_n + t sees
positions 0 .. seq_lens[b] - next_n + t, as in the FP8 variant.

Layout (the kv_fused figure): block j is bs*64 bytes of packed values,
token-major (token i's 64 bytes at i*64; byte m holds element 2m in its low
nibble and element 2m+1 in its high nibble), then bs*4 scale bytes.  Token
order by default: token i's four scales at bs*64 + 4i, byte k for elements
[32k, 32k + 32).  Interleaved (block_size 128 only): scale slot k holds token
(k % 4) * (bs // 4) + k // 4.  q packs each head's 128 elements the same way
(64 bytes); q_sf holds one int32 per (b, t, h) whose byte k is group k's scale.

E2M1 (OCP MX): sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0;
exponent 0 is subnormal (0 or 0.5); magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no
infinity or NaN.

Dot products: an E2M1 x E2M1 product is a multiple of 1/4 below 37 in
magnitude, so a group's 32-term sum is exact in float64, and so is its product
with the two scales (powers of two); the four groups' sum is exact unless the
groups' scale exponents differ by more than about 40.

Precisions (readings, as for the FP8 variant's options; oracle/dtypes.py): the
matrix instruction accumulates in float32 (the page fixes that); with a
float16 or bfloat16 epilogue each head's dot product is rounded to that type,
then the weights, and every product and sum is rounded; the output is rounded
once to output_dtype (bfloat16 by default).  The oracle returns the exact value
on the rounded operands and a per-element bound `tol`:

* float32 epilogue: gamma(D + H + 8, 2^-24) * sum_h |w_h| * sum_d |q^_hd k^_pd|
  (the matrix instruction's float32 accumulation of the 128 scaled products
  and the head sum, in any order);
* float16 / bfloat16 epilogue: gamma(H + 2, u) * sum_h |w'_h| relu(S'_h) with
  u = 2^-11 / 2^-8 (+ 2^-24 for bfloat16: the kernel rounds a float32 fused
  result to bfloat16, a second rounding), plus one unit of the dot product's
  rounding (2^-10 / 2^-7 of sum_h |w'_h| |S_h|), plus the float32 accumulation
  bound above with the rounded weights;
* float16 / bfloat16 output: half a unit of the result, u * (|value| + tol).

Flags may_inf / must_inf as in oracle/dtypes.py, for float16 (65504) only:
bfloat16 and float32 share float32's range, which the test inputs stay far
from.

Pinned by: the E2M1 table (hand values of the OCP definition, and the sum of
the eight positive codes), UE8M0 anchors, the figure's byte offsets (region 2
at 2048, end 2176, token i's scales at 2048 + 4i for block size 32), the nibble
rule on the figure's [e1|e0] picture, the per-token-row misreading failing, the
interleaved slot rule by brute force (and token order read as interleaved
failing), Fraction brute force, per-head ReLU, scale factoring (every group
scale of a key raised by one doubles its logits) and the hand-computed
roundings of oracle/dtypes.py (tests/test_oracle_fp4.py).
"""
import numpy as np

from .dtypes import F16, F32, F16_MAX, F16_OVERFLOW, gamma, round_f16
from .logits import row_ends

BF16 = "bf16"
SF_VEC = 32

def _decode_e2m1_code(code: int) -> float:
    """Value of a 4-bit E2M1 code from its bit fields."""
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * 0.5 * m                       # subnormal: m * 2^(1 - bias) * 2^-1
    return sign * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([_decode_e2m1_code(c) for c in range(16)], dtype=np.float64)


def decode_ue8m0(e):
    """2^(e - 127) of each raw exponent byte; 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, (e - 127).astype(np.int64))
    return np.where(e == 255, np.nan, v)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> float64 [..., 2n]: element 2m from byte m's low nibble,
    2m + 1 from its high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.float64)
    out[..., 0::2] = E2M1_TABLE[p & 0xF]
    out[..., 1::2] = E2M1_TABLE[p >> 4]
    return out


def fp4_region2_offset(block_size: int, head_dim: int = 128) -> int:
    return block_size * head_dim // 2


def fp4_block_bytes(block_size: int, head_dim: int = 128) -> int:
    return block_size * (head_dim // 2 + head_dim // SF_VEC)


def scale_slot(token: int, block_size: int, interleaved: bool) -> int:
    """Scale slot of in-block token `token`: the token itself in token order;
    interleaved, slot k holds token (k % 4) * (bs // 4) + k // 4, so token t
    sits at slot 4 * (t % (bs // 4)) + t // (bs // 4)."""
    if not interleaved:
        return token
    q = block_size // 4
    return 4 * (token % q) + token // q


def parse_fp4_block(block: np.ndarray, block_size: int, head_dim: int = 128, interleaved: bool = False):
    """One block's bytes -> (values float64 [bs, head_dim] dequantised, raw
    codes' values float64 [bs, head_dim], group scales float64 [bs, groups])."""
    b = np.asarray(block, dtype=np.uint8).reshape(-1)
    r2 = fp4_region2_offset(block_size, head_dim)
    groups = head_dim // SF_VEC
    vals = unpack_fp4(b[:r2].reshape(block_size, head_dim // 2))
    slots = np.array([scale_slot(i, block_size, interleaved) for i in range(block_size)])
    sf = b[r2:r2 + block_size * groups].reshape(block_size, groups)[slots]
    scales = decode_ue8m0(sf)
    deq = vals * np.repeat(scales, SF_VEC, axis=1)
    return deq, vals, scales


def gather_fp4_request(kv_fused, block_table_row, seq_len, block_size, head_dim=128, interleaved=False):
    """Dequantised keys float64 [seq_len, head_dim] of one request, with the raw
    element values [seq_len, head_dim] and group scales [seq_len, groups]."""
    nblk = -(-seq_len // block_size)
    deq, vals, sc = [], [], []
    for j in range(nblk):
        d, v, s = parse_fp4_block(kv_fused[int(block_table_row[j])], block_size, head_dim, interleaved)
        deq.append(d)
        vals.append(v)
        sc.append(s)
    if not deq:
        z = np.zeros((0, head_dim))
        return z, z, np.zeros((0, head_dim // SF_VEC))
    return (np.concatenate(deq)[:seq_len], np.concatenate(vals)[:seq_len], np.concatenate(sc)[:seq_len])


def dequant_q(q: np.ndarray, q_sf: np.ndarray) -> np.ndarray:
    """q uint8 [B, nn, H, 64], q_sf int32 [B, nn, H] -> float64 [B, nn, H, 128]."""
    vals = unpack_fp4(q)
    sfb = np.asarray(q_sf, dtype=np.int32).astype("<i4").view(np.uint8).reshape(q_sf.shape + (4,))
    return vals * np.repeat(decode_ue8m0(sfb), SF_VEC, axis=-1)


def round_bits(x, p: int, emin: int, emax: int):
    """Round to a binary format of p significand bits, minimum normal exponent
    emin and maximum exponent emax (nearest, ties to even; subnormals; infinity
    past the range), computed exactly in float64."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        _, e = np.frexp(x)                      # |x| = m * 2^e, 0.5 <= m < 1: leading bit 2^(e-1)
        lead = np.maximum(e - 1, emin)
        quantum = np.ldexp(1.0, lead - (p - 1))
        r = np.rint(x / quantum) * quantum
        top = np.ldexp(2.0 - 2.0 ** (1 - p), emax)
        r = np.where(np.abs(r) > top, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def round_bf16(x):
    return round_bits(x, 8, -126, 127)


_ROUND = {F16: round_f16, BF16: round_bf16}
_UNIT = {F16: 2.0 ** -11, BF16: 2.0 ** -8 + 2.0 ** -24}


def fp4_paged_mqa_logits(q: np.ndarray, q_sf: np.ndarray, kv_fused: np.ndarray, weights: np.ndarray,
                         block_tables: np.ndarray, seq_lens: np.ndarray, block_size: int, max_seq_len: int, *,
                         output_dtype: str = BF16, epi_dtype: str = F32, interleaved: bool = False, rows=None):
    """Returns dict(value, tol, may_inf, must_inf), each [B*next_n, max_seq_len]
    (value NaN where a row sees nothing)."""
    for name, v in (("output_dtype", output_dtype), ("epi_dtype", epi_dtype)):
        if v not in (F32, F16, BF16):
            raise ValueError(f"{name} must be f32, f16 or bf16, got {v!r}")
    B, nn, H, half = q.shape
    D = 2 * half
    R = B * nn
    value = np.full((R, max_seq_len), np.nan)
    tol = np.zeros((R, max_seq_len))
    may_inf = np.zeros((R, max_seq_len), dtype=bool)
    must_inf = np.zeros((R, max_seq_len), dtype=bool)
    ends = row_ends(seq_lens, nn)
    want = set(range(R)) if rows is None else set(int(r) for r in rows)
    qd = dequant_q(q, q_sf)                                   # [B, nn, H, D]
    for b in range(B):
        L = int(seq_lens[b])
        rs = [b * nn + t for t in range(nn)]
        if L == 0 or not any(r in want for r in rs):
            continue
        k, _, _ = gather_fp4_request(kv_fused, block_tables[b], L, block_size, D, interleaved)
        for t, r in enumerate(rs):
            e = int(ends[r])
            if r not in want or e == 0:
                continue
            w = weights[r].astype(np.float64)
            dots = qd[b, t] @ k[:e].T                          # [H, e]
            pabs = np.abs(qd[b, t]) @ np.abs(k[:e]).T          # [H, e]: sum_k |q^_hk k^_pk|
            acc_bound = gamma(D + H + 8, 2.0 ** -24) * (np.abs(w) @ pabs)
            if epi_dtype == F32:
                v = w @ np.maximum(dots, 0.0)
                t_ = acc_bound
                mi = np.zeros(e, dtype=bool)
            else:
                rnd, u = _ROUND[epi_dtype], _UNIT[epi_dtype]
                w2 = rnd(w)
                d2 = rnd(dots)
                rel = np.maximum(d2, 0.0)
                with np.errstate(invalid="ignore", over="ignore"):
                    v = w2 @ rel
                    mag = np.abs(w2) @ rel
                    t_ = (gamma(H + 2, u) * mag + 2 * u * (np.abs(w2) @ np.abs(dots))
                          + gamma(D + H + 8, 2.0 ** -24) * (np.abs(w2) @ pabs) + (H + 2) * 2.0 ** -149)
                if epi_dtype == F16:
                    t_ += (H + 2) * 2.0 ** -25
                    mi = (mag >= F16_MAX) | np.any(np.abs(dots) >= F16_MAX, axis=0)
                else:
                    mi = np.zeros(e, dtype=bool)
            if output_dtype != F32:
                u = _UNIT[output_dtype]
                with np.errstate(invalid="ignore", over="ignore"):
                    t_ = t_ + u * (np.abs(v) + t_) + (2.0 ** -25 if output_dtype == F16 else 2.0 ** -134)
                if output_dtype == F16:
                    mi = mi | (np.abs(v) + t_ >= F16_MAX)
            with np.errstate(invalid="ignore"):
                mu = mi & (np.abs(v) - t_ >= F16_OVERFLOW)
            value[r, :e] = v
            tol[r, :e] = t_
            may_inf[r, :e] = mi
            must_inf[r, :e] = mu
    return {"value": value, "tol": tol, "may_inf": may_inf, "must_inf": must_inf}
