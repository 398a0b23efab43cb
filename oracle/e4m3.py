"""OCP FP8 E4M3 ("e4m3fn") decoding, from the bit-field definition.

The pages only name the dtype (page "flashinfer.attn_scores",
fp8_paged_mqa_logits, parameter q: float8_e4m3fn).  The format (OCP 8-bit
floating point specification, E4M3): sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN;
there is no infinity; the largest finite magnitude is 1.75 * 2^8 = 448.

Pinned by: exhaustive 256-code comparison with torch's own float8_e4m3fn cast,
and the anchors 0x38 = 1.0, 0x7E = 448, 0x01 = 2^-9.
"""
import numpy as np


def _decode_one(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values (exact)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]
