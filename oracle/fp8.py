"""OCP 8-bit floating point E4M3FN decoder — oracle side, test infrastructure.

Follows the OCP 8-bit floating point specification for E4M3 (the "e4m3"
storage format the Triton-TLE HPC-Ops page names for FP8 prefill, §2):
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
holds subnormals m * 2^-9; the single pattern S.1111.111 is NaN; there are
no infinities, so the largest finite magnitude is 1.75 * 2^8 = 448.

Pinned by tests/test_oracle_fp8.py: anchor codes from the definition, sign
symmetry, and equality with torch.float8_e4m3fn -> float32 on all 256 codes.
"""
import numpy as np

EXP_BIAS = 7
MAX_FINITE = 448.0


def _decode_code(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** (1 - EXP_BIAS - 3)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - EXP_BIAS)


DECODE_TABLE = np.array([_decode_code(c) for c in range(256)], dtype=np.float64)


def decode(codes) -> np.ndarray:
    """uint8 E4M3FN codes (any shape) -> float64 values."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3FN codes must be uint8")
    return DECODE_TABLE[codes]
