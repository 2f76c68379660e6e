"""Decoding of the cache's storage formats to float64 (exact).

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: the upper half of an IEEE binary32 word; widening to float64 is exact.
* FP8 E4M3: [d7kj] section 四 (KV Cache 量化) stores KV as FP8 E4M3 with three
  mantissa bits, and [k1-blog] section "KV Cache 量化" treats FP8 as half the
  bytes of FP16.  Scales of absmax/448 fix the variant with largest finite
  value 448: the OCP "E4M3FN" encoding -- sign bit, 4 exponent bits with bias
  7, 3 mantissa bits, subnormals when the exponent field is 0, no infinities,
  and NaN only for exponent and mantissa fields all ones.
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return w.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN codes (uint8) -> float64, exactly."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]
