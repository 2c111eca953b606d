"""Exact decoding of the cache's storage formats to float64.

Test infrastructure only (see the package docstring).

* bf16: the upper 16 bits of an IEEE binary32; widening is exact.
* OCP e4m3 ("FP8 E4M3" of the OCP 8-bit floating point specification, the
  "OCP" variant named beside FNUZ in the joint compressed/window attention
  PR of RL-Kernel, section "Reuse and arithmetic"): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
  m/8 * 2^-6; there are no infinities; S.1111.111 is NaN; the largest finite
  magnitude is 1.75 * 2^8 = 448.
* FNUZ e4m3 (the other variant that page names; the gfx942 format): the
  same fields with exponent bias 8, no infinities, no negative zero, and a
  single NaN at 1.0000.000 (0x80); 0x7F and 0xFF are finite (+-1.875 * 2^7
  = +-240); subnormals are m/8 * 2^-7.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def _e4m3_value(code: int) -> float:
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """The 256-entry OCP e4m3 decode table (float64; NaN at 0x7F and 0xFF)."""
    return _TABLE.copy()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP e4m3 codes (uint8) -> float64, exactly."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def _e4m3fnuz_value(code: int) -> float:
    if code == 0x80:
        return float("nan")
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp_field = (code >> 3) & 0xF
    mant = code & 0x7
    if exp_field == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 8)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 8)


_FNUZ_TABLE = np.array([_e4m3fnuz_value(c) for c in range(256)], dtype=np.float64)


def e4m3fnuz_table() -> np.ndarray:
    """The 256-entry FNUZ e4m3 decode table (float64; NaN only at 0x80)."""
    return _FNUZ_TABLE.copy()


def e4m3fnuz_to_f64(codes: np.ndarray) -> np.ndarray:
    """FNUZ e4m3 codes (uint8) -> float64, exactly."""
    return _FNUZ_TABLE[np.asarray(codes, dtype=np.uint8)]
