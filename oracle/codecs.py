"""Number formats of the fused tail, written from their definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): slow, plain, float64/float32
numpy code; nothing on the product path may import it.

Formats:
  * fp16 (IEEE binary16) and bf16 (the top half of binary32): the activation
    types of the fused case, one type per call (TensorRT-LLM issue #17900,
    Proposal).
  * E4M3FN, the OCP 8-bit float with 4 exponent bits (bias 7) and 3 mantissa
    bits, no infinities, S.1111.111 = NaN, max finite 448. Used for the
    per-tensor FP8 output and for the NVFP4 block scales (the pages say "FP8"
    and "NVFP4"; the E4M3 flavour is the plainest reading for both).
  * E2M1, the 4-bit float of NVFP4: values {0, 0.5, 1, 1.5, 2, 3, 4, 6} with a
    sign bit in bit 3.

Rounding everywhere is round-to-nearest, ties to the even code, with
saturation to the largest finite value (E4M3 +-448, E2M1 +-6). The sign of an
encoded value is the sign bit of the float32 input, so -0.0 encodes to the
negative-zero code.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# fp16 / bf16 <-> float32
# ----------------------------------------------------------------------------


def t_decode(b: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of fp16/bf16 -> float32 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    if dtype == "f16":
        return b.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def t_encode(f: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> fp16/bf16 bit patterns, round to nearest even (RNE_T).

    fp16 uses numpy's binary32->binary16 conversion (IEEE RNE). bf16 keeps the
    top 16 bits of binary32 after adding half an ulp of the kept part, plus one
    more when the kept part is odd: that is round half to even on bit 16.
    Inputs are finite (non-finite activations are outside the op's contract).
    """
    f = np.asarray(f, dtype=np.float32)
    if dtype == "f16":
        with np.errstate(over="ignore"):
            return f.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = f.view(np.uint32).astype(np.uint64)
        u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
        return (u >> np.uint64(16)).astype(np.uint16)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# E4M3FN
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(code) -> np.ndarray:
    """E4M3FN code -> float32.  E >= 1: (-1)^S 2^(E-7) (1 + M/8);
    E = 0: (-1)^S 2^-6 (M/8); S.1111.111 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag).astype(np.float32)


# the 127 non-negative finite E4M3 values, codes 0x00..0x7E, strictly increasing
_E4M3_POS = e4m3_decode(np.arange(0, 0x7F)).astype(np.float64)


def _nearest_code(a: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to a >= 0; ties go to the even index.
    table is increasing and starts at 0; a above the last value gives the
    last index (saturation). All comparisons are exact in float64."""
    top = len(table) - 1
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, top)
    lo = np.clip(hi - 1, 0, top)
    d_lo = a - table[lo]
    d_hi = table[hi] - a
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = d_lo == d_hi
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    return np.where(a >= table[top], top, pick)


def e4m3_encode(v) -> np.ndarray:
    """float32 -> E4M3FN code: nearest, ties to even, saturate to +-448, keep
    subnormals (smallest 2^-9), sign bit copied from the input."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    mag = _nearest_code(a, _E4M3_POS).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, mag | np.uint8(0x80), mag).astype(np.uint8)


# ----------------------------------------------------------------------------
# E2M1
# ----------------------------------------------------------------------------

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def e2m1_decode(code) -> np.ndarray:
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where((c & 8) != 0, -mag, mag).astype(np.float32)


def e2m1_encode(v) -> np.ndarray:
    """float32 -> 4-bit E2M1 code (0..15): nearest of the eight magnitudes,
    ties to the even code, saturate to 6, sign bit (bit 3) copied from input."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    mag = _nearest_code(a, E2M1_VALUES).astype(np.uint8)
    return np.where(np.signbit(v), mag | np.uint8(8), mag).astype(np.uint8)
