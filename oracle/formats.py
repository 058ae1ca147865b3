"""Number formats of block-scaled FP4, written from their definitions.

Scalar forms work on exact rationals (``fractions.Fraction``) and are the
definitions; vectorised numpy forms work on fp64 arrays and are exact under the
argument given in each docstring (pinned against the scalar forms in tests).

E2M1   [V41-NVFP4 s2]: 1 sign, 2 exponent, 1 mantissa bit; the non-negative
       magnitudes are exactly {0, 0.5, 1, 1.5, 2, 3, 4, 6} (the page's table);
       [FP4-101 s1] gives the same 1/2/1 bit split.  Code = sign*8 + index of the
       magnitude in that table.  Rounding to E2M1 = nearest table magnitude,
       ties to the even index, anything >= 6 saturates to 6 (E2M1 has no inf or
       NaN); the sign bit is the input's sign bit (so -0.0 and small negatives
       give code 0x8).
UE8M0  [V41-NVFP4 s3, V4-ARCH s6.3]: the MXFP4 block scale is a power of two
       stored as an unsigned 8-bit exponent: byte b means 2**(b-127); 255 is NaN
       and never produced.
E4M3   [V4-QAT s2.1: E4M3 max is 448]: OCP FP8 E4M3FN, bias 7, normals
       (1+m/8)*2**(e-7) for e in 1..15 except (e=15,m=7) which is NaN,
       subnormals (m/8)*2**-6.  Rounding = nearest, ties to even mantissa,
       saturating at 448.
fp32 / bf16: IEEE binary32 and its 8-significant-bit truncation format, round
       to nearest even.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------- E2M1
# The page's lookup table of non-negative E2M1 magnitudes [V41-NVFP4 s2].
E2M1_MAG = (Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2),
            Fraction(2), Fraction(3), Fraction(4), Fraction(6))
E2M1_MAG_F64 = np.array([float(v) for v in E2M1_MAG], dtype=np.float64)


def e2m1_value(code: int) -> Fraction:
    """Exact value of a 4-bit E2M1 code (bit 3 = sign, bits 2:0 = index)."""
    mag = E2M1_MAG[code & 7]
    return -mag if code & 8 else mag


def e2m1_value_from_fields(code: int) -> Fraction:
    """Same value read through the bit fields (exponent bits 2:1, mantissa bit 0):
    exponent 0 is subnormal m*0.5, otherwise (1 + m/2) * 2**(e-1)."""
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return -mag if code & 8 else mag


def e2m1_encode(negative: bool, magnitude: Fraction) -> int:
    """Round an exact non-negative magnitude to E2M1 (nearest table entry,
    ties to the even index; the largest entry 6 absorbs everything above it)
    and attach the sign bit."""
    assert magnitude >= 0
    best = None
    for i, m in enumerate(E2M1_MAG):
        d = abs(magnitude - m)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return (8 if negative else 0) | best[1]


E2M1_MIDPOINTS_F64 = (E2M1_MAG_F64[1:] + E2M1_MAG_F64[:-1]) / 2     # 0.25, 0.75, ..., 5 (exact)


def e2m1_index_f64(a: np.ndarray) -> np.ndarray:
    """Vectorised E2M1 index of non-negative fp64 magnitudes ``a``.

    Nearest table magnitude with ties to the even index, written as: the index
    is the number of midpoints m_j (between entries j and j+1) that a lies above,
    where a value exactly on m_j counts as above only when j + 1 is even.
    Everything above the last midpoint (5) is index 7, so a >= 6 saturates.
    The midpoints are exact in fp64, so the comparisons are exact for the fp64
    value given; callers pass either the exact quotient or an fp64 value whose
    rounding cannot cross a midpoint (their docstrings give the argument).
    """
    a = np.asarray(a, dtype=np.float64)
    idx = np.zeros(a.shape, dtype=np.uint8)
    for j, m in enumerate(E2M1_MIDPOINTS_F64):
        up = (a > m) | ((a == m) & ((j + 1) % 2 == 0))
        idx += up.astype(np.uint8)
    return idx


# ---------------------------------------------------------------- generic binary float rounding
def floor_log2(q: Fraction) -> int:
    """floor(log2 q) of a positive rational, exactly (no floating point)."""
    assert q > 0
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # now 2**(e-1) < n/d < 2**(e+1); fix up to the exact floor
    if Fraction(n, d) < Fraction(2) ** e:
        e -= 1
    return e


def round_binary(q: Fraction, p: int, emin: int, maxval: Fraction | None,
                 saturate: bool) -> Fraction:
    """Round a non-negative rational to the nearest value of a binary float
    format with p significant bits (implicit bit included) and minimum normal
    exponent emin; ties go to the even significand.  Above ``maxval`` the
    result saturates to ``maxval`` (saturate=True) or is +inf (returned as None).
    """
    assert q >= 0
    if q == 0:
        return Fraction(0)
    e = max(floor_log2(q), emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = q / ulp
    k = n.numerator // n.denominator
    frac = n - k
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and k % 2 == 1):
        k += 1
    r = k * ulp
    if maxval is not None and r > maxval:
        return maxval if saturate else None
    return r


FP32_MAX = (2 - Fraction(2) ** -23) * Fraction(2) ** 127
BF16_MAX = (2 - Fraction(2) ** -7) * Fraction(2) ** 127
E4M3_MAX = Fraction(448)


def round_fp32(q: Fraction) -> Fraction:
    """IEEE binary32 round-to-nearest-even of an exact rational (sign kept)."""
    r = round_binary(abs(q), 24, -126, FP32_MAX, saturate=False)
    assert r is not None, "fp32 overflow"
    return -r if q < 0 else r


def round_bf16(q: Fraction) -> Fraction:
    """bf16 (8 significant bits, fp32 exponent range) round-to-nearest-even."""
    r = round_binary(abs(q), 8, -126, BF16_MAX, saturate=False)
    assert r is not None, "bf16 overflow"
    return -r if q < 0 else r


def round_e4m3_sat(q: Fraction) -> Fraction:
    """Non-negative rational to E4M3FN: nearest, ties to even, saturating at 448."""
    return round_binary(q, 4, -6, E4M3_MAX, saturate=True)


# ---------------------------------------------------------------- E4M3 bytes
def e4m3_decode(byte: int) -> Fraction | None:
    """Exact value of an E4M3FN byte; None for the NaN encodings 0x7F / 0xFF."""
    s, e, m = byte >> 7, (byte >> 3) & 15, byte & 7
    if e == 15 and m == 7:
        return None
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def e4m3_encode(v: Fraction) -> int:
    """Byte of a non-negative value that is exactly representable in E4M3."""
    for b in range(0x7F):
        if e4m3_decode(b) == v:
            return b
    raise ValueError(f"{v} is not an E4M3 value")


# sorted table of the 127 non-negative finite E4M3 values (bytes 0x00..0x7E)
E4M3_POS_F64 = np.array([float(e4m3_decode(b)) for b in range(0x7F)], dtype=np.float64)


def e4m3_rne_sat_f64(q: np.ndarray) -> np.ndarray:
    """Vectorised E4M3 byte of non-negative fp64 values: nearest table value,
    ties to the even byte (= even mantissa), saturating at 448 (byte 0x7E).

    The midpoint of two neighbours has <= 5 significant bits and is exact in
    fp64, so comparing q against it decides exactly for the fp64 q given.
    """
    q = np.asarray(q, dtype=np.float64)
    hi = np.searchsorted(E4M3_POS_F64, q, side="left")      # first value >= q
    hi = np.clip(hi, 1, 0x7E)
    lo = hi - 1
    vlo, vhi = E4M3_POS_F64[lo], E4M3_POS_F64[hi]
    mid = (vlo + vhi) / 2
    pick_hi = (q > mid) | ((q == mid) & (hi % 2 == 0))
    out = np.where(pick_hi, hi, lo)
    out = np.where(q >= 448.0, 0x7E, out)
    out = np.where(q <= 0.0, 0, out)
    return out.astype(np.uint8)


def e4m3_value_f64(b: np.ndarray) -> np.ndarray:
    """fp64 value of non-negative E4M3 bytes (0x00..0x7E)."""
    return E4M3_POS_F64[np.asarray(b, dtype=np.int64)]


# ---------------------------------------------------------------- UE8M0
def ue8m0_value(byte: int) -> Fraction:
    """2**(byte-127); byte 255 (NaN) is rejected."""
    assert 0 <= byte <= 254
    return Fraction(2) ** (byte - 127)


# ---------------------------------------------------------------- bf16 / fp32 bit views
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 bit patterns (uint16): a bf16 is the top half
    of an fp32, so widening through fp32 is exact (subnormals included)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_fraction(bits: int) -> Fraction:
    """Exact rational of one bf16 pattern from its fields."""
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    assert e != 0xFF, "inf/nan not supported"
    v = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
    return -v if s else v


def f64_to_fp32_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 with numpy's IEEE round-to-nearest-even cast (single rounding
    of the fp64 value)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def fp32_to_bf16_bits_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even on the 16 discarded bits.
    (Inputs are finite; the carry out of the mantissa bumps the exponent,
    which is the correct result for both normals and subnormals.)"""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_rne_of_f64(x: np.ndarray) -> np.ndarray:
    """Single correct rounding of fp64 values to bf16 bits.

    fp64 -> fp32 -> bf16 would round twice; instead round the fp64 value to 8
    significant bits directly (exponent range of fp32, subnormals at 2**-133)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.zeros(x.shape, dtype=np.float64)
    nz = a > 0
    _, p = np.frexp(a[nz])                      # a = f * 2**p, f in [0.5, 1)
    e = np.maximum(p - 1, -126)                 # floor(log2 a), clamped to emin
    ulp = np.ldexp(1.0, e - 7)
    n = a[nz] / ulp                              # exact: power-of-two scaling
    k = np.floor(n)
    fr = n - k                                   # exact: n has <= 53 bits
    up = (fr > 0.5) | ((fr == 0.5) & (np.fmod(k, 2) == 1))
    out[nz] = (k + up) * ulp
    out = np.copysign(out, x)
    return fp32_to_bf16_bits_rne(out.astype(np.float32))   # value already on the bf16 grid


def frexp_floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive fp64 a, from the binary exponent (never a
    floating-point log2): a = f * 2**p with f in [0.5, 1) gives p - 1."""
    _, p = np.frexp(np.asarray(a, dtype=np.float64))
    return p.astype(np.int64) - 1


def sign_bit_f64(x: np.ndarray) -> np.ndarray:
    """1 where the sign bit is set (negative values and -0.0)."""
    return np.signbit(np.asarray(x, dtype=np.float64)).astype(np.uint8)


