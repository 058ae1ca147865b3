"""Block-scaled FP4 quantize, MX->NV remap and dequantize (CPU oracle).

Layout conventions (shared with the C ABI by definition, not by code):
  x        bf16 bit patterns, uint16 [R, K], K contiguous.
  codes    uint8 [R, K/2]; byte j holds element 2j in bits 3:0 and 2j+1 in
           bits 7:4 (the pages only say "two FP4 values per byte",
           [V41-NVFP4 s2]; low-nibble-first is this oracle's reading).
  MX       scales uint8 [R, K/32], UE8M0.
  NV       scales uint8 [R, K/16], E4M3FN; one fp32 tensor scale s_t.

Each function below has a scalar exact form (``*_exact``: Fraction arithmetic,
pure-Python loops, for small inputs) that is the definition, and a vectorised
fp64 form used at larger sizes; tests pin one against the other.

MX quantize [V41-NVFP4 s3: 32-element blocks with one UE8M0 scale;
V4-ARCH s6.3: 1x32 tiles along the reduction dimension]:
  amax = max |x| over the block; E = floor(log2 amax) - 2 (from the binary
  exponent), E = -127 when amax = 0, then clamped to [-127, 127]; scale byte is
  E + 127; each code = E2M1_RNE(x * 2**-E).  The "-2" puts amax/2**E in [4, 8),
  so the block maximum maps to the top two E2M1 magnitudes {4, 6} or saturates.

NV quantize [V41-NVFP4 s2: group size 16, per-group scale bringing the group
into [-6, 6], plus a tensor-level scale]:
  s_t = RNE_fp32(amax_t / (6 * 448)) unless supplied (activation scales are
  calibrated, [V41-NVFP4 s4]); per 16-group s_g = RNE_E4M3_sat(amax_g / (6 s_t));
  code = E2M1_RNE(x / (s_g s_t)); s_t = 0 or s_g = 0 gives signed-zero codes.
  Every step is one correct rounding of an exact real number.

MX->NV remap [V41-NVFP4 s1 and s6: NVFP4's finer 16-element groups re-express
MXFP4 weights block by block without loss]:
  codes unchanged; E_max = max block exponent; k = E_max - 8; s_t = 2**k;
  both 16-groups of MX block b get s_g = RNE_E4M3(2**(E_b - k)).  2**j is an
  E4M3 value for j in [-9, 8], so block b is exact iff E_b >= E_max - 17 or all
  of its codes are zero; other blocks are counted as inexact.

MXFP8 (the activations of the W4A8 GEMM) [V4-QAT s4.3: FP4 weights times
FP8 activations; FP4-101: weights in FP4, activations kept in FP8; V4-ARCH
s6.3 and V41-NVFP4 s3: 1x32 blocks with one UE8M0 scale].  The pages do not
spell out the FP8 block rule; the reading taken mirrors the MX rule with E4M3
elements: E = floor(log2 amax) - 8 (8 is E4M3's largest exponent, as 2 is
E2M1's), E = -127 when amax = 0, clamped to [-127, 127]; scale byte E + 127;
each code = E4M3_RNE(x * 2**-E) on the magnitude, saturating at 448 (bytes
0x7F/0xFF, the NaN encodings, never occur), sign copied from the input.

FP4 -> FP8 [V4-QAT s4.2, V4-ARCH s6.3: FP4 data dequantize to FP8 without
loss]: every E2M1 magnitude is an E4M3 value, so an MXFP4 block becomes an
MXFP8 block with the same scale byte and each code re-encoded exactly.

FP4 -> FP8 dequantization through E4M3 block scales [V4-QAT s4.2, its four
steps; V4-ARCH s6.3: lossless while the block scale ratio stays under a
threshold].  The pages re-encode the UE8M0 scale array in E4M3, widen every
E2M1 code to E4M3, and multiply scale by data in FP8.  They name no tensor
scale; E4M3 only spans 2**-9 .. 448, so the reading taken here puts one fp32
power of two s_t = 2**k per tensor in front, k = E_max - 6 (E_max the largest
block exponent), which maps the largest block's top code 6 to 6 * 2**6 = 384
and never saturates.  Per block b with j = E_b - k:
  s8_b = RNE_E4M3(2**j)             (step 2; exact iff j >= -9)
  v8   = RNE_E4M3(MAG * s8_b)       (steps 3-4; sign copied from the code)
The dequantized value is v8 * s_t.  A block is inexact when some element's
v8 * s_t differs from its MX value; every block is exact when its exponent
is at least E_max - 14, i.e. when the ratio of the largest to the smallest
block scale is at most 2**14 (the threshold, under this reading).

Dequantize [V41-NVFP4 s2: the accumulator multiplies scales back;
V4-QAT s4.2 FP4 dequant through the scale]:
  MX: (-1)^s MAG[i] 2**E, exact in fp32 and bf16.
  NV: fp32 = RNE_fp32(MAG[i] s_g s_t) (MAG s_g is exact; one rounding);
      bf16 = RNE_bf16 of that fp32 value.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import formats as F

MX_BLOCK = 32
NV_GROUP = 16
MX8_EMAX = 8                     # largest E4M3 exponent: 448 = 1.75 * 2**8
NV_TENSOR_DIV = 6 * 448          # amax_t / (6 * 448): E2M1 max times E4M3 max


# ====================================================================== packing
def pack_nibbles(codes4: np.ndarray) -> np.ndarray:
    """[R, K] 4-bit codes -> [R, K/2] bytes, even element in the low nibble."""
    c = np.asarray(codes4, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[R, K/2] bytes -> [R, K] 4-bit codes."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = c & 0xF
    out[..., 1::2] = c >> 4
    return out


def code_values_f64(codes4: np.ndarray) -> np.ndarray:
    """Signed E2M1 values of 4-bit codes as fp64 (exact)."""
    c = np.asarray(codes4, dtype=np.uint8)
    v = F.E2M1_MAG_F64[c & 7]
    return np.where(c & 8, -v, v)


# ====================================================================== MX: exact scalar form
def mx_block_exact(bits: list[int]) -> tuple[list[int], int]:
    """One 32-element MX block from bf16 bit patterns: (4-bit codes, scale byte)."""
    vals = [F.bf16_bits_to_fraction(b) for b in bits]
    amax = max(abs(v) for v in vals)
    E = -127 if amax == 0 else F.floor_log2(amax) - 2
    E = min(max(E, -127), 127)
    inv = Fraction(2) ** -E
    codes = [F.e2m1_encode(bool(b >> 15), abs(v) * inv) for b, v in zip(bits, vals)]
    return codes, E + 127


def mx_quantize_exact(xbits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Scalar-loop MX quantize of a small [R, K] bf16 array."""
    R, K = xbits.shape
    assert K % MX_BLOCK == 0
    codes4 = np.zeros((R, K), dtype=np.uint8)
    scales = np.zeros((R, K // MX_BLOCK), dtype=np.uint8)
    for r in range(R):
        for b in range(K // MX_BLOCK):
            c, s = mx_block_exact([int(v) for v in xbits[r, b * 32:(b + 1) * 32]])
            codes4[r, b * 32:(b + 1) * 32] = c
            scales[r, b] = s
    return pack_nibbles(codes4), scales


# ====================================================================== MX: vectorised fp64
def mx_quantize(xbits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MX quantize [R, K] bf16 bits -> (codes [R, K/2], UE8M0 scales [R, K/32]).

    fp64 is exact here: x is a bf16 value and x * 2**-E only shifts its exponent
    (2**-E <= 2**127, |x| >= 2**-133, far inside fp64's range), so the distances
    to the E2M1 table are computed on the exact scaled value.
    """
    xbits = np.asarray(xbits, dtype=np.uint16)
    R, K = xbits.shape
    assert K % MX_BLOCK == 0
    x = F.bf16_bits_to_f64(xbits).reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(x).max(axis=-1)
    E = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    E[nz] = F.frexp_floor_log2(amax[nz]) - 2
    E = np.clip(E, -127, 127)
    v = np.abs(x) * np.ldexp(1.0, -E)[..., None]
    idx = F.e2m1_index_f64(v)
    sign = (xbits.reshape(R, K // MX_BLOCK, MX_BLOCK) >> 15).astype(np.uint8)
    codes4 = (sign << 3) | idx
    return pack_nibbles(codes4.reshape(R, K)), (E + 127).astype(np.uint8)


def mx_dequant_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact real values of MX-coded data as fp64 [R, K] (exact: <= 2 significant
    bits times a power of two in [2**-127, 2**127])."""
    c4 = unpack_nibbles(codes)
    R, K = c4.shape
    e = np.asarray(scales, dtype=np.int64) - 127
    v = code_values_f64(c4).reshape(R, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, e)[..., None]
    return v.reshape(R, K)


# ====================================================================== MXFP8
def mxfp8_block_exact(bits: list[int]) -> tuple[list[int], int]:
    """One 32-element MXFP8 block from bf16 bit patterns: (E4M3 bytes, scale byte)."""
    vals = [F.bf16_bits_to_fraction(b) for b in bits]
    amax = max(abs(v) for v in vals)
    E = -127 if amax == 0 else F.floor_log2(amax) - MX8_EMAX
    E = min(max(E, -127), 127)
    inv = Fraction(2) ** -E
    codes = [F.e4m3_encode(F.round_e4m3_sat(abs(v) * inv)) | (0x80 if b >> 15 else 0)
             for b, v in zip(bits, vals)]
    return codes, E + 127


def mxfp8_quantize_exact(xbits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Scalar-loop MXFP8 quantize of a small [R, K] bf16 array: (E4M3 bytes [R, K],
    UE8M0 scales [R, K/32])."""
    R, K = xbits.shape
    assert K % MX_BLOCK == 0
    codes = np.zeros((R, K), dtype=np.uint8)
    scales = np.zeros((R, K // MX_BLOCK), dtype=np.uint8)
    for r in range(R):
        for b in range(K // MX_BLOCK):
            c, sb = mxfp8_block_exact([int(v) for v in xbits[r, b * 32:(b + 1) * 32]])
            codes[r, b * 32:(b + 1) * 32] = c
            scales[r, b] = sb
    return codes, scales


def mxfp8_quantize(xbits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 quantize [R, K] bf16 bits -> (E4M3 bytes [R, K], UE8M0 scales [R, K/32]).

    fp64 is exact: x * 2**-E only shifts a bf16 value's exponent, and the E4M3
    rounding compares it with exact midpoints of the E4M3 table.
    """
    xbits = np.asarray(xbits, dtype=np.uint16)
    R, K = xbits.shape
    assert K % MX_BLOCK == 0
    x = F.bf16_bits_to_f64(xbits).reshape(R, K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(x).max(axis=-1)
    E = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    E[nz] = F.frexp_floor_log2(amax[nz]) - MX8_EMAX
    E = np.clip(E, -127, 127)
    v = np.abs(x) * np.ldexp(1.0, -E)[..., None]
    mag = F.e4m3_rne_sat_f64(v)
    sign = ((xbits.reshape(R, K // MX_BLOCK, MX_BLOCK) >> 15) & 1).astype(np.uint8)
    codes = (mag | (sign << 7)).astype(np.uint8)
    return codes.reshape(R, K), (E + 127).astype(np.uint8)


def e4m3_signed_f64(codes: np.ndarray) -> np.ndarray:
    """Signed fp64 values of E4M3 bytes (no NaN encodings)."""
    c = np.asarray(codes, dtype=np.uint8)
    v = F.e4m3_value_f64(c & 0x7F)
    return np.where(c & 0x80, -v, v)


def mxfp8_dequant_f64(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact real values of MXFP8 data as fp64 [R, K] (E4M3 value times 2**E)."""
    c = np.asarray(codes, dtype=np.uint8)
    R, K = c.shape
    e = np.asarray(scales, dtype=np.int64) - 127
    v = e4m3_signed_f64(c).reshape(R, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, e)[..., None]
    return v.reshape(R, K)


# E4M3 byte of each E2M1 magnitude index (0, 0.5, 1, 1.5, 2, 3, 4, 6)
E2M1_TO_E4M3 = np.array([F.e4m3_encode(F.E2M1_MAG[i]) for i in range(8)], dtype=np.uint8)


def mx_to_mxfp8(codes: np.ndarray) -> np.ndarray:
    """MXFP4 codes [R, K/2] -> E4M3 bytes [R, K] of the same values (the scale
    bytes carry over unchanged): exact, as E2M1 magnitudes are E4M3 values."""
    c4 = unpack_nibbles(codes)
    return (E2M1_TO_E4M3[c4 & 7] | ((c4 & 8) << 4)).astype(np.uint8)


# ====================================================================== FP4 -> FP8 dequant
MX_FP8_TOP = 6                   # k = E_max - 6: the largest block's code 6 becomes 384


def mx_dequant_fp8(codes: np.ndarray, scales: np.ndarray):
    """MXFP4 (codes [R, K/2], UE8M0 scales [R, K/32]) -> (E4M3 values [R, K],
    E4M3 block scales [R, K/32], fp32 tensor scale s_t, n_inexact blocks).

    fp64 is exact: 2**j and MAG * s8_b are short dyadic numbers, and the E4M3
    rounding compares them with exact midpoints of the E4M3 table."""
    sc = np.asarray(scales, dtype=np.int64)
    R, nb = sc.shape
    if sc.size == 0:
        return np.zeros((R, nb * MX_BLOCK), np.uint8), np.zeros((R, nb), np.uint8), np.float32(1.0), 0
    Emax = int(sc.max()) - 127
    k = Emax - MX_FP8_TOP
    j = sc - 127 - k                                        # <= 6
    s8 = F.e4m3_rne_sat_f64(np.ldexp(1.0, j))               # step 2: the scale array in E4M3
    c4 = unpack_nibbles(codes).reshape(R, nb, MX_BLOCK)
    prod = F.E2M1_MAG_F64[c4 & 7] * F.e4m3_value_f64(s8)[..., None]
    v8 = F.e4m3_rne_sat_f64(prod) | ((c4 & 8) << 4)         # steps 3-4, sign from the code
    exact = e4m3_signed_f64(v8) * np.ldexp(1.0, k) == code_values_f64(c4) * np.ldexp(1.0, sc - 127)[..., None]
    n_inexact = int((~exact.all(axis=-1)).sum())
    return v8.reshape(R, nb * MX_BLOCK).astype(np.uint8), s8.astype(np.uint8), np.float32(np.ldexp(1.0, k)), n_inexact


def mx_dequant_fp8_exact(codes: np.ndarray, scales: np.ndarray):
    """Scalar-loop form of mx_dequant_fp8 for small inputs (Fraction arithmetic)."""
    R, nb = scales.shape
    Emax = max(int(b) - 127 for b in scales.ravel())
    k = Emax - MX_FP8_TOP
    c4 = unpack_nibbles(codes)
    v8 = np.zeros((R, nb * MX_BLOCK), np.uint8)
    s8 = np.zeros((R, nb), np.uint8)
    n_inexact = 0
    for r in range(R):
        for b in range(nb):
            Eb = int(scales[r, b]) - 127
            sb = F.round_e4m3_sat(Fraction(2) ** (Eb - k))
            s8[r, b] = F.e4m3_encode(sb)
            inexact = False
            for i in range(MX_BLOCK):
                c = int(c4[r, b * MX_BLOCK + i])
                v = F.round_e4m3_sat(F.E2M1_MAG[c & 7] * sb)
                v8[r, b * MX_BLOCK + i] = F.e4m3_encode(v) | (0x80 if c & 8 else 0)
                inexact |= v * Fraction(2) ** k != F.E2M1_MAG[c & 7] * Fraction(2) ** Eb
            n_inexact += inexact
    return v8, s8, np.float32(float(Fraction(2) ** k)), n_inexact


# ====================================================================== NV
def nv_tensor_scale_exact(amax_t: Fraction) -> Fraction:
    """s_t = RNE_fp32(amax_t / 2688)."""
    return F.round_fp32(amax_t / NV_TENSOR_DIV)


def nv_tensor_scale(xbits: np.ndarray) -> np.float32:
    """s_t from a bf16 tensor.  amax_t / 2688 in fp64 is rounded once to fp64
    and then to fp32; the fp64 quotient of an 8-bit numerator and 2688 = 21*2**7
    is either exact (numerator divisible by 21) or at least ~2**-30 (relative)
    away from every fp32 rounding midpoint, so the double rounding is exact."""
    amax = float(np.abs(F.bf16_bits_to_f64(xbits)).max()) if np.size(xbits) else 0.0
    return np.float32(amax / NV_TENSOR_DIV)


def nv_group_exact(bits: list[int], s_t: Fraction) -> tuple[list[int], int]:
    """One 16-element NV group: (4-bit codes, E4M3 scale byte) given s_t."""
    vals = [F.bf16_bits_to_fraction(b) for b in bits]
    amax = max(abs(v) for v in vals)
    if s_t == 0:
        return [8 * (b >> 15) for b in bits], 0
    s_g = F.round_e4m3_sat(amax / (6 * s_t))
    if s_g == 0:
        return [8 * (b >> 15) for b in bits], 0
    d = s_g * s_t
    codes = [F.e2m1_encode(bool(b >> 15), abs(v) / d) for b, v in zip(bits, vals)]
    return codes, F.e4m3_encode(s_g)


def nv_quantize_exact(xbits: np.ndarray, s_t: float | None = None):
    """Scalar-loop NV quantize of a small [R, K] bf16 array -> (codes, scales, s_t)."""
    R, K = xbits.shape
    assert K % NV_GROUP == 0
    if s_t is None:
        amax = max((abs(F.bf16_bits_to_fraction(int(b))) for b in xbits.ravel()), default=Fraction(0))
        st = nv_tensor_scale_exact(amax)
    else:
        st = Fraction(float(np.float32(s_t)))
    codes4 = np.zeros((R, K), dtype=np.uint8)
    scales = np.zeros((R, K // NV_GROUP), dtype=np.uint8)
    for r in range(R):
        for g in range(K // NV_GROUP):
            c, s = nv_group_exact([int(v) for v in xbits[r, g * 16:(g + 1) * 16]], st)
            codes4[r, g * 16:(g + 1) * 16] = c
            scales[r, g] = s
    return pack_nibbles(codes4), scales, np.float32(float(st))


def nv_quantize(xbits: np.ndarray, s_t: float | None = None):
    """NV quantize [R, K] bf16 bits -> (codes [R, K/2], E4M3 [R, K/16], s_t fp32).

    fp64 is exact for both roundings: 6*s_t and s_g*s_t are exact (<= 28 bits).
    amax_g/(6 s_t) has an 8-bit numerator and a <= 26-bit denominator, so unless
    it equals an E4M3 midpoint (<= 5 bits) it is >= ~2**-32 (relative) away from
    it; x/(s_g s_t) (8-bit over <= 28-bit) likewise stays >= ~2**-36 from any
    E2M1 midpoint unless equal.  The correctly rounded fp64 quotient (error
    <= 2**-53) therefore lands on the same side of every midpoint, and hits a
    midpoint exactly only when the real quotient does.
    """
    xbits = np.asarray(xbits, dtype=np.uint16)
    R, K = xbits.shape
    assert K % NV_GROUP == 0
    st = nv_tensor_scale(xbits) if s_t is None else np.float32(s_t)
    st64 = float(st)
    x = F.bf16_bits_to_f64(xbits).reshape(R, K // NV_GROUP, NV_GROUP)
    sign = (xbits.reshape(R, K // NV_GROUP, NV_GROUP) >> 15).astype(np.uint8)
    if st64 == 0.0:
        return pack_nibbles((sign << 3).reshape(R, K)), np.zeros((R, K // NV_GROUP), np.uint8), st
    amax = np.abs(x).max(axis=-1)
    sg_b = F.e4m3_rne_sat_f64(amax / (6.0 * st64))
    sg = F.e4m3_value_f64(sg_b)
    d = sg * st64
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(d[..., None] > 0, np.abs(x) / np.where(d > 0, d, 1.0)[..., None], 0.0)
    idx = F.e2m1_index_f64(q)
    codes4 = (sign << 3) | idx
    return pack_nibbles(codes4.reshape(R, K)), sg_b, st


def nv_dequant_exact_f64(codes: np.ndarray, scales: np.ndarray, s_t: float) -> np.ndarray:
    """Exact real values MAG * s_g * s_t as fp64 (<= 6 bits times 24 bits: exact)."""
    c4 = unpack_nibbles(codes)
    R, K = c4.shape
    sg = F.e4m3_value_f64(scales)
    v = code_values_f64(c4).reshape(R, K // NV_GROUP, NV_GROUP) * sg[..., None] * float(np.float32(s_t))
    return v.reshape(R, K)


# ====================================================================== dequant outputs
def dequant_fp32(fmt: str, codes, scales, s_t=None) -> np.ndarray:
    """Dequantize to fp32: MX is exact; NV rounds MAG*s_g*s_t once (exact fp64
    product, then numpy's correctly rounded fp64->fp32 cast)."""
    v = mx_dequant_f64(codes, scales) if fmt == "mx" else nv_dequant_exact_f64(codes, scales, s_t)
    return F.f64_to_fp32_rne(v)


def dequant_bf16_bits(fmt: str, codes, scales, s_t=None) -> np.ndarray:
    """Dequantize to bf16: RNE_bf16 of the fp32 dequantized value."""
    return F.fp32_to_bf16_bits_rne(dequant_fp32(fmt, codes, scales, s_t))


# ====================================================================== remap
def remap_mx_to_nv(codes: np.ndarray, scales: np.ndarray):
    """MX (codes, UE8M0 scales [R, K/32]) -> (E4M3 scales [R, K/16], s_t, n_inexact).

    Codes are reused unchanged.  E_b = byte - 127.  Blocks whose codes are all
    zero never make the remap inexact, and their exponent is still part of E_max
    (a zero block quantized from amax = 0 has E_b = -127 and cannot raise it).
    """
    sc = np.asarray(scales, dtype=np.int64)
    R, nb = sc.shape
    if sc.size == 0:
        return np.zeros((R, nb * 2), np.uint8), np.float32(1.0), 0
    Eb = sc - 127
    Emax = int(Eb.max())
    k = Emax - 8
    j = Eb - k                                           # in [-(254-8), 8]
    sg = F.e4m3_rne_sat_f64(np.ldexp(1.0, j))            # 2**j exact in fp64
    c4 = unpack_nibbles(codes).reshape(R, nb, MX_BLOCK)
    nonzero = (c4 & 7).any(axis=-1)
    n_inexact = int(((j < -9) & nonzero).sum())
    sg2 = np.repeat(sg, 2, axis=1)
    return sg2.astype(np.uint8), np.float32(np.ldexp(1.0, k)), n_inexact


def remap_mx_to_nv_exact(codes: np.ndarray, scales: np.ndarray):
    """Scalar-loop form of the remap for small inputs (Fraction arithmetic)."""
    R, nb = scales.shape
    Emax = max(int(s) - 127 for s in scales.ravel())
    k = Emax - 8
    c4 = unpack_nibbles(codes)
    out = np.zeros((R, nb * 2), np.uint8)
    n_inexact = 0
    for r in range(R):
        for b in range(nb):
            Eb = int(scales[r, b]) - 127
            sg = F.round_e4m3_sat(Fraction(2) ** (Eb - k))
            out[r, 2 * b] = out[r, 2 * b + 1] = F.e4m3_encode(sg)
            exact = sg == Fraction(2) ** (Eb - k)
            if not exact and any(int(c) & 7 for c in c4[r, b * 32:(b + 1) * 32]):
                n_inexact += 1
    return out, np.float32(float(Fraction(2) ** k)), n_inexact


# ====================================================================== QAT fake quant and STE
def fake_quant_fp32(fmt: str, xbits: np.ndarray, s_t: float | None = None) -> np.ndarray:
    """The QAT fake-quantize node [V4-QAT s2.2: quantize-dequantize inserted in
    the forward pass]: the dequantized values of the quantized tensor, fp32 as
    `dequant_fp32` defines them.  NV: s_t computed from the tensor unless given."""
    if fmt == "mx":
        codes, scales = mx_quantize(xbits)
        return dequant_fp32("mx", codes, scales)
    codes, scales, st = nv_quantize(xbits, s_t)
    return dequant_fp32("nv", codes, scales, st)


def fake_quant_bf16_bits(fmt: str, xbits: np.ndarray, s_t: float | None = None) -> np.ndarray:
    """Same, rounded to bf16 (RNE of the fp32 value), as `dequant_bf16_bits`."""
    return F.fp32_to_bf16_bits_rne(fake_quant_fp32(fmt, xbits, s_t))


def ste_backward(grad: np.ndarray, master: np.ndarray | None = None) -> np.ndarray:
    """Straight-through estimator [V4-ARCH s6.3: the gradient of the quantized
    weight goes unchanged to the fp32 master weight]: the incoming gradient
    (fp32 or bf16 values given as float arrays), added to the existing fp32
    master gradient when one is given, one fp32 rounding per element."""
    g = np.asarray(grad, np.float64)
    if master is None:
        return F.f64_to_fp32_rne(g)
    return F.f64_to_fp32_rne(np.asarray(master, np.float64) + g)    # sum of two fp32 is exact in fp64


# ====================================================================== MXFP4 KV cache
def kv_append_mx(cache_codes: np.ndarray, cache_scales: np.ndarray, xbits: np.ndarray, slots) -> tuple:
    """The MXFP4 KV cache [V4-QAT s3.3: new tokens' vectors are quantized as they
    join the cache]: each row of x (one token, d values) is MX-quantized on its
    own and stored at cache row slots[t]; slots outside [0, capacity) are
    padding and skipped.  Returns updated copies of (codes, scales)."""
    codes, scales = cache_codes.copy(), cache_scales.copy()
    cap = codes.shape[0]
    qc, qs = mx_quantize(xbits)
    for t, s in enumerate(np.asarray(slots).tolist()):
        if 0 <= s < cap:
            codes[s], scales[s] = qc[t], qs[t]
    return codes, scales
