"""W4A4 GEMM oracle: C = A_hat . B_hat^T over exact dequantized operands.

[V41-NVFP4 s2] describes the W4A4 product: activations and weights are both
4-bit block-scaled, the products accumulate, and the block scales multiply back
in.  The plain definition is the matrix product of the exact dequantized
values; only the summation order of an fp32 accumulator is free, so the
oracle also returns S[m, n] = sum_k |A_hat[m, k] B_hat[n, k]| for the
tolerance |C - C_ref| <= 1e-5 * S.

Exactness of fp64: every MX product is (<= 2 bits)(<= 2 bits) times a power of
two; with the exponent spans of the workloads here (a few tens of binades) and
K <= 2**13 terms the sum needs < 53 bits, so the fp64 matmul is exact in any
order.  NV operands add a 4-bit group scale per side (still exact) and two
fp32 tensor scales applied after the sum (one rounding of an exact sum).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from . import formats as F
from . import quant as Q


def operand_values(fmt: str, codes, scales, s_t=None) -> np.ndarray:
    """Exact real operand values [R, K] in fp64 (NV without s_t applied);
    fmt "mx8" is MXFP8 (E4M3 bytes [R, K])."""
    if fmt == "mx":
        return Q.mx_dequant_f64(codes, scales)
    if fmt == "mx8":
        return Q.mxfp8_dequant_f64(codes, scales)
    c4 = Q.unpack_nibbles(codes)
    R, K = c4.shape
    sg = F.e4m3_value_f64(scales)
    return (Q.code_values_f64(c4).reshape(R, K // Q.NV_GROUP, Q.NV_GROUP) * sg[..., None]).reshape(R, K)


def gemm_ref(fmt: str, a_codes, a_scales, b_codes, b_scales, a_st=None, b_st=None):
    """C_ref [M, N] (fp64) and the bound S [M, N] for C = A . B^T, B given as [N, K]."""
    A = operand_values(fmt, a_codes, a_scales)
    B = operand_values(fmt, b_codes, b_scales)
    C = A @ B.T
    S = np.abs(A) @ np.abs(B).T
    if fmt == "nv":
        st = float(np.float32(a_st)) * float(np.float32(b_st))
        C, S = C * st, S * st
    return C, S


def gemm_ref_w4a8(a_codes8, a_scales, b_codes, b_scales):
    """W4A4's FP8-activation variant [V4-QAT s4.3]: C = A_hat . B_hat^T with A
    MXFP8 [M, K] and B MXFP4 [N, K/2]; returns C_ref and the bound S in fp64.
    A product of an E4M3 and an E2M1 value has at most 6 significant bits, so
    each term is exact; the fp64 sum's own rounding (at most K * 2**-53 * S)
    is far inside the 1e-5 * S tolerance."""
    A = Q.mxfp8_dequant_f64(a_codes8, a_scales)
    B = Q.mx_dequant_f64(b_codes, b_scales)
    return A @ B.T, np.abs(A) @ np.abs(B).T


def gemm_exact_fraction_w4a8(a_codes8, a_scales, b_codes, b_scales):
    """Brute force for tiny W4A8 inputs in Python ``Fraction``s, element by element
    from the byte fields (independent of the fp64 tables)."""
    cb = Q.unpack_nibbles(b_codes)
    M, K = np.asarray(a_codes8).shape
    N = cb.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                a = F.e4m3_decode(int(a_codes8[m, k])) * F.ue8m0_value(int(a_scales[m, k // Q.MX_BLOCK]))
                b = F.e2m1_value(int(cb[n, k])) * F.ue8m0_value(int(b_scales[n, k // Q.MX_BLOCK]))
                acc += a * b
            out[m][n] = acc
    return out


def gemm_exact_fraction(fmt: str, a_codes, a_scales, b_codes, b_scales, a_st=None, b_st=None):
    """Brute force for tiny inputs: the same sum in Python ``Fraction``s, taken
    block by block as integer dot products of doubled magnitudes times the
    product of the two block scales (an independent formulation)."""
    ca, cb = Q.unpack_nibbles(a_codes), Q.unpack_nibbles(b_codes)
    M, K = ca.shape
    N = cb.shape[0]
    blk = Q.MX_BLOCK if fmt == "mx" else Q.NV_GROUP

    def scale(fmt_, byte):
        return F.ue8m0_value(int(byte)) if fmt_ == "mx" else F.e4m3_decode(int(byte))

    def ival(c):  # 2 * signed magnitude, an integer
        m = int(F.E2M1_MAG[c & 7] * 2)
        return -m if c & 8 else m

    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for b in range(K // blk):
                dot = sum(ival(int(ca[m, k])) * ival(int(cb[n, k])) for k in range(b * blk, (b + 1) * blk))
                acc += Fraction(dot, 4) * scale(fmt, a_scales[m, b]) * scale(fmt, b_scales[n, b])
            if fmt == "nv":
                acc *= Fraction(float(np.float32(a_st))) * Fraction(float(np.float32(b_st)))
            out[m][n] = acc
    return out


def within_tol_f32(C: np.ndarray, C_ref: np.ndarray, S: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """Element mask of fp32 results meeting |C - C_ref| <= rel * S."""
    return np.abs(np.asarray(C, np.float64) - C_ref) <= rel * S


def within_tol_bf16(C_bits: np.ndarray, C_ref: np.ndarray, S: np.ndarray, rel: float = 1e-5) -> np.ndarray:
    """Element mask of bf16 results that some value within the tolerance rounds to:
    RNE_bf16(C_ref - rel*S) <= C <= RNE_bf16(C_ref + rel*S) (rounding is monotone).
    The bracket ends are computed in fp64 and rounded once to bf16."""
    lo = F.bf16_bits_to_f64(F.bf16_rne_of_f64(C_ref - rel * S))
    hi = F.bf16_bits_to_f64(F.bf16_rne_of_f64(C_ref + rel * S))
    c = F.bf16_bits_to_f64(C_bits)
    return (c >= lo) & (c <= hi)
