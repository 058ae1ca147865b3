"""Pins of the oracle's MXFP8 quantizer, FP4 -> FP8 re-encoding and W4A8 GEMM
(the FP8-activation variant of the GEMM): hand-worked blocks, torch's own E4M3
cast, the scale rule's closed form, idempotence, losslessness of FP4 -> FP8,
brute-force Fraction products, and agreement with the W4A4 oracle when the
activations lie on the FP4 grid."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q
from conftest import read_records, parse_float


def _bits(vals):
    v = np.array([parse_float(s) for s in vals], dtype=np.float64)
    bits = F.fp32_to_bf16_bits_rne(v.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(bits), v) and np.array_equal(np.signbit(F.bf16_bits_to_f64(bits)),
                                                                          np.signbit(v))
    return bits


@pytest.mark.parametrize("rec", read_records("mxfp8_worked_blocks.txt"), ids=lambda r: r["name"])
def test_mxfp8_worked_blocks(rec):
    bits = _bits(rec["x"])
    codes, scale = Q.mxfp8_block_exact([int(b) for b in bits])
    assert scale == int(rec["scale"][0])
    assert codes == [int(c) for c in rec["codes"]]
    vc, vs = Q.mxfp8_quantize(bits[None, :])
    assert vs[0, 0] == int(rec["scale"][0])
    assert list(vc[0]) == [int(c) for c in rec["codes"]]


def _random_bits(seed, R, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)) * np.exp2(rng.integers(-20, 20, size=(R, 1)))
    x[rng.random((R, K)) < 0.02] *= 300.0                       # outliers -> saturation
    x[rng.random((R, K)) < 0.02] *= 2.0 ** -30                   # far below the block max -> subnormals, zeros
    x[rng.random((R, K)) < 0.01] = -0.0
    return F.fp32_to_bf16_bits_rne(x.astype(np.float32))


def test_mxfp8_vectorised_matches_exact():
    bits = _random_bits(7, 12, 256)
    c1, s1 = Q.mxfp8_quantize_exact(bits)
    c2, s2 = Q.mxfp8_quantize(bits)
    assert np.array_equal(s1, s2) and np.array_equal(c1, c2)


def test_mxfp8_codes_match_torch_e4m3_cast():
    """The element rounding against torch's float8_e4m3fn cast (round to nearest
    even), on every scaled magnitude inside E4M3's range (the cast does not
    saturate, so the saturating ones are checked against 0x7E)."""
    bits = _random_bits(8, 64, 512)
    codes, scales = Q.mxfp8_quantize(bits)
    x = F.bf16_bits_to_f64(bits).reshape(64, 16, 32)
    v = np.abs(x) * np.ldexp(1.0, 127 - scales.astype(np.int64))[..., None]
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mag = codes.reshape(64, 16, 32) & 0x7F
    inside = v <= 448.0
    assert np.array_equal(mag[inside], ref[inside])
    assert (mag[~inside] == 0x7E).all() and (~inside).any()
    assert np.array_equal(codes.reshape(64, 16, 32) >> 7, (bits.reshape(64, 16, 32) >> 15).astype(np.uint8))


def test_mxfp8_scale_rule_closed_form():
    """amax / 2**E lies in [256, 512) for every block whose E is not clamped."""
    bits = _random_bits(9, 40, 256)
    _, scales = Q.mxfp8_quantize(bits)
    amax = np.abs(F.bf16_bits_to_f64(bits).reshape(40, 8, 32)).max(-1)
    r = amax * np.ldexp(1.0, 127 - scales.astype(np.int64))
    ok = (amax > 0) & (scales > 0)
    assert ok.any() and ((r[ok] >= 256) & (r[ok] < 512)).all()


def test_mxfp8_idempotent_on_grid():
    """Dequantized codes (exact bf16 values) quantize back to the same codes and scales."""
    bits = _random_bits(10, 16, 256)
    codes, scales = Q.mxfp8_quantize(bits)
    vals = Q.mxfp8_dequant_f64(codes, scales)
    back = F.fp32_to_bf16_bits_rne(vals.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(back), vals)      # on the bf16 grid (moderate exponents)
    c2, s2 = Q.mxfp8_quantize(back)
    nonzero_block = np.abs(vals.reshape(16, 8, 32)).max(-1) > 0
    assert np.array_equal(s2[nonzero_block], scales[nonzero_block])
    assert np.array_equal(c2, codes)


def test_fp4_to_fp8_is_lossless():
    """Every E2M1 code re-encodes to the E4M3 byte of the same value, so an MXFP4
    tensor and its MXFP8 re-encoding (same scales) have equal values."""
    for c in range(16):
        e4 = Q.mx_to_mxfp8(np.array([[c | (c << 4)]], dtype=np.uint8))[0, 0]
        assert F.e4m3_decode(int(e4)) == F.e2m1_value(c)
        if c == 8:
            assert e4 == 0x80                                       # -0 keeps its sign
    w = W.random_linear(11, 8, 8, 256).W
    codes, scales = Q.mx_quantize(W.bf16_bits(w))
    a = Q.mx_dequant_f64(codes, scales)
    b = Q.mxfp8_dequant_f64(Q.mx_to_mxfp8(codes), scales)
    assert np.array_equal(a, b)


def _tiny_w4a8(seed, M, N, K):
    wl = W.random_linear(seed, M, N, K, outlier_p=0.02)
    a8, sa = Q.mxfp8_quantize(W.bf16_bits(wl.A))
    b4, sb = Q.mx_quantize(W.bf16_bits(wl.W))
    return a8, sa, b4, sb


@pytest.mark.parametrize("seed", [1, 2])
def test_w4a8_gemm_brute_force(seed):
    a8, sa, b4, sb = _tiny_w4a8(seed, 3, 4, 64)
    C, S = G.gemm_ref_w4a8(a8, sa, b4, sb)
    exact = G.gemm_exact_fraction_w4a8(a8, sa, b4, sb)
    for m in range(3):
        for n in range(4):
            assert Fraction(C[m, n]) == exact[m][n]                # exact at this size
            assert S[m, n] >= abs(C[m, n])


def test_w4a8_equals_w4a4_on_fp4_activations():
    """With activations already on the FP4 grid (an MXFP4 tensor re-encoded to
    MXFP8), the W4A8 product equals the W4A4 oracle's."""
    wl = W.random_linear(12, 16, 24, 512)
    a4, sa = Q.mx_quantize(W.bf16_bits(wl.A))
    b4, sb = Q.mx_quantize(W.bf16_bits(wl.W))
    C8, S8 = G.gemm_ref_w4a8(Q.mx_to_mxfp8(a4), sa, b4, sb)
    C4, S4 = G.gemm_ref("mx", a4, sa, b4, sb)
    assert np.array_equal(C8, C4) and np.array_equal(S8, S4)
