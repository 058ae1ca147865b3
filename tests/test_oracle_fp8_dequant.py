"""Pins of the oracle's MXFP4 -> FP8 dequantization (the four steps of the
"DeepSeek-V4 FP4 quantization-aware training" article, section 4.2, with one
fp32 power-of-two tensor scale): a hand-worked tensor, torch's own E4M3 cast,
the exact MX values (lossless below the 2**14 block scale ratio), the count of
inexact blocks by brute force, and the Fraction form against the fp64 form."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import formats as F
from oracle import quant as Q
from conftest import read_records


def _torch_e4m3_bytes(v: np.ndarray) -> np.ndarray:
    """E4M3FN bytes of non-negative fp64 values below 448 by torch's own cast."""
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_values(b: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("rec", read_records("fp8_dequant_worked_blocks.txt"), ids=lambda r: r["name"])
def test_fp8_dequant_worked_tensor(rec):
    scales = np.array([[int(v) for v in rec["scales"]]], np.uint8)
    nb = scales.shape[1]
    c4 = np.concatenate([[int(v) for v in rec[f"codes{b}"]] for b in range(nb)]).astype(np.uint8)[None, :]
    vals = np.concatenate([[int(v) for v in rec[f"values{b}"]] for b in range(nb)]).astype(np.uint8)[None, :]
    codes = Q.pack_nibbles(c4)
    for fn in (Q.mx_dequant_fp8, Q.mx_dequant_fp8_exact):
        v8, s8, st, n = fn(codes, scales)
        assert np.array_equal(v8, vals)
        assert list(s8[0]) == [int(v) for v in rec["s8"]]
        assert float(st) == float(rec["s_t"][0])
        assert n == int(rec["n_inexact"][0])


def _mx_tensor(seed, R, K, spread):
    """MX codes of N(0,1) data with per-block magnitudes spread over `spread` binades."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)) * np.exp2(rng.integers(0, spread + 1, size=(R, K // 32, 1))).repeat(32, -1).reshape(R, K)
    return Q.mx_quantize(W.bf16_bits(W.to_bf16(x)))


@pytest.mark.parametrize("which", ["A", "W"])
def test_fp8_dequant_lossless_linear_workload(which):
    """The linear workload's tensors (block exponents within 2**14 of the largest)
    dequantize to FP8 without loss: decoded by torch, value * s_t is the exact
    MX value of every element, and no block is counted."""
    bits = W.bf16_bits(getattr(W.workload2(), which))[:512]
    codes, scales = Q.mx_quantize(bits)
    live = (Q.unpack_nibbles(codes) & 7).reshape(512, -1, 32).any(-1)
    assert int(scales.max()) - int(scales[live].min()) <= 14
    v8, s8, st, n = Q.mx_dequant_fp8(codes, scales)
    assert n == 0
    assert np.array_equal(_torch_e4m3_values(v8) * float(st), Q.mx_dequant_f64(codes, scales))


@pytest.mark.parametrize("spread", [10, 14, 15, 16, 20, 40])
def test_fp8_dequant_bytes_match_torch_cast(spread):
    """Every value byte and block scale byte equals torch's float8_e4m3fn cast of
    the same product (all below 448, so torch's NaN range is never reached),
    with the sign taken from the code."""
    codes, scales = _mx_tensor(spread, 16, 512, spread)
    v8, s8, st, n = Q.mx_dequant_fp8(codes, scales)
    k = int(scales.max()) - 127 - 6
    assert float(st) == 2.0 ** k
    j = scales.astype(np.int64) - 127 - k
    assert np.array_equal(s8, _torch_e4m3_bytes(np.ldexp(1.0, j)))
    c4 = Q.unpack_nibbles(codes)
    prod = F.E2M1_MAG_F64[c4 & 7] * np.repeat(_torch_e4m3_values(s8), 32, axis=1)
    assert prod.max() <= 384.0
    assert np.array_equal(v8 & 0x7F, _torch_e4m3_bytes(prod))
    assert np.array_equal(v8 >> 7, c4 >> 3)


@pytest.mark.parametrize("spread", [12, 14, 15, 16, 18])
def test_fp8_dequant_inexact_count_brute_force(spread):
    """n_inexact counts exactly the blocks holding an element whose FP8 value
    times s_t differs from its MX value (Fraction arithmetic per element); it
    is zero whenever every block exponent is within 14 of the largest."""
    codes, scales = _mx_tensor(100 + spread, 6, 256, spread)
    v8, s8, st, n = Q.mx_dequant_fp8(codes, scales)
    c4 = Q.unpack_nibbles(codes)
    cnt = 0
    for r in range(scales.shape[0]):
        for b in range(scales.shape[1]):
            bad = False
            for i in range(32):
                c, v = int(c4[r, b * 32 + i]), int(v8[r, b * 32 + i])
                mx = F.e2m1_value(c) * F.ue8m0_value(int(scales[r, b]))
                bad |= F.e4m3_decode(v) * Fraction(float(st)) != mx
            cnt += bad
    assert n == cnt
    if int(scales.max()) - int(scales.min()) <= 14:
        assert n == 0


def test_fp8_dequant_scale_ratio_threshold():
    """Blocks at E_max - 14 are exact for every code; at E_max - 15 a block with
    code magnitude 0.5 or 1.5 is inexact; at E_max - 16 and below any nonzero
    block is inexact (its E4M3 scale rounds to zero); all-zero blocks never count."""
    c4 = np.zeros((1, 7 * 32), np.uint8)
    allc = np.arange(16, dtype=np.uint8)
    c4[0, 0:16] = allc                     # E_max block, every code
    c4[0, 32:48] = allc                    # E_max - 14, every code: exact
    c4[0, 64:65] = 1                       # E_max - 15, 0.5: inexact
    c4[0, 96:101] = [2, 4, 5, 6, 7]        # E_max - 15, 1..6 without 1.5: exact
    c4[0, 128:129] = 7                     # E_max - 16, 6: inexact (scale 0)
    c4[0, 160:161] = 8                     # -0 only at E_max - 40: exact
    c4[0, 192:193] = 3                     # E_max - 15, 1.5: inexact
    scales = np.array([[140, 126, 125, 125, 124, 100, 125]], np.uint8)
    v8, s8, st, n = Q.mx_dequant_fp8(Q.pack_nibbles(c4), scales)
    assert n == 3
    assert Q.mx_dequant_fp8_exact(Q.pack_nibbles(c4), scales)[3] == 3


def test_fp8_dequant_exact_form_matches_fp64_form():
    for seed, spread in ((1, 3), (2, 17), (3, 30)):
        codes, scales = _mx_tensor(seed, 3, 128, spread)
        a, b = Q.mx_dequant_fp8(codes, scales), Q.mx_dequant_fp8_exact(codes, scales)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert float(a[2]) == float(b[2]) and a[3] == b[3]


def test_fp8_dequant_extreme_exponents():
    """E_max = 127 (s_t = 2**121) and E_max = -127 (s_t = 2**-133, an fp32 subnormal)."""
    c4 = np.tile(np.arange(16, dtype=np.uint8), (2, 4))
    for byte in (254, 0):
        scales = np.full((2, 2), byte, np.uint8)
        v8, s8, st, n = Q.mx_dequant_fp8(Q.pack_nibbles(c4), scales)
        assert n == 0 and float(st) == 2.0 ** (byte - 127 - 6)
        assert np.array_equal(_torch_e4m3_values(v8) * float(st), Q.mx_dequant_f64(Q.pack_nibbles(c4), scales))
