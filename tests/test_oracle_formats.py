"""Pins of the oracle's number formats against the page's E2M1 table, the OCP
E4M3 definition as cast by torch, numpy's IEEE casts, and two independent
formulations of each rounding."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from conftest import read_records, GOLDEN
import os


def _golden_e2m1():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                rows.append((int(c), float(v)))
    return rows


def test_e2m1_table_matches_page():
    rows = _golden_e2m1()
    assert len(rows) == 16
    for code, v in rows:
        assert float(F.e2m1_value(code)) == v
        assert np.signbit(float(F.e2m1_value(code))) == np.signbit(v) or v == 0
        # the bit-field reading (2 exponent + 1 mantissa bits) gives the same table
        assert F.e2m1_value_from_fields(code) == F.e2m1_value(code)


def test_e2m1_encode_table_values_roundtrip():
    for code in range(16):
        v = F.e2m1_value(code)
        assert F.e2m1_encode(bool(code & 8), abs(v)) == code


@pytest.mark.parametrize("mid,expect_idx", [
    (Fraction(1, 4), 0), (Fraction(3, 4), 2), (Fraction(5, 4), 2), (Fraction(7, 4), 4),
    (Fraction(5, 2), 4), (Fraction(7, 2), 6), (Fraction(5), 6)])
def test_e2m1_ties_to_even_index(mid, expect_idx):
    assert F.e2m1_encode(False, mid) == expect_idx
    assert F.e2m1_encode(True, mid) == 8 | expect_idx
    eps = Fraction(1, 2 ** 40)
    assert F.e2m1_encode(False, mid - eps) in (expect_idx, expect_idx - 1) and \
        F.e2m1_encode(False, mid - eps) == (F.E2M1_MAG.index(max(m for m in F.E2M1_MAG if m < mid)))
    assert F.e2m1_encode(False, mid + eps) == F.E2M1_MAG.index(min(m for m in F.E2M1_MAG if m > mid))


def test_e2m1_saturation_and_zero():
    assert F.e2m1_encode(False, Fraction(6)) == 7
    assert F.e2m1_encode(False, Fraction(7)) == 7
    assert F.e2m1_encode(False, Fraction(10 ** 9)) == 7
    assert F.e2m1_encode(True, Fraction(0)) == 8
    assert F.e2m1_encode(False, Fraction(0)) == 0


def test_e2m1_generic_rounding_agrees_with_table():
    """round_binary with E2M1's parameters (2 significant bits, emin 0, max 6,
    saturating) is a second formulation of nearest-in-table rounding."""
    rng = np.random.default_rng(5)
    vals = [Fraction(int(n), 64) for n in rng.integers(0, 64 * 9, 3000)]
    vals += [Fraction(int(n), 1 << 20) for n in rng.integers(0, 9 << 20, 2000)]
    for v in vals:
        r = F.round_binary(v, 2, 0, Fraction(6), saturate=True)
        assert F.E2M1_MAG[F.e2m1_encode(False, v)] == r, v


def test_e2m1_vectorised_matches_scalar():
    rng = np.random.default_rng(6)
    a = np.concatenate([rng.uniform(0, 9, 20000), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, 6, 8, 0]),
                        rng.integers(0, 40, 2000) / 4.0])
    idx = F.e2m1_index_f64(a)
    for x, i in zip(a, idx):
        assert F.e2m1_encode(False, Fraction(float(x))) == i


def test_e4m3_decode_all_bytes_against_torch():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for byte in range(256):
        v = F.e4m3_decode(byte)
        if v is None:
            assert np.isnan(b[byte])
        else:
            assert float(v) == b[byte], byte
    assert max(float(F.e4m3_decode(x)) for x in range(0x7F)) == 448.0


def test_e4m3_rounding_against_torch_cast():
    """torch's float8_e4m3fn cast rounds to nearest even and is finite up to 464;
    above 448 our definition saturates."""
    rng = np.random.default_rng(7)
    q = np.concatenate([rng.uniform(0, 464, 20000), np.exp(rng.uniform(-16, 6, 20000)),
                        F.E4M3_POS_F64, (F.E4M3_POS_F64[1:] + F.E4M3_POS_F64[:-1]) / 2]).astype(np.float32)
    q = q[q <= 464].astype(np.float64)
    ours = F.e4m3_rne_sat_f64(q)
    theirs = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)
    assert F.e4m3_rne_sat_f64(np.array([500.0, 1e9]))[0] == 0x7E


def test_e4m3_exact_vs_vectorised():
    rng = np.random.default_rng(8)
    for _ in range(3000):
        num, den = int(rng.integers(1, 1 << 8)), int(rng.integers(1, 1 << 26))
        q = Fraction(num, den) * Fraction(2) ** int(rng.integers(-12, 20))
        b = F.e4m3_encode(F.round_e4m3_sat(q))
        assert F.e4m3_rne_sat_f64(np.array([float(q)]))[0] == b, q


def test_fp32_rounding_against_numpy():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000),
                        rng.standard_normal(500) * 1e-42])
    for v in x:
        assert float(F.round_fp32(Fraction(float(v)))) == float(np.float32(v))


def test_bf16_bits_against_torch():
    rng = np.random.default_rng(10)
    u = rng.integers(0, 1 << 32, 50000, dtype=np.uint64).astype(np.uint32)
    u = u[((u >> 23) & 0xFF) != 0xFF]
    u = np.concatenate([u, np.array([0x3F808000, 0x3F818000, 0x00008000, 0x00018000, 0x80008000], np.uint32)])
    x = u.view(np.float32)
    ours = F.fp32_to_bf16_bits_rne(x)
    theirs = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_bf16_of_f64_single_rounding():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(3000) * 10.0 ** rng.integers(-38, 38, 3000)
    x = np.concatenate([x, [1 + 2 ** -8, 1 + 2 ** -8 + 2 ** -40, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 ** -133 * 1.5]])
    bits = F.bf16_rne_of_f64(x)
    for v, b in zip(x, bits):
        assert F.bf16_bits_to_fraction(int(b)) == F.round_bf16(Fraction(float(v))), v


def test_floor_log2_exact():
    for num in range(1, 300):
        for den in (1, 3, 7, 64, 1000):
            q = Fraction(num, den)
            e = F.floor_log2(q)
            assert Fraction(2) ** e <= q < Fraction(2) ** (e + 1)
    a = np.array([1.0, 1.5, 2.0, 3.99, 2.0 ** -130, 0.75])
    assert list(F.frexp_floor_log2(a)) == [0, 0, 1, 1, -130, -1]


def test_ue8m0_values():
    assert F.ue8m0_value(127) == 1
    assert F.ue8m0_value(0) == Fraction(2) ** -127
    assert F.ue8m0_value(254) == Fraction(2) ** 127
