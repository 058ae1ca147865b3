"""Pins of the oracle's quantizers, remap and dequantizers: hand-worked blocks,
the scalar exact definition against the vectorised fp64 form, idempotence on
values already on the grid, lossless MX->NV remap, and dequant closed forms."""
from fractions import Fraction

import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import quant as Q
from conftest import read_records, parse_float


def _bits(vals):
    v = np.array([parse_float(s) for s in vals], dtype=np.float64)
    bits = F.fp32_to_bf16_bits_rne(v.astype(np.float32))
    # the fixtures only hold exactly representable bf16 values
    assert np.array_equal(F.bf16_bits_to_f64(bits), v) and np.array_equal(np.signbit(F.bf16_bits_to_f64(bits)), np.signbit(v))
    return bits


@pytest.mark.parametrize("rec", read_records("mx_worked_blocks.txt"), ids=lambda r: r["name"])
def test_mx_worked_blocks(rec):
    bits = _bits(rec["x"])
    codes, scale = Q.mx_block_exact([int(b) for b in bits])
    assert scale == int(rec["scale"][0])
    assert codes == [int(c) for c in rec["codes"]]
    vc, vs = Q.mx_quantize(bits[None, :])
    assert vs[0, 0] == int(rec["scale"][0])
    assert list(Q.unpack_nibbles(vc)[0]) == [int(c) for c in rec["codes"]]


@pytest.mark.parametrize("rec", read_records("nv_worked_groups.txt"), ids=lambda r: r["name"])
def test_nv_worked_groups(rec):
    bits = _bits(rec["x"])
    st = float(rec["st"][0])
    codes, sg = Q.nv_group_exact([int(b) for b in bits], Fraction(st))
    assert sg == int(rec["scale"][0])
    assert codes == [int(c) for c in rec["codes"]]
    vc, vs, vst = Q.nv_quantize(bits[None, :], s_t=st)
    assert vs[0, 0] == int(rec["scale"][0]) and vst == np.float32(st)
    assert list(Q.unpack_nibbles(vc)[0]) == [int(c) for c in rec["codes"]]


def _crafted_rows(rng, K):
    """Rows that stress the rules: exact ties, zero blocks, -0.0, bf16
    subnormals, huge values, clamped exponents, saturating elements."""
    rows = []
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 4.0])
    for scale in (1.0, 2.0 ** -20, 2.0 ** 30, 2.0 ** -126, 2.0 ** -133):
        r = rng.choice(ties, K) * scale * rng.choice([-1, 1], K)
        rows.append(r)
    rows.append(np.zeros(K))
    z = np.zeros(K); z[::3] = -0.0; rows.append(-z)
    rows.append(rng.standard_normal(K) * 2.0 ** -128)
    rows.append(rng.standard_normal(K) * 1e30)
    rows.append(rng.standard_t(3, K) * 0.02)
    return np.array(rows)


def _to_bits(x64):
    return W.bf16_bits(W.to_bf16(x64))


def test_mx_exact_vs_vectorised():
    rng = np.random.default_rng(20)
    x = np.concatenate([_crafted_rows(rng, 128), rng.standard_normal((6, 128)) * 10.0 ** rng.integers(-5, 5, (6, 1))])
    bits = _to_bits(x)
    c1, s1 = Q.mx_quantize_exact(bits)
    c2, s2 = Q.mx_quantize(bits)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def test_nv_exact_vs_vectorised():
    rng = np.random.default_rng(21)
    x = np.concatenate([_crafted_rows(rng, 64), rng.standard_normal((6, 64)) * 10.0 ** rng.integers(-3, 3, (6, 1))])
    bits = _to_bits(x)
    for st in (None, 1.0 / 64, 0.0123, 3.0e-5):
        c1, s1, t1 = Q.nv_quantize_exact(bits, st)
        c2, s2, t2 = Q.nv_quantize(bits, st)
        assert t1 == t2
        assert np.array_equal(s1, s2) and np.array_equal(c1, c2), st


def test_nv_tensor_scale_exact():
    rng = np.random.default_rng(22)
    for _ in range(500):
        b = _to_bits(rng.standard_normal((1, 16)) * 10.0 ** rng.integers(-30, 30))
        amax = max(abs(F.bf16_bits_to_fraction(int(v))) for v in b.ravel())
        assert float(Q.nv_tensor_scale_exact(amax)) == float(Q.nv_tensor_scale(b))


def test_mx_scale_rule_closed_form():
    """amax / 2**E lies in [4, 8) for every block with a normal amax, so the
    block maximum codes to 4 or 6 (index 6 or 7)."""
    rng = np.random.default_rng(23)
    bits = _to_bits(rng.standard_t(3, (64, 256)) * 0.02)
    c, s = Q.mx_quantize(bits)
    x = F.bf16_bits_to_f64(bits).reshape(64, 8, 32)
    amax = np.abs(x).max(-1)
    r = amax / np.ldexp(1.0, s.astype(np.int64) - 127)
    assert np.all((r >= 4) & (r < 8))
    c4 = Q.unpack_nibbles(c).reshape(64, 8, 32) & 7
    assert np.all(c4.max(-1) >= 6)


def test_mx_idempotent_on_grid():
    for wl in (W.workload1(), W.random_linear(24, 64, 96, 512, outlier_p=0.01)):
        for t in (wl.A, wl.W):
            bits = W.bf16_bits(t)
            c, s = Q.mx_quantize(bits)
            back = Q.dequant_bf16_bits("mx", c, s)
            c2, s2 = Q.mx_quantize(back)
            assert np.array_equal(c, c2) and np.array_equal(s, s2)


def test_nv_idempotent_on_grid_fixed_st():
    """With s_t a power of two the dequantized values MAG*s_g*s_t (<= 6 bits) are
    exact bf16 values, and for groups whose s_g is an E4M3 normal (relative
    rounding error <= 1/16) the group maximum codes to 6, so re-quantizing with
    the same s_t returns the same s_g and codes."""
    wl = W.random_linear(25, 64, 96, 512, outlier_p=0.01)
    for t in (wl.A, wl.W):
        bits = W.bf16_bits(t)
        st_dyn = float(Q.nv_tensor_scale(bits))
        st = np.float32(2.0 ** np.floor(np.log2(st_dyn)))
        c, s, _ = Q.nv_quantize(bits, s_t=st)
        back = Q.dequant_bf16_bits("nv", c, s, st)
        assert np.array_equal(F.bf16_bits_to_f64(back), Q.nv_dequant_exact_f64(c, s, st))
        c2, s2, _ = Q.nv_quantize(back, s_t=st)
        normal = s >= 8
        R = bits.shape[0]
        c4a = Q.unpack_nibbles(c).reshape(R, -1, 16)
        c4b = Q.unpack_nibbles(c2).reshape(R, -1, 16)
        assert normal.mean() > 0.9
        assert np.array_equal(c4a[normal], c4b[normal])
        assert np.array_equal(s[normal], s2[normal])


def test_dequant_mx_closed_form():
    codes = Q.pack_nibbles(np.array([[7, 15, 1, 9] + [0] * 28], np.uint8))
    scales = np.array([[130]], np.uint8)               # 2**3
    v = Q.dequant_fp32("mx", codes, scales)
    assert list(v[0, :4]) == [48.0, -48.0, 4.0, -4.0]
    b = Q.dequant_bf16_bits("mx", codes, scales)
    assert list(F.bf16_bits_to_f64(b[0, :4])) == [48.0, -48.0, 4.0, -4.0]


def test_dequant_nv_single_rounding():
    codes = Q.pack_nibbles(np.array([[5] * 16], np.uint8))          # magnitude 3
    scales = np.array([[0x53]], np.uint8)                            # 11
    st = np.float32(1 / 3)                                           # fp32 1/3 (24 bits)
    v = Q.dequant_fp32("nv", codes, scales, st)
    exact = Fraction(3) * 11 * Fraction(float(st))
    assert Fraction(float(v[0, 0])) == F.round_fp32(exact)
    b = Q.dequant_bf16_bits("nv", codes, scales, st)
    assert F.bf16_bits_to_fraction(int(b[0, 0])) == F.round_bf16(F.round_fp32(exact))


def test_remap_lossless_on_workload2():
    wl = W.workload2()
    for t in (wl.W, wl.A):
        bits = W.bf16_bits(t)
        c, s = Q.mx_quantize(bits)
        sg, st, n_inexact = Q.remap_mx_to_nv(c, s)
        assert n_inexact == 0
        assert np.array_equal(Q.dequant_fp32("nv", c, sg, st).view(np.uint32),
                              Q.dequant_fp32("mx", c, s).view(np.uint32))


def test_remap_exact_vs_vectorised_and_inexact_blocks():
    rng = np.random.default_rng(26)
    bits = _to_bits(rng.standard_normal((4, 256)))
    c, s = Q.mx_quantize(bits)
    s = s.copy()
    s[0, 0] = 127 + 10           # E_max = 10 -> k = 2
    s[1, 1] = 127 + 10 - 17      # j = -9: smallest exact power (E4M3 subnormal 2**-9)
    s[1, 2] = 127 + 10 - 18      # j = -10: ties to 0 -> inexact (codes nonzero)
    s[2, 3] = 127 + 10 - 30      # far below -> inexact
    c4 = Q.unpack_nibbles(c)
    c4[3, 4 * 32:5 * 32] &= 8     # block (3, 4): all-zero codes
    s[3, 4] = 0                   # ... with a tiny exponent: stays exact
    c = Q.pack_nibbles(c4)
    sg1, st1, n1 = Q.remap_mx_to_nv(c, s)
    sg2, st2, n2 = Q.remap_mx_to_nv_exact(c, s)
    assert n1 == n2 == 2
    assert st1 == st2 == np.float32(4.0)
    assert np.array_equal(sg1, sg2)
    assert sg1[1, 2] == 1 and sg1[1, 4] == 0 and sg1[0, 0] == F.e4m3_encode(Fraction(256))
    ok = np.ones_like(s, bool); ok[1, 2] = ok[2, 3] = False
    dn = Q.dequant_fp32("nv", c, sg1, st1).reshape(4, 8, 32)
    dm = Q.dequant_fp32("mx", c, s).reshape(4, 8, 32)
    assert np.array_equal(dn[ok], dm[ok])
    assert not np.array_equal(dn[~ok], dm[~ok])


def test_pack_unpack_roundtrip_and_order():
    c4 = np.arange(16, dtype=np.uint8)[None, :]
    p = Q.pack_nibbles(c4)
    assert list(p[0]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert np.array_equal(Q.unpack_nibbles(p), c4)
