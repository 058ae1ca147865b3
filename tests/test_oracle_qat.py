"""Pins of the oracle's QAT fake-quant node and straight-through backward:
the hand-worked MX blocks' codes times the page's E2M1 table, the fixed point
of MX fake quantization, its error bound, NV values already on the grid, and
the STE update against numpy's IEEE float32 addition."""
import numpy as np
import pytest

import workloads as W
from oracle import formats as F
from oracle import quant as Q
from conftest import GOLDEN, parse_float, read_records


def _e2m1_table():
    vals = {}
    with open(f"{GOLDEN}/e2m1_table.txt") as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return vals


@pytest.mark.parametrize("rec", read_records("mx_worked_blocks.txt"), ids=lambda r: r["name"])
def test_fake_quant_mx_worked_blocks(rec):
    """fake_quant = table[code] * 2**(scale - 127) with the fixture's own codes and scale."""
    tab = _e2m1_table()
    x = np.array([parse_float(v) for v in rec["x"]])
    bits = F.fp32_to_bf16_bits_rne(x.astype(np.float32))
    scale = int(rec["scale"][0])
    expect = np.array([tab[int(c)] for c in rec["codes"]]) * 2.0 ** (scale - 127)
    got = Q.fake_quant_fp32("mx", bits[None, :])[0]
    assert np.array_equal(got.astype(np.float64), expect)
    assert np.array_equal(np.signbit(got), np.signbit(expect))


def _bits(seed, R, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, (R, K)) * np.exp2(rng.integers(-30, 30, size=(R, 1)))
    x[rng.random((R, K)) < 0.01] *= 500.0
    return F.fp32_to_bf16_bits_rne(x.astype(np.float32))


def test_fake_quant_mx_fixed_point():
    """An MX block's largest code is 4 or 6, so the dequantized block has the
    same exponent and quantizes to itself."""
    bits = _bits(1, 16, 512)
    once = Q.fake_quant_bf16_bits("mx", bits)
    assert np.array_equal(Q.fake_quant_bf16_bits("mx", once), once)


def test_fake_quant_mx_error_bound():
    """|x - fq(x)| <= 2**E (half the widest E2M1 spacing at the block scale),
    and < 2**(E+1) for saturated values (scaled |x| in (6, 8))."""
    bits = _bits(2, 16, 512)
    x = F.bf16_bits_to_f64(bits)
    fq = Q.fake_quant_fp32("mx", bits).astype(np.float64)
    _, scales = Q.mx_quantize(bits)
    E = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    err = np.abs(x - fq)
    sat = np.abs(x) * np.ldexp(1.0, -E) > 6
    assert (err[~sat] <= np.ldexp(1.0, E[~sat])).all()
    assert (err[sat] < np.ldexp(1.0, E[sat] + 1)).all() and sat.any()


def test_fake_quant_nv_on_grid_values_unchanged():
    """x = code * s_g * s_t with the group max at code 6 and s_g an E4M3 value:
    the fake-quantized tensor is x itself (s_t supplied)."""
    rng = np.random.default_rng(3)
    st = 2.0 ** -7
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    e4m3 = np.array([F.e4m3_decode(b) for b in range(1, 0x7F)])
    sg = rng.choice(e4m3[(e4m3 >= 2.0 ** -6) & (e4m3 <= 64)], (8, 32))
    codes = rng.choice(mags, (8, 32, 16)) * rng.choice([-1, 1], (8, 32, 16))
    codes[:, :, 0] = 6.0
    x = (codes * sg[..., None] * st).reshape(8, 512)
    bits = F.fp32_to_bf16_bits_rne(x.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(bits), x)            # on the bf16 grid
    assert np.array_equal(Q.fake_quant_fp32("nv", bits, st).astype(np.float64), x)


def test_fake_quant_nv_is_quantize_then_dequantize_of_workload():
    """Against the two entry-point definitions it fuses (computed s_t)."""
    bits = W.bf16_bits(W.workload1().W)
    c, s, st = Q.nv_quantize(bits)
    assert np.array_equal(Q.fake_quant_bf16_bits("nv", bits), Q.dequant_bf16_bits("nv", c, s, st))


def test_ste_backward_against_float32_addition():
    rng = np.random.default_rng(4)
    g = (rng.standard_normal((64, 96)) * 1e-3).astype(np.float32)
    m = rng.standard_normal((64, 96)).astype(np.float32)
    assert np.array_equal(Q.ste_backward(g), g)
    assert np.array_equal(Q.ste_backward(g, m), m + g)             # numpy: IEEE fp32 add, RNE
    gb = F.bf16_bits_to_f64(F.fp32_to_bf16_bits_rne(g))
    assert np.array_equal(Q.ste_backward(gb, m), m + gb.astype(np.float32))
