"""Pins of the GEMM and MoE oracles: exact Fraction brute force, an integer
matmul special case, the tolerance bracket, and MoE invariants (single-expert
dense chain, identical experts, token permutation, brute-force gate/up)."""
from fractions import Fraction

import numpy as np
import scipy.special
import torch
import pytest

import workloads as W
from oracle import formats as F
from oracle import gemm as G
from oracle import moe as M
from oracle import quant as Q


def test_gemm_fraction_brute_force_mx_workload1():
    wl = W.workload1()
    ac, as_ = Q.mx_quantize(W.bf16_bits(wl.A))
    bc, bs = Q.mx_quantize(W.bf16_bits(wl.W))
    rows, cols = slice(0, 6), slice(100, 112)
    C, S = G.gemm_ref("mx", ac, as_, bc, bs)
    ex = G.gemm_exact_fraction("mx", ac[rows], as_[rows], bc[cols], bs[cols])
    for i in range(6):
        for j in range(12):
            assert Fraction(C[i, 100 + j]) == ex[i][j]      # fp64 sum is exact here
    assert np.all(S >= np.abs(C))


def test_gemm_fraction_brute_force_nv():
    wl = W.random_linear(30, 5, 7, 64)
    ac, as_, ast = Q.nv_quantize(W.bf16_bits(wl.A))
    bc, bs, bst = Q.nv_quantize(W.bf16_bits(wl.W))
    C, S = G.gemm_ref("nv", ac, as_, bc, bs, ast, bst)
    ex = G.gemm_exact_fraction("nv", ac, as_, bc, bs, ast, bst)
    for i in range(5):
        for j in range(7):
            # one rounding (fp64) of the exact value after the tensor-scale product
            assert abs(Fraction(C[i, j]) - ex[i][j]) <= abs(ex[i][j]) * Fraction(1, 2 ** 51)


def test_gemm_integer_special_case_non_square():
    """Scale byte 127 (2**0) everywhere: values are the table magnitudes, so
    4*C is the integer matmul of doubled magnitudes.  M != N != K catches a
    transposed operand."""
    rng = np.random.default_rng(31)
    M_, N_, K_ = 24, 40, 96
    ca = rng.integers(0, 16, (M_, K_), dtype=np.uint8)
    cb = rng.integers(0, 16, (N_, K_), dtype=np.uint8)
    sa = np.full((M_, K_ // 32), 127, np.uint8)
    sb = np.full((N_, K_ // 32), 127, np.uint8)
    C, _ = G.gemm_ref("mx", Q.pack_nibbles(ca), sa, Q.pack_nibbles(cb), sb)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)
    ia = np.where(ca & 8, -1, 1) * twice[ca & 7]
    ib = np.where(cb & 8, -1, 1) * twice[cb & 7]
    assert np.array_equal((4 * C).astype(np.int64), ia @ ib.T)
    assert np.all(4 * C == np.round(4 * C))


def test_gemm_block_scale_placement():
    """One nonzero block per row: C picks up exactly that block's two scales."""
    K_ = 128
    ca = np.zeros((2, K_), np.uint8); cb = np.zeros((3, K_), np.uint8)
    ca[0, 32:64] = 2; ca[1, 96:128] = 4                   # values 1 and 2
    cb[:, 32:64] = 2; cb[2, 96:128] = 6                   # values 1 and 4
    sa = np.full((2, 4), 127, np.uint8); sa[0, 1] = 130; sa[1, 3] = 120
    sb = np.full((3, 4), 127, np.uint8); sb[1, 1] = 125; sb[2, 3] = 131
    C, _ = G.gemm_ref("mx", Q.pack_nibbles(ca), sa, Q.pack_nibbles(cb), sb)
    assert C[0, 0] == 32 * 8 and C[0, 1] == 32 * 8 / 4 and C[0, 2] == 32 * 8
    assert C[1, 0] == 0 and C[1, 2] == 32 * 2 * 4 * 2.0 ** (-7 + 4)


def test_tolerance_brackets():
    Cref = np.array([[1.0, 3.0e-3, -7.5]])
    S = np.array([[10.0, 1.0, 100.0]])
    exact_bits = F.bf16_rne_of_f64(Cref)
    assert G.within_tol_bf16(exact_bits, Cref, S).all()
    far = F.bf16_rne_of_f64(Cref + 1e-3 * S)
    assert not G.within_tol_bf16(far, Cref, S).any()
    assert G.within_tol_f32(Cref.astype(np.float32), Cref, S).all()
    assert not G.within_tol_f32((Cref + 2e-5 * S).astype(np.float32), Cref, S).any()


# ------------------------------------------------------------------ MoE
def _experts(num_e, hidden, inter, fmt, seed=40, same=False):
    w13c, w13s, w2c, w2s, st13, st2 = [], [], [], [], [], []
    for e in range(num_e):
        a, b = W.expert_weights(seed, 0 if same else e, hidden, inter)
        ab, bb = W.bf16_bits(a), W.bf16_bits(b)
        if fmt == "mx":
            c1, s1 = Q.mx_quantize(ab); c2, s2 = Q.mx_quantize(bb); t1 = t2 = None
        else:
            c1, s1, t1 = Q.nv_quantize(ab); c2, s2, t2 = Q.nv_quantize(bb)
        w13c.append(c1); w13s.append(s1); w2c.append(c2); w2s.append(s2); st13.append(t1); st2.append(t2)
    st = (np.array(st13, np.float32), np.array(st2, np.float32)) if fmt == "nv" else (None, None)
    return np.stack(w13c), np.stack(w13s), np.stack(w2c), np.stack(w2s), st[0], st[1]


def _act_st(fmt, xbits):
    return (Q.nv_tensor_scale(xbits), np.float32(0.01)) if fmt == "nv" else (None, None)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_moe_single_expert_is_dense_chain(fmt):
    T, H, I, E = 8, 64, 96, 3
    m = W.small_moe(41, T, H, I, E, 1)
    ids = np.zeros((T, 1), np.int32)
    wts = np.ones((T, 1), np.float32)
    w13c, w13s, w2c, w2s, st13, st2 = _experts(E, H, I, fmt)
    xb = W.bf16_bits(m.X)
    act = _act_st(fmt, xb)
    r = M.moe_forward(fmt, xb, ids, wts, w13c, w13s, w2c, w2s, st13, st2, act)
    # dense chain through the GEMM oracle
    if fmt == "mx":
        xc, xs = Q.mx_quantize(xb); xst = None
    else:
        xc, xs, xst = Q.nv_quantize(xb, s_t=act[0])
    gu, _ = G.gemm_ref(fmt, xc, xs, w13c[0], w13s[0], xst, None if st13 is None else st13[0])
    h = M.silu_mul_bf16(gu[:, :I], gu[:, I:])
    if fmt == "mx":
        hc, hs = Q.mx_quantize(h); hst = None
    else:
        hc, hs, hst = Q.nv_quantize(h, s_t=act[1])
    y, _ = G.gemm_ref(fmt, hc, hs, w2c[0], w2s[0], hst, None if st2 is None else st2[0])
    assert np.array_equal(r["h_bits"][:, 0], h)
    assert np.allclose(r["out_f64"], y, rtol=0, atol=0)
    assert np.array_equal(r["out_bits"], F.bf16_rne_of_f64(y))


def test_moe_identical_experts_independent_of_routing():
    T, H, I, E, k = 10, 64, 64, 5, 2
    m = W.small_moe(42, T, H, I, E, k)
    w13c, w13s, w2c, w2s, _, _ = _experts(E, H, I, "mx", same=True)
    xb = W.bf16_bits(m.X)
    r1 = M.moe_forward("mx", xb, m.ids, m.weights, w13c, w13s, w2c, w2s)
    ids2 = (m.ids + 1) % E
    r2 = M.moe_forward("mx", xb, ids2, m.weights, w13c, w13s, w2c, w2s)
    assert np.array_equal(r1["out_f64"], r2["out_f64"])
    # and weights summing to one over identical slots give back the single-slot y
    assert np.allclose(r1["out_f64"], r1["y"][:, 0] * m.weights.astype(np.float64).sum(1, keepdims=True), rtol=1e-12, atol=1e-30)


def test_moe_token_permutation_equivariant():
    T, H, I, E, k = 12, 64, 32, 6, 3
    m = W.small_moe(43, T, H, I, E, k)
    w13c, w13s, w2c, w2s, _, _ = _experts(E, H, I, "mx")
    xb = W.bf16_bits(m.X)
    r = M.moe_forward("mx", xb, m.ids, m.weights, w13c, w13s, w2c, w2s)
    p = np.random.default_rng(0).permutation(T)
    rp = M.moe_forward("mx", xb[p], m.ids[p], m.weights[p], w13c, w13s, w2c, w2s)
    assert np.array_equal(rp["out_bits"], r["out_bits"][p])
    # a token subset gives the same rows as the full run
    rs = M.moe_forward("mx", xb, m.ids, m.weights, w13c, w13s, w2c, w2s, tokens=np.array([3, 7]))
    assert np.array_equal(rs["out_bits"], r["out_bits"][[3, 7]])


def test_moe_gate_up_brute_force_fraction():
    """Tiny case: g and u from exact rational dot products of the block-scaled
    values, independent of the fp64 matmul."""
    T, H, I, E, k = 4, 64, 32, 4, 2
    m = W.small_moe(44, T, H, I, E, k)
    w13c, w13s, w2c, w2s, _, _ = _experts(E, H, I, "mx")
    xb = W.bf16_bits(m.X)
    r = M.moe_forward("mx", xb, m.ids, m.weights, w13c, w13s, w2c, w2s)
    xc, xs = Q.mx_quantize(xb)
    for t in range(T):
        for j in range(k):
            e = int(m.ids[t, j])
            ex = G.gemm_exact_fraction("mx", xc[t:t + 1], xs[t:t + 1], w13c[e], w13s[e])[0]
            assert [Fraction(v) for v in r["g"][t, j]] == ex[:I]
            assert [Fraction(v) for v in r["u"][t, j]] == ex[I:]


def test_silu_mul_reference_values():
    g = np.array([0.0, 1.0, -1.0, 20.0, -800.0])
    u = np.array([3.0, 2.0, 2.0, 1.0, 1.0])
    h = F.bf16_bits_to_f64(M.silu_mul_bf16(g, u))
    expect = [0.0, 2 / (1 + np.exp(-1.0)), -2 / (1 + np.e), 20 / (1 + np.exp(-20.0)), -0.0]
    for a, b in zip(h, expect):
        assert F.bf16_bits_to_fraction(int(F.bf16_rne_of_f64(np.array([b]))[0])) == Fraction(a)


def _silu_mul_expit_bf16(g, u):
    """SiLU(g)*u from scipy's logistic function z*expit(z) (fp64), rounded to bf16
    by torch's own float64 -> bfloat16 cast: no code shared with the oracle."""
    h = g * scipy.special.expit(g) * u
    return torch.from_numpy(h).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_silu_mul_against_scipy_expit():
    """h = bf16(SiLU(g) u) against an independent evaluation, z*expit(z), over a
    sweep of g that spans saturation on both sides (|g| up to 1e4, past the
    fp64 overflow of exp(-g) at g < -709) and a spread of u."""
    rng = np.random.default_rng(51)
    g = np.concatenate([np.linspace(-40, 40, 4001), -np.logspace(-3, 4, 800), np.logspace(-3, 4, 800),
                        rng.standard_normal(20000) * 3, [-700.0, -709.5, -745.0, -750.0, 709.5, 1e4]])
    u = rng.choice([-7.0, -1.0, 0.37, 1.0, 2.5, 1e3], g.size) * rng.uniform(0.5, 2.0, g.size)
    got = M.silu_mul_bf16(g, u)
    exp = _silu_mul_expit_bf16(g, u)
    assert np.array_equal(got, exp)


def test_silu_closed_forms():
    """Closed forms of SiLU(z) = z*sigmoid(z) through the oracle's h with u = 1:
    SiLU(0) = 0; SiLU(z) rounds to z for large z and to zero for very negative
    z; 0 < SiLU(z) <= z for z > 0 (after rounding); and SiLU(z) - SiLU(-z) = z (sigmoid(z) +
    sigmoid(-z) = 1), up to the two bf16 roundings."""
    one = lambda z: np.ones_like(z)
    assert M.silu_mul_bf16(np.array([0.0]), np.array([5.0]))[0] & 0x7FFF == 0
    big = np.array([40.0, 100.0, 1000.0])
    assert np.array_equal(M.silu_mul_bf16(big, one(big)), F.bf16_rne_of_f64(big))
    neg = np.array([-200.0, -1000.0, -1e5])
    assert np.all((M.silu_mul_bf16(neg, one(neg)) & 0x7FFF) == 0)
    z = np.array([0.5, 1.0, 2.0, 3.0, 8.0])
    hp = F.bf16_bits_to_f64(M.silu_mul_bf16(z, one(z)))
    assert np.all(hp <= z) and np.all(hp > 0)
    zz = np.array([-3.0, -0.75, 0.125, 1.5, 6.0])
    d = F.bf16_bits_to_f64(M.silu_mul_bf16(zz, one(zz))) - F.bf16_bits_to_f64(M.silu_mul_bf16(-zz, one(zz)))
    assert np.all(np.abs(d - zz) <= 2.0 ** -8 * 2 * np.abs(zz))


def test_routing_metadata_brute_force():
    m = W.small_moe(45, 50, 16, 16, 9, 3)
    counts, offsets, perm = M.routing_metadata(m.ids, 9)
    assert counts.sum() == 150 and offsets[-1] == 150
    slots = []
    for e in range(9):
        for s in range(150):
            if m.ids.ravel()[s] == e:
                slots.append(s)
    assert list(perm) == slots
    for e in range(9):
        assert counts[e] == (m.ids == e).sum()
        assert offsets[e + 1] - offsets[e] == counts[e]
