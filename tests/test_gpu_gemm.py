"""GPU parity of the W4A4 GEMM against the oracle: every output element within
|C - C_ref| <= 1e-5 * sum_k |a b| (bf16 output: inside the rounded bracket)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W
from oracle import gemm as G
from oracle import quant as Q
from gpu_util import DEV, chunked, dev_bf16, quantize_mx, quantize_nv

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _run_gemm(fmt, a, b, dtype, st=(None, None)):
    m, n = a[0].shape[0], b[0].shape[0]
    c = torch.empty((m, n), dtype=dtype, device=DEV)
    F.fp4_gemm(F.FMT_MX if fmt == "mx" else F.FMT_NV, a[0], a[1], b[0], b[1], c, st[0], st[1])
    torch.cuda.synchronize()
    return c


def _assert_within(c, Cref, S, rows=None, cols=None):
    got = c if rows is None else c[rows][:, cols]
    if got.dtype == torch.float32:
        ok = G.within_tol_f32(got.cpu().numpy(), Cref, S, TOL)
    else:
        ok = G.within_tol_bf16(W.bf16_bits(got), Cref, S, TOL)
    if not ok.all():
        bad = np.argwhere(~ok)[:8]
        g = got.float().cpu().numpy()
        msg = "\n".join(f"  {tuple(i)}: got {g[tuple(i)]!r} ref {Cref[tuple(i)]!r} S {S[tuple(i)]!r}" for i in bad)
        raise AssertionError(f"{(~ok).sum()} of {ok.size} outside tolerance\n{msg}")


def _mx_case(wl, dtype):
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    a = quantize_mx(dev_bf16(ab))
    b = quantize_mx(dev_bf16(wb))
    c = _run_gemm("mx", a, b, dtype)
    ea, eb = Q.mx_quantize(ab), Q.mx_quantize(wb)
    Cref, S = G.gemm_ref("mx", *ea, *eb)
    _assert_within(c, Cref, S)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gemm_mx_workload1(dtype):
    _mx_case(W.workload1(), dtype)


@pytest.mark.parametrize("m,n,k", [(1, 1, 32), (37, 75, 96), (130, 260, 160), (16, 512, 4096), (300, 200, 544)])
def test_gemm_mx_ragged(m, n, k):
    _mx_case(W.random_linear(m * 1000 + n + k, m, n, k, outlier_p=0.01), torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pad", [0, 4, 16])
def test_gemm_mx_tiled_ragged_strided(dtype, pad):
    """K a multiple of 512 and at least 64 tiles: the 256x256 LDS-staged tile,
    with ragged M and N, both output types and a padded output row pitch (pad 4
    leaves bf16 rows off 16-byte alignment, which takes the scalar stores)."""
    m, n, k = 2000, 2100, 1024
    wl = W.random_linear(4242 + pad, m, n, k, outlier_p=0.01)
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    a = quantize_mx(dev_bf16(ab))
    b = quantize_mx(dev_bf16(wb))
    buf = torch.full((m, n + pad), float("nan"), dtype=dtype, device=DEV)
    c = buf[:, :n]
    F.fp4_gemm(F.FMT_MX, a[0], a[1], b[0], b[1], c)
    torch.cuda.synchronize()
    Cref, S = G.gemm_ref("mx", *Q.mx_quantize(ab), *Q.mx_quantize(wb))
    _assert_within(c, Cref, S)
    if pad:
        assert torch.isnan(buf[:, n:].float()).all()    # the padding is never written


def test_gemm_mx_workload3_full_sampled():
    """Workload 3 (4096^3) at full size, in the launch the bench times; every
    output of 48 sampled rows and 48 sampled columns is checked."""
    wl = W.workload3()
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    a = quantize_mx(dev_bf16(ab))
    b = quantize_mx(dev_bf16(wb))
    c = _run_gemm("mx", a, b, torch.bfloat16)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(4096, 48, replace=False))
    cols = np.sort(rng.choice(4096, 48, replace=False))
    ea = Q.mx_quantize(ab[rows])
    eb = chunked(Q.mx_quantize, wb)
    Cref, S = G.gemm_ref("mx", *ea, *eb)
    _assert_within(c[rows], Cref, S)
    Cref2, S2 = G.gemm_ref("mx", *chunked(Q.mx_quantize, ab), eb[0][cols], eb[1][cols])
    _assert_within(c[:, cols], Cref2, S2)


def test_gemm_mx_deterministic():
    wl = W.random_linear(77, 256, 384, 1024)
    a = quantize_mx(dev_bf16(W.bf16_bits(wl.A)))
    b = quantize_mx(dev_bf16(W.bf16_bits(wl.W)))
    c1 = _run_gemm("mx", a, b, torch.float32)
    c2 = _run_gemm("mx", a, b, torch.float32)
    assert torch.equal(c1, c2)


def _nv_case(wl, dtype):
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    ac, as_, ats = quantize_nv(dev_bf16(ab))
    bc, bs, bts = quantize_nv(dev_bf16(wb))
    c = _run_gemm("nv", (ac, as_), (bc, bs), dtype, (ats, bts))
    ea, eb = Q.nv_quantize(ab), Q.nv_quantize(wb)
    Cref, S = G.gemm_ref("nv", ea[0], ea[1], eb[0], eb[1], ea[2], eb[2])
    _assert_within(c, Cref, S)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gemm_nv_small(dtype):
    _nv_case(W.random_linear(91, 64, 96, 512, outlier_p=0.01), dtype)


@pytest.mark.parametrize("m,n,k", [(1, 3, 16), (37, 75, 112), (130, 260, 4096)])
def test_gemm_nv_ragged(m, n, k):
    _nv_case(W.random_linear(m * 7 + n + k, m, n, k), torch.float32)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pad", [0, 4])
def test_gemm_nv_tiled_ragged_strided(dtype, pad):
    """K a multiple of 128 and at least 16 tiles: the 128x512 wide NV tile (both
    operands staged as NVFP4 codes, A expanded to fp16 in LDS one step ahead, B
    expanded in registers), ragged M and N (24 tiles here), both output types
    and a padded output row pitch."""
    m, n, k = 1000, 1100, 1024
    wl = W.random_linear(5151 + pad, m, n, k, outlier_p=0.01)
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    ac, as_, ats = quantize_nv(dev_bf16(ab))
    bc, bs, bts = quantize_nv(dev_bf16(wb))
    buf = torch.full((m, n + pad), float("nan"), dtype=dtype, device=DEV)
    c = buf[:, :n]
    F.fp4_gemm(F.FMT_NV, ac, as_, bc, bs, c, ats, bts)
    torch.cuda.synchronize()
    ea, eb = Q.nv_quantize(ab), Q.nv_quantize(wb)
    Cref, S = G.gemm_ref("nv", ea[0], ea[1], eb[0], eb[1], ea[2], eb[2])
    _assert_within(c, Cref, S)
    if pad:
        assert torch.isnan(buf[:, n:].float()).all()


@pytest.mark.parametrize("m,n,k", [(700, 1500, 128), (640, 2048, 384), (2000, 520, 256)])
def test_gemm_nv_tiled_short_k(m, n, k):
    """The tiled NV path with one, two and three K steps (the three-stage copy
    ring before it is full) and N tails of 476 and 8 columns."""
    _nv_case(W.random_linear(m + n + k, m, n, k, outlier_p=0.01), torch.float32)


@pytest.mark.parametrize("r", [16, 29, 48, 61, 80, 93, 112])
def test_gemm_nv_tiled_last_tile_fragments(r):
    """The tiled NV path whose last row tile holds 1 to 7 row fragments of 16
    (its K loop is instantiated per fragment count, odd counts with half a
    fragment pair), some with a ragged last fragment; 16 tiles, three K steps."""
    m, n, k = 128 + r, 4096, 384
    _nv_case(W.random_linear(7000 + r, m, n, k, outlier_p=0.01), torch.float32)


def test_gemm_nv_4096_sampled():
    """NVFP4 GEMM at 4096^3 (the tiled path): every output of 32 sampled rows
    and 32 sampled columns within the bound."""
    wl = W.workload3()
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    ac, as_, ats = quantize_nv(dev_bf16(ab))
    bc, bs, bts = quantize_nv(dev_bf16(wb))
    c = _run_gemm("nv", (ac, as_), (bc, bs), torch.bfloat16, (ats, bts))
    rng = np.random.default_rng(4)
    rows = np.sort(rng.choice(4096, 32, replace=False))
    cols = np.sort(rng.choice(4096, 32, replace=False))
    sa, sb = Q.nv_tensor_scale(ab), Q.nv_tensor_scale(wb)
    ea = Q.nv_quantize(ab[rows], s_t=sa)
    eb = chunked(Q.nv_quantize, wb, s_t=sb)
    Cref, S = G.gemm_ref("nv", ea[0], ea[1], eb[0], eb[1], sa, sb)
    _assert_within(c[rows], Cref, S)
    ea2 = chunked(Q.nv_quantize, ab, s_t=sa)
    Cref2, S2 = G.gemm_ref("nv", ea2[0], ea2[1], eb[0][cols], eb[1][cols], sa, sb)
    _assert_within(c[:, cols], Cref2, S2)


@pytest.mark.parametrize("m,n,k,dtype,pad", [(1, 4096, 128, torch.float32, 0), (5, 4097, 384, torch.float32, 3),
                                             (64, 8200, 512, torch.bfloat16, 0), (100, 5000, 256, torch.bfloat16, 5),
                                             (128, 4160, 1024, torch.float32, 0), (33, 6000, 7168, torch.float32, 0)])
def test_gemm_mx_skinny_streaming(m, n, k, dtype, pad):
    """Few A rows against at least 4096 B rows: up to 64 A rows (k % 128 == 0)
    take the streaming kernel (one pass over B), 100 and 128 rows the fallback
    kernel (fewer than 64 tiles of 256 x 256); ragged m and n, both output
    types and an output pitch that forces the element-wise stores."""
    wl = W.random_linear(m * 7 + n + k, m, n, k, outlier_p=0.01)
    ab, wb = W.bf16_bits(wl.A), W.bf16_bits(wl.W)
    a = quantize_mx(dev_bf16(ab))
    b = quantize_mx(dev_bf16(wb))
    buf = torch.full((m, n + pad), float("nan"), dtype=dtype, device=DEV)
    c = buf[:, :n]
    F.fp4_gemm(F.FMT_MX, a[0], a[1], b[0], b[1], c)
    torch.cuda.synchronize()
    Cref, S = G.gemm_ref("mx", *Q.mx_quantize(ab), *chunked(Q.mx_quantize, wb))
    _assert_within(c, Cref, S)
    if pad:
        assert torch.isnan(buf[:, n:].float()).all()


# ---------------------------------------------------------------- crafted blocks
def _crafted_operands(seed, m, n, k, pairs, zero_p=0.1, sat_p=0.1, huge_zero_blocks=()):
    """MX operands written directly as codes and scale bytes.  K block b gets
    scale byte alpha_b in every A row and beta_b in every B row, cycling through
    `pairs`, so the two extremes of a pair (e.g. 254 with 0, 1 with 253) put a
    product's scale 2^(alpha + beta - 254) where the pair says while A's rows
    mix bytes 0, 1, 253 and 254.  Some blocks are all zero codes (signed zeros
    included), some saturated (every code +-6).  huge_zero_blocks: K blocks in
    which every A row holds only zero codes under byte 254 while B's rows hold
    nonzero codes under byte 254 (a scale product of 2^254 multiplying zeros)."""
    rng = np.random.default_rng(seed)
    nb = k // 32
    al = np.array([pairs[b % len(pairs)][0] for b in range(nb)], np.uint8)
    be = np.array([pairs[b % len(pairs)][1] for b in range(nb)], np.uint8)

    def side(rows, sc):
        c4 = rng.integers(0, 16, (rows, k), dtype=np.uint8)
        s = np.tile(sc, (rows, 1))
        blk = c4.reshape(rows, nb, 32)
        zero = rng.random((rows, nb)) < zero_p
        sat = (rng.random((rows, nb)) < sat_p) & ~zero
        blk[zero] = rng.choice(np.array([0, 8], np.uint8), (int(zero.sum()), 32))
        blk[sat] = rng.choice(np.array([7, 15], np.uint8), (int(sat.sum()), 32))
        return blk, s

    ab, as_ = side(m, al)
    bb, bs = side(n, be)
    for b in huge_zero_blocks:
        ab[:, b] = rng.choice(np.array([0, 8], np.uint8), (m, 32))
        bb[:, b] = rng.choice(np.array([1, 7, 9, 15], np.uint8), (n, 32))
        as_[:, b] = bs[:, b] = 254
    return (Q.pack_nibbles(ab.reshape(m, k)), as_), (Q.pack_nibbles(bb.reshape(n, k)), bs)


_PAIRS = [(254, 0), (0, 254), (253, 1), (1, 253), (254, 3), (0, 250), (127, 127), (200, 60), (30, 221)]
_SHAPES = [(37, 75, 288), (2048, 2048, 512), (48, 4096, 512)]     # fallback, 256x256 tile, skinny


def _crafted_case(a, b, dtype):
    at = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in a)
    bt = tuple(torch.from_numpy(np.ascontiguousarray(t)).to(DEV) for t in b)
    c = _run_gemm("mx", at, bt, dtype)
    Cref, S = G.gemm_ref("mx", *a, *b)
    return c, Cref, S


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("m,n,k", _SHAPES)
def test_gemm_mx_crafted_extreme_scale_bytes(m, n, k, dtype):
    """Scale bytes 0, 1, 253 and 254 mixed within each row (2^-127 is an fp32
    subnormal, 2^127 the largest power of two), zero and saturated blocks, on
    the fallback kernel, the 256x256 tile and the skinny kernel; every product
    lies in fp32's normal range, so the usual bar holds."""
    a, b = _crafted_operands(m + n + k, m, n, k, _PAIRS)
    c, Cref, S = _crafted_case(a, b, dtype)
    _assert_within(c, Cref, S)


def test_gemm_mx_crafted_brute_force_fraction():
    """A slice of the crafted case against exact Fraction dot products."""
    a, b = _crafted_operands(5, 37, 75, 288, _PAIRS)
    c, Cref, S = _crafted_case(a, b, torch.float32)
    ex = G.gemm_exact_fraction("mx", a[0][:4], a[1][:4], b[0][:6], b[1][:6])
    got = c.cpu().numpy()
    for i in range(4):
        for j in range(6):
            assert abs(float(got[i, j]) - float(ex[i][j])) <= TOL * S[i, j]


@pytest.mark.parametrize("m,n,k", _SHAPES)
def test_gemm_mx_zero_blocks_under_huge_scales(m, n, k):
    """K blocks where A holds only (signed) zero codes under byte 254 and B
    nonzero codes under byte 254: a scale product of 2^254, beyond fp32, times
    zeros contributes exactly zero (no inf * 0 reaches the accumulator)."""
    a, b = _crafted_operands(7 + m, m, n, k, [(120, 130), (127, 127)], zero_p=0.1, sat_p=0.05,
                             huge_zero_blocks=(0, 3, k // 32 - 1))
    c, Cref, S = _crafted_case(a, b, torch.float32)
    assert torch.isfinite(c).all()
    _assert_within(c, Cref, S)


@pytest.mark.parametrize("m,n,k", _SHAPES)
def test_gemm_mx_results_beyond_fp32_are_infinite(m, n, k):
    """Exact results beyond fp32's range come out as the infinity of their sign,
    as fp32 rounding defines (bf16 output likewise).  Every A row holds codes of
    one sign and every B code is positive, so partial sums never change sign
    (with mixed signs, a partial sum that overflows can make inf - inf)."""
    rng = np.random.default_rng(17 + m)
    sign = np.where(rng.random((m, 1)) < 0.5, 8, 0).astype(np.uint8)
    a4 = rng.choice(np.array([5, 6, 7], np.uint8), (m, k)) | sign
    b4 = rng.choice(np.array([4, 5, 6, 7], np.uint8), (n, k))
    a = (Q.pack_nibbles(a4), np.full((m, k // 32), 254, np.uint8))
    b = (Q.pack_nibbles(b4), np.full((n, k // 32), 125, np.uint8))      # products of 6 * 2^125 and up
    for dtype in (torch.float32, torch.bfloat16):
        c, Cref, S = _crafted_case(a, b, dtype)
        assert (np.abs(Cref) >= 2.0 ** 129).all()
        got = c.float().cpu().numpy()
        assert np.array_equal(got, np.copysign(np.inf, Cref))


@pytest.mark.parametrize("m,n,k", _SHAPES)
def test_gemm_mx_results_near_fp32_limits(m, n, k):
    """Outputs near the top of fp32 (block scale products 2^110 .. 2^111, sums
    up to about 2^126) and near the bottom of its normal range (block scale
    products 2^-119 .. 2^-117, single products down to 2^-121; a cancelling sum
    can land among the subnormals, where 1e-5 * S, about 2^-126, is still far
    above their spacing 2^-149): the bar holds there too."""
    for pairs in ([(254, 111), (253, 110), (230, 130)], [(0, 136), (1, 134), (20, 117)]):
        a, b = _crafted_operands(11 + k, m, n, k, pairs, zero_p=0.0, sat_p=0.3)
        c, Cref, S = _crafted_case(a, b, torch.float32)
        assert np.isfinite(Cref).all() and np.abs(Cref).max() < 2.0 ** 128
        assert torch.isfinite(c).all()
        _assert_within(c, Cref, S)
