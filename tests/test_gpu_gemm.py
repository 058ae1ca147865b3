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
    """K a multiple of 128 and at least 32 tiles: the 64x512 LDS-staged NV tile
    (A expanded to fp16 in LDS, B in registers), ragged M and N, both output
    types and a padded output row pitch."""
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
    """At most 128 A rows and at least 4096 B rows (k % 128 == 0): the
    streaming kernel (one pass over B), ragged m and n, both output types and
    an output pitch that forces the element-wise stores."""
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
