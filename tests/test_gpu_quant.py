"""GPU parity of quantize / dequantize / remap against the CPU oracle:
codes and scales bit-exact at the workloads' full sizes and on edge cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W
from oracle import formats as OF
from oracle import quant as Q
import bf16_patterns as BP
from gpu_util import (DEV, chunked, describe_mismatch, dev_bf16, empty_u8, host_u8, quantize_mx,
                      quantize_nv)

pytestmark = pytest.mark.gpu


def _crafted(K, seed=0):
    rng = np.random.default_rng(seed)
    rows = []
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 4.0, 0.5, 3.0])
    for scale in (1.0, 2.0 ** -20, 2.0 ** 30, 2.0 ** -126, 2.0 ** -128, 2.0 ** -133, 2.0 ** 100):
        rows.append(rng.choice(ties, K) * scale * rng.choice([-1, 1], K))
    rows.append(np.zeros(K))
    rows.append(np.where(np.arange(K) % 2 == 1, -0.0, 0.0))
    rows.append(rng.standard_normal(K) * 2.0 ** -130)
    rows.append(rng.standard_normal(K) * 1e35)
    rows.append(rng.standard_t(3, K) * 0.02)
    rows.append(rng.standard_normal(K) * np.where(rng.random(K) < 0.05, 1000.0, 1.0))
    return W.bf16_bits(W.to_bf16(np.array(rows)))


def _check_mx(bits):
    x = dev_bf16(bits)
    c, s = quantize_mx(x)
    torch.cuda.synchronize()
    ec, es = chunked(Q.mx_quantize, bits)
    gs, gc = host_u8(s), host_u8(c)
    assert np.array_equal(gs, es), describe_mismatch("mx scales", gs, es)
    assert np.array_equal(gc, ec), describe_mismatch("mx codes", gc, ec)


def _check_nv(bits, s_t=None):
    x = dev_bf16(bits)
    c, s, ts = quantize_nv(x, s_t)
    torch.cuda.synchronize()
    ec, es, est = chunked(Q.nv_quantize, bits, s_t=(Q.nv_tensor_scale(bits) if s_t is None else s_t))
    assert ts.item() == float(est), (ts.item(), float(est))
    gs, gc = host_u8(s), host_u8(c)
    assert np.array_equal(gs, es), describe_mismatch("nv scales", gs, es)
    assert np.array_equal(gc, ec), describe_mismatch("nv codes", gc, ec)


@pytest.mark.parametrize("which", ["A", "W"])
def test_mx_quantize_workload1(which):
    wl = W.workload1()
    _check_mx(W.bf16_bits(getattr(wl, which)))


@pytest.mark.parametrize("which", ["A", "W"])
def test_mx_quantize_workload2_full(which):
    wl = W.workload2()
    _check_mx(W.bf16_bits(getattr(wl, which)))


def test_mx_quantize_crafted_edges():
    _check_mx(_crafted(256))


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (37, 160), (130, 4096)])
def test_mx_quantize_ragged(rows, k):
    rng = np.random.default_rng(rows * 7 + k)
    _check_mx(W.bf16_bits(W.to_bf16(rng.standard_normal((rows, k)))))


def test_mx_quantize_strided_rows():
    rng = np.random.default_rng(3)
    full = W.to_bf16(rng.standard_normal((40, 200)))
    bits = W.bf16_bits(full)[:, :160]
    x = W.from_bits(W.bf16_bits(full)).to(DEV)[:, :160]
    assert x.stride(0) == 200
    c, s = quantize_mx(x)
    torch.cuda.synchronize()
    ec, es = Q.mx_quantize(bits)
    assert np.array_equal(host_u8(s), es) and np.array_equal(host_u8(c), ec)


def _rows_of(blocks, per_row):
    pad = (-blocks.shape[0]) % per_row
    blocks = np.concatenate([blocks, np.zeros((pad, blocks.shape[1]), np.uint16)])
    return blocks.reshape(-1, per_row * blocks.shape[1])


def test_mx_quantize_exhaustive_bf16_patterns():
    """All 65,280 finite bf16 patterns: as their own block maximum (sorted
    blocks), 0, 1, 2, 3, 4, 5 and 8 binades below the block maximum (every
    pattern whose binade leaves room for the offset), and in random blocks.
    The offsets run through normal, subnormal and clamped block exponents."""
    sb, rb = BP.sorted_blocks(32), BP.random_blocks(32, 7)
    ob, _ = BP.offset_blocks(32, [0, 1, 2, 3, 4, 5, 8])
    assert BP.covered(sb) == BP.covered(rb) == BP.covered(ob[:, 1:]) == BP.N_FINITE
    _check_mx(_rows_of(np.concatenate([sb, rb, ob]), 128))


def test_nv_quantize_exhaustive_bf16_patterns():
    """All 65,280 finite bf16 patterns in 16-element groups 0, 1, 2, 3, 4 and 6
    binades below the group maximum, under supplied tensor scales that put the
    group scale amax / (6 s_t) in E4M3's normal range, its subnormal range, and
    past 448 (saturated); plus every pattern as its own group maximum and in
    random groups under a computed tensor scale."""
    ob, ea = BP.offset_blocks(16, [0, 1, 2, 3, 4, 6])
    assert BP.covered(ob[:, 1:]) == BP.N_FINITE
    calls = []
    for f in np.unique(ea):
        grp = ob[ea == f]
        a = float(OF.bf16_bits_to_f64(grp[:1, 0])[0])
        lg = int(np.frexp(a)[1]) - 1
        for shift in (-4, 6, -12):                       # normal, subnormal, saturated group scales
            s_t = float(np.float32(np.ldexp(1.0, int(np.clip(lg + shift, -149, 127)))))
            calls.append((_rows_of(grp, 8), s_t))
    outs = []
    for bits, s_t in calls:
        x = dev_bf16(bits)
        outs.append((bits, s_t) + quantize_nv(x, s_t))
    torch.cuda.synchronize()
    bad = []
    for bits, s_t, c, s, ts in outs:
        ec, es, _ = Q.nv_quantize(bits, s_t=s_t)
        if not (np.array_equal(host_u8(s), es) and np.array_equal(host_u8(c), ec)):
            bad.append((s_t, describe_mismatch("nv scales", host_u8(s), es), describe_mismatch("nv codes", host_u8(c), ec)))
    assert not bad, f"{len(bad)} of {len(outs)} calls differ; first: {bad[0]}"
    sb, rb = BP.sorted_blocks(16), BP.random_blocks(16, 8)
    _check_nv(_rows_of(np.concatenate([sb, rb]), 64))


@pytest.mark.parametrize("which", ["A", "W"])
def test_nv_quantize_workload2_full(which):
    wl = W.workload2()
    _check_nv(W.bf16_bits(getattr(wl, which)))


@pytest.mark.parametrize("s_t", [1.0 / 64, 0.0123, 2.0 ** -20, 3.0e-30])
def test_nv_quantize_supplied_scale_crafted(s_t):
    _check_nv(_crafted(256, seed=5), s_t=s_t)


def test_nv_quantize_dynamic_scale_crafted():
    _check_nv(_crafted(128, seed=6))


@pytest.mark.parametrize("rows,k", [(1, 16), (5, 48), (33, 272)])
def test_nv_quantize_ragged(rows, k):
    rng = np.random.default_rng(rows + k)
    _check_nv(W.bf16_bits(W.to_bf16(rng.standard_t(3, (rows, k)) * 0.02)))


def test_nv_quantize_power_of_two_scale_ties():
    """A power-of-two s_t makes exact E2M1 midpoints common: the exact tie path."""
    rng = np.random.default_rng(9)
    bits = W.bf16_bits(W.to_bf16(rng.choice([0.25, 0.75, 1.25, 2.5, 3.5, 5.0], (64, 256)) * rng.choice([1, 2, 4, 8], (64, 256))))
    _check_nv(bits, s_t=2.0 ** -3)


def test_nv_quantize_group_scale_midpoints():
    """Group maxima whose quotient amax_g / (6 s_t) is exactly an E4M3 rounding
    midpoint (normal and subnormal, even and odd neighbours): with s_t = 2^-3,
    amax_g = 0.75 m is a bf16 value for every midpoint m.  Both tie directions
    and the neighbours just above and below each midpoint are covered."""
    pos = OF.E4M3_POS_F64
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(11)
    centre = W.bf16_bits(W.to_bf16(0.75 * mids)).astype(np.int64)      # exact: 0.75 m has <= 7 bits
    rows = []
    for c in centre:
        for amax_bits in (c - 1, c, c + 1):                            # bf16 neighbours of the tie
            amax = OF.bf16_bits_to_f64(np.array([amax_bits], np.uint16))[0]
            g = W.bf16_bits(W.to_bf16(rng.uniform(-1, 1, 16) * amax))
            g[rng.integers(16)] = amax_bits | (0x8000 if rng.random() < 0.5 else 0)
            rows.append(g)
    flat = np.concatenate(rows)
    bits = np.concatenate([flat, np.zeros((-flat.size) % 256, np.uint16)]).reshape(-1, 256).astype(np.uint16)
    _check_nv(bits, s_t=2.0 ** -3)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dequant_bit_exact(fmt, dtype):
    wl = W.random_linear(50, 96, 8, 512, outlier_p=0.01)
    bits = W.bf16_bits(wl.A)
    x = dev_bf16(bits)
    if fmt == "mx":
        c, s = quantize_mx(x)
        ts = None
        ec, es = Q.mx_quantize(bits)
        est = None
    else:
        c, s, ts = quantize_nv(x)
        ec, es, est = Q.nv_quantize(bits)
    out = torch.empty((96, 520), dtype=dtype, device=DEV)[:, :512]
    F.fp4_dequant(F.FMT_MX if fmt == "mx" else F.FMT_NV, c, s, ts, out)
    torch.cuda.synchronize()
    if dtype == torch.float32:
        exp = Q.dequant_fp32(fmt, ec, es, est)
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), describe_mismatch("deq f32", got, exp)
    else:
        exp = Q.dequant_bf16_bits(fmt, ec, es, est)
        got = W.bf16_bits(out)
        assert np.array_equal(got, exp), describe_mismatch("deq bf16", got, exp)


def test_dequant_mx_extreme_scales():
    codes = np.tile(np.arange(16, dtype=np.uint8), (4, 8))
    packed = Q.pack_nibbles(codes)
    scales = np.array([[0, 1, 127, 252]] * 4, np.uint8)
    c = torch.from_numpy(packed).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    out = torch.empty((4, 128), dtype=torch.float32, device=DEV)
    F.fp4_dequant(F.FMT_MX, c, s, None, out)
    torch.cuda.synchronize()
    exp = Q.dequant_fp32("mx", packed, scales)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("with_ws", [False, True], ids=["three_launch", "workspace"])
@pytest.mark.parametrize("which", ["A", "W"])
def test_remap_workload2_lossless(which, with_ws):
    wl = W.workload2()
    bits = W.bf16_bits(getattr(wl, which))
    x = dev_bf16(bits)
    c, s = quantize_mx(x)
    snv = empty_u8(bits.shape[0], bits.shape[1] // 16)
    ts = torch.zeros(1, dtype=torch.float32, device=DEV)
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = None
    if with_ws:
        ws = torch.full((F.fp4_scale_max_workspace_bytes(*bits.shape),), 0xFF, dtype=torch.uint8, device=DEV)
    F.fp4_remap_mx_to_nv(c, s, snv, ts, n, workspace=ws)
    torch.cuda.synchronize()
    ec, es = chunked(Q.mx_quantize, bits)
    esnv, est, en = Q.remap_mx_to_nv(ec, es)
    assert n.item() == en == 0
    assert ts.item() == float(est)
    assert np.array_equal(host_u8(snv), esnv)
    # lossless: the NV reading of the same codes dequantizes to identical fp32 values
    o1 = torch.empty(x.shape, dtype=torch.float32, device=DEV)
    o2 = torch.empty(x.shape, dtype=torch.float32, device=DEV)
    F.fp4_dequant(F.FMT_MX, c, s, None, o1)
    F.fp4_dequant(F.FMT_NV, c, snv, ts, o2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


def test_remap_inexact_blocks_counted():
    rng = np.random.default_rng(26)
    bits = W.bf16_bits(W.to_bf16(rng.standard_normal((4, 256))))
    ec, es = Q.mx_quantize(bits)
    es = es.copy()
    es[0, 0] = 137; es[1, 1] = 120; es[1, 2] = 119; es[2, 3] = 107; es[3, 4] = 0
    c4 = Q.unpack_nibbles(ec); c4[3, 128:160] &= 8; ec = Q.pack_nibbles(c4)
    c = torch.from_numpy(ec).to(DEV)
    s = torch.from_numpy(es).to(DEV)
    snv = empty_u8(4, 16)
    ts = torch.zeros(1, dtype=torch.float32, device=DEV)
    n = torch.zeros(1, dtype=torch.int32, device=DEV)
    F.fp4_remap_mx_to_nv(c, s, snv, ts, n)
    torch.cuda.synchronize()
    esnv, est, en = Q.remap_mx_to_nv(ec, es)
    assert en == 2 and n.item() == 2
    assert ts.item() == float(est)
    assert np.array_equal(host_u8(snv), esnv)


def test_quantize_deterministic_run_to_run():
    wl = W.workload2()
    x = dev_bf16(W.bf16_bits(wl.A))
    c1, s1 = quantize_mx(x)
    c2, s2 = quantize_mx(x)
    n1, ns1, t1 = quantize_nv(x)
    n2, ns2, t2 = quantize_nv(x)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    assert torch.equal(n1, n2) and torch.equal(ns1, ns2) and torch.equal(t1, t2)


def test_zero_size_calls_are_noops():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c = empty_u8(0, 32); s = empty_u8(0, 2)
    F.fp4_quantize_mx(x, c, s)
    torch.cuda.synchronize()
