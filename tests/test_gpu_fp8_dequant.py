"""GPU parity of fp4_mx_dequant_fp8 (MXFP4 -> FP8 values with E4M3 block scales
and a power-of-two tensor scale) and of the remap's tensor-wide passes against
the CPU oracle: value bytes, block scale bytes, tensor scale and inexact-block
count bit-exact, from one block to many workgroups, with inexact blocks inside
and outside the blocks the last workgroup finishes, with and without the
optional workspace that holds the partial maxima."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W
from conftest import read_records
from gpu_util import DEV, chunked, describe_mismatch, dev_bf16, empty_u8, host_u8, quantize_mx
from oracle import quant as Q

pytestmark = pytest.mark.gpu


def _workspace(R, K, fill=0xFF):
    """A workspace of the required size, filled with bytes that would raise
    E_max if a stale one were read."""
    return torch.full((F.fp4_scale_max_workspace_bytes(R, K),), fill, dtype=torch.uint8, device=DEV)


def _run(codes, scales, with_s8=True, ws=None):
    R, nb = scales.shape
    c = torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    v8 = empty_u8(R, nb * 32)
    s8 = empty_u8(R, nb) if with_s8 else None
    ts = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    F.fp4_mx_dequant_fp8(c, s, v8, ts, n, s8, workspace=ws)
    torch.cuda.synchronize()
    return host_u8(v8), None if s8 is None else host_u8(s8), ts.item(), n.item()


def _check(codes, scales, with_s8=True, ws=None):
    ev, es, est, en = Q.mx_dequant_fp8(codes, scales)
    gv, gs, gts, gn = _run(codes, scales, with_s8, ws)
    assert gts == float(est), (gts, float(est))
    assert gn == en, (gn, en)
    if with_s8:
        assert np.array_equal(gs, es), describe_mismatch("block scales", gs, es)
    assert np.array_equal(gv, ev), describe_mismatch("fp8 values", gv, ev)
    return en


@pytest.mark.parametrize("rec", read_records("fp8_dequant_worked_blocks.txt"), ids=lambda r: r["name"])
def test_fp8_dequant_worked_tensor(rec):
    scales = np.array([[int(v) for v in rec["scales"]]], np.uint8)
    nb = scales.shape[1]
    c4 = np.concatenate([[int(v) for v in rec[f"codes{b}"]] for b in range(nb)]).astype(np.uint8)[None, :]
    assert _check(Q.pack_nibbles(c4), scales) == int(rec["n_inexact"][0])


@pytest.mark.parametrize("which", ["A", "W"])
def test_fp8_dequant_workload2_lossless(which):
    """The linear workload's tensors: bit-exact bytes, no inexact block, and the
    FP8 values times the tensor scale equal the MX dequantization in fp32."""
    bits = W.bf16_bits(getattr(W.workload2(), which))
    x = dev_bf16(bits)
    c, s = quantize_mx(x)
    v8 = empty_u8(*bits.shape)
    s8 = empty_u8(bits.shape[0], bits.shape[1] // 32)
    ts = torch.zeros(1, dtype=torch.float32, device=DEV)
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    F.fp4_mx_dequant_fp8(c, s, v8, ts, n, s8)
    deq = torch.empty(bits.shape, dtype=torch.float32, device=DEV)
    F.fp4_dequant(F.FMT_MX, c, s, None, deq)
    torch.cuda.synchronize()
    ec, es_ = chunked(Q.mx_quantize, bits)
    ev, es, est, en = Q.mx_dequant_fp8(ec, es_)
    assert n.item() == en == 0 and ts.item() == float(est)
    assert np.array_equal(host_u8(s8), es)
    assert np.array_equal(host_u8(v8), ev)
    got = v8.view(torch.float8_e4m3fn).to(torch.float32) * ts
    assert torch.equal(got, deq)


def _spread(seed, R, K, spread, every=None):
    rng = np.random.default_rng(seed)
    c4 = rng.integers(0, 16, (R, K), dtype=np.uint8)
    sc = (200 - rng.integers(0, spread + 1, (R, K // 32))).astype(np.uint8)
    if every:                                   # a few far-below blocks, block 0 among them
        flat = sc.reshape(-1)
        flat[::every] = 200 - spread - 1 - rng.integers(0, 3, flat[::every].shape)
    return Q.pack_nibbles(c4), sc


@pytest.mark.parametrize("with_ws", [False, True], ids=["three_launch", "workspace"])
@pytest.mark.parametrize("R,K", [(1, 32), (1, 64), (3, 96), (5, 1024), (777, 4096), (2048, 16384)])
def test_fp8_dequant_shapes(R, K, with_ws):
    """One block up to 1M blocks (256 pass-1 workgroups): without workspace the
    blocks whose output bytes hold the pass-1 maxima (finished by the last
    workgroup) include block 0; with it the maxima sit in the workspace."""
    codes, scales = _spread(R * 31 + K, R, K, 15, every=97)
    n = _check(codes, scales, ws=_workspace(R, K) if with_ws else None)
    if R * K // 32 > 97:
        assert n > 0


@pytest.mark.parametrize("spread", [0, 14, 15, 16, 40, 200])
def test_fp8_dequant_scale_ratio_sweep(spread):
    codes, scales = _spread(spread, 64, 2048, spread)
    n = _check(codes, scales)
    if spread <= 14:
        assert n == 0


def test_fp8_dequant_extremes_and_null_block_scales():
    c4 = np.tile(np.arange(16, dtype=np.uint8), (4, 16))
    for lo, hi in ((254, 254), (0, 0), (0, 254), (240, 254)):
        scales = np.full((4, 8), lo, np.uint8)
        scales[1, 3] = hi
        _check(Q.pack_nibbles(c4), scales)
        _check(Q.pack_nibbles(c4), scales, with_s8=False)


def test_fp8_dequant_back_to_back_calls():
    """The tensor-scale and count words double as the call's counters: two calls
    in a row on the same outputs, the second on a smaller tensor."""
    a = _spread(1, 512, 4096, 16, every=13)
    b = _spread(2, 7, 256, 20, every=3)
    for codes, scales in (a, b, a):
        _check(codes, scales)


def test_fp8_dequant_workspace_reused():
    """One workspace through three calls, the second on a smaller tensor (fewer
    pass-1 workgroups, so bytes of the first call stay behind) and a call with
    the workspace and one without agreeing on the same tensor."""
    a = _spread(3, 2048, 16384, 16, every=13)
    b = _spread(4, 33, 512, 20, every=3)
    ws = _workspace(2048, 16384, fill=0)
    assert ws.numel() == 256
    for codes, scales in (a, b, a):
        _check(codes, scales, ws=ws)
    assert all(x == y if isinstance(x, float) else np.array_equal(x, y)
               for x, y in zip(_run(*b, ws=ws), _run(*b)))


@pytest.mark.parametrize("with_ws", [False, True], ids=["three_launch", "workspace"])
@pytest.mark.parametrize("R,K", [(1, 32), (2, 64), (777, 4096), (4096, 8192)])
def test_remap_inexact_blocks_in_every_region(R, K, with_ws):
    """Remap over one block to 1M blocks with inexact blocks at block 0 (without
    workspace, output bytes that held the pass-1 maxima) and spread through the
    tensor."""
    rng = np.random.default_rng(R + K)
    c4 = rng.integers(1, 16, (R, K), dtype=np.uint8)
    sc = (150 - rng.integers(0, 10, (R, K // 32))).astype(np.uint8)
    flat = sc.reshape(-1)
    if flat.size > 1:
        flat[::max(1, flat.size // 50)] = 120
        flat[1] = 150
    codes = Q.pack_nibbles(c4)
    snv = empty_u8(R, K // 16)
    ts = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    F.fp4_remap_mx_to_nv(torch.from_numpy(codes).to(DEV), torch.from_numpy(sc).to(DEV), snv, ts, n,
                         workspace=_workspace(R, K) if with_ws else None)
    torch.cuda.synchronize()
    esnv, est, en = Q.remap_mx_to_nv(codes, sc)
    assert n.item() == en and ts.item() == float(est)
    if flat.size > 1:
        assert en > 0
    assert np.array_equal(host_u8(snv), esnv), describe_mismatch("remap scales", host_u8(snv), esnv)


@pytest.mark.parametrize("with_ws", [False, True], ids=["three_launch", "workspace"])
@pytest.mark.parametrize("R,K", [(3, 96), (777, 4096)])
def test_scale_passes_write_only_their_outputs(R, K, with_ws):
    """Guard bands around every output of the remap and the FP8 dequant (and
    past the workspace bytes the query asks for) keep their sentinel bytes:
    the pass-1 maxima land in the workspace or in the output's own first
    bytes, and nothing is written past an output's end."""
    codes, sc = _spread(R + K, R, K, 12, every=37)
    c = torch.from_numpy(codes).to(DEV)
    s = torch.from_numpy(sc).to(DEV)
    G = 4096
    need = F.fp4_scale_max_workspace_bytes(R, K)

    def guarded(n):
        buf = torch.full((n + 2 * G,), 0xA5, dtype=torch.uint8, device=DEV)
        return buf, buf[G:G + n]

    ws_buf, ws = guarded(need + 64) if with_ws else (None, None)
    snv_buf, snv = guarded(R * K // 16)
    v8_buf, v8 = guarded(R * K)
    s8_buf, s8 = guarded(R * K // 32)
    ts = torch.zeros(2, dtype=torch.float32, device=DEV)
    n = torch.zeros(2, dtype=torch.int32, device=DEV)
    F.fp4_remap_mx_to_nv(c, s, snv.view(R, K // 16), ts[:1], n[:1], workspace=ws)
    F.fp4_mx_dequant_fp8(c, s, v8.view(R, K), ts[1:], n[1:], s8.view(R, K // 32), workspace=ws)
    torch.cuda.synchronize()
    for name, buf, m in (("remap scales", snv_buf, R * K // 16), ("fp8 values", v8_buf, R * K),
                         ("fp8 block scales", s8_buf, R * K // 32)):
        h = host_u8(buf)
        assert (h[:G] == 0xA5).all() and (h[G + m:] == 0xA5).all(), name
    if with_ws:
        assert (host_u8(ws_buf)[:G] == 0xA5).all() and (host_u8(ws_buf)[G + need:] == 0xA5).all(), "workspace"
    esnv, est, en = Q.remap_mx_to_nv(codes, sc)
    assert np.array_equal(host_u8(snv).reshape(R, K // 16), esnv) and ts[0].item() == float(est) and n[0].item() == en
    ev, es, est8, en8 = Q.mx_dequant_fp8(codes, sc)
    assert np.array_equal(host_u8(v8).reshape(R, K), ev) and np.array_equal(host_u8(s8).reshape(R, K // 32), es)
    assert ts[1].item() == float(est8) and n[1].item() == en8
