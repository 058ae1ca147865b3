"""GPU parity of the QAT fake-quant node (fused quantize -> dequantize) and the
straight-through backward against the oracle: every output bit-exact (the
fused node rounds exactly as quantize followed by dequantize)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W
from oracle import formats as OF
from oracle import quant as Q
from gpu_util import DEV, chunked, describe_mismatch, dev_bf16
from test_gpu_quant import _crafted

pytestmark = pytest.mark.gpu


def _fake(fmt, x, dtype, s_t=None, out=None):
    rows, k = x.shape
    if out is None:
        out = torch.full((rows, k), float("nan"), dtype=dtype, device=DEV)
    ts = torch.full((1,), float("nan") if s_t is None else float(np.float32(s_t)), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.fp4_quantize_nv_workspace_bytes(rows, k), dtype=torch.uint8, device=DEV)
    F.fp4_fake_quant(F.FMT_MX if fmt == "mx" else F.FMT_NV, x, out, ts, s_t is not None, ws)
    torch.cuda.synchronize()
    return out, ts


def _expect(fmt, bits, dtype, s_t=None):
    if fmt == "nv" and s_t is None:
        s_t = Q.nv_tensor_scale(bits)
    fn = Q.fake_quant_fp32 if dtype == torch.float32 else Q.fake_quant_bf16_bits
    return chunked(lambda b: fn(fmt, b, s_t), bits)      # s_t of the whole tensor, not per chunk


def _got(out):
    return out.cpu().numpy() if out.dtype == torch.float32 else W.bf16_bits(out)


def _check(fmt, bits, dtype, s_t=None):
    out, ts = _fake(fmt, dev_bf16(bits), dtype, s_t)
    exp = _expect(fmt, bits, dtype, s_t)
    got = _got(out)
    if dtype == torch.float32:
        same = (got.view(np.uint32) == exp.view(np.uint32))
        assert same.all(), describe_mismatch("fake-quant f32 bits", got.view(np.uint32), exp.view(np.uint32))
    else:
        assert np.array_equal(got, exp), describe_mismatch("fake-quant bf16", got, exp)
    if fmt == "nv" and s_t is None:
        assert ts.item() == float(Q.nv_tensor_scale(bits))


@pytest.mark.parametrize("fmt", ["mx", "nv"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fake_quant_workload2_weight_full(fmt, dtype):
    _check(fmt, W.bf16_bits(W.workload2().W), dtype)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_fake_quant_crafted_edges(fmt):
    _check(fmt, _crafted(256), torch.bfloat16)
    _check(fmt, _crafted(256, seed=1), torch.float32)


@pytest.mark.parametrize("s_t", [1.0 / 64, 0.0123, 2.0 ** -20])
def test_fake_quant_nv_supplied_scale(s_t):
    _check("nv", _crafted(160, seed=2), torch.float32, s_t)
    _check("nv", W.bf16_bits(W.workload1().A), torch.bfloat16, s_t)


@pytest.mark.parametrize("fmt,rows,k", [("mx", 1, 32), ("mx", 37, 160), ("nv", 3, 48), ("nv", 130, 4096)])
def test_fake_quant_ragged(fmt, rows, k):
    rng = np.random.default_rng(rows + k)
    _check(fmt, W.bf16_bits(W.to_bf16(rng.standard_t(3, (rows, k)) * 0.02)), torch.bfloat16)


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_fake_quant_in_place_and_strided(fmt):
    rng = np.random.default_rng(9)
    full = W.bf16_bits(W.to_bf16(rng.standard_normal((48, 208))))
    bits = full[:, :192]
    exp = _expect(fmt, bits, torch.bfloat16)
    base = W.from_bits(full).to(DEV)
    x = base[:, :192]                                              # row pitch 208
    _fake(fmt, x, torch.bfloat16, out=x)                           # in place
    assert np.array_equal(W.bf16_bits(x.contiguous()), exp)
    assert np.array_equal(W.bf16_bits(base[:, 192:].contiguous()), full[:, 192:])
    buf = torch.full((48, 200), float("nan"), dtype=torch.float32, device=DEV)
    out, _ = _fake(fmt, W.from_bits(full).to(DEV)[:, :192], torch.float32, out=buf[:, :192])
    got = np.ascontiguousarray(out.cpu().numpy()).view(np.uint32)
    assert np.array_equal(got, _expect(fmt, bits, torch.float32).view(np.uint32))
    assert torch.isnan(buf[:, 192:]).all()


def test_fake_quant_rejects_partial_overlap():
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(F.Fp4Error):
        F.fp4_fake_quant(F.FMT_MX, x[:, :32], x[:, 32:], None, False, None, rows=8, k=32)


@pytest.mark.parametrize("gdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("accumulate", [False, True])
def test_ste_backward(gdt, accumulate):
    rng = np.random.default_rng(11)
    g = (rng.standard_normal((300, 520)) * 1e-3).astype(np.float32)
    m = rng.standard_normal((300, 520)).astype(np.float32)
    gt = torch.from_numpy(g).to(DEV).to(gdt)
    mbuf = torch.full((300, 528), float("nan"), dtype=torch.float32, device=DEV)
    mbuf[:, :520] = torch.from_numpy(m).to(DEV)
    F.fp4_ste_backward(gt, mbuf[:, :520], accumulate=accumulate)
    torch.cuda.synchronize()
    gv = gt.float().cpu().numpy()
    exp = Q.ste_backward(gv, m if accumulate else None)
    got = np.ascontiguousarray(mbuf[:, :520].cpu().numpy()).view(np.uint32)
    assert np.array_equal(got, np.ascontiguousarray(exp, np.float32).view(np.uint32))
    assert torch.isnan(mbuf[:, 520:]).all()
