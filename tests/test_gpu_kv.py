"""GPU parity of the MXFP4 KV-cache append (bit-exact cache bytes after a
prefill and several decode appends, padding slots skipped, strided input) and
of FP4 QK scores over the cache rows (fp4_gemm, within 1e-5 * sum|q k|)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W
from oracle import gemm as G
from oracle import quant as Q
from gpu_util import DEV, chunked, describe_mismatch, dev_bf16, host_u8, quantize_mx

pytestmark = pytest.mark.gpu


def _rows(seed, n, d):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)) * np.where(rng.random((n, 1)) < 0.1, 30.0, 1.0)
    return W.bf16_bits(W.to_bf16(x))


def _append(cc, cs, bits, slots, x=None):
    x = dev_bf16(bits) if x is None else x
    F.fp4_kv_append_mx(x, torch.tensor(slots, dtype=torch.int32, device=DEV), cc, cs)
    torch.cuda.synchronize()


def test_kv_append_prefill_then_decode_steps():
    cap, d = 1024, 512
    cc = torch.full((cap, d // 2), 0xA5, dtype=torch.uint8, device=DEV)
    cs = torch.full((cap, d // 32), 0x5A, dtype=torch.uint8, device=DEV)
    ec, es = host_u8(cc), host_u8(cs)
    rng = np.random.default_rng(0)
    steps = [(300, 0), (1, 300), (7, 301), (64, 308), (130, 372)]
    for i, (n, start) in enumerate(steps):
        bits = _rows(10 + i, n, d)
        slots = np.arange(start, start + n)
        if n > 1:
            slots = rng.permutation(slots)                            # tokens land out of order
            slots[rng.random(n) < 0.1] = -1                           # padding tokens
            slots[0] = cap + 5                                        # out of range: skipped
        _append(cc, cs, bits, slots.tolist())
        ec, es = Q.kv_append_mx(ec, es, bits, slots)
        gc, gs = host_u8(cc), host_u8(cs)
        assert np.array_equal(gs, es), describe_mismatch(f"scales after step {i}", gs, es)
        assert np.array_equal(gc, ec), describe_mismatch(f"codes after step {i}", gc, ec)


def test_kv_append_strided_input_and_small_d():
    cap, d = 64, 96
    full = _rows(3, 20, 128)
    bits = full[:, :d]
    x = W.from_bits(full).to(DEV)[:, :d]
    cc = torch.full((cap, d // 2), 0xA5, dtype=torch.uint8, device=DEV)
    cs = torch.full((cap, d // 32), 0x5A, dtype=torch.uint8, device=DEV)
    slots = list(range(40, 60))
    _append(cc, cs, bits, slots, x=x)
    ec, es = Q.kv_append_mx(np.full((cap, d // 2), 0xA5, np.uint8), np.full((cap, d // 32), 0x5A, np.uint8), bits, slots)
    assert np.array_equal(host_u8(cc), ec) and np.array_equal(host_u8(cs), es)


def test_kv_append_shape_error():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(F.Fp4Error):
        F.fp4_kv_append_mx(x, torch.zeros(4, dtype=torch.int32, device=DEV),
                           torch.zeros((8, 24), dtype=torch.uint8, device=DEV),
                           torch.zeros((8, 2), dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("nq,n,d", [(5, 300, 96), (64, 32768, 512)])
def test_fp4_qk_scores_over_cache(nq, n, d):
    """Indexer-style scores: MXFP4 queries against the first n cache rows (fp32
    out).  64 x 32768 x 512 is a 128K-token context at compression 4."""
    cap = n + 64
    cc = torch.zeros((cap, d // 2), dtype=torch.uint8, device=DEV)
    cs = torch.full((cap, d // 32), 127, dtype=torch.uint8, device=DEV)
    kbits = _rows(21, n, d)
    _append(cc, cs, kbits, list(range(n)))
    qbits = _rows(22, nq, d)
    qc, qs = quantize_mx(dev_bf16(qbits))
    scores = torch.empty((nq, n), dtype=torch.float32, device=DEV)
    F.fp4_gemm(F.FMT_MX, qc, qs, cc, cs, scores, n=n, k=d)
    torch.cuda.synchronize()
    ek = chunked(Q.mx_quantize, kbits)
    Cref, S = G.gemm_ref("mx", *Q.mx_quantize(qbits), *ek)
    ok = G.within_tol_f32(scores.cpu().numpy(), Cref, S, 1e-5)
    assert ok.all(), f"{(~ok).sum()} scores outside tolerance"
