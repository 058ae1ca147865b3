"""The allocation-free NV quantize (fp4_quantize_nv_noalloc, scratch in the
library's static device array) against fp4_quantize_nv with a caller
workspace: codes, scales and tensor scale bit-exact, on consecutive calls of
decreasing size, with computed and supplied tensor scales."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W
from gpu_util import DEV, dev_bf16, empty_u8, host_u8
from oracle import quant as Q

pytestmark = pytest.mark.gpu


def _noalloc(x, s_t=None):
    rows, k = x.shape
    codes, scales = empty_u8(rows, k // 2), empty_u8(rows, k // 16)
    ts = torch.full((1,), float("nan") if s_t is None else s_t, dtype=torch.float32, device=DEV)
    st = F.lib.fp4_quantize_nv_noalloc(x.data_ptr(), rows, k, x.stride(0), codes.data_ptr(), scales.data_ptr(),
                                       ts.data_ptr(), int(s_t is not None), torch.cuda.current_stream().cuda_stream)
    assert st == 0, F.lib.fp4_last_error()
    return codes, scales, ts


def _with_workspace(x, s_t=None):
    rows, k = x.shape
    codes, scales = empty_u8(rows, k // 2), empty_u8(rows, k // 16)
    ts = torch.full((1,), float("nan") if s_t is None else s_t, dtype=torch.float32, device=DEV)
    ws = torch.empty(F.fp4_quantize_nv_workspace_bytes(rows, k), dtype=torch.uint8, device=DEV)
    F.fp4_quantize_nv(x, codes, scales, ts, s_t is not None, ws)
    return codes, scales, ts


@pytest.mark.parametrize("s_t", [None, 0.0123])
def test_noalloc_nv_quantize_matches_workspace_entry_point(s_t):
    wl = W.workload2()
    shapes = [W.bf16_bits(wl.A), W.bf16_bits(W.random_linear(77, 37, 8, 272, outlier_p=0.02).A)]
    for bits in shapes:                         # the second call is the smaller one
        x = dev_bf16(bits)
        a = _noalloc(x, s_t)
        b = _with_workspace(x, s_t)
        torch.cuda.synchronize()
        assert torch.equal(a[2].view(torch.int32), b[2].view(torch.int32))
        assert torch.equal(a[1], b[1]) and torch.equal(a[0], b[0])
    # the last (small) call against the oracle as well
    ec, es, est = Q.nv_quantize(bits, s_t=None if s_t is None else np.float32(s_t))
    assert a[2].item() == float(est)
    assert np.array_equal(host_u8(a[1]), es) and np.array_equal(host_u8(a[0]), ec)


def test_noalloc_nv_quantize_strided_rows_and_empty():
    full = dev_bf16(W.bf16_bits(W.random_linear(78, 40, 8, 320).A))
    x = full[:, :256]
    a, b = _noalloc(x), _with_workspace(x)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    assert F.lib.fp4_quantize_nv_noalloc(e.data_ptr(), 0, 64, 64, None, None, None, 0, None) == 0
