"""Helpers for GPU parity tests: move oracle-side numpy data to the device and
back, and run the library entry points on torch-allocated device buffers."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_fp4_mx_amd as F
import workloads as W

DEV = "cuda"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return W.from_bits(bits).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return W.bf16_bits(t)


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def empty_u8(*shape) -> torch.Tensor:
    # poison value so unwritten bytes show up
    return torch.full(shape, 0xA5, dtype=torch.uint8, device=DEV)


def quantize_mx(x: torch.Tensor, k=None):
    rows = x.shape[0]
    k = x.shape[1] if k is None else k
    codes = empty_u8(rows, k // 2)
    scales = empty_u8(rows, k // 32)
    F.fp4_quantize_mx(x, codes, scales, rows=rows, k=k)
    return codes, scales


def quantize_nv(x: torch.Tensor, s_t=None, k=None):
    rows = x.shape[0]
    k = x.shape[1] if k is None else k
    codes = empty_u8(rows, k // 2)
    scales = empty_u8(rows, k // 16)
    ts = torch.full((1,), float("nan") if s_t is None else float(np.float32(s_t)), dtype=torch.float32, device=DEV)
    ws = torch.empty(F.fp4_quantize_nv_workspace_bytes(rows, k), dtype=torch.uint8, device=DEV)
    F.fp4_quantize_nv(x, codes, scales, ts, tensor_scale_is_input=s_t is not None, workspace=ws, rows=rows, k=k)
    return codes, scales, ts


def chunked(fn, bits: np.ndarray, rows_per_chunk: int = 512, **kw):
    """Run a row-wise oracle function over row chunks (bounded host memory) and
    concatenate each returned array along the row axis."""
    outs = [fn(bits[i:i + rows_per_chunk], **kw) for i in range(0, bits.shape[0], rows_per_chunk)]
    if isinstance(outs[0], tuple):
        return tuple(np.concatenate([o[j] for o in outs]) if np.ndim(outs[0][j]) else outs[0][j]
                     for j in range(len(outs[0])))
    return np.concatenate(outs)


def describe_mismatch(name, got, exp, max_show=8):
    bad = np.argwhere(got != exp)
    lines = [f"{name}: {len(bad)} mismatches of {got.size}"]
    for idx in bad[:max_show]:
        t = tuple(idx)
        lines.append(f"  at {t}: got {got[t]!r} expected {exp[t]!r}")
    return "\n".join(lines)
