"""Python binding of libfp4 (block-scaled FP4 on MI355X / gfx950).

Argument marshalling only: every function passes device pointers, sizes and the
current HIP stream to the C ABI declared in include/fp4.h and raises on a
non-zero status.  All computation happens in the library's HIP kernels; there
is no fallback.  Tensors are torch tensors used as device memory.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib", "Fp4Error", "FMT_MX", "FMT_NV", "DT_BF16", "DT_F32",
    "fp4_quantize_mx", "fp4_quantize_nv", "fp4_quantize_nv_workspace_bytes", "fp4_remap_mx_to_nv",
    "fp4_dequant", "fp4_gemm", "fp4_quantize_mxfp8", "fp4_mx_to_mxfp8", "fp4_gemm_w4a8", "fp4_fake_quant",
    "fp4_ste_backward", "fp4_kv_append_mx", "fp4_moe_grouped_gemm", "fp4_moe_workspace_bytes", "MoeDebug",
    "fp4_abi_version", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfp4.so")
FMT_MX, FMT_NV = 0, 1
DT_BF16, DT_F32 = 0, 1

_c = ctypes
_vp, _i64, _i32, _sz = _c.c_void_p, _c.c_int64, _c.c_int, _c.c_size_t


class MoeDebug(_c.Structure):
    """Mirror of struct fp4_moe_debug (all members nullable device pointers)."""
    _fields_ = [("x_codes", _vp), ("x_scales", _vp), ("counts", _vp), ("offsets", _vp), ("perm", _vp), ("gate_up", _vp),
                ("h_bf16", _vp), ("h_codes", _vp), ("h_scales", _vp), ("y", _vp),
                ("gate_up_in", _vp), ("h_codes_in", _vp), ("h_scales_in", _vp), ("stage_events", _vp * 6)]


_SIGS = {
    "fp4_abi_version": (_i32, []),
    "fp4_status_string": (_c.c_char_p, [_i32]),
    "fp4_last_error": (_c.c_char_p, []),
    "fp4_quantize_mx": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp4_quantize_nv": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _sz, _vp]),
    "fp4_quantize_nv_workspace_bytes": (_sz, [_i64, _i64]),
    "fp4_remap_mx_to_nv": (_i32, [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]),
    "fp4_dequant": (_i32, [_i32, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i64, _vp]),
    "fp4_gemm": (_i32, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp]),
    "fp4_kv_append_mx": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "fp4_fake_quant": (_i32, [_i32, _vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp, _i32, _vp, _sz, _vp]),
    "fp4_ste_backward": (_i32, [_vp, _i32, _i64, _i64, _i64, _vp, _i64, _i32, _vp]),
    "fp4_quantize_mxfp8": (_i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp]),
    "fp4_mx_to_mxfp8": (_i32, [_vp, _i64, _i64, _vp, _vp]),
    "fp4_gemm_w4a8": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i32, _i64, _vp]),
    "fp4_moe_grouped_gemm": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _i32, _i32, _i64, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, _vp, _sz, _c.POINTER(MoeDebug), _vp]),
    "fp4_moe_workspace_bytes": (_sz, [_i32, _i64, _i64, _i32, _i32, _i64]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    h = _c.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        f = getattr(h, name)
        f.restype, f.argtypes = res, args
    return h


lib = _load()


class Fp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib.fp4_last_error().decode() or lib.fp4_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({lib.fp4_status_string(status).decode()}): {msg}")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(fn, status):
    if status != 0:
        raise Fp4Error(fn, status)


def fp4_abi_version() -> int:
    return lib.fp4_abi_version()


def fp4_quantize_mx(x, codes, scales, rows=None, k=None, ld_x=None, stream=None):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    ld_x = x.stride(0) if ld_x is None else ld_x
    _check("fp4_quantize_mx", lib.fp4_quantize_mx(_ptr(x), rows, k, ld_x, _ptr(codes), _ptr(scales), _stream(stream)))


def fp4_quantize_nv_workspace_bytes(rows: int, k: int) -> int:
    return lib.fp4_quantize_nv_workspace_bytes(rows, k)


def fp4_quantize_nv(x, codes, scales, tensor_scale, tensor_scale_is_input=False, workspace=None,
                    rows=None, k=None, ld_x=None, stream=None):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    ld_x = x.stride(0) if ld_x is None else ld_x
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fp4_quantize_nv", lib.fp4_quantize_nv(_ptr(x), rows, k, ld_x, _ptr(codes), _ptr(scales),
                                                  _ptr(tensor_scale), int(bool(tensor_scale_is_input)),
                                                  _ptr(workspace), wsb, _stream(stream)))


def fp4_remap_mx_to_nv(codes, scales_e8m0, scales_e4m3, tensor_scale, n_inexact, rows=None, k=None, stream=None):
    rows = codes.shape[0] if rows is None else rows
    k = codes.shape[1] * 2 if k is None else k
    _check("fp4_remap_mx_to_nv", lib.fp4_remap_mx_to_nv(_ptr(codes), _ptr(scales_e8m0), rows, k, _ptr(scales_e4m3),
                                                        _ptr(tensor_scale), _ptr(n_inexact), _stream(stream)))


def fp4_dequant(fmt, codes, scales, tensor_scale, out, rows=None, k=None, ld_out=None, stream=None):
    rows = codes.shape[0] if rows is None else rows
    k = codes.shape[1] * 2 if k is None else k
    ld_out = out.stride(0) if ld_out is None else ld_out
    dt = DT_F32 if out.dtype == torch.float32 else DT_BF16
    _check("fp4_dequant", lib.fp4_dequant(fmt, _ptr(codes), _ptr(scales), _ptr(tensor_scale), rows, k, _ptr(out), dt,
                                          ld_out, _stream(stream)))


def fp4_gemm(fmt, a_codes, a_scales, b_codes, b_scales, c, a_tensor_scale=None, b_tensor_scale=None,
             m=None, n=None, k=None, ldc=None, stream=None):
    m = a_codes.shape[0] if m is None else m
    n = b_codes.shape[0] if n is None else n
    k = a_codes.shape[1] * 2 if k is None else k
    ldc = c.stride(0) if ldc is None else ldc
    dt = DT_F32 if c.dtype == torch.float32 else DT_BF16
    _check("fp4_gemm", lib.fp4_gemm(fmt, _ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), _ptr(b_codes),
                                    _ptr(b_scales), _ptr(b_tensor_scale), m, n, k, _ptr(c), dt, ldc,
                                    _stream(stream)))


def fp4_kv_append_mx(x, slots, cache_codes, cache_scales, tokens=None, d=None, ld_x=None, stream=None):
    tokens = x.shape[0] if tokens is None else tokens
    d = x.shape[1] if d is None else d
    ld_x = x.stride(0) if ld_x is None else ld_x
    _check("fp4_kv_append_mx", lib.fp4_kv_append_mx(_ptr(x), tokens, d, ld_x, _ptr(slots), _ptr(cache_codes),
                                                    _ptr(cache_scales), cache_codes.shape[0], _stream(stream)))


def fp4_fake_quant(fmt, x, out, tensor_scale=None, tensor_scale_is_input=False, workspace=None, rows=None, k=None,
                   ld_x=None, ld_out=None, stream=None):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    ld_x = x.stride(0) if ld_x is None else ld_x
    ld_out = out.stride(0) if ld_out is None else ld_out
    dt = DT_F32 if out.dtype == torch.float32 else DT_BF16
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("fp4_fake_quant", lib.fp4_fake_quant(fmt, _ptr(x), rows, k, ld_x, _ptr(out), dt, ld_out, _ptr(tensor_scale),
                                                int(bool(tensor_scale_is_input)), _ptr(workspace), wsb,
                                                _stream(stream)))


def fp4_ste_backward(grad, grad_master, accumulate=True, rows=None, k=None, ld_grad=None, ld_master=None,
                     stream=None):
    rows = grad.shape[0] if rows is None else rows
    k = grad.shape[1] if k is None else k
    ld_grad = grad.stride(0) if ld_grad is None else ld_grad
    ld_master = grad_master.stride(0) if ld_master is None else ld_master
    dt = DT_F32 if grad.dtype == torch.float32 else DT_BF16
    _check("fp4_ste_backward", lib.fp4_ste_backward(_ptr(grad), dt, rows, k, ld_grad, _ptr(grad_master), ld_master,
                                                    int(bool(accumulate)), _stream(stream)))


def fp4_quantize_mxfp8(x, codes8, scales, rows=None, k=None, ld_x=None, stream=None):
    rows = x.shape[0] if rows is None else rows
    k = x.shape[1] if k is None else k
    ld_x = x.stride(0) if ld_x is None else ld_x
    _check("fp4_quantize_mxfp8", lib.fp4_quantize_mxfp8(_ptr(x), rows, k, ld_x, _ptr(codes8), _ptr(scales),
                                                        _stream(stream)))


def fp4_mx_to_mxfp8(codes, codes8, rows=None, k=None, stream=None):
    rows = codes.shape[0] if rows is None else rows
    k = codes.shape[1] * 2 if k is None else k
    _check("fp4_mx_to_mxfp8", lib.fp4_mx_to_mxfp8(_ptr(codes), rows, k, _ptr(codes8), _stream(stream)))


def fp4_gemm_w4a8(a_codes8, a_scales, b_codes, b_scales, c, m=None, n=None, k=None, ldc=None, stream=None):
    m = a_codes8.shape[0] if m is None else m
    n = b_codes.shape[0] if n is None else n
    k = a_codes8.shape[1] if k is None else k
    ldc = c.stride(0) if ldc is None else ldc
    dt = DT_F32 if c.dtype == torch.float32 else DT_BF16
    _check("fp4_gemm_w4a8", lib.fp4_gemm_w4a8(_ptr(a_codes8), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), m, n, k,
                                              _ptr(c), dt, ldc, _stream(stream)))


def fp4_moe_workspace_bytes(fmt, tokens, hidden, topk, num_experts, inter) -> int:
    return lib.fp4_moe_workspace_bytes(fmt, tokens, hidden, topk, num_experts, inter)


def fp4_moe_grouped_gemm(fmt, x, topk_ids, topk_weights, num_experts, inter, w13_codes, w13_scales, w2_codes,
                         w2_scales, out, workspace, w13_tensor_scales=None, w2_tensor_scales=None,
                         act_tensor_scales=None, debug: MoeDebug | None = None, stream=None):
    tokens, hidden = x.shape
    topk = topk_ids.shape[1]
    wsb = workspace.numel() * workspace.element_size()
    dbg = _c.byref(debug) if debug is not None else None
    _check("fp4_moe_grouped_gemm", lib.fp4_moe_grouped_gemm(
        fmt, _ptr(x), tokens, hidden, _ptr(topk_ids), _ptr(topk_weights), topk, num_experts, inter,
        _ptr(w13_codes), _ptr(w13_scales), _ptr(w13_tensor_scales), _ptr(w2_codes), _ptr(w2_scales),
        _ptr(w2_tensor_scales), _ptr(act_tensor_scales), _ptr(out), _ptr(workspace), wsb, dbg, _stream(stream)))
