"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function that include/fp4.h declares, and
reject bad arguments with the documented status before it makes any HIP call
(so these calls are safe without a device: no pointer is dereferenced).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4.h")

OK, INVALID, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4, -5, -6


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    names = re.findall(r"\b(fp4_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


@pytest.fixture(scope="module")
def F():
    import block_scaled_fp4_mx_amd as pkg
    return pkg


def test_header_declares_the_six_entry_points():
    names = declared_functions()
    for n in ("fp4_quantize_mx", "fp4_quantize_nv", "fp4_remap_mx_to_nv", "fp4_dequant", "fp4_gemm",
              "fp4_moe_grouped_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol(F):
    lib = ctypes.CDLL(F.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    # the binding wraps every declared entry point under the same name
    for n in declared_functions():
        if n not in ("fp4_status_string", "fp4_last_error"):
            assert hasattr(F, n), n


def test_version_and_status_strings(F):
    assert F.lib.fp4_abi_version() == 2
    for st in (OK, INVALID, SHAPE, ALIGN, UNSUPPORTED, WORKSPACE, HIPERR):
        assert F.lib.fp4_status_string(st)
    assert F.lib.fp4_status_string(12345) == b"unknown status"


FAKE = 1 << 20          # 16-byte aligned, never dereferenced by rejected calls
MISALIGNED = FAKE + 8


def test_quantize_mx_rejections(F):
    q = F.lib.fp4_quantize_mx
    assert q(FAKE, 4, 48, 48, FAKE, FAKE, None) == SHAPE            # k % 32
    assert q(FAKE, -1, 32, 32, FAKE, FAKE, None) == INVALID
    assert q(None, 4, 32, 32, FAKE, FAKE, None) == INVALID
    assert b"x_bf16" in F.lib.fp4_last_error()
    assert q(MISALIGNED, 4, 32, 32, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 4, 32, 16, FAKE, FAKE, None) == INVALID          # ld_x < k
    assert q(FAKE, 4, 32, 36, FAKE, FAKE, None) == ALIGN            # ld_x % 8
    assert q(None, 0, 32, 32, None, None, None) == OK               # empty: no-op
    assert q(None, 5, 0, 0, None, None, None) == OK


def test_quantize_nv_rejections(F):
    q = F.lib.fp4_quantize_nv
    assert q(FAKE, 4, 40, 40, FAKE, FAKE, FAKE, 0, FAKE, 4096, None) == SHAPE   # k % 16
    assert q(FAKE, 4, 32, 32, FAKE, FAKE, None, 0, FAKE, 4096, None) == INVALID  # no tensor scale
    assert q(FAKE, 4, 32, 32, FAKE, FAKE, FAKE + 2, 0, FAKE, 4096, None) == ALIGN
    need = F.lib.fp4_quantize_nv_workspace_bytes(4, 32)
    assert need > 0
    assert q(FAKE, 4, 32, 32, FAKE, FAKE, FAKE, 0, None, 0, None) == WORKSPACE
    assert q(FAKE, 4, 32, 32, FAKE, FAKE, FAKE, 0, FAKE, need - 1, None) == WORKSPACE
    assert q(None, 0, 32, 32, None, None, None, 0, None, 0, None) == OK


def test_remap_and_dequant_rejections(F):
    r = F.lib.fp4_remap_mx_to_nv
    assert r(FAKE, FAKE, 4, 48, FAKE, FAKE, FAKE, None, 0, None) == SHAPE
    assert r(FAKE, FAKE, 4, 64, FAKE, FAKE, None, None, 0, None) == INVALID
    # the optional workspace: one byte per partial-maximum workgroup
    need = F.lib.fp4_scale_max_workspace_bytes(4096, 4096)
    assert need == 128 and F.lib.fp4_scale_max_workspace_bytes(1 << 20, 4096) == 256
    assert F.lib.fp4_scale_max_workspace_bytes(4, 64) == 1 and F.lib.fp4_scale_max_workspace_bytes(0, 64) == 0
    assert r(FAKE, FAKE, 4096, 4096, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert r(FAKE, FAKE, 4096, 4096, FAKE, FAKE, FAKE, None, need, None) == WORKSPACE   # NULL with a size
    d = F.lib.fp4_dequant
    assert d(7, FAKE, FAKE, FAKE, 4, 32, FAKE, 0, 32, None) == INVALID         # format
    assert d(0, FAKE, FAKE, FAKE, 4, 32, FAKE, 9, 32, None) == INVALID         # dtype
    assert d(1, FAKE, FAKE, FAKE, 4, 24, FAKE, 0, 24, None) == SHAPE           # NV k % 16
    assert d(1, FAKE, FAKE, None, 4, 32, FAKE, 0, 32, None) == INVALID         # NV needs s_t
    assert d(0, FAKE, FAKE, None, 4, 32, FAKE, 0, 16, None) == INVALID         # ld_out < k


def test_gemm_rejections(F):
    g = F.lib.fp4_gemm
    args = lambda fmt, m, n, k, ldc, ats=FAKE, c=FAKE: (fmt, FAKE, FAKE, ats, FAKE, FAKE, FAKE, m, n, k, c, 0, ldc,
                                                        None)
    assert g(*args(0, 8, 8, 48, 8)) == SHAPE
    assert g(*args(1, 8, 8, 40, 8)) == SHAPE
    assert g(*args(0, 8, 8, 64, 4)) == INVALID     # ldc < n
    assert g(*args(1, 8, 8, 64, 8, ats=None)) == INVALID
    assert g(*args(0, 8, 8, 64, 8, c=MISALIGNED)) == ALIGN
    assert g(*args(0, 0, 8, 64, 8, c=None)) == OK  # empty


def test_moe_rejections_and_workspace(F):
    m = F.lib.fp4_moe_grouped_gemm
    ws = F.lib.fp4_moe_workspace_bytes(0, 64, 256, 2, 8, 128)
    assert ws > 0
    assert F.lib.fp4_moe_workspace_bytes(0, 64, 256, 0, 8, 128) == 0

    def call(fmt=0, tokens=64, hidden=256, topk=2, E=8, inter=128, ws_bytes=ws, ws_ptr=FAKE, act=None):
        return m(fmt, FAKE, tokens, hidden, FAKE, FAKE, topk, E, inter, FAKE, FAKE, None, FAKE, FAKE, None, act,
                 FAKE, ws_ptr, ws_bytes, None, None)

    assert call(hidden=192) == SHAPE
    assert call(topk=17) == INVALID
    assert call(E=2000) == INVALID
    assert call(ws_bytes=ws - 1) == WORKSPACE
    assert call(ws_ptr=None) == WORKSPACE
    assert call(fmt=1) == INVALID                   # NV needs tensor scales
    assert call(tokens=0, ws_ptr=None, ws_bytes=0) == OK
    # operands past the 32-bit tile offsets: 163840 tokens x top-8 at H=4096,
    # I=8192 puts Q(h) at 5.4e9 bytes; NV's fp16 activations at 2^31 bytes
    assert call(tokens=163840, hidden=4096, topk=8, E=64, inter=8192) == SHAPE
    assert b"32-bit" in F.lib.fp4_last_error()
    assert call(fmt=1, tokens=131072, hidden=8192, topk=1, E=8, inter=128, act=FAKE) == SHAPE
    assert call(tokens=8, hidden=65536, topk=1, E=8, inter=32768) == SHAPE          # one expert slab of 2^31 bytes


def test_w4a8_rejections(F):
    q = F.lib.fp4_quantize_mxfp8
    assert q(FAKE, 4, 48, 48, FAKE, FAKE, None) == SHAPE            # k % 32
    assert q(MISALIGNED, 4, 32, 32, FAKE, FAKE, None) == ALIGN
    assert q(FAKE, 4, 32, 16, FAKE, FAKE, None) == INVALID          # ld_x < k
    assert q(None, 0, 32, 32, None, None, None) == OK
    r = F.lib.fp4_mx_to_mxfp8
    assert r(FAKE, 4, 40, FAKE, None) == SHAPE
    assert r(None, 4, 32, FAKE, None) == INVALID
    assert r(None, 0, 32, None, None) == OK
    g = F.lib.fp4_gemm_w4a8
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 8, 48, FAKE, 0, 8, None) == SHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 5, 8, None) == INVALID      # dtype
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 8, 64, FAKE, 0, 4, None) == INVALID      # ldc < n
    assert g(FAKE, FAKE, MISALIGNED, FAKE, 8, 8, 64, FAKE, 0, 8, None) == ALIGN
    assert g(None, None, None, None, 0, 8, 64, None, 0, 8, None) == OK


def test_fake_quant_ste_and_kv_rejections(F):
    fq = F.lib.fp4_fake_quant
    assert fq(0, FAKE, 4, 48, 48, FAKE + 4096, 0, 48, None, 0, None, 0, None) == SHAPE     # MX k % 32
    assert fq(1, FAKE, 4, 40, 40, FAKE + 4096, 0, 40, FAKE, 1, None, 0, None) == SHAPE     # NV k % 16
    assert fq(3, FAKE, 4, 32, 32, FAKE + 4096, 0, 32, None, 0, None, 0, None) == INVALID   # format
    assert fq(1, FAKE, 4, 32, 32, FAKE + 4096, 0, 32, FAKE, 0, None, 0, None) == WORKSPACE  # computed s_t
    assert fq(1, FAKE, 4, 32, 32, FAKE + 4096, 0, 32, None, 1, None, 0, None) == INVALID   # NV needs s_t
    # out overlapping x without being x (same buffer shifted by 16 bytes)
    assert fq(0, FAKE, 4, 32, 32, FAKE + 16, 0, 32, None, 0, None, 0, None) == INVALID
    assert b"overlaps" in F.lib.fp4_last_error()
    assert fq(0, FAKE, 4, 32, 32, FAKE, 1, 32, None, 0, None, 0, None) == INVALID          # in place needs bf16
    assert fq(0, None, 0, 32, 32, None, 0, 32, None, 0, None, 0, None) == OK
    st = F.lib.fp4_ste_backward
    assert st(FAKE, 0, 4, 12, 16, FAKE, 16, 1, None) == SHAPE       # k % 8
    assert st(FAKE, 7, 4, 16, 16, FAKE, 16, 1, None) == INVALID     # dtype
    assert st(FAKE, 0, 4, 16, 16, FAKE, 12, 1, None) == INVALID     # ld_master < k
    assert st(None, 0, 0, 16, 16, None, 16, 1, None) == OK
    kv = F.lib.fp4_kv_append_mx
    assert kv(FAKE, 4, 48, 48, FAKE, FAKE, FAKE, 16, None) == SHAPE
    assert kv(FAKE, 4, 32, 32, None, FAKE, FAKE, 16, None) == INVALID      # slots
    assert kv(FAKE, 4, 32, 32, FAKE + 2, FAKE, FAKE, 16, None) == ALIGN    # slots need 4-byte alignment
    assert kv(FAKE, 4, 32, 32, FAKE, FAKE, FAKE, -1, None) == INVALID
    assert kv(None, 0, 32, 32, None, None, None, 16, None) == OK


def test_fp8_dequant_rejections(F):
    d = F.lib.fp4_mx_dequant_fp8
    assert d(FAKE, FAKE, 4, 48, FAKE, None, FAKE, FAKE, None, 0, None) == SHAPE            # k % 32
    assert d(FAKE, FAKE, 4, 64, FAKE, None, None, FAKE, None, 0, None) == INVALID          # tensor scale
    assert d(FAKE, FAKE, 4, 64, FAKE, None, FAKE, None, None, 0, None) == INVALID          # count
    assert d(FAKE, FAKE, 4, 64, MISALIGNED, None, FAKE, FAKE, None, 0, None) == ALIGN
    assert d(FAKE, FAKE, 8192, 4096, FAKE, None, FAKE, FAKE, FAKE, 255, None) == WORKSPACE   # needs 256
    assert d(FAKE, FAKE, 4, 64, FAKE, None, FAKE, FAKE, None, 1, None) == WORKSPACE
    assert d(None, None, 0, 64, None, None, None, None, None, 0, None) == OK


def test_binding_rejects_what_the_c_side_would_misread(F):
    """The Python wrappers check dtype, device, layout and operand agreement
    before any pointer is passed (these calls never reach the library)."""
    import torch
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    x = torch.zeros((8, 64), dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="bfloat16"):
        F.fp4_quantize_mx(x.float(), u8(8, 32), u8(8, 2))
    with pytest.raises(ValueError, match="GPU"):
        F.fp4_quantize_mx(x, u8(8, 32), u8(8, 2))
    with pytest.raises(TypeError, match="int32"):
        F.fp4_moe_grouped_gemm(F.FMT_MX, x, torch.zeros((8, 2), dtype=torch.int64), torch.zeros((8, 2)), 4, 128,
                               u8(4, 256, 32), u8(4, 256, 2), u8(4, 64, 64), u8(4, 64, 4), x.clone(), u8(64))
    with pytest.raises(TypeError, match="float32"):
        F.fp4_moe_grouped_gemm(F.FMT_MX, x, torch.zeros((8, 2), dtype=torch.int32),
                               torch.zeros((8, 2), dtype=torch.bfloat16), 4, 128, u8(4, 256, 32), u8(4, 256, 2),
                               u8(4, 64, 64), u8(4, 64, 4), x.clone(), u8(64))
    with pytest.raises(ValueError, match="contiguous"):
        F.fp4_moe_grouped_gemm(F.FMT_MX, torch.zeros((8, 128), dtype=torch.bfloat16)[:, :64],
                               torch.zeros((8, 2), dtype=torch.int32), torch.zeros((8, 2)), 4, 128, u8(4, 256, 32),
                               u8(4, 256, 2), u8(4, 64, 64), u8(4, 64, 4), x.clone(), u8(64))
    with pytest.raises(TypeError, match="uint8"):
        F.fp4_gemm(F.FMT_MX, u8(8, 32), u8(8, 2), torch.zeros((8, 32), dtype=torch.int8), u8(8, 2),
                   torch.zeros((8, 8)))
    # top-1 routing: a [T, 1] id tensor is dense whatever the stride of its size-1
    # axis (numpy may hand over 0 there); only the device check remains to fail
    import numpy as np
    ids1 = torch.from_numpy(np.ascontiguousarray((np.arange(8, dtype=np.int32) % 4)[:, None]))
    w1 = torch.from_numpy(np.ascontiguousarray(np.ones(8, np.float32)[:, None]))
    assert ids1.stride(-1) == 0 and w1.stride(-1) == 0
    with pytest.raises(ValueError, match="GPU"):
        F.fp4_moe_grouped_gemm(F.FMT_MX, x, ids1, w1, 4, 128, u8(4, 256, 32), u8(4, 256, 2), u8(4, 64, 64),
                               u8(4, 64, 4), x.clone(), u8(64))


def test_binding_checks_operand_shapes():
    """Shape agreement is checked with the tensors' shapes alone (no device needed):
    a B operand narrower than A's K would make the kernels read past it."""
    import torch
    import block_scaled_fp4_mx_amd as F
    with pytest.raises(ValueError, match="b_codes"):
        F._shape("fp4_gemm", "b_codes", torch.zeros((8, 16)), (8, 32), rows_at_least=True)
    F._shape("fp4_gemm", "b_codes", torch.zeros((12, 32)), (8, 32), rows_at_least=True)
    with pytest.raises(ValueError, match="w13_codes"):
        F._shape("fp4_moe_grouped_gemm", "w13_codes", torch.zeros((4, 256, 16)), (4, 256, 32))


def test_peak_probe_library_exports():
    """The peak-rate microbenchmark library (not part of the ABI) is built
    beside libfp4.so and exports its four entry points."""
    lib = ctypes.CDLL(os.path.join(ROOT, "block_scaled_fp4_mx_amd", "probes", "libfp4_peak.so"))
    for n in ("peak_mfma", "peak_copy", "peak_lds_dma", "peak_lds_read"):
        assert hasattr(lib, n), n
