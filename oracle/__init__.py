"""Plain CPU oracle for block-scaled FP4 (MXFP4 / NVFP4) quantization, remap,
dequantization, W4A4 GEMM and the MoE expert path.

THIS PACKAGE IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The HIP library never calls it and it never calls
the HIP library: the two share no code, tables, helpers or constants.

Every routine is written from the pages' definitions, step by step, in exact
arithmetic (Python ``Fraction`` / ``int``) for the scalar definitions and in
numpy fp64 for the vectorised forms, each fp64 use exact by the argument stated
next to it.  Page citations use the short keys defined in ``oracle/cite.py``.

Modules
  formats  -- E2M1 / E4M3 / UE8M0 / fp32 / bf16 encodings and correct rounding
  quant    -- MX and NV quantize, MX->NV remap, dequantize
  gemm     -- C = A . B^T over dequantized operands, error bound S
  moe      -- routed-expert SwiGLU MoE (gate/up, SiLU*mul, down, weighted sum)

Parity pins: every function here is pinned by tests under ``tests/`` marked
``not gpu`` against the page's printed E2M1 table, library casts, closed forms,
invariants and brute force; none of them is "parity unpinned".
"""
