"""Pins of the oracle's MXFP4 KV-cache append: every stored row against the
scalar block definition, padding slots skipped, untouched rows kept, and FP4
QK scores over the cache rows against brute-force Fraction dot products."""
from fractions import Fraction

import numpy as np

from oracle import formats as F
from oracle import gemm as G
from oracle import quant as Q


def _bits(seed, R, K):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)) * np.exp2(rng.integers(-8, 8, size=(R, 1)))
    return F.fp32_to_bf16_bits_rne(x.astype(np.float32))


def test_kv_append_rows_against_block_definition():
    cap, d = 10, 64
    codes0 = np.full((cap, d // 2), 0xA5, np.uint8)
    scales0 = np.full((cap, d // 32), 0x5A, np.uint8)
    x = _bits(1, 5, d)
    slots = [7, -1, 2, 10, 0]                      # -1 and 10 (= capacity) are padding
    codes, scales = Q.kv_append_mx(codes0, scales0, x, slots)
    for t, s in enumerate(slots):
        if not 0 <= s < cap:
            continue
        for b in range(d // 32):
            c4, sc = Q.mx_block_exact([int(v) for v in x[t, 32 * b:32 * b + 32]])
            assert sc == scales[s, b]
            assert list(Q.unpack_nibbles(codes[s:s + 1, 16 * b:16 * b + 16])[0]) == c4
    untouched = [r for r in range(cap) if r not in (7, 2, 0)]
    assert (codes[untouched] == 0xA5).all() and (scales[untouched] == 0x5A).all()
    assert (codes0 == 0xA5).all()                  # inputs not modified


def test_fp4_qk_scores_over_cache_brute_force():
    cap, d = 6, 64
    codes, scales = np.zeros((cap, d // 2), np.uint8), np.full((cap, d // 32), 127, np.uint8)
    codes, scales = Q.kv_append_mx(codes, scales, _bits(2, 4, d), [0, 1, 2, 3])
    codes, scales = Q.kv_append_mx(codes, scales, _bits(3, 2, d), [4, 5])
    q_codes, q_scales = Q.mx_quantize(_bits(4, 3, d))
    C, S = G.gemm_ref("mx", q_codes, q_scales, codes, scales)
    qv = Q.mx_dequant_f64(q_codes, q_scales)
    kv = Q.mx_dequant_f64(codes, scales)
    for i in range(3):
        for j in range(cap):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[i], kv[j]))
            assert Fraction(C[i, j]) == exact
