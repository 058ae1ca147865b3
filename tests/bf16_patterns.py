"""Every finite bf16 bit pattern (65,280 of them) arranged in quantization
blocks, for the exhaustive quantizer tests.  Input construction only: no
quantization arithmetic.

A block-scaled quantizer maps an element through its block's maximum, so each
pattern p is placed
  * as the block maximum itself (all patterns sorted by magnitude and cut into
    blocks, so each block holds neighbouring magnitudes),
  * below a block maximum that lies d binades above p's own binade, for every
    offset d in a given list (one anchor element of exponent e + d and the
    largest mantissa, then block-1 patterns of exponent field e, both signs),
  * in random mixtures.
Patterns of exponent field 0 are the bf16 subnormals; anchors of exponent
field 0 or 1 give blocks with subnormal or clamped block exponents.
"""
from __future__ import annotations

import numpy as np

N_FINITE = 65280


def finite_patterns() -> np.ndarray:
    p = np.arange(1 << 16, dtype=np.uint32)
    return p[((p >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def _chunk(vals: np.ndarray, per: int) -> np.ndarray:
    pad = (-len(vals)) % per
    return np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, per)


def sorted_blocks(block: int) -> np.ndarray:
    p = finite_patterns()
    order = np.argsort(p & 0x7FFF, kind="stable")
    return _chunk(p[order], block)


def random_blocks(block: int, seed: int) -> np.ndarray:
    p = finite_patterns()
    return _chunk(np.random.default_rng(seed).permutation(p), block)


def offset_blocks(block: int, offsets, exponents=range(0, 255)) -> tuple[np.ndarray, np.ndarray]:
    """Blocks [anchor, block-1 patterns of exponent field e] for each e and each
    d in offsets with e + d <= 254; returns (blocks, exponent field of each
    block's anchor)."""
    p = finite_patterns()
    field = (p >> 7) & 0xFF
    rows, efield = [], []
    for e in exponents:
        pe = p[field == e]
        for d in offsets:
            ea = max(e, 1) + d if e == 0 and d > 0 else e + d
            if ea > 254:
                continue
            anchor = np.uint16((ea << 7) | 0x7F)          # largest mantissa of binade ea
            body = _chunk(pe, block - 1)
            blk = np.concatenate([np.full((body.shape[0], 1), anchor, np.uint16), body], axis=1)
            rows.append(blk)
            efield += [ea] * blk.shape[0]
    return np.concatenate(rows), np.array(efield)


def covered(blocks: np.ndarray) -> int:
    """Number of distinct finite patterns present."""
    return len(np.unique(blocks.ravel()))
