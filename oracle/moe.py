"""Routed-expert MoE oracle (the expert path that the pages' NVFP4/MXFP4 layers feed).

[V41-NVFP4 s3] the quantized layers are the routed experts' w1, w2, w3
projections; [V4-ARCH s2] 384 routed experts with 6 active per token;
[V4-ARCH s5.1] the experts are SwiGLU; [V4-QAT s3.1] top-k routing then
per-expert linear layers; [V4-ARCH s6.1] tokens are dispatched to experts and
combined back.  Steps per (token t, slot j), expert e = ids[t, j]:

  x_hat  = deq(Q(X[t]))                      activation quantized per token row
  g, u   = x_hat . w1_hat[e]^T, x_hat . w3_hat[e]^T      (exact sums)
  h      = RNE_bf16( SiLU(g) * u ),  SiLU(z) = z / (1 + exp(-z))   (fp64)
  h_hat  = deq(Q(h))                          quantized along the intermediate dim
  y      = h_hat . w2_hat[e]^T
  out[t] = RNE_bf16( sum_j w[t, j] * y[t, j] )

Weights are given already quantized, per expert: w13 codes [E, 2I, H/2] whose
rows 0..I-1 are w1 (gate) and I..2I-1 are w3 (up), w2 codes [E, H, I/2]; for
NV each expert matrix is its own tensor with its own fp32 s_t.  NV activation
tensor scales (for X and for h) are calibrated inputs [V41-NVFP4 s4].

The per-expert functions (gate/up, SiLU*mul, down) let a test compute each
stage's expectation on its own inputs; the weighted sum over a token's slots
is the last step of moe_forward.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import gemm as G
from . import quant as Q


def quantize_rows(fmt: str, xbits: np.ndarray, s_t=None):
    """Q(x) row-wise: MX (codes, scales, None) or NV with the given tensor scale."""
    if fmt == "mx":
        c, s = Q.mx_quantize(xbits)
        return c, s, None
    c, s, st = Q.nv_quantize(xbits, s_t=s_t)
    return c, s, st


def silu_mul_bf16(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = RNE_bf16(SiLU(g) * u) in fp64 (g, u given as fp32/fp64 values)."""
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return F.bf16_rne_of_f64(silu * u)


def expert_gate_up(fmt, xq, w13c, w13s, w13_st, e: int, rows: np.ndarray, inter: int):
    """g, u for the tokens ``rows`` routed to expert e, with their bounds S_g, S_u,
    through the GEMM oracle.  xq = (codes, scales, s_t) of the quantized X."""
    gu, S = G.gemm_ref(fmt, xq[0][rows], xq[1][rows], w13c[e], w13s[e],
                       xq[2], None if w13_st is None else w13_st[e])
    return gu[:, :inter], gu[:, inter:], S[:, :inter], S[:, inter:]


def expert_down(fmt, hq, w2c, w2s, w2_st, e: int):
    """y = h_hat . w2_hat[e]^T and its bound S_y; hq = (codes, scales, s_t)."""
    return G.gemm_ref(fmt, hq[0], hq[1], w2c[e], w2s[e], hq[2], None if w2_st is None else w2_st[e])


def moe_forward(fmt: str, xbits: np.ndarray, ids: np.ndarray, weights: np.ndarray,
                w13c, w13s, w2c, w2s, w13_st=None, w2_st=None, act_st=(None, None),
                tokens: np.ndarray | None = None):
    """Full MoE oracle for the token subset ``tokens`` (default: all).

    Returns dict with per-slot g, u, h (bf16 bits), y and the per-token output
    (bf16 bits) plus its bound  B[t] = sum_j |w[t,j]| * S_y[t,j].  X is quantized
    per token row; the quantized rows do not depend on which tokens are picked.
    """
    T, H = xbits.shape
    topk = ids.shape[1]
    inter = w2c.shape[2] * 2
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens)
    xq = quantize_rows(fmt, xbits[tokens], act_st[0])
    nt = len(tokens)
    g = np.zeros((nt, topk, inter))
    u = np.zeros_like(g)
    y = np.zeros((nt, topk, H))
    Sy = np.zeros_like(y)
    h_bits = np.zeros((nt, topk, inter), np.uint16)
    local = np.arange(nt)
    for e in np.unique(ids[tokens]):
        ti, tj = np.nonzero(ids[tokens] == e)
        gg, uu, _, _ = expert_gate_up(fmt, xq, w13c, w13s, w13_st, int(e), local[ti], inter)
        g[ti, tj], u[ti, tj] = gg, uu
        h_bits[ti, tj] = silu_mul_bf16(gg, uu)
    hq = quantize_rows(fmt, h_bits.reshape(nt * topk, inter), act_st[1])
    hq = (hq[0].reshape(nt, topk, -1), hq[1].reshape(nt, topk, -1), hq[2])
    for e in np.unique(ids[tokens]):
        ti, tj = np.nonzero(ids[tokens] == e)
        yy, ss = expert_down(fmt, (hq[0][ti, tj], hq[1][ti, tj], hq[2]), w2c, w2s, w2_st, int(e))
        y[ti, tj], Sy[ti, tj] = yy, ss
    w = np.asarray(weights, np.float32).astype(np.float64)[tokens]
    out = np.einsum("tj,tjh->th", w, y)
    bound = np.einsum("tj,tjh->th", np.abs(w), Sy)
    return dict(g=g, u=u, h_bits=h_bits, h_codes=hq[0], h_scales=hq[1], h_st=hq[2],
                y=y, S_y=Sy, out_f64=out, out_bound=bound,
                out_bits=F.bf16_rne_of_f64(out), x_codes=xq[0], x_scales=xq[1], x_st=xq[2])


def routing_metadata(ids: np.ndarray, num_experts: int):
    """Expert histogram, exclusive offsets and the stable slot permutation.

    Slots are numbered s = t*topk + j; ``perm`` lists them grouped by expert in
    increasing expert order, and in increasing slot order within an expert
    (the stable order, which makes the permutation unique)."""
    flat = np.asarray(ids, np.int64).ravel()
    counts = np.bincount(flat, minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = np.argsort(flat, kind="stable")
    return counts.astype(np.int32), offsets.astype(np.int32), perm.astype(np.int32)
