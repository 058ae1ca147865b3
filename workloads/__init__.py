"""Seeded synthetic inputs for the five block-scaled FP4 workloads.

This module only draws random numbers and shapes them; it holds none of the
quantization, GEMM or MoE arithmetic.  Both the HIP path's tests/bench and the
CPU oracle read their inputs from here.

Recipe (every value: fp64 sample -> fp32 (numpy RNE cast) -> bf16 (torch RNE
cast)); seed = 1000 + workload number, child streams from SeedSequence.spawn
in the order A, W, outliers, router noise, router permutation:

  w1  tiny MX:   A 32x256, W 512x256 ~ N(0,1); each element independently an
                 outlier with probability 0.01, outliers multiplied by 50.
  w2  linear:    W 4096x4096 ~ Student-t(3) x 0.02; A 2048x4096 ~ N(0,1) with
                 round(0.005*4096) = 20 input-feature columns multiplied by 30.
  w3  GEMM:      A 4096x4096 ~ N(0,1); W 4096x4096 ~ Student-t(3) x 0.02.
  w4  MoE MX:    X 8192x4096 ~ N(0,1); 384 experts, top-6, I = 2048.
  w5  MoE NV:    X {64, 16384}x7168 ~ N(0,1); 384 experts, top-6, I = 3072.
  router:        logits = N(0,1) + b_e with b_e = -1.1 ln(rank_e), rank a seeded
                 permutation of 1..384 (so expert popularity follows a Zipf(1.1)
                 law); ids = top-6 logits, descending, ties to the lower index;
                 weights = softmax over the 6 selected logits (fp64 -> fp32).
  experts:       w13 [2I, H] (rows 0..I-1 gate w1, I..2I-1 up w3) and w2 [H, I]
                 ~ Student-t(3) x 0.02, seeded per expert index.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

NUM_EXPERTS = 384
TOPK = 6


def to_bf16(x64: np.ndarray) -> torch.Tensor:
    """fp64 samples -> fp32 (RNE) -> bf16 (RNE) CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (CPU copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(bits: np.ndarray) -> torch.Tensor:
    """bf16 CPU tensor with the given uint16 bit patterns."""
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def streams(workload: int, n: int = 5):
    ss = np.random.SeedSequence(1000 + workload)
    return [np.random.default_rng(s) for s in ss.spawn(n)]


def student_t3(rng, shape, scale=0.02):
    return rng.standard_t(3, size=shape) * scale


@dataclass
class Linear:
    A: torch.Tensor      # bf16 [M, K]
    W: torch.Tensor      # bf16 [N, K]


def workload1() -> Linear:
    rA, rW, rO, _, _ = streams(1)
    A = rA.standard_normal((32, 256))
    W = rW.standard_normal((512, 256))
    A = np.where(rO.random(A.shape) < 0.01, A * 50.0, A)
    W = np.where(rO.random(W.shape) < 0.01, W * 50.0, W)
    return Linear(to_bf16(A), to_bf16(W))


def workload2() -> Linear:
    rA, rW, rO, _, _ = streams(2)
    W = student_t3(rW, (4096, 4096))
    A = rA.standard_normal((2048, 4096))
    cols = rO.permutation(4096)[:round(0.005 * 4096)]
    A[:, cols] *= 30.0
    return Linear(to_bf16(A), to_bf16(W))


def workload3() -> Linear:
    rA, rW, _, _, _ = streams(3)
    A = rA.standard_normal((4096, 4096))
    W = student_t3(rW, (4096, 4096))
    return Linear(to_bf16(A), to_bf16(W))


def random_linear(seed: int, m: int, n: int, k: int, outlier_p: float = 0.0) -> Linear:
    """Extra parity shapes (ragged tiles, several blocks): N(0,1) activations,
    t(3)x0.02 weights, optional elementwise x50 outliers."""
    rA, rW, rO = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    A = rA.standard_normal((m, k))
    W = student_t3(rW, (n, k))
    if outlier_p:
        A = np.where(rO.random(A.shape) < outlier_p, A * 50.0, A)
    return Linear(to_bf16(A), to_bf16(W))


# ---------------------------------------------------------------- MoE
@dataclass
class MoE:
    workload: int
    X: torch.Tensor          # bf16 [T, H]
    ids: np.ndarray          # int32 [T, 6]
    weights: np.ndarray      # float32 [T, 6]
    hidden: int
    inter: int
    num_experts: int = NUM_EXPERTS
    topk: int = TOPK


def router(rng_noise, rng_perm, tokens: int, num_experts: int = NUM_EXPERTS, topk: int = TOPK):
    """Seeded skewed router (input generation, not part of the expert path)."""
    rank = rng_perm.permutation(num_experts) + 1
    bias = -1.1 * np.log(rank.astype(np.float64))
    logits = rng_noise.standard_normal((tokens, num_experts)) + bias
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]   # ties -> lower index
    sel = np.take_along_axis(logits, order, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def moe_workload(workload: int, tokens: int | None = None) -> MoE:
    """workload 4 (MX, H=4096, I=2048, 8192 tokens) or 5 (NV, H=7168, I=3072,
    64 decode tokens or 16384 prefill tokens)."""
    if workload == 4:
        H, I, T = 4096, 2048, 8192 if tokens is None else tokens
    elif workload == 5:
        H, I, T = 7168, 3072, 64 if tokens is None else tokens
    else:
        raise ValueError(workload)
    rA, _, _, rN, rP = streams(workload)
    X = rA.standard_normal((T, H))
    ids, w = router(rN, rP, T)
    return MoE(workload, to_bf16(X), ids, w, H, I)


def small_moe(seed: int, tokens: int, hidden: int, inter: int, num_experts: int, topk: int) -> MoE:
    """Small MoE cases for parity at sizes the oracle finishes in seconds."""
    rA, rN, rP = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3)]
    X = rA.standard_normal((tokens, hidden))
    ids, w = router(rN, rP, tokens, num_experts, topk)
    return MoE(0, to_bf16(X), ids, w, hidden, inter, num_experts, topk)


def expert_weights(workload_seed: int, e: int, hidden: int, inter: int):
    """bf16 (w13 [2I, H], w2 [H, I]) of expert e, seeded per expert (CPU)."""
    r13, r2 = [np.random.default_rng(s) for s in np.random.SeedSequence([workload_seed, 99, e]).spawn(2)]
    return to_bf16(student_t3(r13, (2 * inter, hidden))), to_bf16(student_t3(r2, (hidden, inter)))


def expert_weights_device(seed: int, num_experts: int, hidden: int, inter: int, device="cuda"):
    """All experts' bf16 weights drawn on the device (t(3)x0.02 built from normals
    as N / sqrt(chi2_3 / 3)) for timing runs, where the values only need the
    right distribution.  Yields (e, w13, w2) one expert at a time."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def t3(shape):
        z = torch.randn(shape, generator=g, device=device)
        c = torch.randn((3,) + tuple(shape), generator=g, device=device).square().sum(0) / 3.0
        return (z / c.sqrt() * 0.02).to(torch.bfloat16)

    for e in range(num_experts):
        yield e, t3((2 * inter, hidden)), t3((hidden, inter))
