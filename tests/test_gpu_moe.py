"""GPU parity of the routed-expert MoE path (fp4_moe_grouped_gemm) against the
oracle: an end-to-end run (routing, Q(X), g/u, h validity, output statistics)
and each fused stage on injected oracle data (h and Q(h) exact; y and out within
tolerance).  Expectations come from the oracle on the seeded inputs only."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import workloads as W
from moe_check import (Case, calibrate_act_scales, check_down_stage, check_end_to_end, check_gate_up_stage,
                       oracle_expect, oracle_expert_quant, run_gpu)

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=64)
def _expert(seed, e, H, I):
    a, b = W.expert_weights(seed, e, H, I)
    return W.bf16_bits(a), W.bf16_bits(b)


def _small_case(fmt, seed, T, H, I, E, topk, ids=None, weights=None):
    m = W.small_moe(seed, T, H, I, E, topk)
    ids = m.ids if ids is None else ids
    wts = m.weights if weights is None else weights
    experts = {e: _expert(seed, e, H, I) for e in range(E)}
    case = Case(fmt, W.bf16_bits(m.X), ids, wts, E, H, I, experts)
    eq = oracle_expert_quant(case)
    if fmt == "nv":
        case.act_st = calibrate_act_scales(case, eq, np.arange(case.T))
    return case, eq


def _all_checks(case, exp, fill=False):
    st = {"e2e": check_end_to_end(case, run_gpu(case, fill_other_experts=fill), exp)}
    st["gate_up"] = check_gate_up_stage(case, run_gpu(case, fill_other_experts=fill, inject="gate_up", exp=exp), exp)
    st["down"] = check_down_stage(case, run_gpu(case, fill_other_experts=fill, inject="h", exp=exp), exp)
    print(case.fmt, st)
    return st


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_moe_small(fmt):
    case, eq = _small_case(fmt, 100, 40, 256, 256, 8, 3)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq))


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_moe_multi_tile_segments(fmt):
    """Experts with more than one 128-row tile and ragged last tiles."""
    case, eq = _small_case(fmt, 101, 300, 128, 128, 4, 2)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq))


def test_moe_tiled_mx_segments():
    """Hidden and intermediate multiples of 512 take the 256-row LDS-staged MX
    tiles: segments spanning several tiles, ragged last tiles, and last tiles of
    at most 128 rows (whose second row band skips the matrix work)."""
    case, eq = _small_case("mx", 104, 700, 512, 512, 4, 2)
    counts = np.bincount(case.ids.ravel(), minlength=4)
    assert counts.max() > 256 and ((counts % 256) <= 128).any()
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq))


def test_moe_tiled_nv_segments():
    """Hidden and intermediate multiples of 256 take the 128-row LDS-staged NV
    tiles (A read as NVFP4 codes and expanded in the tile): segments spanning several tiles,
    ragged last tiles of several row-fragment counts, and last tiles of at most
    64 rows (whose second staging pass of the down tile is skipped)."""
    case, eq = _small_case("nv", 105, 300, 256, 256, 4, 2)
    counts = np.bincount(case.ids.ravel(), minlength=4)
    last = counts % 128
    assert counts.max() > 128 and len(set((last + 15) // 16)) > 2 and ((last > 0) & (last <= 64)).any()
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq))


def test_moe_decode_nv_segments():
    """Batches of at most 128 tokens take the 32-row, three-stage NV tiles:
    several tiles per expert, ragged last tiles, and K loops of 4 (gate/up)
    and 3 (down) steps, which exercise the copy waits with two steps in flight."""
    case, eq = _small_case("nv", 106, 100, 1024, 768, 8, 6)
    counts = np.bincount(case.ids.ravel(), minlength=8)
    assert counts.max() > 64 and (counts % 32 != 0).any()
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq))


def test_moe_single_expert_topk1():
    T, H, I, E = 33, 128, 256, 5
    ids = np.full((T, 1), 3, np.int32)
    case, eq = _small_case("mx", 102, T, H, I, E, 1, ids=ids, weights=np.ones((T, 1), np.float32))
    _all_checks(case, oracle_expect(case, np.arange(T), eq))


def test_moe_ids_outside_range_route_nowhere():
    T, H, I, E, k = 24, 128, 128, 6, 3
    m = W.small_moe(103, T, H, I, E, k)
    ids = m.ids.copy()
    ids[::5, 1] = -1
    ids[::7, 2] = E + 3
    case, eq = _small_case("mx", 103, T, H, I, E, k, ids=ids)
    _all_checks(case, oracle_expect(case, np.arange(T), eq))


def _full_case(workload, fmt, tokens=None, sample=(0,)):
    m = W.moe_workload(workload, tokens)
    sample = np.asarray(sample)
    need = sorted(set(int(e) for e in m.ids[sample].ravel()))
    experts = {e: _expert(1000 + workload, e, m.hidden, m.inter) for e in need}
    case = Case(fmt, W.bf16_bits(m.X), m.ids, m.weights, m.num_experts, m.hidden, m.inter, experts)
    eq = oracle_expert_quant(case)
    if fmt == "nv":
        case.act_st = calibrate_act_scales(case, eq, sample)
    return case, eq, sample


@pytest.mark.timeout(400)
def test_moe_workload4_full_size_sampled():
    """MoE at hidden 4096 (8192 tokens, 384 experts, top-6, MXFP4) in the launch
    the benchmark times: routing checked whole, two tokens checked per stage."""
    case, eq, sample = _full_case(4, "mx", sample=(5, 4321))
    _all_checks(case, oracle_expect(case, sample, eq), fill=True)


@pytest.mark.timeout(400)
def test_moe_workload5_decode_sampled():
    """NVFP4 MoE at hidden 7168, decode batch of 64 tokens; one token per stage."""
    case, eq, sample = _full_case(5, "nv", sample=(17,))
    _all_checks(case, oracle_expect(case, sample, eq), fill=True)


@pytest.mark.timeout(600)
def test_moe_workload5_prefill_sampled():
    """NVFP4 MoE at hidden 7168 on a prefill batch of 16384 tokens (98,304
    routed slots, the 128-row wide NV tiles), in the launch the benchmark
    times: routing checked whole, two tokens checked per stage."""
    case, eq, sample = _full_case(5, "nv", tokens=16384, sample=(3, 12345))
    _all_checks(case, oracle_expect(case, sample, eq), fill=True)
