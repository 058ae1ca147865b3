"""GPU parity of the routed-expert MoE path (fp4_moe_grouped_gemm) against the
oracle: an end-to-end run (routing, Q(X), g/u, h validity, output statistics)
and each fused stage on injected oracle data (h and Q(h) exact; y and out within
tolerance).  Expectations come from the oracle on the seeded inputs only."""
from __future__ import annotations

import functools

import numpy as np
import pytest

import workloads as W
from moe_check import (DEV, Case, check_down_stage, check_end_to_end, check_gate_up_stage, device_weight_quant,
                       oracle_expect, oracle_expert_quant, run_gpu)
from oracle import moe as M

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
    return case, oracle_expert_quant(case)


def _all_checks(case, exp, fill=False):
    st = {"e2e": check_end_to_end(case, run_gpu(case, fill_other_experts=fill), exp)}
    st["gate_up"] = check_gate_up_stage(case, run_gpu(case, fill_other_experts=fill, inject="gate_up", exp=exp), exp)
    st["down"] = check_down_stage(case, run_gpu(case, fill_other_experts=fill, inject="h", exp=exp), exp)
    print(case.fmt, st)
    return st


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_moe_small(fmt):
    case, eq = _small_case(fmt, 100, 40, 256, 256, 8, 3)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_moe_multi_tile_segments(fmt):
    """Experts with more than one 128-row tile and ragged last tiles."""
    case, eq = _small_case(fmt, 101, 300, 128, 128, 4, 2)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def test_moe_tiled_mx_segments():
    """Hidden and intermediate multiples of 512 take the 256-row LDS-staged MX
    tiles: segments spanning several tiles, ragged last tiles, and last tiles of
    at most 128 rows (whose second row band skips the matrix work)."""
    case, eq = _small_case("mx", 104, 700, 512, 512, 4, 2)
    counts = np.bincount(case.ids.ravel(), minlength=4)
    assert counts.max() > 256 and ((counts % 256) <= 128).any()
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def test_moe_tiled_nv_segments():
    """Hidden and intermediate multiples of 256 take the 128-row LDS-staged NV
    tiles (A read as NVFP4 codes and expanded in the tile): segments spanning several tiles,
    ragged last tiles of several row-fragment counts, and last tiles of at most
    64 rows (whose second staging pass of the down tile is skipped)."""
    case, eq = _small_case("nv", 105, 300, 256, 256, 4, 2)
    counts = np.bincount(case.ids.ravel(), minlength=4)
    last = counts % 128
    assert counts.max() > 128 and len(set((last + 15) // 16)) > 2 and ((last > 0) & (last <= 64)).any()
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def test_moe_decode_nv_segments():
    """Batches of at most 128 tokens take the 32-row, three-stage NV tiles:
    several tiles per expert, ragged last tiles, and K loops of 4 (gate/up)
    and 3 (down) steps, which exercise the copy waits with two steps in flight."""
    case, eq = _small_case("nv", 106, 100, 1024, 768, 8, 6)
    counts = np.bincount(case.ids.ravel(), minlength=8)
    assert counts.max() > 64 and (counts % 32 != 0).any()
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def test_moe_decode_nv_two_step_k():
    """Hidden and intermediate 512 on the 32-row decode tiles: K loops of
    exactly two steps, so the prologue's two copies are the whole loop and the
    first step's wait leaves the last step's copies in flight."""
    case, eq = _small_case("nv", 109, 100, 512, 512, 8, 6)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def _segment_case(fmt, seed, counts, H, I):
    """topk 1, expert e routed exactly counts[e] tokens (in shuffled order)."""
    counts = np.asarray(counts)
    ids = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    np.random.default_rng(seed).shuffle(ids)
    case, eq = _small_case(fmt, seed, len(ids), H, I, len(counts), 1, ids=np.ascontiguousarray(ids[:, None]))
    assert (np.bincount(case.ids.ravel(), minlength=len(counts)) == counts).all()
    return case, eq


@pytest.mark.parametrize("fmt,counts,H", [
    # 256-row MX tiles: 16-row fragments, 128-row bands, a second tile of one row
    ("mx", [1, 15, 16, 17, 127, 128, 129, 255, 257], 512),
    # 128-row wide NV tiles: 16-row fragments, 64-row staging passes, a second tile of one row
    ("nv", [1, 15, 16, 17, 63, 64, 65, 127, 129], 256),
])
def test_moe_segments_at_fragment_boundaries(fmt, counts, H):
    """Expert segments that end exactly on, just past and just before a 16-row
    fragment, a row band or staging pass, and a whole tile: the epilogues work
    only on the fragments and rows inside the segment, and the down tiles take
    each stored row's slot from a per-lane load."""
    case, eq = _segment_case(fmt, 107, counts, H, H)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def test_moe_tiled_mx_hidden_1024():
    """Hidden and intermediate 1024 on the 256-row MX tiles: K loops of four
    steps (two scale loads each), eight gate/up column blocks, and segments at
    fragment, band and tile boundaries."""
    case, eq = _segment_case("mx", 110, [1, 16, 17, 128, 129, 255, 257, 300], 1024, 1024)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


@pytest.mark.parametrize("fmt", ["mx", "nv"])
def test_moe_topk_above_eight(fmt):
    """Top-12 routing over 16 experts: the combine sums a token's slots in two
    batches of loads (slots 0-7, then 8-11), in slot order."""
    case, eq = _small_case(fmt, 108, 40, 256, 256, 16, 12)
    _all_checks(case, oracle_expect(case, np.arange(case.T), eq, calibrate_h=True))


def test_moe_single_expert_topk1():
    T, H, I, E = 33, 128, 256, 5
    ids = np.full((T, 1), 3, np.int32)
    case, eq = _small_case("mx", 102, T, H, I, E, 1, ids=ids, weights=np.ones((T, 1), np.float32))
    _all_checks(case, oracle_expect(case, np.arange(T), eq, calibrate_h=True))


def test_moe_ids_outside_range_route_nowhere():
    T, H, I, E, k = 24, 128, 128, 6, 3
    m = W.small_moe(103, T, H, I, E, k)
    ids = m.ids.copy()
    ids[::5, 1] = -1
    ids[::7, 2] = E + 3
    case, eq = _small_case("mx", 103, T, H, I, E, k, ids=ids)
    _all_checks(case, oracle_expect(case, np.arange(T), eq, calibrate_h=True))


def _sample_tokens(ids, E):
    """Tokens whose slots reach the tiles most likely to go wrong: one slot of
    every expert with at most 4 routed slots (cold experts, nearly empty
    tiles), the first and the last slot of the four busiest experts (the last
    one is the last row of the expert's ragged last tile); checked on the host."""
    topk = ids.shape[1]
    counts, offsets, perm = M.routing_metadata(ids, E)
    cold = np.nonzero((counts > 0) & (counts <= 4))[0]
    hot = np.argsort(-counts, kind="stable")[:4]
    toks = {int(perm[offsets[e]]) // topk for e in cold}
    for e in hot:
        toks |= {int(perm[offsets[e]]) // topk, int(perm[offsets[e + 1] - 1]) // topk}
    toks = np.array(sorted(toks))
    reached = set(int(v) for v in ids[toks].ravel())
    assert all(int(e) in reached for e in cold)
    last = {int(perm[offsets[e + 1] - 1]) for e in hot}
    slots = set((toks[:, None] * topk + np.arange(topk)[None, :]).ravel().tolist())
    assert last <= slots
    return toks, len(cold)


def _full_case(workload, fmt, tokens=None, all_tokens=False):
    """The full-size workload with every active expert's weights drawn on the
    device (seeded); the oracle reads back the exact bf16 of the experts it checks."""
    m = W.moe_workload(workload, tokens)
    active = set(int(v) for v in np.unique(m.ids))
    wdev = {e: (a, b) for e, a, b in W.expert_weights_device(1000 + workload, m.num_experts, m.hidden, m.inter, DEV)
            if e in active}
    case = Case(fmt, W.bf16_bits(m.X), m.ids, m.weights, m.num_experts, m.hidden, m.inter, {}, wdev=wdev)
    if all_tokens:
        sample, ncold = np.arange(m.X.shape[0]), -1
    else:
        sample, ncold = _sample_tokens(m.ids, m.num_experts)
    exp = oracle_expect(case, sample, device_weight_quant(case), calibrate_h=fmt == "nv")
    print(f"workload {workload} {fmt}: {len(sample)} tokens checked, {ncold} cold experts reached, "
          f"{len(set(int(v) for v in m.ids[sample].ravel()))} experts")
    return case, exp


@pytest.mark.timeout(600)
def test_moe_workload4_full_size_sampled():
    """MoE at hidden 4096 (8192 tokens, 384 experts, top-6, MXFP4) in the launch
    the benchmark times: routing checked whole; every stage checked on the
    tokens that reach each cold expert and the busiest experts' first and last
    tile rows."""
    case, exp = _full_case(4, "mx")
    _all_checks(case, exp)


@pytest.mark.timeout(600)
def test_moe_workload5_decode_all_tokens():
    """NVFP4 MoE at hidden 7168, decode batch of 64 tokens: every token checked
    at every stage."""
    case, exp = _full_case(5, "nv", all_tokens=True)
    _all_checks(case, exp)


@pytest.mark.timeout(900)
def test_moe_workload5_prefill_sampled():
    """NVFP4 MoE at hidden 7168 on a prefill batch of 16384 tokens (98,304
    routed slots, the 128-row wide NV tiles), in the launch the benchmark
    times: routing checked whole; every stage checked on the tokens that reach
    each cold expert and the busiest experts' first and last tile rows."""
    case, exp = _full_case(5, "nv", tokens=16384)
    _all_checks(case, exp)
