"""MoE test support: build a case, run the library, and compute the oracle's
expectations from the seeded inputs alone (no GPU result is ever an oracle input).

Three checks:
  end to end   Q(X) and the routing metadata (counts, offsets, stable perm)
               exact; g, u within TOL * sum|a b| (only fp32 summation order is
               free); h must be the bf16 rounding of some value within eps_h of
               the exact SiLU(g) u, eps_h covering the allowed g/u error, an fp32
               SiLU (a few ulp) and the fp32 product.  Because the allowed g error
               makes many h positions legitimately round either way, the output
               of this run is reported as statistics (fraction inside the
               tolerance bracket, max error / bound) with a gross-error limit.
  gate/up stage  the oracle's g|u (rounded to fp32) are injected; h must equal
               the oracle's bf16 rounding of SiLU(g) u computed from the same
               fp32 values, except where that exact value lies within 4 fp32 ulp
               (8 * 2^-24 relative) of a bf16 rounding boundary (the kernel's
               fp32 exp, add, divide and multiply); those positions are counted
               and listed (token, choice, column); Q(h) must be bit-exact in
               every block without such a position.
  down stage   the oracle's Q(h) is injected; y within TOL * sum|h w2| and out
               inside the bf16 bracket of TOL * sum_j |w_j| sum|h w2|.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import block_scaled_fp4_mx_amd as F
import workloads as W
from oracle import formats as OF
from oracle import gemm as G
from oracle import moe as M
from oracle import quant as Q

DEV = "cuda"
TOL = 1e-5
SILU_DERIV_MAX = 1.1        # max |d/dz z sigmoid(z)| is about 1.0998


def blk_of(fmt):
    return 32 if fmt == "mx" else 16


class Case:
    def __init__(self, fmt, X_bits, ids, weights, E, H, I, experts, act_st=(None, None), wdev=None):
        self.fmt, self.X, self.ids, self.w = fmt, X_bits, ids, weights
        self.E, self.H, self.I = E, H, I
        self.T, self.topk = ids.shape
        self.experts = experts            # e -> (w13 bits [2I, H], w2 bits [H, I]) on the host
        self.wdev = wdev                  # e -> (w13, w2) bf16 device tensors (full-size cases)
        self.act_st = act_st
        if fmt == "nv" and act_st[0] is None:
            self.act_st = (np.float32(Q.nv_tensor_scale(X_bits)), None)


def device_weight_quant(case):
    """e -> oracle-quantized weights of the device-drawn expert e (its exact bf16
    read back to the host), for oracle_expect."""
    def q(e):
        a, b = case.wdev[e]
        a, b = W.bf16_bits(a), W.bf16_bits(b)
        if case.fmt == "mx":
            c1, s1 = Q.mx_quantize(a); c2, s2 = Q.mx_quantize(b); return c1, s1, None, c2, s2, None
        c1, s1, t1 = Q.nv_quantize(a); c2, s2, t2 = Q.nv_quantize(b)
        return c1, s1, t1, c2, s2, t2
    return q


def oracle_expert_quant(case):
    out = {}
    for e, (a, b) in case.experts.items():
        if case.fmt == "mx":
            c1, s1 = Q.mx_quantize(a); c2, s2 = Q.mx_quantize(b); t1 = t2 = None
        else:
            c1, s1, t1 = Q.nv_quantize(a); c2, s2, t2 = Q.nv_quantize(b)
        out[e] = (c1, s1, t1, c2, s2, t2)
    return out


def _ref_h(g, u):
    """Exact SiLU(g) u in fp64 and its bf16 rounding."""
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    hx = silu * u
    return silu, hx, OF.bf16_rne_of_f64(hx)


def _quant(fmt, hb, s_h):
    if fmt == "mx":
        c, s_ = Q.mx_quantize(hb); return c, s_, None
    return Q.nv_quantize(hb, s_t=s_h)


H_WINDOW = 8 * 2.0 ** -24    # 4 fp32 ulp (ulp <= 2^-23 |h|): SiLU's fp32 exp, add, divide and product


def _expert_stage1(fmt, I, wq, xc, xs, xst):
    """Gate/up of the token rows (xc, xs) routed to one expert: g, u, their
    bounds, the exact h and its window, and the injected-g|u stage's h."""
    c1, s1, t1 = wq[:3]
    gu, S = G.gemm_ref(fmt, xc, xs, c1, s1, xst, t1)
    g, u, Sg, Su = gu[:, :I], gu[:, I:], S[:, :I], S[:, I:]
    silu, hx, hb = _ref_h(g, u)
    eps = SILU_DERIV_MAX * TOL * Sg * np.abs(u) + np.abs(silu) * TOL * Su + H_WINDOW * np.abs(hx) + 2.0 ** -140
    g32, u32 = g.astype(np.float32), u.astype(np.float32)
    _, hx2, hb2 = _ref_h(g32.astype(np.float64), u32.astype(np.float64))
    eps2 = H_WINDOW * np.abs(hx2) + 2.0 ** -140
    return dict(g=g, u=u, Sg=Sg, Su=Su, h_bits=hb, h_lo=OF.bf16_rne_of_f64(hx - eps),
                h_hi=OF.bf16_rne_of_f64(hx + eps), g32=g32, u32=u32, hi_bits=hb2,
                hi_amb=OF.bf16_rne_of_f64(hx2 - eps2) != OF.bf16_rne_of_f64(hx2 + eps2),
                hmax=float(np.abs(OF.bf16_bits_to_f64(hb)).max()) if hb.size else 0.0)


def _expert_stage2(fmt, wq, hb, hb2, s_h):
    """Down stage of one expert's slots on the oracle's own Q(h), and Q of the
    injected-g|u stage's h."""
    c2, s2, t2 = wq[3:]
    hc, hs, hst = _quant(fmt, hb, s_h)
    y, Sy = G.gemm_ref(fmt, hc, hs, c2, s2, hst, t2)
    ic, is_, _ = _quant(fmt, hb2, s_h)
    return dict(h_codes=hc, h_scales=hs, y=y, Sy=Sy, hi_codes=ic, hi_scales=is_)


def oracle_expect(case, tokens, eq=None, threads=None, calibrate_h=False):
    """Per-slot expectations for the token subset `tokens`, computed expert by
    expert (each expert's weights quantized once, its slots batched), experts in
    parallel threads.  eq maps expert -> quantized weights, or is a callable
    e -> quantized weights (called once per expert).  calibrate_h (NV): set
    case.act_st[1] from the oracle's h over these tokens first, as a
    calibration would."""
    fmt, I, H, topk = case.fmt, case.I, case.H, case.topk
    eq = eq if eq is not None else oracle_expert_quant(case)
    get = eq if callable(eq) else eq.__getitem__
    tokens = np.asarray(tokens)
    s_x = case.act_st[0]
    if fmt == "mx":
        xc, xs = Q.mx_quantize(case.X[tokens]); xst = None
    else:
        xc, xs, xst = Q.nv_quantize(case.X[tokens], s_t=s_x)
    nt = len(tokens)
    ids = case.ids[tokens]
    valid = (ids >= 0) & (ids < case.E)
    experts = sorted(set(int(e) for e in ids[valid]))
    threads = threads or min(16, os.cpu_count() or 1)
    wq, st1 = {}, {}

    def one(e):
        ti, tj = np.nonzero(ids == e)
        q = get(e)
        with threadpool_limits(1):
            return e, q, (ti, tj), _expert_stage1(fmt, I, q, xc[ti], xs[ti], xst)

    with cf.ThreadPoolExecutor(threads) as ex:
        for e, q, idx, r in ex.map(one, experts):
            wq[e] = q[3:]
            st1[e] = (idx, r)
    if calibrate_h:
        hmax = max((r["hmax"] for _, r in st1.values()), default=0.0)
        case.act_st = (case.act_st[0], np.float32(hmax / 2688.0))
    s_h = case.act_st[1]

    def two(e):
        (ti, tj), r = st1[e]
        with threadpool_limits(1):
            return e, _expert_stage2(fmt, (None, None, None) + tuple(wq[e]), r["h_bits"], r["hi_bits"], s_h)

    with cf.ThreadPoolExecutor(threads) as ex:
        st2 = dict(ex.map(two, experts))
    shp = (nt, topk, I)
    res = dict(tokens=tokens, x_codes=xc, x_scales=xs, valid=valid,
               g=np.zeros(shp), u=np.zeros(shp), Sg=np.zeros(shp), Su=np.zeros(shp),
               h_lo=np.zeros(shp, np.uint16), h_hi=np.zeros(shp, np.uint16), h_bits=np.zeros(shp, np.uint16),
               g32=np.zeros(shp, np.float32), u32=np.zeros(shp, np.float32),
               hi_bits=np.zeros(shp, np.uint16), hi_amb=np.zeros(shp, bool),
               hi_codes=np.zeros((nt, topk, I // 2), np.uint8),
               hi_scales=np.zeros((nt, topk, I // blk_of(fmt)), np.uint8),
               h_codes=np.zeros((nt, topk, I // 2), np.uint8),
               h_scales=np.zeros((nt, topk, I // blk_of(fmt)), np.uint8),
               y=np.zeros((nt, topk, H)), Sy=np.zeros((nt, topk, H)),
               out_f64=np.zeros((nt, H)), bound=np.zeros((nt, H)))
    for e in experts:
        (ti, tj), r1 = st1[e]
        for k_, v in list(r1.items()) + list(st2[e].items()):
            if k_ != "hmax":
                res[k_][ti, tj] = v
    wts = np.asarray(case.w, np.float32).astype(np.float64)[tokens] * valid
    res["out_f64"] = np.einsum("tj,tjh->th", wts, res["y"])
    res["bound"] = np.einsum("tj,tjh->th", np.abs(wts), res["Sy"])
    return res


def run_gpu(case, fill_other_experts=False, seed=7, debug=True, inject=None, exp=None):
    """Run fp4_moe_grouped_gemm on the case.  Experts in `case.experts` are
    uploaded as bf16 and quantized by the library; other experts are zero (or
    device-random when fill_other_experts).  inject = "gate_up" or "h" feeds
    the oracle's per-slot values of `exp` for its tokens (zeros elsewhere)."""
    fmt, E, H, I, T, topk = case.fmt, case.E, case.H, case.I, case.T, case.topk
    blk = blk_of(fmt)
    fm = F.FMT_MX if fmt == "mx" else F.FMT_NV
    w13c = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
    w13s = torch.full((E, 2 * I, H // blk), 127 if fmt == "mx" else 0, dtype=torch.uint8, device=DEV)
    w2c = torch.zeros((E, H, I // 2), dtype=torch.uint8, device=DEV)
    w2s = torch.full((E, H, I // blk), 127 if fmt == "mx" else 0, dtype=torch.uint8, device=DEV)
    w13ts = torch.ones(E, dtype=torch.float32, device=DEV)
    w2ts = torch.ones(E, dtype=torch.float32, device=DEV)
    nvws = torch.empty(F.fp4_quantize_nv_workspace_bytes(1, 1), dtype=torch.uint8, device=DEV)

    def put(e, a, b):
        if fmt == "mx":
            F.fp4_quantize_mx(a, w13c[e], w13s[e])
            F.fp4_quantize_mx(b, w2c[e], w2s[e])
        else:
            F.fp4_quantize_nv(a, w13c[e], w13s[e], w13ts[e:e + 1], False, nvws)
            F.fp4_quantize_nv(b, w2c[e], w2s[e], w2ts[e:e + 1], False, nvws)

    if case.wdev is not None:
        for e, (a, b) in case.wdev.items():
            put(e, a, b)
    elif fill_other_experts:
        active = set(int(v) for v in np.unique(case.ids))
        for e, a, b in W.expert_weights_device(seed, E, H, I, DEV):
            if e in active and e not in case.experts:
                put(e, a, b)
    for e, (a, b) in case.experts.items():
        put(e, W.from_bits(a).to(DEV), W.from_bits(b).to(DEV))
    X = W.from_bits(case.X).to(DEV)
    ids = torch.from_numpy(np.ascontiguousarray(case.ids, np.int32)).to(DEV)
    wts = torch.from_numpy(np.ascontiguousarray(case.w, np.float32)).to(DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(F.fp4_moe_workspace_bytes(fm, T, H, topk, E, I), dtype=torch.uint8, device=DEV)
    act = None
    if fmt == "nv":
        act = torch.tensor([float(case.act_st[0]), float(case.act_st[1])], dtype=torch.float32, device=DEV)
    S = T * topk
    bufs = {}
    if debug:
        bufs = dict(
            x_codes=torch.empty((T, H // 2), dtype=torch.uint8, device=DEV),
            x_scales=torch.empty((T, H // blk), dtype=torch.uint8, device=DEV),
            counts=torch.empty(E, dtype=torch.int32, device=DEV),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
            perm=torch.empty(S, dtype=torch.int32, device=DEV),
            gate_up=torch.full((S, 2 * I), float("nan"), dtype=torch.float32, device=DEV),
            h_bf16=torch.zeros((S, I), dtype=torch.bfloat16, device=DEV),
            h_codes=torch.zeros((S, I // 2), dtype=torch.uint8, device=DEV),
            h_scales=torch.zeros((S, I // blk), dtype=torch.uint8, device=DEV),
            y=torch.full((S, H), float("nan"), dtype=torch.float32, device=DEV))
    ptrs = {k: v.data_ptr() for k, v in bufs.items()}
    keep = []
    if inject is not None:
        toks = exp["tokens"]
        slots = (toks[:, None] * topk + np.arange(topk)[None, :])
        if inject == "gate_up":
            gu = np.zeros((S, 2 * I), np.float32)
            gu[slots, :I] = exp["g32"]
            gu[slots, I:] = exp["u32"]
            t_ = torch.from_numpy(gu).to(DEV)
            keep.append(t_)
            ptrs["gate_up_in"] = t_.data_ptr()
        else:
            hc = np.zeros((S, I // 2), np.uint8); hs = np.zeros((S, I // blk), np.uint8)
            hc[slots] = exp["h_codes"]; hs[slots] = exp["h_scales"]
            tc, tsc = torch.from_numpy(hc).to(DEV), torch.from_numpy(hs).to(DEV)
            keep += [tc, tsc]
            ptrs["h_codes_in"], ptrs["h_scales_in"] = tc.data_ptr(), tsc.data_ptr()
    dbg = F.MoeDebug(**ptrs) if ptrs else None
    F.fp4_moe_grouped_gemm(fm, X, ids, wts, E, I, w13c, w13s, w2c, w2s, out, ws, w13ts if fmt == "nv" else None,
                           w2ts if fmt == "nv" else None, act, debug=dbg)
    torch.cuda.synchronize()
    res = {"out": W.bf16_bits(out)}
    for k, v in bufs.items():
        res[k] = W.bf16_bits(v) if v.dtype == torch.bfloat16 else v.cpu().numpy()
    return res


def _slots(case, exp):
    toks = exp["tokens"]
    return toks[:, None] * case.topk + np.arange(case.topk)[None, :]


def _out_bracket(exp):
    lo = OF.bf16_bits_to_f64(OF.bf16_rne_of_f64(exp["out_f64"] - TOL * exp["bound"]))
    hi = OF.bf16_bits_to_f64(OF.bf16_rne_of_f64(exp["out_f64"] + TOL * exp["bound"]))
    return lo, hi


def check_end_to_end(case, gpu, exp):
    fmt, I = case.fmt, case.I
    toks, valid = exp["tokens"], exp["valid"]
    assert np.array_equal(gpu["x_codes"][toks], exp["x_codes"]), "Q(X) codes differ"
    assert np.array_equal(gpu["x_scales"][toks], exp["x_scales"]), "Q(X) scales differ"
    ids = np.where((case.ids >= 0) & (case.ids < case.E), case.ids, case.E)
    counts, offsets, perm = M.routing_metadata(ids, case.E + 1)
    assert np.array_equal(gpu["counts"], counts[:case.E]), "expert counts differ"
    assert np.array_equal(gpu["offsets"], offsets[:case.E + 1]), "expert offsets differ"
    nvalid = int(offsets[case.E])
    assert np.array_equal(gpu["perm"][:nvalid], perm[:nvalid]), "routing permutation differs"
    slots = _slots(case, exp)
    gu = gpu["gate_up"][slots]
    eg = np.abs(gu[..., :I] - exp["g"]) <= TOL * exp["Sg"]
    eu = np.abs(gu[..., I:] - exp["u"]) <= TOL * exp["Su"]
    bad = ~(eg & eu) & valid[..., None]
    assert not bad.any(), f"g/u outside tolerance at {np.argwhere(bad)[:5]}"
    h = OF.bf16_bits_to_f64(gpu["h_bf16"][slots])
    lo, hi = OF.bf16_bits_to_f64(exp["h_lo"]), OF.bf16_bits_to_f64(exp["h_hi"])
    hv = ((h >= np.minimum(lo, hi)) & (h <= np.maximum(lo, hi))) | ~valid[..., None]
    assert hv.all(), f"h is not a rounding of SiLU(g)u within eps_h at {np.argwhere(~hv)[:5]}"
    o = OF.bf16_bits_to_f64(gpu["out"][toks])
    blo, bhi = _out_bracket(exp)
    inside = (o >= blo) & (o <= bhi)
    err = np.abs(o - exp["out_f64"])
    rel_l2 = float(np.linalg.norm(o - exp["out_f64"]) / max(np.linalg.norm(exp["out_f64"]), 1e-300))
    stats = dict(h_equal_fraction=float((gpu["h_bf16"][slots] == exp["h_bits"])[valid].mean()),
                 out_within_tol_fraction=float(inside.mean()),
                 out_max_err_over_bound=float((err / np.maximum(exp["bound"], 1e-300)).max()),
                 out_rel_l2=rel_l2)
    assert rel_l2 < 1e-2, f"end-to-end output far from the oracle: {stats}"
    return stats


def check_gate_up_stage(case, gpu, exp):
    fmt, I = case.fmt, case.I
    valid = exp["valid"]
    slots = _slots(case, exp)
    h = gpu["h_bf16"][slots]
    ok = (h == exp["hi_bits"]) | exp["hi_amb"] | ~valid[..., None]
    assert ok.all(), f"h differs at {np.argwhere(~ok)[:5]}"
    blk = blk_of(fmt)
    nt, k = valid.shape
    bamb = exp["hi_amb"].reshape(nt, k, I // blk, blk).any(-1) | ~valid[..., None]
    gc = Q.unpack_nibbles(gpu["h_codes"][slots].reshape(-1, I // 2)).reshape(nt, k, I // blk, blk)
    ec = Q.unpack_nibbles(exp["hi_codes"].reshape(-1, I // 2)).reshape(nt, k, I // blk, blk)
    gs = gpu["h_scales"][slots]
    assert np.array_equal(gs[~bamb], exp["hi_scales"][~bamb]), "Q(h) scales differ"
    assert np.array_equal(gc[~bamb], ec[~bamb]), "Q(h) codes differ"
    amb = np.argwhere(exp["hi_amb"] & valid[..., None])
    return dict(h_ambiguous=len(amb), h_ambiguous_at=[(int(exp["tokens"][t]), int(j), int(c)) for t, j, c in amb[:20]],
                h_checked=int(valid.sum()) * I, blocks_checked=int((~bamb).sum()))


def check_down_stage(case, gpu, exp):
    valid = exp["valid"]
    slots = _slots(case, exp)
    y = gpu["y"][slots]
    ok = (np.abs(y - exp["y"]) <= TOL * exp["Sy"]) | ~valid[..., None]
    assert ok.all(), f"y outside tolerance at {np.argwhere(~ok)[:5]}"
    o = OF.bf16_bits_to_f64(gpu["out"][exp["tokens"]])
    lo, hi = _out_bracket(exp)
    inside = (o >= lo) & (o <= hi)
    assert inside.all(), f"out outside tolerance at {np.argwhere(~inside)[:5]}"
    return dict(out_checked=int(inside.size))
