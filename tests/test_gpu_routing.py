"""GPU parity of the MoE routing metadata (expert counts, exclusive offsets and
the stable slot permutation) against the oracle's definition, over expert
counts from 7 to 1024 and batches of 3 to 313 routing blocks of 512 slots
(whole and partial batches of the scan's 16-block loads).  Expert ids are
skewed (most slots on a few experts) and about 1% are outside [0, E), which
routes those slots nowhere.  The GEMMs run on all-zero weights at the smallest
hidden/intermediate sizes; only the routing is checked."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import block_scaled_fp4_mx_amd as F
from oracle import moe as M

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROUTE_SLOTS = 512      # slots per routing block of the device scan


def _skewed_ids(rng, T, k, E):
    w = 1.0 / np.arange(1, E + 1) ** 1.1
    ids = rng.choice(E, size=(T, k), p=w / w.sum()).astype(np.int32)
    bad = rng.random((T, k)) < 0.01
    ids[bad] = rng.choice(np.array([-1, E, E + 7], np.int32), size=int(bad.sum()))
    return ids


@pytest.mark.parametrize("E,T,k,H", [
    (384, 8192, 6, 128),     # 96 routing blocks
    (7, 3000, 3, 128),       # 18 blocks, 7 experts
    (1024, 20000, 8, 128),   # 313 blocks, the most experts
    (300, 16384, 6, 128),    # 192 blocks
    (520, 8000, 6, 128),     # 94 blocks
    (64, 600, 2, 128),       # 3 blocks
    (100, 4000, 8, 128),     # 63 blocks
    (33, 20000, 8, 128),     # 313 blocks, 33 experts
    (384, 8192, 6, 512),     # 256-row tiles (the MX tile path's tile list)
])
def test_routing_metadata_exact(E, T, k, H):
    S = T * k
    nblk = -(-S // ROUTE_SLOTS)
    print(f"routing E={E} T={T} topk={k} H={H}: {nblk} routing blocks", flush=True)
    rng = np.random.default_rng(5000 + E + T)
    ids = _skewed_ids(rng, T, k, E)
    I = H
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    idt = torch.from_numpy(ids).to(DEV)
    wts = torch.full((T, k), 1.0 / k, dtype=torch.float32, device=DEV)
    w13c = torch.zeros((E, 2 * I, H // 2), dtype=torch.uint8, device=DEV)
    w13s = torch.full((E, 2 * I, H // 32), 127, dtype=torch.uint8, device=DEV)
    w2c = torch.zeros((E, H, I // 2), dtype=torch.uint8, device=DEV)
    w2s = torch.full((E, H, I // 32), 127, dtype=torch.uint8, device=DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(F.fp4_moe_workspace_bytes(F.FMT_MX, T, H, k, E, I), dtype=torch.uint8, device=DEV)
    counts = torch.full((E,), -1, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device=DEV)
    perm = torch.full((S,), -1, dtype=torch.int32, device=DEV)
    dbg = F.MoeDebug(counts=counts.data_ptr(), offsets=offsets.data_ptr(), perm=perm.data_ptr())
    F.fp4_moe_grouped_gemm(F.FMT_MX, x, idt, wts, E, I, w13c, w13s, w2c, w2s, out, ws, debug=dbg)
    torch.cuda.synchronize()

    mapped = np.where((ids >= 0) & (ids < E), ids, E)
    ec, eo, ep = M.routing_metadata(mapped, E + 1)
    nvalid = int(eo[E])
    assert np.array_equal(counts.cpu().numpy(), ec[:E]), "expert counts differ"
    assert np.array_equal(offsets.cpu().numpy(), eo[:E + 1]), "expert offsets differ"
    assert np.array_equal(perm.cpu().numpy()[:nvalid], ep[:nvalid]), "routing permutation differs"
    assert not torch.isnan(out.float()).any()
