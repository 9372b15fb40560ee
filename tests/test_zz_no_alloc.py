"""The allocation-free routing entry point (fva_route_static, for callers that
cannot allocate device memory) against fva_route, through the C ABI: lists,
base counts, head totals and masks bit for bit, on two calls in a row, the
second with a smaller problem (the static scratch keeps the first call's
contents), into output buffers pre-filled with garbage."""
import numpy as np
import pytest
import torch

import block_sparse_attention_22_amd as fva
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _garbage_like(lists):
    def g(t):
        return None if t is None else torch.full_like(t, -7)
    return fva.BlockLists(row_ptr=g(lists.row_ptr), col_idx=g(lists.col_idx), base_count=g(lists.base_count),
                          head_kept=g(lists.head_kept), mask=g(lists.mask), nq=lists.nq, nk=lists.nk,
                          grid=lists.grid, tile=lists.tile, order=lists.order)


def test_route_static_matches_route():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    dev = torch.device("cuda:0")
    for cid in (4, 2):            # the 720p 5-head shard (33 MB of scratch), then the 12-head mid layer
        w = WORKLOADS[cid]
        print(f"\n[static] config {cid} {w.name}", flush=True)
        q, k, _, _ = make_inputs(w)
        qd, kd = q.to(dev), k.to(dev)
        ref = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile, want_mask=True)
        out = _garbage_like(ref)
        torch.cuda.synchronize()
        got = fva.route_static(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile, out=out)
        torch.cuda.synchronize()
        assert got is out
        n = int(ref.row_ptr[-1].item())
        assert torch.equal(out.row_ptr, ref.row_ptr)
        assert torch.equal(out.col_idx[:n], ref.col_idx[:n])
        assert torch.equal(out.base_count, ref.base_count)
        assert torch.equal(out.head_kept, ref.head_kept)
        assert torch.equal(out.mask, ref.mask)
        print(f"[static] config {cid}: {len(ref.row_ptr) - 1} rows, {n} kept blocks identical", flush=True)


def test_route_static_rejects_problems_above_its_scratch():
    dev = torch.device("cuda:0")
    w = WORKLOADS[3]          # 40 heads x 660 blocks: 264 MB of routing scratch
    q = torch.zeros((1, 40, w.N, 128), dtype=torch.bfloat16, device=dev)
    lists = fva.route(q, q, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    with pytest.raises(fva.FvaError) as e:
        fva.route_static(q, q, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile, out=lists)
    assert e.value.status == fva.FVA_ERR_SCRATCH
