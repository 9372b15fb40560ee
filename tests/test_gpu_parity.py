"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every workload runs at its full size in the launch configuration the bench
times (default balancer options).  Block lists are compared in full; outputs
on every row for the small workloads and on a seeded sample of query blocks
per head for the 75,600- and 171,360-token layers.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_22_amd as fva
from oracle import BlockLayout, HilbertLayout, attention, routing
from workloads import WORKLOADS, make_inputs, sample_qblocks, tiny_random

from parity import assert_exact, attention_error, compare_lists, gpu_lists_to_host, to_numpy

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}
SAMPLE = {1: None, 2: None, 3: 16, 4: 16, 5: 64}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _rows_sample(w, nb, n):
    if n is None:
        return None
    rng = np.random.default_rng((260716190, w.cid, 1))
    return {bh: np.sort(rng.choice(nb, min(n, nb), replace=False)) for bh in range(w.B * w.H)}


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_parity(dev, cid):
    w = WORKLOADS[cid]
    print(f"\n[parity] config {cid} {w.name}: generating", flush=True)
    q, k, v, _ = make_inputs(w)
    lay = BlockLayout(w.grid, w.tile)
    npdt = np.float64 if cid <= 2 else np.float32
    qn, kn, vn = (to_numpy(t, npdt) for t in (q, k, v))
    ref = routing.route(qn, kn, lay, w.p, w.kmin, w.budget)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    print(f"[parity] config {cid}: route on GPU", flush=True)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    g = gpu_lists_to_host(lists)
    rep = compare_lists(g, ref, w.p, w.budget, lay, w.B, w.H)
    print(f"[parity] config {cid}: lists {rep}", flush=True)
    assert_exact(rep)
    # determinism of the routing
    lists2 = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    g2 = gpu_lists_to_host(lists2)
    assert np.array_equal(g["row_ptr"], g2["row_ptr"]) and np.array_equal(g["col_idx"], g2["col_idx"])

    print(f"[parity] config {cid}: attention on GPU", flush=True)
    o = fva.sparse_attn(qd, kd, vd, lists)
    st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile), dtype=torch.uint8, device=dev)
    o2 = fva.sparse_attn(qd, kd, vd, lists, stats=st)
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "attention is not deterministic"
    # the library's count of kept valid token pairs (the flop count) against the oracle's
    info, _ = fva.parse_stats(st)
    pairs, _ = attention.kept_pairs(lay, g["row_ptr"], g["col_idx"], lay.Nb)
    print(f"[parity] config {cid}: kept pairs {info.kept_pairs} (oracle {pairs})", flush=True)
    assert info.kept_pairs == pairs
    rows = _rows_sample(w, lay.Nb, SAMPLE[cid])
    prec = "fp64" if cid <= 2 else "fp32"
    err = attention_error(o, qn, kn, vn, lay, g["row_ptr"], g["col_idx"], rows=rows, precision=prec)
    print(f"[parity] config {cid}: max|o - oracle| = {err:.3e} (tol {TOL[w.dtype]})", flush=True)
    assert err <= TOL[w.dtype]


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _oracle_errors(tmp_path, cid, lay, q, k, v, o, g, rows, hilbert=False):
    """|o - oracle| of every query block in ``rows`` [(b*H + h, i), ...],
    computed by tests/oracle_pool.py in a child process (a pool of CPU
    workers); returns (errors in the order of rows, worker count)."""
    stem = str(tmp_path / f"c{cid}")
    for n, t in (("q", q), ("k", k), ("v", v)):
        np.save(f"{stem}_{n}.npy", t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16
                else t.numpy())
    H = q.shape[1]
    parts = []
    for bh, i in rows:
        b, h = divmod(bh, H)
        parts.append(torch.as_tensor(lay.members[i], device=o.device) + (b * H + h) * lay.N)
    flat = o.reshape(-1, o.shape[-1])
    out = flat.index_select(0, torch.cat(parts)).float().cpu().numpy()
    np.savez(f"{stem}.npz", cid=cid, hilbert=int(hilbert), row_ptr=g["row_ptr"], col_idx=g["col_idx"],
             rows=np.asarray(rows, dtype=np.int64), out=out)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "oracle_pool.py"), f"{stem}.npz"],
                       capture_output=True, text=True, timeout=1500)
    assert r.returncode == 0, r.stderr[-3000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    return np.asarray(res["err"]), res["processes"]


def test_shard_outputs_on_every_row(dev, tmp_path):
    """The 720p 5-head shard (every head dense after the match-max budget):
    every output of all 3,300 query blocks against the oracle, on the GPU's
    own lists, in the launch configuration the bench times."""
    w = WORKLOADS[4]
    q, k, v, _ = make_inputs(w)
    lay = BlockLayout(w.grid, w.tile)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    o = fva.sparse_attn(qd, kd, vd, lists)
    torch.cuda.synchronize()
    g = gpu_lists_to_host(lists)
    rows = [(bh, i) for bh in range(w.B * w.H) for i in range(lay.Nb)]
    err, nproc = _oracle_errors(tmp_path, 4, lay, q, k, v, o, g, rows)
    per_head = err.reshape(w.B * w.H, lay.Nb).max(axis=1)
    print(f"\n[shard] {len(rows)} query blocks on {nproc} processes: max|o - oracle| per head "
          f"{[f'{x:.2e}' for x in per_head]}", flush=True)
    assert err.max() <= TOL["bf16"]


def _pair_leads(sizes):
    """First blocks of the greedy pairs of neighbouring <= 64-token blocks."""
    small = np.asarray(sizes) <= 64
    lead, i = [], 0
    while i < len(small) - 1:
        if small[i] and small[i + 1]:
            lead.append(i)
            i += 2
        else:
            i += 1
    return lead


def test_720p_outputs_on_every_special_row(dev, tmp_path):
    """The 720p layer where the kernel takes its special paths: every row the
    plan splits into chunks, one paired item per head (both rows), every edge
    class of query block (40, 64, 80 and 128 tokens; two rows of each per
    head), plus the seeded sample of 16 rows per head; worst error per class."""
    w = WORKLOADS[3]
    q, k, v, _ = make_inputs(w)
    lay = BlockLayout(w.grid, w.tile)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile), dtype=torch.uint8, device=dev)
    o = fva.sparse_attn(qd, kd, vd, lists, stats=st)
    torch.cuda.synchronize()
    info, _ = fva.parse_stats(st)
    g = gpu_lists_to_host(lists)
    rp, ci, nb, H = g["row_ptr"], g["col_idx"], lay.Nb, w.B * w.H
    C = info.chunk_blocks
    counts = np.diff(rp).reshape(H, nb)
    leads = _pair_leads(lay.sizes)
    rng = np.random.default_rng((260716190, 3, 7))
    cls = {}
    for bh in range(H):
        paired = set()
        for i in leads:
            r = bh * nb + i
            if len(np.union1d(ci[rp[r]:rp[r + 1]], ci[rp[r + 1]:rp[r + 2]])) <= C:
                paired |= {i, i + 1}
        for i in range(nb):
            if counts[bh, i] > C and i not in paired:
                cls.setdefault((bh, i), "split")
        if paired:
            i0 = min(paired)
            cls.setdefault((bh, i0), "paired")
            cls.setdefault((bh, i0 + 1), "paired")
        for size in (40, 64, 80, 128):
            cand = np.nonzero(lay.sizes == size)[0]
            for i in rng.choice(cand, min(2, len(cand)), replace=False):
                cls.setdefault((bh, int(i)), f"edge{size}")
    for bh, sel in _rows_sample(w, nb, SAMPLE[3]).items():
        for i in sel:
            cls.setdefault((bh, int(i)), "sample")
    n_split = sum(1 for c in cls.values() if c == "split")
    assert n_split == info.n_split_rows, (n_split, info.n_split_rows)
    rows = sorted(cls)
    err, nproc = _oracle_errors(tmp_path, 3, lay, q, k, v, o, g, rows)
    worst = {}
    for rc, e in zip(rows, err):
        worst[cls[rc]] = max(worst.get(cls[rc], 0.0), float(e))
    counts_by = {c: sum(1 for x in cls.values() if x == c) for c in worst}
    print(f"\n[720p special rows] {len(rows)} query blocks on {nproc} processes; worst |o - oracle| by class: "
          + ", ".join(f"{c} ({counts_by[c]} rows) {worst[c]:.2e}" for c in sorted(worst)), flush=True)
    assert set(worst) >= {"split", "paired", "edge40", "edge64", "edge80", "edge128"}
    assert max(worst.values()) <= TOL["bf16"]


@pytest.mark.parametrize("grid,tile,H", [((5, 20, 20), (2, 8, 8), 3), ((8, 128, 128), (1, 8, 8), 1)],
                         ids=["27_blocks", "2048_blocks"])
def test_route_mask_matches_the_lists(dev, grid, tile, H):
    """The materialised mask (want_mask): bit j of row r is set exactly when
    block j is in the row's CSR list, and no bit at or past Nk is set; on a
    ragged grid (one partial word) and at 2,048 blocks (64 words)."""
    q, k, _ = _small_case(grid, tile, H, 128, "bf16", 160, scale=2.0)
    lay = BlockLayout(grid, tile)
    lists = fva.route(q.to(dev), k.to(dev), 0.8, 2, ("frac", 0.1), grid=grid, tile=tile, want_mask=True)
    g = gpu_lists_to_host(lists)
    nb = lay.Nb
    words = (nb + 31) // 32
    R = H * nb
    mask = lists.mask[: R * words].cpu().numpy().view(np.uint32).reshape(R, words)
    bits = np.unpackbits(mask.view(np.uint8).reshape(R, words, 4)[..., ::-1], axis=-1)[..., ::-1]
    bits = bits.reshape(R, words * 32)             # bits[r, j] = bit j of row r
    for r in range(R):
        expect = np.zeros(words * 32, dtype=np.uint8)
        expect[g["col_idx"][g["row_ptr"][r]:g["row_ptr"][r + 1]]] = 1
        assert np.array_equal(bits[r], expect), r
    assert not bits[:, nb:].any()


def test_equal_load_plan_balances_exactly(dev):
    """A synthetic equal-load plan: 64 heads of 256 full blocks, every row
    keeping the same 4 blocks, rows never split, so that each workgroup gets
    32 equal items from the queues.  The plan's own prediction is exactly 1
    and the measured per-CU imbalance stays within the 1.10 bound (a
    workgroup that starts late leaves at most an item or so to the others)."""
    grid, tile, H = (8, 64, 64), (2, 8, 8), 64             # 4 x 8 x 8 = 256 blocks of 128 tokens
    q, k, v = (t.to(dev) for t in _small_case(grid, tile, H, 128, "bf16", 170))
    nb = 256
    st = torch.zeros(fva.stats_bytes(q, grid, tile, chunk_blocks=-1), dtype=torch.uint8, device=dev)
    R = H * nb
    rp = np.arange(R + 1, dtype=np.int64) * 4
    ci = np.concatenate([np.arange(4) * 64 + (r % 64) for r in range(R)])
    lists = fva.lists_from_csr(rp, ci, nq=nb, grid=grid, tile=tile, device=dev)
    fva.sparse_attn(q, k, v, lists, chunk_blocks=-1, row_pairs=False)     # warm-up
    fva.sparse_attn(q, k, v, lists, chunk_blocks=-1, row_pairs=False, stats=st)
    torch.cuda.synchronize()
    info, ctas = fva.parse_stats(st)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    assert R % info.num_ctas == 0 and info.n_items == R
    imb, busy = fva.per_cu_imbalance(ctas, ncu)
    print(f"\n[equal load] {R} items on {info.num_ctas} workgroups: predicted {info.predicted_imbalance:.4f}, "
          f"measured per-CU {imb:.4f}", flush=True)
    assert info.predicted_imbalance == 1.0
    assert imb <= 1.10


def _host_plan_counts(rp, ci, Nb, BH, C, sizes, pairs_on):
    """The balancer's counts recomputed on the host from the lists, by the rule
    the plan states: a row of more than C kept blocks becomes ceil(cnt / C)
    work items, each with a partial slot; with row pairs, neighbouring query
    blocks of at most 64 tokens are paired two by two from the start of each
    run of such blocks, and a pair is one item when its union list holds at
    most C blocks.  Returns (items, partial slots, split rows, pairs)."""
    firsts = []
    if pairs_on:
        i = 0
        while i < Nb - 1:
            if sizes[i] <= 64 and sizes[i + 1] <= 64:
                firsts.append(i)
                i += 2
            else:
                i += 1
    items = parts = splits = npairs = 0
    for bh in range(BH):
        paired = set()
        for i in firsts:
            r = bh * Nb + i
            union = set(ci[rp[r]:rp[r + 1]].tolist()) | set(ci[rp[r + 1]:rp[r + 2]].tolist())
            if len(union) <= C:
                paired.update((i, i + 1))
                npairs += 1
                items += 1
        for i in range(Nb):
            if i in paired:
                continue
            r = bh * Nb + i
            cnt = int(rp[r + 1] - rp[r])
            n = -(-cnt // C) if cnt > C else 1
            items += n
            if n > 1:
                splits += 1
                parts += n
    return items, parts, splits, npairs


@pytest.mark.parametrize("cid", [2, 4])
def test_plan_counts_match_host(dev, cid):
    """The plan's work-item, split-row, partial-slot and pair counts, its chunk
    size and its total equal the balancer rule applied on the host to the
    GPU's own lists: every chunk mode (automatic, unsplit, fixed 1, 3 and 7
    blocks) with row pairs on and off on the mid size, and the automatic mode
    on the 5-head 720p shard, whose long rows are split."""
    w = WORKLOADS[cid]
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lay = BlockLayout(w.grid, w.tile)
    sizes = [len(m) for m in lay.members]
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    g = gpu_lists_to_host(lists)
    rp, ci = g["row_ptr"], g["col_idx"]
    BH = w.B * w.H
    modes = [(0, True), (0, False), (-1, True), (-1, False), (1, False), (3, False), (7, False)] if cid == 2 \
        else [(0, True)]
    for chunk, pairs in modes:
        st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile, chunk_blocks=chunk), dtype=torch.uint8, device=dev)
        fva.sparse_attn(qd, kd, vd, lists, stats=st, chunk_blocks=chunk, row_pairs=pairs)
        torch.cuda.synchronize()
        info, _ = fva.parse_stats(st)
        total = int(rp[-1])
        C = {0: max(16, -(-total // (8 * info.num_ctas))), -1: 2 ** 31 - 1}.get(chunk, chunk)
        items, parts, splits, npairs = _host_plan_counts(rp, ci, lay.Nb, BH, C, sizes, pairs and chunk <= 0)
        got = (info.n_items, info.n_partials, info.n_split_rows, info.n_row_pairs, info.chunk_blocks,
               info.total_blocks)
        print(f"\n[plan] config {cid} chunk {chunk} pairs {pairs}: {got}", flush=True)
        assert got == (items, parts, splits, npairs, C, total), (chunk, pairs, got)
        if cid == 4:
            assert splits > 0


def _small_case(grid, tile, H, d, dtype, seed, scale=1.0, B=1):
    N = grid[0] * grid[1] * grid[2]
    q = tiny_random((B, H, N, d), seed, dtype, scale)
    k = tiny_random((B, H, N, d), seed + 1, dtype, scale)
    v = tiny_random((B, H, N, d), seed + 2, dtype)
    return q, k, v


def _run_and_check(dev, q, k, v, grid, tile, p, kmin, budget, tol, chunk=0, strided=False, hilbert=False):
    from oracle import HilbertLayout
    lay = HilbertLayout(grid) if hilbert else BlockLayout(grid, tile)
    blk = dict(grid=grid, order=fva.hilbert_order(grid, dev)) if hilbert else dict(grid=grid, tile=tile)
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    B, H = q.shape[:2]
    ref = routing.route(qn, kn, lay, p, kmin, budget)
    if strided:     # views whose token stride is wider than the head dimension
        d = q.shape[-1]
        def wide(t):
            big = torch.zeros(t.shape[:-1] + (d + 64,), dtype=t.dtype, device=dev)
            big[..., :d] = t.to(dev)
            return big[..., :d]
        qd, kd, vd = wide(q), wide(k), wide(v)
    else:
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, p, kmin, budget, **blk)
    g = gpu_lists_to_host(lists)
    compare_lists(g, ref, p, budget, lay, B, H)
    out = wide(torch.zeros_like(q)) if strided else torch.empty_like(qd)
    o = fva.sparse_attn(qd, kd, vd, lists, out=out, chunk_blocks=chunk)
    assert o.data_ptr() == out.data_ptr()
    torch.cuda.synchronize()
    err = attention_error(o, qn, kn, vn, lay, g["row_ptr"], g["col_idx"])
    assert err <= tol, err
    return g, o, ref


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128), ("fp32", 64)])
def test_p_one_is_dense_attention(dev, dtype, d):
    grid, tile = (3, 20, 20), (2, 8, 8)          # 18 blocks, ragged on every axis
    q, k, v = _small_case(grid, tile, 2, d, dtype, 50)
    g, o, _ = _run_and_check(dev, q, k, v, grid, tile, 1.0, 0, ("none", 0.0), TOL[dtype])
    nb = BlockLayout(grid, tile).Nb
    assert np.all(np.diff(g["row_ptr"]) == nb)
    # dense reference: torch CPU scaled_dot_product_attention in float64
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double())
    assert (o.double().cpu() - ref).abs().max().item() <= TOL[dtype]


@pytest.mark.parametrize("grid,tile,p,kmin,budget", [
    ((1, 5, 5), (2, 8, 8), 0.9, 4, ("none", 0.0)),            # one partial block: the whole grid
    ((2, 16, 16), (1, 8, 8), 1e-12, 3, ("none", 0.0)),        # p -> 0+: fixed Top-3
    ((2, 16, 16), (1, 8, 8), 0.5, 50, ("none", 0.0)),         # floor above the block count
    ((4, 24, 24), (2, 8, 8), 0.6, 1, ("frac", 1e6)),          # budget capped at every block
    ((4, 24, 40), (2, 8, 8), 0.8, 2, ("match_max", 0.0)),
    ((3, 13, 21), (2, 4, 8), 0.7, 2, ("frac", 0.25)),         # 64-token tiles, ragged
    ((5, 9, 11), (1, 3, 5), 0.9, 1, ("frac", 0.5)),           # 15-token tiles
])
def test_edge_cases(dev, grid, tile, p, kmin, budget):
    q, k, v = _small_case(grid, tile, 3, 128, "bf16", 60, scale=2.0)
    g, _, _ = _run_and_check(dev, q, k, v, grid, tile, p, kmin, budget, TOL["bf16"])
    nb = BlockLayout(grid, tile).Nb
    counts = np.diff(g["row_ptr"])
    if p < 1e-6:
        assert np.all(counts == min(nb, max(kmin, 1)))
    if kmin >= nb or budget[1] >= 1e6:
        assert np.all(counts == nb)


@pytest.mark.parametrize("case", ["constant_keys", "duplicate_block"])
def test_tied_masses_follow_block_order(dev, case):
    """Equal routing masses are ordered by the lower block index (the routing
    sort's keys carry the index below the mass, so exact ties come out in
    index order from the first pass).
    constant_keys: every mass of every row is equal, and p = 0.5 falls on a
    sum that is exact in floating point; duplicate_block: key block 5 is a
    copy of key block 2, so every row holds one tie."""
    grid, tile, H = (4, 16, 16), (1, 8, 8), 2          # 16 blocks of 64 tokens
    q, k, v = _small_case(grid, tile, H, 128, "bf16", 80, scale=2.0)
    lay = BlockLayout(grid, tile)
    if case == "constant_keys":
        k = torch.full_like(k, 0.25)
        p, kmin, budget = 0.5, 1, ("frac", 0.25)
    else:
        members = lay.members
        k[:, :, torch.as_tensor(members[5])] = k[:, :, torch.as_tensor(members[2])]
        p, kmin, budget = 0.8, 2, ("frac", 0.2)
    qn, kn = to_numpy(q), to_numpy(k)
    ref = routing.route(qn, kn, lay, p, kmin, budget)
    lists = fva.route(q.to(dev), k.to(dev), p, kmin, budget, grid=grid, tile=tile)
    g = gpu_lists_to_host(lists)
    rep = compare_lists(g, ref, p, budget, lay, 1, H)
    print(f"\n[ties] {case}: {rep}", flush=True)
    assert rep["exact_rows"] == rep["rows"]
    if case == "constant_keys":
        counts = np.diff(g["row_ptr"]).reshape(H, lay.Nb)
        base = lists.base_count[: H * lay.Nb].cpu().numpy().reshape(H, lay.Nb)
        assert np.all(base == 8)                       # 8 of 16 equal masses reach 0.5
        for h in range(H):                             # every row keeps a prefix of the block order
            for i in range(lay.Nb):
                cols = g["col_idx"][g["row_ptr"][h * lay.Nb + i]:g["row_ptr"][h * lay.Nb + i + 1]]
                assert list(cols) == list(range(counts[h, i]))


@pytest.mark.parametrize("grid,H,big", [((4, 16, 16), 2, 20.0), ((4, 160, 128), 1, 60.0)],
                         ids=["16_blocks", "1280_blocks"])
def test_near_tied_masses_take_the_exact_order(dev, grid, H, big):
    """Two masses that agree in all but the low 11 bits of their bit patterns:
    key block 5 is key block 2 with one coordinate of one token raised by one
    float32 ulp (1 -> 1 + 2^-23), along a query coordinate that is 3e-4
    everywhere, so block 5 holds the larger mass in every row by a relative
    5e-14 or so (far above fp64 rounding of the scores, below 2^-41).  The
    routing sort's first pass orders on a key truncated to the high 53 bits,
    which puts the lower index first in most rows; the exact order must win.
    With p below the top mass and no augmentation each row keeps exactly one
    block, so a misorder changes it.  16 blocks sort one slot per lane, 1,280
    blocks 32 slots per lane."""
    tile = (1, 8, 8)                                   # blocks of 64 tokens
    q, k, v = _small_case(grid, tile, H, 128, "fp32", 90)
    lay = BlockLayout(grid, tile)
    m2, m5 = (torch.as_tensor(lay.members[j]) for j in (2, 5))
    q[..., 0] = q[..., 0].abs() + 1.0
    q[..., 1] = 3e-4
    k[:, :, m2, 0] = big
    k[:, :, m2, 1] = 1.0
    k[:, :, m5] = k[:, :, m2]
    k[:, :, m5[0], 1] = float(np.nextafter(np.float32(1.0), np.float32(2.0)))
    p, kmin, budget = 0.2, 1, ("none", 0.0)
    qn, kn = to_numpy(q), to_numpy(k)
    ref = routing.route(qn, kn, lay, p, kmin, budget)
    for hd in ref["heads"][0]:
        P = hd["P"]
        assert np.all(P[:, 5] > P[:, 2]) and np.all(np.abs(P[:, 5] / P[:, 2] - 1) < 1e-13)
        assert np.all(hd["base"] == 1)
    lists = fva.route(q.to(dev), k.to(dev), p, kmin, budget, grid=grid, tile=tile)
    g = gpu_lists_to_host(lists)
    rep = compare_lists(g, ref, p, budget, lay, 1, H)
    print(f"\n[near ties] {rep}", flush=True)
    assert rep["exact_rows"] == rep["rows"]
    assert np.all(np.diff(g["row_ptr"]) == 1) and np.all(g["col_idx"][: H * lay.Nb] == 5)


def test_masses_down_to_denormals_and_zeros(dev):
    """Routing masses spanning the whole fp64 range: every query block scores
    key block j at -90 j, so its masses are e^(-90 j) / sum: normal down to
    j = 7, a denormal at j = 8 (e^-720) and exact zeros beyond.  With p = 0.9,
    a floor of 2 and a budget of 5x the base count, augmentation takes every
    row's j = 2..8 and then 16 of the 112 equal zero masses, which go to the
    lowest rows first (ties to lower (i, j)): rows 0 and 1 take all 7 of
    theirs and row 2 takes 2."""
    grid, tile, H = (4, 16, 16), (1, 8, 8), 1           # 16 blocks of 64 tokens
    lay = BlockLayout(grid, tile)
    N = grid[0] * grid[1] * grid[2]
    q = torch.zeros((1, H, N, 128), dtype=torch.float32)
    k = torch.zeros_like(q)
    q[..., 0] = 1.0
    for j in range(lay.Nb):
        k[:, :, torch.as_tensor(lay.members[j]), 0] = -90.0 * j * np.sqrt(128.0)
    p, kmin, budget = 0.9, 2, ("frac", 4.0)
    ref = routing.route(to_numpy(q), to_numpy(k), lay, p, kmin, budget)
    P = ref["heads"][0][0]["P"]
    assert 0 < P[0, 8] < np.finfo(np.float64).tiny and np.all(P[:, 9:] == 0) and P[0, 7] >= np.finfo(np.float64).tiny
    lists = fva.route(q.to(dev), k.to(dev), p, kmin, budget, grid=grid, tile=tile)
    g = gpu_lists_to_host(lists)
    rep = compare_lists(g, ref, p, budget, lay, 1, H)
    print(f"\n[denormals] {rep}", flush=True)
    assert rep["exact_rows"] == rep["rows"]
    counts = np.diff(g["row_ptr"])
    assert list(counts[:4]) == [16, 16, 11, 9] and np.all(counts[3:] == 9)


def test_batch_and_strided_views(dev):
    grid, tile = (3, 16, 24), (2, 8, 8)
    q, k, v = _small_case(grid, tile, 3, 128, "bf16", 70, scale=2.0, B=2)
    _run_and_check(dev, q, k, v, grid, tile, 0.85, 2, ("match_max", 0.0), TOL["bf16"], strided=True)
    qf, kf, vf = _small_case(grid, tile, 2, 64, "fp32", 71, scale=2.0, B=2)
    _run_and_check(dev, qf, kf, vf, grid, tile, 0.85, 2, ("frac", 0.3), TOL["fp32"], strided=True)


@pytest.mark.parametrize("cid,dtype,chunks", [(2, "bf16", (-1, 0, 3, 7)), (1, "fp32", (-1, 0, 3, 1))])
def test_balancer_does_not_change_results(dev, cid, dtype, chunks):
    """Splitting rows into work items changes where work runs, not what is kept
    or computed (within float32 merge rounding)."""
    w = WORKLOADS[cid]
    q, k, v, _ = make_inputs(w)
    lay = BlockLayout(w.grid, w.tile)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    outs = {}
    for chunk in chunks:
        st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile, chunk_blocks=chunk), dtype=torch.uint8, device=dev)
        outs[chunk] = fva.sparse_attn(qd, kd, vd, lists, chunk_blocks=chunk, stats=st)
        torch.cuda.synchronize()
        info, _ = fva.parse_stats(st)
        R = w.B * w.H * lay.Nb
        if chunk == -1:
            assert info.n_items == R - info.n_row_pairs and info.n_partials == 0
        if chunk in (1, 3):
            assert info.n_partials > 0 and info.n_items > R
            assert info.chunk_blocks == chunk
    # bf16: each chunk of a split row rounds its probabilities to bf16
    # against its own softmax offset (_rounding_bound); float32: merge
    # rounding only.
    base = outs[-1].double()
    vmax = v.abs().max().item()
    for chunk, o in outs.items():
        if dtype == "bf16":
            bound = _rounding_bound(base, vmax)
        else:
            bound = base.abs().clamp(min=1.0) * 1e-5
        excess = ((o.double() - base).abs() - bound).max().item()
        assert excess <= 0, (chunk, excess)
    g = gpu_lists_to_host(lists)
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    for o in outs.values():
        assert attention_error(o, qn, kn, vn, lay, g["row_ptr"], g["col_idx"]) <= TOL[dtype]


def _greedy_pairs(sizes):
    """Pairs of neighbouring query blocks of at most 64 tokens, taken two by
    two from the start of every run of such blocks."""
    small = np.asarray(sizes) <= 64
    n, i = 0, 0
    while i < len(small) - 1:
        if small[i] and small[i + 1]:
            n, i = n + 1, i + 2
        else:
            i += 1
    return n


def _rounding_bound(base, vmax):
    """Largest difference between two bf16 runs of the same rows that round
    their probabilities against different softmax offsets (chunks of a split
    row, or a pair's union stream against a row's own): every weight carries
    a relative rounding error of at most 2^-9 in either run, so each output
    lies within 2^-9 * max_u |v_u - o| of the unrounded-weight result and the
    two within 2^-8 * (max|v| + |o|), plus half an output ulp each
    (2^-9 |o|): 2^-8 * max|v| + 2^-7 * |o|, with 1% and 1e-6 for float32
    accumulation and merge rounding."""
    return (2 ** -8 * vmax + 2 ** -7 * base.abs()) * 1.01 + 1e-6


@pytest.mark.parametrize("case", ["config2", "all64_odd_run", "mixed_edges", "hilbert"])
def test_row_pairs_match_unpaired(dev, case):
    """Query blocks of at most 64 tokens paired into one work item give the
    unpaired results up to the rounding of the probabilities (each run rounds
    them against its own offsets), and as many pairs as the greedy rule."""
    hilbert = case == "hilbert"
    if case == "config2":
        w = WORKLOADS[2]
        q, k, v, _ = make_inputs(w)
        grid, tile, p, kmin, budget, B, H = w.grid, w.tile, w.p, w.kmin, w.budget, w.B, w.H
    else:
        grid, tile = {"all64_odd_run": ((3, 24, 40), (1, 8, 8)), "mixed_edges": ((5, 20, 20), (2, 8, 8)),
                      "hilbert": ((5, 20, 20), None)}[case]
        B, H = 2, 3
        q, k, v = _small_case(grid, tile, H, 128, "bf16", 90, scale=2.0, B=B)
        p, kmin, budget = 0.85, 2, ("frac", 0.2)
    print(f"\n[pairs] {case}: grid {grid} tile {tile}", flush=True)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    order = fva.hilbert_order(grid, dev) if hilbert else None
    blk = dict(grid=grid, order=order) if hilbert else dict(grid=grid, tile=tile)
    lists = fva.route(qd, kd, p, kmin, budget, **blk)
    outs, infos = {}, {}
    for chunk in (-1, 0):          # rows never split / the automatic split the bench uses
        for on in (True, False):
            st = torch.zeros(fva.stats_bytes(qd, grid, tile, chunk_blocks=chunk, order=order), dtype=torch.uint8,
                             device=dev)
            outs[chunk, on] = fva.sparse_attn(qd, kd, vd, lists, stats=st, chunk_blocks=chunk, row_pairs=on)
            torch.cuda.synchronize()
            infos[chunk, on], _ = fva.parse_stats(st)
    sizes = fva.block_sizes(grid, tile, ordered=hilbert)
    expect = 0 if hilbert else B * H * _greedy_pairs(sizes)
    for chunk in (-1, 0):
        assert infos[chunk, False].n_row_pairs == 0
    # without splitting, every pair runs as one item and replaces two items
    # by one
    assert infos[-1, True].n_row_pairs == expect
    assert infos[-1, True].n_items == infos[-1, False].n_items - expect
    base = outs[-1, False].double()
    excess = ((outs[-1, True].double() - base).abs() - _rounding_bound(base, v.abs().max().item())).max().item()
    assert excess <= 0, excess
    # with the automatic split, only pairs whose union fits the chunk size run
    # together, and such an item replaces at least two
    n0 = infos[0, True].n_row_pairs
    assert 0 <= n0 <= expect
    assert infos[0, True].n_items <= infos[0, False].n_items - n0
    lay = HilbertLayout(grid) if hilbert else BlockLayout(grid, tile)
    g = gpu_lists_to_host(lists)
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    for chunk in (-1, 0):
        err = attention_error(outs[chunk, True], qn, kn, vn, lay, g["row_ptr"], g["col_idx"])
        assert err <= TOL["bf16"], (chunk, err)


def test_row_pairs_with_descending_columns(dev):
    """Unordered columns: a pair walks the union in ascending order, so the
    sum order differs from the unpaired run; both stay within tolerance."""
    grid, tile, B, H = (3, 24, 40), (1, 8, 8), 1, 2
    q, k, v = _small_case(grid, tile, H, 128, "bf16", 95, scale=2.0, B=B)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, 0.8, 2, None, grid=grid, tile=tile)
    g = gpu_lists_to_host(lists)
    rp, ci = g["row_ptr"], g["col_idx"].copy()
    for r in range(len(rp) - 1):
        ci[rp[r]:rp[r + 1]] = ci[rp[r]:rp[r + 1]][::-1]
    rev = fva.lists_from_csr(rp, ci, nq=lists.nq, grid=grid, tile=tile, device=dev)
    lay = BlockLayout(grid, tile)
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    for on in (True, False):
        o = fva.sparse_attn(qd, kd, vd, rev, row_pairs=on)
        torch.cuda.synchronize()
        assert attention_error(o, qn, kn, vn, lay, rp, ci) <= TOL["bf16"]


def test_many_heads_keep_head_order(dev):
    """More heads than the plan orders by density (1,100 > 1,024): the plan
    keeps (b, h) order; 64-token blocks still pair."""
    grid, tile, B, H = (2, 8, 16), (1, 8, 8), 2, 550          # 4 blocks of 64 tokens per head
    q, k, v = _small_case(grid, tile, H, 128, "bf16", 110, scale=2.0, B=B)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, 0.7, 1, ("frac", 0.5), grid=grid, tile=tile)
    st = torch.zeros(fva.stats_bytes(qd, grid, tile), dtype=torch.uint8, device=dev)
    o = fva.sparse_attn(qd, kd, vd, lists, stats=st)
    o_np = fva.sparse_attn(qd, kd, vd, lists, row_pairs=False)
    torch.cuda.synchronize()
    info, _ = fva.parse_stats(st)
    assert info.n_row_pairs > 0
    assert torch.equal(o, o_np)
    lay = BlockLayout(grid, tile)
    g = gpu_lists_to_host(lists)
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    ref = routing.route(qn, kn, lay, 0.7, 1, ("frac", 0.5))
    rep = compare_lists(g, ref, 0.7, ("frac", 0.5), lay, B, H)
    assert_exact(rep)
    err = attention_error(o, qn, kn, vn, lay, g["row_ptr"], g["col_idx"])
    print(f"\n[many heads] {rep} max|o - oracle| = {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("scale", [2.0, 3.0])
def test_sharp_softmax_bf16(dev, scale):
    """Sharp rows (q, k at scale 2 and 3: score spreads of 4 and 9 nats per
    unit of the 1/sqrt(d)-scaled product) with |v| up to 6, on ragged
    tiles: every output within 2e-2 of the oracle.  Half an ulp of a bf16
    output in [4, 8) is already 0.0156, so the weights the kernel rounds for
    P V must be the ones it normalises by."""
    grid, tile, H = (5, 20, 20), (2, 8, 8), 4                 # 27 blocks, ragged on two axes
    q, k, _ = _small_case(grid, tile, H, 128, "bf16", 120, scale=scale)
    v = tiny_random((1, H, grid[0] * grid[1] * grid[2], 128), 123, "fp32", 2.0).clamp(-6.0, 6.0)
    v = v.to(torch.bfloat16)
    _run_and_check(dev, q, k, v, grid, tile, 0.9, 2, ("frac", 0.2), TOL["bf16"])


def test_one_hot_rows_reproduce_v(dev):
    """Each query's own key scores far above every other (q = k with a large
    norm): the softmax is one-hot on the query's own token, so every output
    is that token's value row, which is exact in bf16.  With the normaliser
    summing the same rounded weights as P V, the kernel returns v itself
    whatever its softmax offset; a normaliser of unrounded weights would be
    off by up to 2^-9 |v| (0.012 at |v| = 6)."""
    grid, tile, H = (4, 16, 24), (2, 8, 8), 2                  # 12 full blocks
    N, d = grid[0] * grid[1] * grid[2], 128
    x = tiny_random((1, H, N, d), 130, "fp32", 1.0)
    x = 40.0 * x / x.norm(dim=-1, keepdim=True)                # |q|^2 / sqrt(d) = 141 for the own key
    q = x.to(torch.bfloat16)
    k = q.clone()
    v = tiny_random((1, H, N, d), 131, "fp32", 2.0).clamp(-6.0, 6.0).to(torch.bfloat16)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, 1.0, 0, None, grid=grid, tile=tile)     # every block: the whole row
    o = fva.sparse_attn(qd, kd, vd, lists)
    torch.cuda.synchronize()
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    s = np.einsum("bhnd,bhmd->bhnm", qn, kn) / np.sqrt(d)
    gap = np.sort(s, axis=-1)[..., -1] - np.sort(s, axis=-1)[..., -2]
    assert gap.min() > 60.0, gap.min()                 # every other weight below e^-60
    err = (o.double().cpu() - v.double()).abs().max().item()
    print(f"\n[one-hot] max|o - v| = {err:.3e}", flush=True)
    assert err <= 1e-6


@pytest.mark.parametrize("case", ["config1", "config2", "config4", "ragged64", "hilbert"])
def test_layer_is_route_then_attention(dev, case):
    """fva_layer (route and attention in one call, one shared read of q, k and
    v for bf16 d = 128) gives the lists and outputs of fva_route followed by
    fva_sparse_attn bit for bit."""
    if case.startswith("config"):
        w = WORKLOADS[int(case[-1])]
        q, k, v, _ = make_inputs(w)
        grid, tile, p, kmin, budget = w.grid, w.tile, w.p, w.kmin, w.budget
    else:
        grid, tile = ((3, 13, 21), (2, 4, 8)) if case == "ragged64" else ((5, 20, 20), None)
        q, k, v = _small_case(grid, tile, 3, 128, "bf16", 180, scale=2.0, B=2)
        p, kmin, budget = 0.8, 2, ("frac", 0.25)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    order = fva.hilbert_order(grid, dev) if case == "hilbert" else None
    blk = dict(grid=grid, order=order) if order is not None else dict(grid=grid, tile=tile)
    lists = fva.route(qd, kd, p, kmin, budget, **blk)
    o = fva.sparse_attn(qd, kd, vd, lists)
    for rep in range(2):
        l2, o2 = fva.layer(qd, kd, vd, p, kmin, budget, **blk)
        torch.cuda.synchronize()
        n = int(lists.row_ptr[-1].item())
        assert torch.equal(l2.row_ptr, lists.row_ptr) and torch.equal(l2.col_idx[:n], lists.col_idx[:n]), rep
        assert torch.equal(l2.base_count, lists.base_count) and torch.equal(l2.head_kept, lists.head_kept), rep
        assert torch.equal(o2, o), (rep, (o2.float() - o.float()).abs().max().item())


def test_empty_problem(dev):
    q = torch.empty((1, 0, 256, 128), dtype=torch.bfloat16, device=dev)
    lists = fva.route(q, q, 0.9, 1, None, grid=(4, 8, 8), tile=(1, 8, 8))
    torch.cuda.synchronize()
    assert lists.row_ptr.cpu().tolist() == [0]
    o = fva.sparse_attn(q, q, q, lists)
    assert o.shape == q.shape
    l2, o2 = fva.layer(q, q, q, 0.9, 1, None, grid=(4, 8, 8), tile=(1, 8, 8))
    torch.cuda.synchronize()
    assert l2.row_ptr.cpu().tolist() == [0] and o2.shape == q.shape


def test_stats_and_per_cu_imbalance(dev):
    w = WORKLOADS[2]
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile), dtype=torch.uint8, device=dev)
    fva.sparse_attn(qd, kd, vd, lists, stats=st)
    torch.cuda.synchronize()
    info, ctas = fva.parse_stats(st)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    assert info.num_ctas in (ncu, 2 * ncu) and len(ctas) == info.num_ctas     # 1 or 2 workgroups per CU
    assert sum(c.items for c in ctas) == info.n_items
    assert sum(c.blocks for c in ctas) == info.total_blocks == int(lists.row_ptr[-1].item())
    assert all(c.t_end >= c.t_start for c in ctas)
    imb, busy = fva.per_cu_imbalance(ctas, ncu)
    print(f"\n[stats] ctas={len(ctas)} distinct CU keys={len(busy)} imbalance={imb:.3f}", flush=True)
    assert imb >= 1.0


@pytest.mark.parametrize("cid", [1, 2])
def test_prepare_on_a_side_stream(dev, cid):
    """attn_prepare on a second stream, overlapped with route on the main
    stream and joined before sparse_attn(prepared=True), gives the same bits
    as sparse_attn doing everything itself (the same kernels run on the same
    data; only the stream of the K/V copies changes)."""
    w = WORKLOADS[cid]
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    ref = fva.sparse_attn(qd, kd, vd, lists)
    torch.cuda.synchronize()
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)
    for it in range(3):
        side.wait_stream(main)              # the last sparse_attn is done with the workspace
        with torch.cuda.stream(side):
            fva.attn_prepare(kd, vd, grid=w.grid, tile=w.tile, stream=main)
        lists2 = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
        main.wait_stream(side)
        o = fva.sparse_attn(qd, kd, vd, lists2, prepared=True)
        torch.cuda.synchronize()
        assert torch.equal(lists2.row_ptr, lists.row_ptr)
        assert torch.equal(o, ref), (cid, it, (o.float() - ref.float()).abs().max().item())


def test_graph_capture_replays(dev):
    """route -> attn_prepare (second stream) -> sparse_attn captured in one
    HIP graph: every replay, with other eager calls on the same workspaces and
    host synchronisations in between, reproduces the eager lists and output
    bit for bit.  The library records no memset or copy, only kernels."""
    w = WORKLOADS[2]
    q, k, v, _ = make_inputs(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    out = torch.empty_like(qd)
    fva.sparse_attn(qd, kd, vd, lists, out=out)
    torch.cuda.synchronize()
    ref_o, ref_rp = out.clone(), lists.row_ptr.clone()
    ref_ci = lists.col_idx[: int(ref_rp[-1].item())].clone()
    # other inputs for the eager calls between replays
    q2, k2 = qd.flip(2).contiguous(), kd.flip(2).contiguous()
    side = torch.cuda.Stream(dev)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            main = torch.cuda.current_stream(dev)
            side.wait_stream(main)
            with torch.cuda.stream(side):
                fva.attn_prepare(kd, vd, grid=w.grid, tile=w.tile, stream=main)
            fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile, out=lists)
            main.wait_stream(side)
            fva.sparse_attn(qd, kd, vd, lists, out=out, prepared=True)
    torch.cuda.current_stream(dev).wait_stream(cap)
    torch.cuda.synchronize()
    for rep in range(4):
        out.zero_()
        lists.row_ptr.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lists.row_ptr, ref_rp), rep
        assert torch.equal(lists.col_idx[: ref_ci.numel()], ref_ci), rep
        assert torch.equal(out, ref_o), (rep, (out.float() - ref_o.float()).abs().max().item())
        # eager work on the same workspaces between replays
        l2 = fva.route(q2, k2, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
        fva.sparse_attn(q2, k2, vd, l2)
        torch.cuda.synchronize()


def test_layer_graph_capture_replays(dev, tmp_path):
    """fva_layer captured in one HIP graph: every replay, with eager layer
    calls on other inputs between them on the same workspace, reproduces the
    eager lists and output bit for bit, at 720p (the 5-head shard) and at the
    mid bf16 size; the replayed lists equal the oracle's and the replayed
    output is within tolerance of the oracle (every query block of the mid
    size, 64 seeded ones of the shard)."""
    for cid in (4, 2):
        w = WORKLOADS[cid]
        q, k, v, _ = make_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        blk = dict(grid=w.grid, tile=w.tile)
        lists, out = fva.layer(qd, kd, vd, w.p, w.kmin, w.budget, **blk)
        torch.cuda.synchronize()
        ref_o, ref_rp = out.clone(), lists.row_ptr.clone()
        ref_ci = lists.col_idx[: int(ref_rp[-1].item())].clone()
        q2, k2 = qd.flip(2).contiguous(), kd.flip(2).contiguous()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            fva.layer(qd, kd, vd, w.p, w.kmin, w.budget, **blk, lists=lists, out=out)   # the stream's workspace
        cap.synchronize()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                fva.layer(qd, kd, vd, w.p, w.kmin, w.budget, **blk, lists=lists, out=out)
        torch.cuda.current_stream(dev).wait_stream(cap)
        torch.cuda.synchronize()
        for rep in range(3):
            out.zero_()
            lists.row_ptr.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(lists.row_ptr, ref_rp), (cid, rep)
            assert torch.equal(lists.col_idx[: ref_ci.numel()], ref_ci), (cid, rep)
            assert torch.equal(out, ref_o), (cid, rep)
            with torch.cuda.stream(cap):
                fva.layer(q2, k2, vd, w.p, w.kmin, w.budget, **blk)
            torch.cuda.synchronize()
        # the last replay against the oracle
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        del g
        lay = BlockLayout(w.grid, w.tile)
        gl = gpu_lists_to_host(lists)
        ref = routing.route(to_numpy(q), to_numpy(k), lay, w.p, w.kmin, w.budget)
        rep = compare_lists(gl, ref, w.p, w.budget, lay, w.B, w.H)
        assert_exact(rep)
        nb = lay.Nb
        if cid == 2:
            rows = [(bh, i) for bh in range(w.B * w.H) for i in range(nb)]
        else:
            pick = np.random.default_rng(160).choice(w.B * w.H * nb, 64, replace=False)
            rows = [(int(x) // nb, int(x) % nb) for x in np.sort(pick)]
        errs, _ = _oracle_errors(tmp_path, cid, lay, q, k, v, out, gl, rows)
        err = float(errs.max())
        print(f"\n[graph] {w.name}: 3 replays of the layer bit-exact; replayed lists exact, "
              f"max|o - oracle| = {err:.3e} on {len(rows)} query blocks", flush=True)
        assert err <= TOL["bf16"]


def test_two_streams_with_different_problems(dev):
    """Route + attention of two different problems issued on two streams with
    no ordering between them, small first and then large, three times: each
    stream has its own workspaces, so every result equals the same call run
    alone."""
    w = WORKLOADS[2]
    qa, ka, va, _ = make_inputs(w)
    qa, ka, va = qa.to(dev), ka.to(dev), va.to(dev)
    grid_b, tile_b = (3, 16, 24), (2, 8, 8)
    qb, kb, vb = (t.to(dev) for t in _small_case(grid_b, tile_b, 3, 128, "bf16", 150, scale=2.0))
    la = fva.route(qa, ka, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
    ref_a = fva.sparse_attn(qa, ka, va, la)
    lb = fva.route(qb, kb, 0.85, 2, ("frac", 0.3), grid=grid_b, tile=tile_b)
    ref_b = fva.sparse_attn(qb, kb, vb, lb)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    for rep in range(3):
        sa.wait_stream(torch.cuda.current_stream(dev))
        sb.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(sb):
            lb2 = fva.route(qb, kb, 0.85, 2, ("frac", 0.3), grid=grid_b, tile=tile_b)
            ob = fva.sparse_attn(qb, kb, vb, lb2)
        with torch.cuda.stream(sa):
            la2 = fva.route(qa, ka, w.p, w.kmin, w.budget, grid=w.grid, tile=w.tile)
            oa = fva.sparse_attn(qa, ka, va, la2)
        torch.cuda.synchronize()
        assert torch.equal(la2.row_ptr, la.row_ptr) and torch.equal(lb2.row_ptr, lb.row_ptr), rep
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b), rep


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_hilbert_block_parity(dev, cid):
    """Hilbert-curve blocks (128-token runs of the curve order from the
    library's host helper) against the oracle's own Hilbert layout: lists by
    the list rule, outputs within the dtype's tolerance."""
    from oracle import HilbertLayout
    w = WORKLOADS[cid]
    print(f"\n[parity] config {cid} {w.name} with Hilbert blocks", flush=True)
    q, k, v, _ = make_inputs(w)
    lay = HilbertLayout(w.grid)
    npdt = np.float64 if cid <= 2 else np.float32
    qn, kn, vn = (to_numpy(t, npdt) for t in (q, k, v))
    ref = routing.route(qn, kn, lay, w.p, w.kmin, w.budget)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    order = fva.hilbert_order(w.grid, dev)
    assert np.array_equal(order.cpu().numpy().astype(np.int64), lay.order)
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, grid=w.grid, order=order)
    assert lists.nq == lay.Nb
    g = gpu_lists_to_host(lists)
    rep = compare_lists(g, ref, w.p, w.budget, lay, w.B, w.H)
    print(f"[parity] config {cid} hilbert: lists {rep}", flush=True)
    assert_exact(rep)
    o = fva.sparse_attn(qd, kd, vd, lists)
    torch.cuda.synchronize()
    print(f"[parity] config {cid} hilbert: density {np.diff(g['row_ptr']).sum() / (w.B * w.H * lay.Nb ** 2):.4f} "
          f"(tiles: see the workload test)", flush=True)
    rows = _rows_sample(w, lay.Nb, SAMPLE[cid])
    prec = "fp64" if cid <= 2 else "fp32"
    err = attention_error(o, qn, kn, vn, lay, g["row_ptr"], g["col_idx"], rows=rows, precision=prec)
    print(f"[parity] config {cid} hilbert: max|o - oracle| = {err:.3e} (tol {TOL[w.dtype]})", flush=True)
    assert err <= TOL[w.dtype]


@pytest.mark.parametrize("grid,p,kmin,budget,dtype,d,B,strided", [
    ((3, 20, 20), 1.0, 0, ("none", 0.0), "bf16", 128, 1, False),      # dense, last block 48 tokens
    ((1, 5, 5), 0.9, 4, ("none", 0.0), "bf16", 128, 1, False),        # one block smaller than 128
    ((3, 16, 24), 0.85, 2, ("match_max", 0.0), "bf16", 128, 2, True),  # batch 2, wide token stride
    ((3, 16, 24), 0.85, 2, ("frac", 0.3), "fp32", 64, 2, True),
    ((2, 16, 16), 1e-12, 3, ("none", 0.0), "bf16", 64, 1, False),     # p -> 0+: fixed Top-3
])
def test_hilbert_edge_cases(dev, grid, p, kmin, budget, dtype, d, B, strided):
    q, k, v = _small_case(grid, None, 3, d, dtype, 80, scale=2.0, B=B)
    g, _, _ = _run_and_check(dev, q, k, v, grid, None, p, kmin, budget, TOL[dtype], strided=strided,
                             hilbert=True)
    counts = np.diff(g["row_ptr"])
    nb = -(-grid[0] * grid[1] * grid[2] // 128)
    if p >= 1.0:
        assert np.all(counts == nb)
    if p < 1e-6:
        assert np.all(counts == min(nb, max(kmin, 1)))


def test_maximum_block_count(dev):
    """The largest supported list width: 2,048 key blocks per row (the row sort
    then has no padding at all), one head; lists against the oracle, outputs
    on sampled rows."""
    grid, tile = (8, 128, 128), (1, 8, 8)          # 8 x 16 x 16 = 2048 blocks of 64 tokens
    assert fva.num_blocks(grid, tile) == 2048
    q, k, v = _small_case(grid, tile, 1, 128, "bf16", 90, scale=2.0)
    lay = BlockLayout(grid, tile)
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    ref = routing.route(qn, kn, lay, 0.8, 3, ("frac", 0.05))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, 0.8, 3, ("frac", 0.05), grid=grid, tile=tile)
    g = gpu_lists_to_host(lists)
    rep = compare_lists(g, ref, 0.8, ("frac", 0.05), lay, 1, 1)
    assert_exact(rep)
    o = fva.sparse_attn(qd, kd, vd, lists)
    torch.cuda.synchronize()
    rows = {0: np.sort(np.random.default_rng(91).choice(2048, 24, replace=False))}
    err = attention_error(o, qn, kn, vn, lay, g["row_ptr"], g["col_idx"], rows=rows)
    assert err <= TOL["bf16"], err


def test_nonfinite_token_keeps_every_block(dev):
    """A NaN key token at 2,048 blocks per row (32 sort slots per lane): every
    row of its head has a NaN routing score, keeps every key block in block
    order and takes no augmentation, as the oracle reads it; the other head
    routes normally.  Lists bit-exact against the oracle; the clean head's
    outputs within tolerance; the attention call on the NaN head completes."""
    grid, tile = (8, 128, 128), (1, 8, 8)          # 2048 blocks of 64 tokens
    q, k, v = _small_case(grid, tile, 2, 128, "bf16", 140, scale=2.0)
    lay = BlockLayout(grid, tile)
    k[0, 0, int(lay.members[700][3]), 5] = float("nan")
    qn, kn, vn = (to_numpy(t) for t in (q, k, v))
    with np.errstate(invalid="ignore"):
        ref = routing.route(qn, kn, lay, 0.8, 3, ("frac", 0.05))
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    lists = fva.route(qd, kd, 0.8, 3, ("frac", 0.05), grid=grid, tile=tile)
    g = gpu_lists_to_host(lists)
    nb = lay.Nb
    assert np.array_equal(g["row_ptr"], ref["row_ptr"]) and np.array_equal(g["col_idx"], ref["col_idx"])
    assert np.all(np.diff(g["row_ptr"])[:nb] == nb)
    assert np.array_equal(g["col_idx"][: nb * nb], np.tile(np.arange(nb), nb))
    o = fva.sparse_attn(qd, kd, vd, lists)
    torch.cuda.synchronize()
    rows = {1: np.sort(np.random.default_rng(141).choice(nb, 16, replace=False))}
    hrp, hci = (g["row_ptr"][nb:] - g["row_ptr"][nb]), g["col_idx"][g["row_ptr"][nb]:]
    ref_o = attention.sparse_attention_head(qn[0, 1], kn[0, 1], vn[0, 1], lay, hrp, hci, rows=rows[1])
    toks = np.concatenate([lay.members[i] for i in rows[1]])
    got = o[0, 1].index_select(0, torch.as_tensor(toks, device=dev)).double().cpu().numpy()
    err = float(np.abs(got - ref_o[toks]).max())
    print(f"\n[nan] clean head max|o - oracle| = {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
