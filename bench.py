"""Benchmark of the FVAttn block-sparse attention hot path on one MI355X.

One step = the whole path on one synthetic layer: fva_route (pool, block
scores, Top-p + floor, slack augmentation, CSR) then fva_sparse_attn (plan,
block-sparse flash attention, combine), with the inputs already resident in
HBM.  The list-independent K/V copies (fva_attn_prepare) run on a second
stream while the routing runs, joined before the attention.  The step is
timed eagerly (ms_per_layer, `value`), then captured once in a HIP graph
and timed as replays (ms_per_layer_graph; graph_replay_bit_exact says
whether a replay reproduced the eager lists and output bit for bit).  The
same step on one stream is timed too (ms_per_layer_one_stream).

Workload (default): the 720p-shaped DiT self-attention layer - B=1, 40 heads,
d=128, bf16, 21x45x80 latent tokens in 2x8x8 tiles, p=0.9, floor 8, +10%
slack.  Metric: ms per layer and effective sparse TFLOP/s, with
FLOPs = 4 * d * (kept valid query-key token pairs over all heads), as a
fraction of the MI355X dense bf16 MFMA peak (2516.6 TFLOP/s = 256 CUs x
2.4 GHz x 4096 flop/clk).

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--config 3] [--no-cpu-baseline] [--no-dense]

Besides the step, it times the same attention kernel on dense lists (p = 1,
every key block kept) once, for the sparse-over-dense attention speedup.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # 256 CUs * 2.4 GHz * 4096 bf16 flop/clk/CU, dense
PEAK_F32_VALU_TFLOPS = 157.3   # fp32 vector, packed (256 CUs * 2.4 GHz * 256 flop/clk/CU)
KERNEL_NAME = "attn_bf16_d128_kernel"     # the dominant kernel of the path (bf16, d=128)
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_bf16_d128_kernel_720p_layer_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "block_sparse_attention_22_amd", "csrc", "attn.hip")


def measured_traffic():
    """HBM-side bytes per launch of the attention kernel from the committed
    FETCH_SIZE/WRITE_SIZE summary (copy-calibrated), or None when the kernel
    source has changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_PROFILE).read()
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    m_sha = re.search(r"attn\.hip sha256 ([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch attn_bf16_d128_kernel: ([0-9.e+]+)", text)
    if not (m_sha and m_val) or m_sha.group(1) != src:
        return None
    return float(m_val.group(1))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kept_pairs(row_ptr: np.ndarray, col_idx: np.ndarray, sizes: np.ndarray, nb: int):
    """Kept valid query-key token pairs: sum over kept (i, j) of n_i * n_j."""
    counts = np.diff(row_ptr)
    rows = np.repeat(np.arange(len(counts)) % nb, counts)
    pairs = sizes[rows].astype(np.int64) * sizes[col_idx].astype(np.int64)
    per_row = np.add.reduceat(pairs, row_ptr[:-1]) if len(pairs) else np.zeros(len(counts), np.int64)
    return int(pairs.sum()), per_row


def simulate_queue(costs, ncta):
    """Makespan / mean load of workers that each take the next item when idle."""
    import heapq
    h = [(0.0, c) for c in range(ncta)]
    heapq.heapify(h)
    for x in costs:
        t, c = heapq.heappop(h)
        heapq.heappush(h, (t + x, c))
    loads = [t for t, _ in h]
    mean = sum(loads) / ncta
    return max(loads) / mean if mean > 0 else 1.0


def cpu_baseline(w, q, k, v, g_row_ptr, g_col_idx, budget_s=12.0, hilbert=False):
    """Time the CPU oracle (unchanged) on a bounded sample of this workload and
    extrapolate to the whole layer: routing of the first heads, attention of a
    seeded sample of query blocks, each until its time budget is used."""
    from oracle import BlockLayout, HilbertLayout, attention, routing

    lay = HilbertLayout(w.grid) if hilbert else BlockLayout(w.grid, w.tile)

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    nb = lay.Nb
    H = w.B * w.H
    # routing: whole heads until ~1/4 of the budget
    t0 = time.perf_counter()
    h_done = 0
    while h_done < H and time.perf_counter() - t0 < budget_s / 4:
        b, h = divmod(h_done, w.H)
        routing.route_head(q[b, h].float().numpy(), k[b, h].float().numpy(), lay, w.p, w.kmin)
        h_done += 1
    t_route = time.perf_counter() - t0
    route_full = t_route * H / h_done
    # attention: seeded (head, query block) sample until the rest of the budget
    rng = np.random.default_rng((260716190, w.cid, 2))
    order = rng.permutation(H * nb)
    sizes = lay.sizes
    t1 = time.perf_counter()
    pairs_done = 0
    rows_done = 0
    cache = {}
    for r in order:
        if time.perf_counter() - t1 > budget_s * 3 / 4:
            break
        bh, i = divmod(int(r), nb)
        b, h = divmod(bh, w.H)
        if bh not in cache:
            cache.clear()
            cache[bh] = tuple(t[b, h].float().numpy() for t in (q, k, v))
        qh, kh, vh = cache[bh]
        r0 = bh * nb
        hrp = g_row_ptr[r0:r0 + nb + 1] - g_row_ptr[r0]
        hci = g_col_idx[g_row_ptr[r0]:g_row_ptr[r0 + nb]]
        attention.sparse_attention_head(qh, kh, vh, lay, hrp, hci, rows=[i], precision="fp32")
        js = hci[hrp[i]:hrp[i + 1]]
        pairs_done += int(sizes[i]) * int(sizes[js].sum())
        rows_done += 1
    t_attn = time.perf_counter() - t1
    return dict(route_s=t_route, route_heads=h_done, route_full_s=route_full, attn_s=t_attn, attn_rows=rows_done,
                attn_pairs=pairs_done, cores=cores, blas_threads=blas_threads)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense (p = 1) comparison")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--blocks", choices=("tiles", "hilbert"), default="tiles",
                    help="block organisation: the workload's 3D tiles, or 128-token runs of the Hilbert-curve order")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(every step of the path is independent per (batch, head), so more GPUs would each run it on "
              "their own heads; this benchmark measures the one-GPU share)", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_22_amd as fva
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: B={w.B} H={w.H} d={w.d} grid={w.grid} tile={w.tile}")
    q, k, v, gains = make_inputs(w)
    hilbert = args.blocks == "hilbert"
    order = fva.hilbert_order(w.grid, dev) if hilbert else None
    blk = dict(grid=w.grid, order=order) if hilbert else dict(grid=w.grid, tile=w.tile)
    sizes = fva.block_sizes(w.grid, w.tile, ordered=hilbert)
    nb = len(sizes)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()

    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, **blk)
    out = torch.empty_like(qd)

    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)          # default priority, like the main stream

    def step(ev=None):
        # K/V copies on the side stream once the last attention has released
        # the workspace; routing meanwhile on the main stream; join, attend.
        side.wait_stream(main)
        with torch.cuda.stream(side):
            if ev:
                ev[5].record()
            fva.attn_prepare(kd, vd, **blk, stream=main)
            if ev:
                ev[6].record()
        if ev:
            ev[0].record()
        fva.route(qd, kd, w.p, w.kmin, w.budget, **blk, out=lists)
        if ev:
            ev[1].record()
        main.wait_stream(side)
        fva.sparse_attn(qd, kd, vd, lists, out=out, prepared=True,
                        kernel_events=(ev[3], ev[4]) if ev else None)
        if ev:
            ev[2].record()

    def step_one_stream():
        fva.route(qd, kd, w.p, w.kmin, w.budget, **blk, out=lists)
        fva.sparse_attn(qd, kd, vd, lists, out=out)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
        step_one_stream()
    torch.cuda.synchronize()

    # Per step: events around the routing call and the attention call (main
    # stream, where the library launches), the pair the library records right
    # around the attention kernel proper, and a pair around the K/V copies on
    # the side stream.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for e in ev:                      # create the kernel events before the timed region
        e[3].record()
        e[4].record()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(ev[s])
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    route_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    attn_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    kernel_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in ev]))
    prepare_ms = float(np.mean([e[5].elapsed_time(e[6]) for e in ev]))
    # The same step on one stream (everything in order), for comparison.
    start.record()
    for s in range(args.steps):
        step_one_stream()
    stop.record()
    torch.cuda.synchronize()
    ms_one_stream = start.elapsed_time(stop) / args.steps

    # The overlapped step captured once in a HIP graph and replayed: the same
    # kernels without host launch gaps.
    step()
    torch.cuda.synchronize()
    eager_o, eager_rp = out.clone(), lists.row_ptr.clone()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(main)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            main = torch.cuda.current_stream(dev)
            step()
    main = torch.cuda.current_stream(dev)
    main.wait_stream(cap)
    torch.cuda.synchronize()
    out.zero_()
    graph.replay()
    torch.cuda.synchronize()
    graph_ok = bool(torch.equal(out, eager_o) and torch.equal(lists.row_ptr, eager_rp))
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms_graph = start.elapsed_time(stop) / args.steps
    log(f"[bench] eager {ms_step:.3f} ms, one stream {ms_one_stream:.3f} ms, graph {ms_graph:.3f} ms "
        f"(replay {'matches' if graph_ok else 'DIFFERS FROM'} eager)")
    ms_eager = ms_step

    # Lists, pair count and balance (one more call with per-workgroup stats).
    rp = lists.row_ptr.cpu().numpy().astype(np.int64)
    ci = lists.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    pairs, per_row = kept_pairs(rp, ci, sizes, nb)
    flops = 4.0 * w.d * pairs
    exe_sizes = ((sizes + 31) // 32) * 32        # work the kernel issues: 32-token sub-tiles
    executed_pairs, _ = kept_pairs(rp, ci, exe_sizes, nb)
    st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile, order=order), dtype=torch.uint8, device=dev)
    fva.sparse_attn(qd, kd, vd, lists, out=out, stats=st)
    torch.cuda.synchronize()
    info, ctas = fva.parse_stats(st)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    imb, busy = fva.per_cu_imbalance(ctas, ncu)
    counts = np.diff(rp)
    C = info.chunk_blocks
    # items in the plan's order: heads by kept blocks, densest first (ties to
    # the lower head), rows of a head in order
    per_head = counts.reshape(w.B * w.H, nb)
    head_order = sorted(range(w.B * w.H), key=lambda bh: (-int(per_head[bh].sum()), bh))
    # neighbouring query blocks of <= 64 tokens run as one item over the union
    # of their lists when it holds at most C blocks (bf16, d = 128 only)
    lead = set()
    if info.n_row_pairs > 0:
        small, i = sizes <= 64, 0
        while i < nb - 1:
            if small[i] and small[i + 1]:
                lead.add(i)
                i += 2
            else:
                i += 1
    item_costs = []
    for bh in head_order:
        i = 0
        while i < nb:
            if i in lead:
                r = bh * nb + i
                union = len(np.union1d(ci[rp[r]:rp[r + 1]], ci[rp[r + 1]:rp[r + 2]]))
                if union <= C:
                    item_costs.append(union)
                    i += 2
                    continue
            c = per_head[bh][i]
            n = 1 if c <= C else -(-int(c) // C)
            item_costs += [c / n] * n
            i += 1
    pred_imb = simulate_queue(item_costs, info.num_ctas)
    dens = counts.reshape(w.B * w.H, nb).sum(axis=1) / (nb * nb)
    base_dens = lists.base_count[: len(counts)].cpu().numpy().reshape(w.B * w.H, nb).sum(axis=1) / (nb * nb)

    tflops = flops / (ms_step * 1e-3) / 1e12
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
    # the kernel that runs and the peak of its arithmetic: bf16 on the matrix
    # cores, float32 on the vector ALUs
    if w.dtype == "bf16":
        bound, peak = "mfma", PEAK_BF16_TFLOPS
        kernel_name = KERNEL_NAME if w.d == 128 else "attn_bf16_kernel<64>"
    else:
        bound, peak, kernel_name = "alu", PEAK_F32_VALU_TFLOPS, f"attn_f32_kernel<{w.d}>"
    res = {
        "metric": "ms/layer + effective sparse TFLOP/s (% bf16 MFMA peak) at 75,600 tok x 40 heads",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded RFF-plus-noise q/k, N(0,1) v; stands in for Wan2.2 activations)",
        "config": {"workload": w.name + ("-hilbert" if hilbert else ""), "B": w.B, "heads": w.H, "head_dim": w.d,
                   "grid": list(w.grid), "blocks": "hilbert-128" if hilbert else "tiles",
                   "tile": None if hilbert else list(w.tile), "p": w.p, "kmin": w.kmin, "budget": list(w.budget), "tokens": w.N},
        "ms_per_layer": round(ms_step, 4),
        "ms_per_layer_graph": round(ms_graph, 4),
        "graph_replay_bit_exact": graph_ok,
        "ms_per_layer_one_stream": round(ms_one_stream, 4),
        "route_ms": round(route_ms, 4),
        "attn_prepare_ms_side_stream": round(prepare_ms, 4),
        "attn_ms": round(attn_ms, 4),
        "attn_kernel_ms": round(kernel_ms, 4),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "kept_valid_pairs": pairs,
        "effective_flop": flops,
        "executed_pairs_32_padded": executed_pairs,
        "executed_mfma_tflops": round(4.0 * w.d * executed_pairs / (kernel_ms * 1e-3) / 1e12, 2),
        "block_density": round(float(counts.sum()) / (w.B * w.H * nb * nb), 4),
        "block_density_per_head": [round(float(x), 4) for x in dens],
        "base_density_per_head": [round(float(x), 4) for x in base_dens],
        "per_cu_imbalance": round(imb, 4),
        "per_cu_imbalance_predicted": round(pred_imb, 4),
        "distinct_cus": len(busy),
        "plan": {"n_items": info.n_items, "chunk_blocks": C, "n_split_rows": info.n_split_rows,
                 "n_partials": info.n_partials, "n_row_pairs": info.n_row_pairs, "num_ctas": info.num_ctas},
        "roofline": {"bound": bound, "achieved": round(kernel_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / peak, 4),
                     "traffic": measured_traffic() if (w.dtype == "bf16" and w.d == 128 and w.cid == 3 and not hilbert) else None,
                     "kernel": kernel_name, "per_launch_flop": flops, "avg_launch_ms": round(kernel_ms, 4)},
    }
    if not args.no_dense:
        # Dense comparator: the same kernel on every key block (p = 1), after
        # the timed region; its lists replace nothing the step uses.
        log("[bench] dense comparison (p = 1)")
        dlists = fva.route(qd, kd, 1.0, 0, ("none", 0.0), **blk)
        dout = torch.empty_like(qd)
        dev0, dev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fva.sparse_attn(qd, kd, vd, dlists, out=dout, kernel_events=(dev0, dev1))   # warm-up
        dts = []
        for _ in range(2):
            fva.sparse_attn(qd, kd, vd, dlists, out=dout, kernel_events=(dev0, dev1))
            torch.cuda.synchronize()
            dts.append(dev0.elapsed_time(dev1))
        dense_ms = float(np.mean(dts))
        dense_pairs = int(sizes.sum()) ** 2 * w.B * w.H
        res["dense"] = {
            "attn_kernel_ms": round(dense_ms, 3),
            "tflops": round(4.0 * w.d * dense_pairs / (dense_ms * 1e-3) / 1e12, 2),
            "sparse_attn_speedup": round(dense_ms / kernel_ms, 3),
        }
        del dlists, dout
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, bounded sample)")
        cb = cpu_baseline(w, q, k, v, rp, ci, budget_s=args.cpu_budget, hilbert=hilbert)
        attn_full_s = cb["attn_s"] * pairs / max(cb["attn_pairs"], 1)
        full_s = cb["route_full_s"] + attn_full_s
        res["cpu_baseline"] = {
            "value": round(flops / full_s / 1e12, 6), "unit": "TFLOP/s", "cores": cb["blas_threads"],
            "kind": "oracle",
            "sample": (f"routing oracle on {cb['route_heads']} of {w.B * w.H} heads ({cb['route_s']:.1f}s) and "
                       f"attention oracle (fp32 products, fp64 row stats) on {cb['attn_rows']} seeded query blocks "
                       f"({cb['attn_pairs']} pairs, {cb['attn_s']:.1f}s), linearly extrapolated to the layer: "
                       f"{full_s:.1f}s/layer; host affinity {cb['cores']} cores"),
            "ms_per_layer_extrapolated": round(full_s * 1e3, 1),
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
