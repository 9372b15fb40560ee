"""Benchmark of the FVAttn block-sparse attention hot path on one MI355X.

One step = the whole path on one synthetic layer, as one fva_layer call:
a prologue that reads Q, K and V once (pooled block means for the routing,
the attention's packed K/V copies), the routing (block scores, Top-p +
floor, slack augmentation, CSR lists), then the attention (plan,
block-sparse flash attention, combine), with the inputs already resident in
HBM.  The step is timed eagerly (ms_per_layer, `value`), then captured once
in a HIP graph and timed as replays (ms_per_layer_graph;
graph_replay_bit_exact says whether a replay reproduced the eager lists and
output bit for bit).  For comparison the same work is timed as two calls:
fva_route then fva_sparse_attn on one stream (ms_per_layer_one_stream), and
with the K/V copies (fva_attn_prepare) on a second stream beside the
routing (ms_per_layer_two_calls_overlapped).

Workload (default): the 720p-shaped DiT self-attention layer - B=1, 40 heads,
d=128, bf16, 21x45x80 latent tokens in 2x8x8 tiles, p=0.9, floor 8, +10%
slack.  Metric: ms per layer and effective sparse TFLOP/s, with
FLOPs = 4 * d * (kept valid query-key token pairs over all heads, counted by
the library), as a fraction of the MI355X dense bf16 MFMA peak
(2516.6 TFLOP/s = 256 CUs x 2.4 GHz x 4096 flop/clk).

After the layer, the same step runs on one GPU's 5-head shard of the 720p
layer (skewed head gains, match-max budget), whose per-CU imbalance the
workload asks for; its figures are the `shard_*` keys of the same line.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--config 3] [--no-cpu-baseline] [--no-dense]
                    [--no-shard] [--blocks tiles|hilbert]

Besides the step, it times the same attention kernel on dense lists (p = 1,
every key block kept) once, for the sparse-over-dense attention speedup, and
the CPU oracle on a bounded sample of the workload in a pool of processes.
"""
from __future__ import annotations

import argparse
import json
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
SHARD_CONFIG = 4              # one GPU's 5-head shard of the 720p layer
CPU_POOL_MAX = 16             # worker processes of the CPU baseline (the machine's CPU share for one GPU)


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


# --------------------------------------------------------------- CPU baseline
# The oracle runs in a pool of worker processes forked before the GPU is
# touched; the workers inherit the workload and the raw bf16 (or fp32) input
# arrays below and convert one head at a time.
_CPU = {}


def _cpu_head(name, bh):
    w = _CPU["w"]
    b, h = divmod(bh, w.H)
    x = _CPU[name][b, h]
    if x.dtype == np.uint16:           # bf16 bits -> float32, exactly
        return (x.astype(np.uint32) << 16).view(np.float32)
    return np.asarray(x, dtype=np.float32)


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    _CPU["limits"] = threadpool_limits(1)       # one BLAS thread per worker process


def _cpu_route_task(bh):
    from oracle import routing
    w = _CPU["w"]
    t0 = time.perf_counter()
    routing.route_head(_cpu_head("q", bh), _cpu_head("k", bh), _CPU["lay"], w.p, w.kmin)
    return time.perf_counter() - t0


def _cpu_attn_task(task):
    from oracle import attention
    bh, rows, hrp, hci = task
    t0 = time.perf_counter()
    attention.sparse_attention_head(_cpu_head("q", bh), _cpu_head("k", bh), _cpu_head("v", bh), _CPU["lay"], hrp,
                                    hci, rows=rows, precision="fp32")
    return time.perf_counter() - t0


def start_cpu_pool(w, q, k, v, hilbert):
    """Fork the oracle's worker pool (before any GPU call)."""
    import multiprocessing as mp

    import torch
    from oracle import BlockLayout, HilbertLayout

    def raw(t):
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    _CPU.update(w=w, q=raw(q), k=raw(k), v=raw(v),
                lay=HilbertLayout(w.grid) if hilbert else BlockLayout(w.grid, w.tile))
    n = max(1, min(CPU_POOL_MAX, len(os.sched_getaffinity(0))))
    return mp.get_context("fork").Pool(n, initializer=_cpu_worker_init), n


def cpu_baseline(pool, n_proc, w, rp, ci, sizes, pairs_total, budget_s):
    """The unchanged oracle on this workload: routing of every head, then
    attention on seeded query blocks until the time budget is spent,
    extrapolated to the layer by kept pairs."""
    nb = len(sizes)
    H = w.B * w.H
    t0 = time.perf_counter()
    pool.map(_cpu_route_task, range(H))
    t_route = time.perf_counter() - t0
    rng = np.random.default_rng((260716190, w.cid, 2))
    order = rng.permutation(H * nb)
    tasks = []
    for r in order:
        bh, i = divmod(int(r), nb)
        r0 = bh * nb
        hrp = rp[r0:r0 + nb + 1] - rp[r0]
        hci = ci[rp[r0]:rp[r0 + nb]]
        js = hci[hrp[i]:hrp[i + 1]]
        tasks.append(((bh, [i], hrp, hci), int(sizes[i]) * int(sizes[js].sum())))
    t1 = time.perf_counter()
    done_rows, done_pairs, pos = 0, 0, 0
    while pos < len(tasks) and time.perf_counter() - t1 < budget_s:
        batch = tasks[pos:pos + 2 * n_proc]
        pool.map(_cpu_attn_task, [t for t, _ in batch])
        done_rows += len(batch)
        done_pairs += sum(p for _, p in batch)
        pos += len(batch)
    t_attn = time.perf_counter() - t1
    attn_full = t_attn * pairs_total / max(done_pairs, 1)
    return dict(route_s=t_route, attn_s=t_attn, attn_rows=done_rows, attn_pairs=done_pairs,
                attn_full_s=attn_full, full_s=t_route + attn_full)


# ------------------------------------------------------------------ GPU step
def run_workload(w, args, q, k, v, hilbert, full):
    """Time the layer step on workload w.  full: also the one-stream and graph
    timings.  Returns the figures and the host copy of the lists."""
    import torch

    import block_sparse_attention_22_amd as fva

    dev = torch.device("cuda:0")
    order = fva.hilbert_order(w.grid, dev) if hilbert else None
    blk = dict(grid=w.grid, order=order) if hilbert else dict(grid=w.grid, tile=w.tile)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    lists = fva.route(qd, kd, w.p, w.kmin, w.budget, **blk)
    out = torch.empty_like(qd)
    main = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(dev)          # default priority, like the main stream

    def step(ev=None):
        # One call: prologue, routing and attention on the main stream.  The
        # library records ev[3] / ev[4] right around the attention kernel.
        if ev:
            ev[0].record()
        fva.layer(qd, kd, vd, w.p, w.kmin, w.budget, **blk, lists=lists, out=out,
                  kernel_events=(ev[3], ev[4]) if ev else None)
        if ev:
            ev[2].record()

    def step_overlapped():
        # Two calls, K/V copies on the side stream (into the main stream's
        # workspace) once the last attention has released it, routing
        # meanwhile on the main stream; join, attend.
        side.wait_stream(main)
        with torch.cuda.stream(side):
            fva.attn_prepare(kd, vd, **blk, stream=main)
        fva.route(qd, kd, w.p, w.kmin, w.budget, **blk, out=lists)
        main.wait_stream(side)
        fva.sparse_attn(qd, kd, vd, lists, out=out, prepared=True)

    def step_one_stream():
        fva.route(qd, kd, w.p, w.kmin, w.budget, **blk, out=lists)
        fva.sparse_attn(qd, kd, vd, lists, out=out)

    log(f"[bench] {w.name}: warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
        if full:
            step_overlapped()
            step_one_stream()
    torch.cuda.synchronize()
    # Per step: events around the call (main stream, where the library
    # launches) and the pair the library records right around the attention
    # kernel proper; what precedes that kernel is the prologue, the routing
    # and the plan.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for e in ev:                      # create the kernel events before the timed region
        e[3].record()
        e[4].record()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] {w.name}: timing {args.steps} steps")
    torch.cuda.synchronize()
    start.record()
    for s in range(args.steps):
        step(ev[s])
    stop.record()
    torch.cuda.synchronize()
    res = dict(ms_step=start.elapsed_time(stop) / args.steps,
               route_ms=float(np.mean([e[0].elapsed_time(e[3]) for e in ev])),
               attn_ms=float(np.mean([e[3].elapsed_time(e[2]) for e in ev])),
               kernel_ms=float(np.mean([e[3].elapsed_time(e[4]) for e in ev])))
    if full:
        # The same work as two calls, overlapped and on one stream.
        start.record()
        for s in range(args.steps):
            step_overlapped()
        stop.record()
        torch.cuda.synchronize()
        res["ms_overlapped"] = start.elapsed_time(stop) / args.steps
        start.record()
        for s in range(args.steps):
            step_one_stream()
        stop.record()
        torch.cuda.synchronize()
        res["ms_one_stream"] = start.elapsed_time(stop) / args.steps
        # The step captured once in a HIP graph and replayed; one eager call
        # on the capture stream first gives that stream its workspace.
        step()
        torch.cuda.synchronize()
        eager_o, eager_rp = out.clone(), lists.row_ptr.clone()
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(main)
        with torch.cuda.stream(cap):
            step()
        cap.synchronize()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                step()
        main.wait_stream(cap)
        torch.cuda.synchronize()
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        res["graph_ok"] = bool(torch.equal(out, eager_o) and torch.equal(lists.row_ptr, eager_rp))
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        start.record()
        for s in range(args.steps):
            graph.replay()
        stop.record()
        torch.cuda.synchronize()
        res["ms_graph"] = start.elapsed_time(stop) / args.steps
        del graph
        log(f"[bench] {w.name}: eager {res['ms_step']:.3f} ms, two calls {res['ms_overlapped']:.3f} ms "
            f"overlapped / {res['ms_one_stream']:.3f} ms one stream, "
            f"graph {res['ms_graph']:.3f} ms (replay {'matches' if res['graph_ok'] else 'DIFFERS FROM'} eager)")
    else:
        log(f"[bench] {w.name}: eager {res['ms_step']:.3f} ms")
    # Balance and the pair count: one more call with per-workgroup stats.
    st = torch.zeros(fva.stats_bytes(qd, w.grid, w.tile, order=order), dtype=torch.uint8, device=dev)
    fva.sparse_attn(qd, kd, vd, lists, out=out, stats=st)
    torch.cuda.synchronize()
    info, ctas = fva.parse_stats(st)
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    imb, busy = fva.per_cu_imbalance(ctas, ncu)
    rp = lists.row_ptr.cpu().numpy().astype(np.int64)
    ci = lists.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    nb = lists.nq
    counts = np.diff(rp)
    res.update(info=info, imbalance=imb, distinct_cus=len(busy), rp=rp, ci=ci, nb=nb,
               density=float(counts.sum()) / (w.B * w.H * nb * nb),
               density_per_head=counts.reshape(w.B * w.H, nb).sum(axis=1) / (nb * nb),
               base_density_per_head=lists.base_count[: len(counts)].cpu().numpy().reshape(w.B * w.H, nb).sum(axis=1)
               / (nb * nb),
               sizes=fva.block_sizes(w.grid, w.tile, ordered=hilbert), blk=blk, dev_tensors=(qd, kd, vd))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense (p = 1) comparison")
    ap.add_argument("--no-shard", action="store_true", help="skip the 5-head shard measurement")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of attention oracle work in the CPU baseline (routing runs in full)")
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
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.config]
    hilbert = args.blocks == "hilbert"
    log(f"[bench] generating {w.name}: B={w.B} H={w.H} d={w.d} grid={w.grid} tile={w.tile}")
    q, k, v, _ = make_inputs(w)
    pool = None
    if not args.no_cpu_baseline:
        pool, n_proc = start_cpu_pool(w, q, k, v, hilbert)      # forked before the GPU is touched

    import block_sparse_attention_22_amd as fva
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read + {args.copy_calibration_mib} MiB written")
        del src, dst

    r = run_workload(w, args, q, k, v, hilbert, full=True)
    info = r["info"]
    pairs = int(info.kept_pairs)
    flops = 4.0 * w.d * pairs
    sizes = r["sizes"]
    exe = ((sizes + 31) // 32) * 32                  # work the kernel issues: 32-query sub-tiles
    rows = np.repeat(np.arange(len(r["rp"]) - 1) % r["nb"], np.diff(r["rp"]))
    executed_pairs = int((exe[rows] * sizes[r["ci"]]).sum())
    ms_step, kernel_ms = r["ms_step"], r["kernel_ms"]
    tflops = flops / (ms_step * 1e-3) / 1e12
    kernel_tflops = flops / (kernel_ms * 1e-3) / 1e12
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
                   "tile": None if hilbert else list(w.tile), "p": w.p, "kmin": w.kmin, "budget": list(w.budget),
                   "tokens": w.N},
        "ms_per_layer": round(ms_step, 4),
        "ms_per_layer_graph": round(r["ms_graph"], 4),
        "graph_replay_bit_exact": r["graph_ok"],
        "ms_per_layer_two_calls_overlapped": round(r["ms_overlapped"], 4),
        "ms_per_layer_one_stream": round(r["ms_one_stream"], 4),
        "pre_attn_ms": round(r["route_ms"], 4),
        "attn_ms": round(r["attn_ms"], 4),
        "attn_kernel_ms": round(kernel_ms, 4),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "kept_valid_pairs": pairs,
        "effective_flop": flops,
        "executed_pairs_32_padded": executed_pairs,
        "executed_mfma_tflops": round(4.0 * w.d * executed_pairs / (kernel_ms * 1e-3) / 1e12, 2),
        "block_density": round(r["density"], 4),
        "block_density_per_head": [round(float(x), 4) for x in r["density_per_head"]],
        "base_density_per_head": [round(float(x), 4) for x in r["base_density_per_head"]],
        "per_cu_imbalance": round(r["imbalance"], 4),
        "per_workgroup_imbalance_predicted": round(float(info.predicted_imbalance), 4),
        "distinct_cus": r["distinct_cus"],
        "plan": {"n_items": info.n_items, "chunk_blocks": info.chunk_blocks, "n_split_rows": info.n_split_rows,
                 "n_partials": info.n_partials, "n_row_pairs": info.n_row_pairs, "num_ctas": info.num_ctas},
        "roofline": {"bound": bound, "achieved": round(kernel_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(kernel_tflops / peak, 4),
                     "traffic": measured_traffic() if (w.dtype == "bf16" and w.d == 128 and w.cid == 3
                                                       and not hilbert) else None,
                     "kernel": kernel_name, "per_launch_flop": flops, "avg_launch_ms": round(kernel_ms, 4)},
    }
    qd, kd, vd = r["dev_tensors"]
    if not args.no_dense:
        # Dense comparator: the same kernel on every key block (p = 1), after
        # the timed region; its lists replace nothing the step uses.
        log("[bench] dense comparison (p = 1)")
        dlists = fva.route(qd, kd, 1.0, 0, ("none", 0.0), **r["blk"])
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
    del qd, kd, vd, r["dev_tensors"]
    if args.config == 3 and not hilbert and not args.no_shard:
        ws = WORKLOADS[SHARD_CONFIG]
        log(f"[bench] shard: generating {ws.name}")
        qs, ks, vs, _ = make_inputs(ws)
        rs = run_workload(ws, args, qs, ks, vs, False, full=False)
        sflops = 4.0 * ws.d * int(rs["info"].kept_pairs)
        res.update({
            "shard_workload": ws.name,
            "shard_ms_per_layer": round(rs["ms_step"], 4),
            "shard_tflops": round(sflops / (rs["ms_step"] * 1e-3) / 1e12, 2),
            "shard_attn_kernel_ms": round(rs["kernel_ms"], 4),
            "shard_pre_attn_ms": round(rs["route_ms"], 4),
            "shard_per_cu_imbalance": round(rs["imbalance"], 4),
            "shard_per_workgroup_imbalance_predicted": round(float(rs["info"].predicted_imbalance), 4),
            "shard_block_density_per_head": [round(float(x), 4) for x in rs["density_per_head"]],
        })
        del rs
    if pool is not None:
        log(f"[bench] cpu baseline (oracle, {n_proc} processes)")
        cb = cpu_baseline(pool, n_proc, w, r["rp"], r["ci"], sizes, pairs, args.cpu_budget)
        pool.close()
        pool.join()
        res["cpu_baseline"] = {
            "value": round(flops / cb["full_s"] / 1e12, 6), "unit": "TFLOP/s", "cores": n_proc, "kind": "oracle",
            "sample": (f"routing oracle on all {w.B * w.H} heads ({cb['route_s']:.1f}s) and attention oracle "
                       f"(fp32 products, fp64 row stats) on {cb['attn_rows']} seeded query blocks "
                       f"({cb['attn_pairs']} of {pairs} kept pairs, {cb['attn_s']:.1f}s), on {n_proc} worker "
                       f"processes with one BLAS thread each; attention extrapolated to the layer by kept pairs: "
                       f"{cb['full_s']:.1f}s/layer"),
            "ms_per_layer_extrapolated": round(cb["full_s"] * 1e3, 1),
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
