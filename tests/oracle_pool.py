"""Oracle attention on many query blocks at once, in a pool of worker
processes (test infrastructure).

A GPU test that checks outputs at full size writes the GPU's lists, the
query blocks to check and the GPU's output rows to an .npz file, then runs

    python tests/oracle_pool.py <file.npz>

as a child process, which regenerates the seeded inputs, runs the CPU
oracle (fp32 products, fp64 row statistics) on every listed query block and
prints one JSON line: the largest |o_gpu - o_oracle| of every listed block.
The child never touches the GPU, so its workers are plain forked processes.

npz fields: cid (workload id), hilbert (0/1), row_ptr, col_idx (the GPU's
CSR over all (b, h, i) rows), rows (int64 [n, 2]: (b*H + h, i) per checked
query block) and out (the GPU's output of those blocks' tokens, float32,
concatenated in the order of `rows`, each block's tokens in layout order).
The inputs themselves sit beside it as <stem>_q.npy, <stem>_k.npy and
<stem>_v.npy ([B, H, N, d]; uint16 bf16 bit patterns or float32), memory-
mapped by the workers.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

POOL_MAX = 16
_S = {}


def _init():
    from threadpoolctl import threadpool_limits
    _S["limits"] = threadpool_limits(1)


def _f32(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:             # bf16 bits -> float32, exactly
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float32)


def _check(task):
    from oracle import attention
    bh, rows, offs = task
    w, lay = _S["w"], _S["lay"]
    b, h = divmod(bh, w.H)
    q, k, v = (_f32(_S[n][b, h]) for n in ("q", "k", "v"))
    nb = lay.Nb
    rp, ci = _S["row_ptr"], _S["col_idx"]
    r0 = bh * nb
    hrp = rp[r0:r0 + nb + 1] - rp[r0]
    hci = ci[rp[r0]:rp[r0 + nb]]
    ref = attention.sparse_attention_head(q, k, v, lay, hrp, hci, rows=rows, precision="fp32")
    out = []
    for i, off in zip(rows, offs):
        toks = lay.members[i]
        got = _S["out"][off:off + len(toks)].astype(np.float64)
        err = np.abs(got - ref[toks])
        out.append(float(err.max()) if np.isfinite(err).all() else float("inf"))
    return bh, rows, out


def main(path):
    import multiprocessing as mp

    from oracle import BlockLayout, HilbertLayout
    from workloads import WORKLOADS

    z = np.load(path)
    w = WORKLOADS[int(z["cid"])]
    lay = HilbertLayout(w.grid) if int(z["hilbert"]) else BlockLayout(w.grid, w.tile)
    stem = path[:-4] if path.endswith(".npz") else path
    _S.update(w=w, lay=lay, row_ptr=z["row_ptr"].astype(np.int64), col_idx=z["col_idx"].astype(np.int64),
              out=z["out"])
    for n in ("q", "k", "v"):
        _S[n] = np.load(f"{stem}_{n}.npy", mmap_mode="r")
    rows = z["rows"].astype(np.int64)
    sizes = lay.sizes[rows[:, 1]]
    offs = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    # tasks of up to 8 query blocks of one head
    tasks, by_head = [], {}
    for (bh, i), off in zip(rows.tolist(), offs.tolist()):
        by_head.setdefault(bh, []).append((i, off))
    for bh, lst in by_head.items():
        for s in range(0, len(lst), 8):
            part = lst[s:s + 8]
            tasks.append((bh, [i for i, _ in part], [o for _, o in part]))
    n = max(1, min(POOL_MAX, len(os.sched_getaffinity(0))))
    errs = {}
    with mp.get_context("fork").Pool(n, initializer=_init) as pool:
        for bh, rs, es in pool.imap_unordered(_check, tasks):
            for i, e in zip(rs, es):
                errs[(bh, i)] = e
    print(json.dumps({"processes": n, "err": [errs[(bh, i)] for bh, i in rows.tolist()]}), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
