"""Parity helpers (test infrastructure): compare the HIP path's block lists and
outputs with the CPU oracle.

List rule: bit-exact, except that a row's Top-p count may differ where the
oracle's cumulative mass lies within 1e-5 of p, and two masses that agree to
a relative 1e-12 may swap at a cut (the two sides sum the float64 pooled
means and scores in different orders, which moves a mass by ~1e-16 of
itself); augmentation is re-derived by the oracle from the GPU's own base
counts so one excused row cannot cascade.  Every use of either excuse is
counted; the workload tests require both counts to be zero.
Output rule: max |o_gpu - o_oracle| over the checked rows, the oracle run on
the GPU's own lists, in float64 (float32 products for the large layers).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import BlockLayout, attention, routing

P_WINDOW = 1e-5
TIE_REL = 1e-12   # relative: |P_a - P_b| <= TIE_REL * max(P_a, P_b)


def to_numpy(t: torch.Tensor, dtype=np.float64) -> np.ndarray:
    """Exact upcast of CPU bf16/fp32 tensors to numpy."""
    return t.to(torch.float64 if dtype == np.float64 else torch.float32).numpy()


def gpu_lists_to_host(lists):
    rp = lists.row_ptr.cpu().numpy().astype(np.int64)
    ci = lists.col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
    return dict(row_ptr=rp, col_idx=ci, base=lists.base_count[: len(rp) - 1].cpu().numpy().astype(np.int64),
                head_kept=lists.head_kept.cpu().numpy().astype(np.int64))


def compare_lists(gpu: dict, ref: dict, p: float, budget, layout: BlockLayout, B: int, H: int) -> dict:
    """Check GPU lists against the oracle; returns a report, raises on failure."""
    Nb = layout.Nb
    mode, frac = budget
    rep = dict(rows=B * H * Nb, exact_rows=0, excused_count_rows=0, excused_tie_rows=0)
    rp, ci = gpu["row_ptr"], gpu["col_idx"]
    assert rp[0] == 0 and np.all(np.diff(rp) >= 1), "every row keeps at least one block"
    for b in range(B):
        base_g = gpu["base"][b * H * Nb:(b + 1) * H * Nb].reshape(H, Nb)
        K_g = base_g.sum(axis=1)
        B_g = routing.head_budget(K_g, mode, frac, Nb, Nb)
        for h in range(H):
            hd = ref["heads"][b][h]
            bh = b * H + h
            assert gpu["head_kept"][bh] == B_g[h], f"head {bh}: total {gpu['head_kept'][bh]} != budget {B_g[h]}"
            m_g, m_r = base_g[h], hd["base"]
            for i in np.nonzero(m_g != m_r)[0]:
                lo, hi = sorted((int(m_g[i]), int(m_r[i])))
                c = hd["cum"][i]
                ok = all(abs(c[m - 1] - p) <= P_WINDOW for m in range(max(lo, 1), hi))
                assert ok, f"head {bh} row {i}: base count {m_g[i]} vs oracle {m_r[i]} (cum {c[lo - 1:hi]})"
                rep["excused_count_rows"] += 1
            A = int(B_g[h] - K_g[h])
            add = routing.augment(hd["P"], hd["order"], m_g, A)
            cnt = m_g + add
            # threshold mass of the augmentation (for tie excuses across rows)
            tau = None
            if A > 0:
                vals = np.concatenate([hd["P"][i, hd["order"][i, m_g[i]:cnt[i]]] for i in range(Nb)])
                tau = vals.min()
            r0 = bh * Nb
            assert rp[r0 + Nb] - rp[r0] == int(cnt.sum())
            for i in range(Nb):
                got = ci[rp[r0 + i]:rp[r0 + i + 1]]
                assert np.all(np.diff(got) > 0), f"head {bh} row {i}: columns not ascending/unique"
                exp = np.sort(hd["order"][i, :cnt[i]])
                if len(got) == len(exp) and np.array_equal(got, exp):
                    rep["exact_rows"] += 1
                    continue
                diff = np.setxor1d(got, exp)
                P = hd["P"][i]
                bnd = [P[exp].min()] + ([tau] if tau is not None else [])
                ok = all(any(abs(P[x] - t) <= TIE_REL * max(P[x], t) for t in bnd) for x in diff)
                assert ok, f"head {bh} row {i}: lists differ beyond near-ties: gpu {got} oracle {exp}"
                rep["excused_tie_rows"] += 1
    return rep


def assert_exact(rep: dict) -> None:
    """Every row matched the oracle without either excuse."""
    assert rep["excused_count_rows"] == 0 and rep["excused_tie_rows"] == 0, rep
    assert rep["exact_rows"] == rep["rows"], rep


def head_csr(rp, ci, bh, Nb):
    r0 = bh * Nb
    hrp = rp[r0:r0 + Nb + 1] - rp[r0]
    hci = ci[rp[r0]:rp[r0 + Nb]]
    return hrp, hci


def attention_error(o_gpu: torch.Tensor, q, k, v, layout: BlockLayout, rp, ci, rows=None, precision="fp64"):
    """Max |o_gpu - oracle| over the given rows (dict bh -> row list, None = all).

    q, k, v: numpy [B, H, N, d]; o_gpu: device or CPU tensor [B, H, N, d]."""
    B, H = q.shape[:2]
    Nb = layout.Nb
    worst = 0.0
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            sel = range(Nb) if rows is None else rows[bh]
            hrp, hci = head_csr(rp, ci, bh, Nb)
            ref = attention.sparse_attention_head(q[b, h], k[b, h], v[b, h], layout, hrp, hci, rows=sel,
                                                  precision=precision)
            toks = np.concatenate([layout.members[i] for i in sel])
            idx = torch.as_tensor(toks, device=o_gpu.device)
            got = o_gpu[b, h].index_select(0, idx).double().cpu().numpy()
            err = float(np.abs(got - ref[toks]).max())
            assert np.isfinite(err), f"non-finite output in head {bh}"
            worst = max(worst, err)
    return worst
