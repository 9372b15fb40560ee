"""Sparse-routing front end (oracle, float64 numpy).

TEST INFRASTRUCTURE ONLY: see the package docstring.

Steps, in the pages' order (paperlayer.ai summary of FVAttn, section 3 "FVAttn
Design": Pipeline and Sparse-routing frontend; section 2 "Background and
Related Work": Sparse Attention):

  O2 pool     mean of Q and of K over each block's tokens;
  O3 scores   block similarity s_ij = qbar_i . kbar_j / sqrt(d) and its row
              softmax P_ij (how each query block's similarity spreads over the
              key blocks);
  O4 order    per query block, key blocks by P descending, ties to lower j
              (the routing importance order that augmentation follows);
  O5 cut      Top-p: the smallest prefix whose cumulative mass reaches p,
              then a Top-k floor that keeps at least kmin blocks;
  O6 augment  slack-aware augmentation: per head, add the next-highest-mass
              not-yet-kept blocks up to a per-head budget, without changing p;
  O7 csr      per-row kept key blocks, ascending, as CSR.

Readings where the pages are silent:
  * the score has no block-size correction and uses the same 1/sqrt(d) scale
    as attention;
  * the cut is c_m >= p; p >= 1 (or no prefix reaching p because of
    rounding) keeps every block; the floor is m = min(Nk, max(m_p, kmin));
  * augmentation ranks candidates by the row-normalised mass P_ij, ties to
    lower (i, j); budgets: none, +floor(frac*K_h), or the largest K_h' of
    the same batch item ("match_max").
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

from .blocks import BlockLayout


def pool(x: np.ndarray, layout: BlockLayout) -> np.ndarray:
    """O2: mean of x [N, d] over each block's valid tokens -> [Nb, d] float64."""
    x = np.asarray(x, dtype=np.float64)
    return np.stack([x[m].mean(axis=0) for m in layout.members])


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """O3 (first half): s_ij = qbar_i . kbar_j / sqrt(d), float64 [Nq, Nk]."""
    d = qbar.shape[1]
    return (qbar @ kbar.T) / math.sqrt(d)


def row_softmax(s: np.ndarray) -> np.ndarray:
    """O3 (second half): P_ij = exp(s_ij - max_j s_ij) / sum_j exp(...)."""
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def importance_order(P: np.ndarray) -> np.ndarray:
    """O4: per row, key-block indices by P descending; equal P -> lower j first.

    A stable sort of -P keeps equal keys in ascending j.  A row whose masses
    are all NaN (the softmax of a row holding a non-finite score) stays in
    block order.
    """
    return np.argsort(-P, axis=1, kind="stable")


def topp_floor(P: np.ndarray, order: np.ndarray, p: float, kmin: int):
    """O5: base count m_i per row and the sorted cumulative masses c.

    c_m is the sum of the m largest P of the row, accumulated in sorted order.
    m_p = min{m : c_m >= p}; m_p = Nk when p >= 1 or no prefix reaches p.
    m_i = min(Nk, max(m_p, kmin)).
    """
    Nq, Nk = P.shape
    Ps = np.take_along_axis(P, order, axis=1)
    c = np.cumsum(Ps, axis=1)
    if p >= 1.0:
        m_p = np.full(Nq, Nk, dtype=np.int64)
    else:
        reached = c >= p
        m_p = np.where(reached.any(axis=1), reached.argmax(axis=1) + 1, Nk)
    m = np.minimum(Nk, np.maximum(m_p, int(kmin)))
    # A row whose masses are not finite numbers (a non-finite q or k token
    # upstream) has no prefix whose mass reaches p, so it keeps every block;
    # importance_order leaves such a row in block order.
    assert np.all(m[~np.isfinite(P).all(axis=1)] == Nk)
    return m.astype(np.int64), c


def head_budget(K: np.ndarray, mode: str, frac: float, Nq: int, Nk: int) -> np.ndarray:
    """Per-head block budget B_h for one batch item; K = base totals [H].

    none:      B_h = K_h
    frac:      B_h = min(Nq*Nk, K_h + floor(frac * K_h))   (frac as float64)
    match_max: B_h = max over heads h' of K_h'
    """
    K = np.asarray(K, dtype=np.int64)
    if mode == "none":
        return K.copy()
    if mode == "frac":
        add = np.array([math.floor(float(frac) * int(x)) for x in K], dtype=np.int64)
        return np.minimum(Nq * Nk, K + add)
    if mode == "match_max":
        return np.full_like(K, K.max())
    raise ValueError(mode)


def augment(P: np.ndarray, order: np.ndarray, m: np.ndarray, A: int) -> np.ndarray:
    """O6 for one head: number of blocks added to each row.

    Candidates are the not-yet-kept entries (i, order[i, r]) with r >= m_i.
    The A candidates with the largest P are taken, equal P broken by lower i,
    then lower j.  Returns add[i] (taken entries of row i, always a prefix of
    the row's remaining order).
    """
    Nq, Nk = P.shape
    add = np.zeros(Nq, dtype=np.int64)
    if A <= 0:
        return add
    ii, rr = [], []
    for i in range(Nq):
        r = np.arange(m[i], Nk)
        ii.append(np.full(len(r), i))
        rr.append(r)
    ii = np.concatenate(ii)
    rr = np.concatenate(rr)
    jj = order[ii, rr]
    pv = P[ii, jj]
    assert A <= len(pv)
    sel = np.lexsort((jj, ii, -pv))[:A]      # primary -P, then i, then j
    np.add.at(add, ii[sel], 1)
    return add


def to_csr(order: np.ndarray, counts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """O7: CSR over rows; each row's kept key blocks in ascending order."""
    Nq = order.shape[0]
    row_ptr = np.zeros(Nq + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col = np.concatenate([np.sort(order[i, :counts[i]]) for i in range(Nq)]) if Nq else np.zeros(0, np.int64)
    return row_ptr, col.astype(np.int64)


def route_head(q: np.ndarray, k: np.ndarray, layout: BlockLayout, p: float, kmin: int) -> Dict:
    """O2-O5 for one (batch, head); q, k: [N, d] (any float dtype)."""
    qbar = pool(q, layout)
    kbar = pool(k, layout)
    s = block_scores(qbar, kbar)
    P = row_softmax(s)
    order = importance_order(P)
    m, c = topp_floor(P, order, p, kmin)
    return dict(qbar=qbar, kbar=kbar, s=s, P=P, order=order, base=m, cum=c)


def _route_head_args(args):
    return route_head(*args)


def route(q, k, layout: BlockLayout, p: float, kmin: int, budget=("none", 0.0), map_fn=map) -> Dict:
    """Full front end (O2-O7) over q, k [B, H, N, d].

    ``map_fn`` evaluates the independent per-head steps O2-O5 (e.g. a process
    pool's ``map``); augmentation and CSR then run in (b, h) order.

    Returns a dict with per-head lists (``heads[b][h]``) and the flattened
    (b, h, i)-ordered arrays ``base`` [B*H*Nq], ``count`` [B*H*Nq],
    ``row_ptr`` [B*H*Nq+1], ``col_idx``, ``head_kept`` [B*H].
    """
    q = np.asarray(q)
    k = np.asarray(k)
    B, H = q.shape[:2]
    Nq = Nk = layout.Nb
    mode, frac = budget
    flat = list(map_fn(_route_head_args, [(q[b, h], k[b, h], layout, p, kmin) for b in range(B) for h in range(H)]))
    heads = [flat[b * H:(b + 1) * H] for b in range(B)]
    base, count, cols, kept = [], [], [], []
    for b in range(B):
        K = np.array([heads[b][h]["base"].sum() for h in range(H)], dtype=np.int64)
        Bh = head_budget(K, mode, frac, Nq, Nk)
        for h in range(H):
            r = heads[b][h]
            A = int(Bh[h] - K[h])
            add = augment(r["P"], r["order"], r["base"], A)
            cnt = r["base"] + add
            rp, ci = to_csr(r["order"], cnt)
            r.update(add=add, count=cnt, row_ptr=rp, col_idx=ci, budget=int(Bh[h]))
            base.append(r["base"])
            count.append(cnt)
            cols.append(ci)
            kept.append(int(cnt.sum()))
    base = np.concatenate(base) if base else np.zeros(0, np.int64)
    count = np.concatenate(count) if count else np.zeros(0, np.int64)
    row_ptr = np.zeros(len(count) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(count)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    return dict(heads=heads, base=base, count=count, row_ptr=row_ptr, col_idx=col_idx,
                head_kept=np.asarray(kept, dtype=np.int64), Nq=Nq, Nk=Nk)

