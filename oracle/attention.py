"""Exact softmax attention over the kept key blocks (oracle).

TEST INFRASTRUCTURE ONLY: see the package docstring.

FVAttn runs dynamic block-sparse attention: exact attention restricted to the
(query block, key block) pairs the router kept (paperlayer.ai summary of
FVAttn, section 2 "Background and Related Work", Sparse Attention; section 3
"FVAttn Design", Pipeline).  For a query token t in block i and the set U of
valid tokens of row i's kept key blocks:

    o_t = sum_{u in U} exp(q_t.k_u/sqrt(d) - M_t) v_u / sum_{u in U} exp(q_t.k_u/sqrt(d) - M_t)

with M_t = max_u q_t.k_u/sqrt(d).  Attention is bidirectional (no causal mask).
"""
from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

from .blocks import BlockLayout


def _rows_softmax_av(qi, kk, vv, precision):
    d = qi.shape[1]
    if precision == "fp64":
        s = (qi.astype(np.float64) @ kk.astype(np.float64).T) / math.sqrt(d)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        return (e @ vv.astype(np.float64)) / e.sum(axis=1, keepdims=True)
    # float32 products, float64 row statistics
    s = (qi.astype(np.float32) @ kk.astype(np.float32).T).astype(np.float64) / math.sqrt(d)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    o = (e.astype(np.float32) @ vv.astype(np.float32)).astype(np.float64)
    return o / e.sum(axis=1, keepdims=True)


def sparse_attention_head(q, k, v, layout: BlockLayout, row_ptr, col_idx,
                          rows: Optional[Iterable[int]] = None, precision: str = "fp64"):
    """O8 for one (batch, head).  q, k, v: [N, d].  row_ptr/col_idx: this head's CSR.

    Returns o [N, d] float64; tokens of rows not in ``rows`` are NaN.
    """
    N, d = q.shape
    o = np.full((N, d), np.nan, dtype=np.float64)
    rows = range(layout.Nb) if rows is None else rows
    for i in rows:
        js = col_idx[row_ptr[i]:row_ptr[i + 1]]
        qi_tok = layout.members[i]
        if len(js) == 0:
            continue
        keys = np.concatenate([layout.members[j] for j in js])
        o[qi_tok] = _rows_softmax_av(q[qi_tok], k[keys], v[keys], precision)
    return o


def kept_pairs(layout: BlockLayout, row_ptr, col_idx, nrows_per_head: int):
    """Kept valid query-key token pairs: sum over kept (i, j) of n_i * n_j.

    row_ptr/col_idx span every (b, h) row in order; returns the total and the
    per-head totals.
    """
    sizes = layout.sizes
    nrows = len(row_ptr) - 1
    per_row = np.zeros(nrows, dtype=np.int64)
    for r in range(nrows):
        js = col_idx[row_ptr[r]:row_ptr[r + 1]]
        per_row[r] = sizes[r % nrows_per_head] * int(sizes[js].sum())
    per_head = per_row.reshape(-1, nrows_per_head).sum(axis=1)
    return int(per_row.sum()), per_head
