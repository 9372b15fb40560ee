"""Pins for the CPU oracle: hand-worked fixtures, closed forms, brute force and
library routines that do not share the oracle's own code paths.

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
transposed operand, a wrong axis, > instead of >=, a wrong tie rule, a divisor
that counts padding) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import BlockLayout, routing, attention
from workloads import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- blocks (O1)

@pytest.mark.parametrize("cid,nb,padded", [(1, 4, 256), (2, 84, 10752), (3, 660, 84480),
                                            (4, 660, 84480), (5, 1485, 190080)])
def test_block_counts_closed_form(cid, nb, padded):
    w = WORKLOADS[cid]
    lay = BlockLayout(w.grid, w.tile)
    assert lay.Nb == nb
    assert lay.padded_N == padded
    assert int(lay.sizes.sum()) == w.N


@pytest.mark.parametrize("grid,tile", [((21, 45, 80), (2, 8, 8)), ((5, 30, 52), (2, 8, 8)),
                                       ((3, 2, 5), (2, 2, 4)), ((1, 5, 5), (2, 8, 8))])
def test_blocks_partition_tokens(grid, tile):
    lay = BlockLayout(grid, tile)
    allm = np.concatenate(lay.members)
    assert np.array_equal(np.sort(allm), np.arange(lay.N))      # each token exactly once
    T, Y, X = grid
    for b, m in enumerate(lay.members):                          # every member lies in its tile
        it, iy, ix = b // (lay.nY * lay.nX), (b // lay.nX) % lay.nY, b % lay.nX
        t, y, x = m // (Y * X), (m // X) % Y, m % X
        assert np.all(t // tile[0] == it) and np.all(y // tile[1] == iy) and np.all(x // tile[2] == ix)


def test_720p_block_size_mix():
    lay = BlockLayout((21, 45, 80), (2, 8, 8))
    vals, cnt = np.unique(lay.sizes, return_counts=True)
    assert dict(zip(vals.tolist(), cnt.tolist())) == {40: 10, 64: 50, 80: 100, 128: 500}


def test_golden_blocks_and_pooling():
    g = _load("blocks_scores_attention_cases.json")["blocks"]
    lay = BlockLayout(g["grid"], g["tile"])
    assert lay.Nb == g["Nb"] and lay.sizes.tolist() == g["sizes"]
    T, Y, X = g["grid"]
    n = np.arange(lay.N)
    coords = np.stack([n // (Y * X), (n // X) % Y, n % X, np.ones_like(n)], 1).astype(np.float64)
    cen = routing.pool(coords, lay)
    assert np.allclose(cen[:, :3], np.asarray(g["centroids_tyx"]), atol=0, rtol=0)
    assert np.all(cen[:, 3] == 1.0)      # divides by the valid count, not the padded tile size


# ---------------------------------------------------------------- scores (O3)

def test_golden_scores_orientation():
    g = _load("blocks_scores_attention_cases.json")["scores"]
    s = routing.block_scores(np.asarray(g["qbar"], float), np.asarray(g["kbar"], float))
    assert s.shape == (2, 3)
    assert np.array_equal(s, np.asarray(g["s"]))


def test_golden_softmax_closed_form():
    g = _load("blocks_scores_attention_cases.json")["softmax"]
    P = routing.row_softmax(np.asarray([g["s"]]))
    assert np.allclose(P[0], g["P"], rtol=1e-15, atol=1e-15)


def test_softmax_rows_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(0)
    s = rng.normal(0, 30, size=(7, 13))
    P = routing.row_softmax(s)
    assert np.allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(routing.row_softmax(s + rng.normal(0, 5, size=(7, 1))), P, atol=1e-14)
    # textbook routine: torch.softmax on the same rows (fp64)
    assert np.allclose(torch.softmax(torch.from_numpy(s), dim=1).numpy(), P, rtol=1e-13, atol=1e-300)


def test_constant_inputs_give_uniform_routing():
    lay = BlockLayout((2, 8, 8), (1, 8, 8))
    q = np.ones((lay.N, 8))
    r = routing.route_head(q, q, lay, 0.5, 0)
    assert np.allclose(r["P"], 1.0 / lay.Nb, rtol=0, atol=1e-15)


# ----------------------------------------------------- order and Top-p (O4, O5)

def test_golden_topp_floor():
    for c in _load("topp_floor_cases.json")["cases"]:
        P = np.asarray([c["P"]], dtype=np.float64)
        order = routing.importance_order(P)
        m, _ = routing.topp_floor(P, order, c["p"], c["kmin"])
        assert int(m[0]) == c["m"], c["why"]
        assert sorted(order[0, :m[0]].tolist()) == c["kept"], c["why"]


def _brute_min_size(P, p):
    """Smallest subset size whose total mass reaches p (exhaustive)."""
    Nk = len(P)
    if p >= 1.0:
        return Nk
    for size in range(1, Nk + 1):
        best = max(math.fsum(P[list(S)]) for S in itertools.combinations(range(Nk), size))
        if best >= p:
            return size
    return Nk


def _ref_order(Prow):
    return sorted(range(len(Prow)), key=lambda j: (-Prow[j], j))


@pytest.mark.parametrize("seed", range(40))
def test_topp_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    Nk = int(rng.integers(1, 11))
    # dyadic masses (exact sums) with frequent ties
    w = rng.integers(1, 5, size=Nk).astype(np.float64)
    tot = 2.0 ** math.ceil(math.log2(w.sum()))
    w[0] += tot - w.sum()
    P = w / tot
    assert math.fsum(P) == 1.0
    p = float(rng.choice([1e-9, 0.25, 0.5, 0.6, 0.75, 0.9, 0.95, 1.0]))
    kmin = int(rng.integers(0, Nk + 2))
    order = routing.importance_order(P[None, :])
    m, c = routing.topp_floor(P[None, :], order, p, kmin)
    m_expected = min(Nk, max(_brute_min_size(P, p), kmin))
    assert int(m[0]) == m_expected
    kept = order[0, :m[0]].tolist()
    assert kept == _ref_order(P)[:m_expected]
    # the kept set has the largest mass among all sets of its size
    best = max(math.fsum(P[list(S)]) for S in itertools.combinations(range(Nk), m_expected))
    assert math.fsum(P[kept]) == best


def test_p_to_zero_is_fixed_topk():
    rng = np.random.default_rng(3)
    P = routing.row_softmax(rng.normal(0, 2, size=(50, 37)))
    for kmin in (0, 1, 5, 37, 40):
        order = routing.importance_order(P)
        m, _ = routing.topp_floor(P, order, 1e-300, kmin)
        assert np.all(m == min(37, max(kmin, 1)))
        for i in range(50):
            assert sorted(order[i, :m[i]].tolist()) == sorted(_ref_order(P[i])[:m[i]])


def test_p_one_keeps_all():
    rng = np.random.default_rng(4)
    P = routing.row_softmax(rng.normal(0, 9, size=(20, 30)))
    m, _ = routing.topp_floor(P, routing.importance_order(P), 1.0, 0)
    assert np.all(m == 30)


# ------------------------------------------------------------ augmentation (O6)

def test_golden_augment():
    g = _load("augment_cases.json")
    for c in g["cases"]:
        P = np.asarray(c["P"], dtype=np.float64)
        order = routing.importance_order(P)
        for A, exp in c["add"].items():
            add = routing.augment(P, order, np.asarray(c["base"]), int(A))
            assert add.tolist() == exp, (A, c["why"])
    for b in g["budgets"]:
        Bh = routing.head_budget(np.asarray(b["K"]), b["mode"], b["frac"], b["Nq"], b["Nk"])
        assert Bh.tolist() == b["B"], b["why"]


@pytest.mark.parametrize("seed", range(25))
def test_augment_is_max_mass_prefix(seed):
    rng = np.random.default_rng(100 + seed)
    Nq, Nk = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    w = rng.integers(1, 4, size=(Nq, Nk)).astype(np.float64)
    P = w / w.sum(axis=1, keepdims=True)
    order = routing.importance_order(P)
    base = np.asarray([int(rng.integers(1, Nk + 1)) for _ in range(Nq)])
    cands = [(i, int(order[i, r])) for i in range(Nq) for r in range(base[i], Nk)]
    for A in range(len(cands) + 1):
        add = routing.augment(P, order, base, A)
        assert int(add.sum()) == A                                # exact total
        assert np.all(base + add <= Nk)
        taken = [(i, int(order[i, r])) for i in range(Nq) for r in range(base[i], base[i] + add[i])]
        mass = math.fsum(P[i, j] for i, j in taken)
        best = max((math.fsum(P[i, j] for i, j in S) for S in itertools.combinations(cands, A)), default=0.0)
        assert abs(mass - best) < 1e-12                           # maximal added mass
        # tie rule: any candidate left out has mass <= every candidate taken,
        # and equal mass only if it comes later in (i, j) order
        left = [c for c in cands if c not in taken]
        for (i, j) in taken:
            for (a, b) in left:
                assert P[i, j] > P[a, b] or (P[i, j] == P[a, b] and (i, j) < (a, b))


# --------------------------------------------------------------- CSR and route

def test_route_end_to_end_invariants():
    lay = BlockLayout((3, 16, 16), (1, 8, 8))
    rng = np.random.default_rng(7)
    q = rng.normal(size=(2, 3, lay.N, 16))
    k = q + 0.3 * rng.normal(size=q.shape)
    for budget in (("none", 0.0), ("frac", 0.25), ("match_max", 0.0)):
        r = routing.route(q, k, lay, 0.8, 2, budget)
        Nb = lay.Nb
        assert np.array_equal(np.diff(r["row_ptr"]), r["count"])
        assert np.all(r["count"] >= r["base"]) and np.all(r["base"] >= 2)
        for b in range(2):
            K = np.array([r["heads"][b][h]["base"].sum() for h in range(3)])
            for h in range(3):
                hd = r["heads"][b][h]
                if budget[0] == "none":
                    assert hd["count"].sum() == K[h]
                elif budget[0] == "frac":
                    assert hd["count"].sum() == min(Nb * Nb, K[h] + math.floor(0.25 * K[h]))
                else:
                    assert hd["count"].sum() == K.max()
                for i in range(Nb):
                    cols = hd["col_idx"][hd["row_ptr"][i]:hd["row_ptr"][i + 1]]
                    assert np.all(np.diff(cols) > 0)                       # ascending, unique
                    assert set(cols.tolist()) == set(hd["order"][i, :hd["count"][i]].tolist())


# ------------------------------------------------------------- attention (O8)

def test_golden_attention():
    g = _load("blocks_scores_attention_cases.json")["attention"]
    lay = BlockLayout((1, 1, 2), (1, 1, 1))
    q = np.stack([np.asarray(g["q"]), np.zeros(4)])
    k = np.asarray(g["k"], dtype=np.float64)
    v = np.asarray(g["v"], dtype=np.float64)
    o = attention.sparse_attention_head(q, k, v, lay, np.array([0, 2, 3]), np.array([0, 1, 1]))
    assert np.allclose(o[0], g["o"], rtol=1e-14, atol=1e-14)
    assert np.allclose(o[1], v[1])          # row 1 keeps only block 1: softmax over one key


def _sdpa(q, k, v):
    """torch CPU scaled_dot_product_attention in float64 (a library routine)."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()


def test_p_one_is_dense_attention():
    lay = BlockLayout((2, 5, 9), (1, 4, 4))
    rng = np.random.default_rng(11)
    q, k, v = (rng.normal(size=(1, 1, lay.N, 16)) * s for s in (1.5, 1.5, 1.0))
    r = routing.route(q, k, lay, 1.0, 0)
    assert np.all(r["count"] == lay.Nb)
    o = attention.sparse_attention_head(q[0, 0], k[0, 0], v[0, 0], lay, r["row_ptr"], r["col_idx"])
    assert np.allclose(o, _sdpa(q[0, 0], k[0, 0], v[0, 0]), rtol=1e-12, atol=1e-12)
    o32 = attention.sparse_attention_head(q[0, 0], k[0, 0], v[0, 0], lay, r["row_ptr"], r["col_idx"],
                                          precision="fp32")
    assert np.abs(o32 - o).max() < 1e-5


def test_single_block_and_identical_keys():
    lay = BlockLayout((1, 4, 8), (1, 4, 4))       # 2 blocks of 16 tokens
    rng = np.random.default_rng(12)
    q, k, v = (rng.normal(size=(lay.N, 8)) for _ in range(3))
    rp, ci = np.array([0, 1, 2]), np.array([1, 0])  # row 0 keeps block 1, row 1 keeps block 0
    o = attention.sparse_attention_head(q, k, v, lay, rp, ci)
    m0, m1 = lay.members
    assert np.allclose(o[m0], _sdpa(q[m0], k[m1], v[m1]), atol=1e-12)
    assert np.allclose(o[m1], _sdpa(q[m1], k[m0], v[m0]), atol=1e-12)
    k_same = np.tile(k[:1], (lay.N, 1))            # identical keys -> plain mean of V
    o = attention.sparse_attention_head(q, k_same, v, lay, np.array([0, 2, 4]), np.array([0, 1, 0, 1]))
    assert np.allclose(o, np.tile(v.mean(axis=0), (lay.N, 1)), atol=1e-12)


def test_csr_order_does_not_matter():
    lay = BlockLayout((2, 8, 8), (1, 4, 4))
    rng = np.random.default_rng(13)
    q, k, v = (rng.normal(size=(lay.N, 8)) for _ in range(3))
    rp = np.array([0, 3] + [3] * (lay.Nb - 1))
    o1 = attention.sparse_attention_head(q, k, v, lay, rp, np.array([1, 4, 6]), rows=[0])
    o2 = attention.sparse_attention_head(q, k, v, lay, rp, np.array([6, 1, 4]), rows=[0])
    m0 = lay.members[0]
    assert np.allclose(o1[m0], o2[m0], atol=1e-13)


def test_kept_pairs_counts_valid_tokens():
    lay = BlockLayout((3, 2, 5), (2, 2, 4))         # sizes 16, 4, 8, 2
    rp = np.array([0, 4, 5, 6, 8])
    ci = np.array([0, 1, 2, 3, 1, 2, 0, 3])
    tot, per_head = attention.kept_pairs(lay, rp, ci, 4)
    assert tot == 16 * 30 + 4 * 4 + 8 * 8 + 2 * (16 + 2)
    assert per_head.tolist() == [tot]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kept_pairs_by_token_enumeration(seed):
    """Brute force: count every (query token, key token) pair whose key's
    block is kept by the query's block, over ragged tiles and two heads."""
    lay = BlockLayout((3, 5, 7), (2, 2, 4))          # 2 x 3 x 2 = 12 blocks of 16, 8, 4, 12, 6, 3 tokens
    rng = np.random.default_rng(40 + seed)
    H = 2
    rows = []
    for _ in range(H * lay.Nb):
        rows.append(np.sort(rng.choice(lay.Nb, rng.integers(0, lay.Nb + 1), replace=False)))
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
    ci = np.concatenate(rows)
    owner = np.empty(lay.N, dtype=np.int64)
    for b, m in enumerate(lay.members):
        owner[m] = b
    expect = []
    for h in range(H):
        kept = [set(rows[h * lay.Nb + i].tolist()) for i in range(lay.Nb)]
        expect.append(sum(1 for t in range(lay.N) for u in range(lay.N) if owner[u] in kept[owner[t]]))
    tot, per_head = attention.kept_pairs(lay, rp, ci, lay.Nb)
    assert per_head.tolist() == expect and tot == sum(expect)


# --------------------------------------------------------------- Hilbert order
# The curve's defining properties, each of which a plausible slip breaks: a
# bijection onto the cube (a lost bit), unit steps between consecutive points
# (a missing exchange or Gray step; Morton order fails it), and every aligned
# sub-cube visited as one contiguous run (a snake order fails it).
import itertools  # noqa: E402

from oracle.hilbert import HilbertLayout, cube_bits, hilbert_index, hilbert_token_order  # noqa: E402


@pytest.mark.parametrize("n,bits", [(2, 1), (2, 3), (3, 1), (3, 2), (3, 3), (3, 4)])
def test_hilbert_is_a_unit_step_bijection(n, bits):
    pts = np.array(list(itertools.product(range(1 << bits), repeat=n)))
    h = hilbert_index(pts, bits)
    assert np.array_equal(np.sort(h), np.arange(len(pts)))
    walk = pts[np.argsort(h)]
    assert np.array_equal(walk[0], np.zeros(n, dtype=walk.dtype))          # starts at the origin
    assert (np.abs(np.diff(walk, axis=0)).sum(axis=1) == 1).all()          # one axis, one step


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_hilbert_visits_aligned_subcubes_contiguously(bits):
    pts = np.array(list(itertools.product(range(1 << bits), repeat=3)))
    walk = pts[np.argsort(hilbert_index(pts, bits))]
    for k in range(1, bits):
        runs = walk.reshape(-1, 8 ** k, 3) >> k            # runs of 8^k consecutive points
        assert (runs == runs[:, :1, :]).all()             # one aligned 2^k cube per run


def test_hilbert_order_on_a_non_power_of_two_grid():
    grid = (3, 5, 6)
    order = hilbert_token_order(grid)
    assert np.array_equal(np.sort(order), np.arange(90))
    # the kept tokens follow the curve of the enclosing 8^3 cube
    full = np.array(list(itertools.product(range(8), repeat=3)))
    walk = full[np.argsort(hilbert_index(full, 3))]
    inside = walk[(walk[:, 0] < 3) & (walk[:, 1] < 5) & (walk[:, 2] < 6)]
    assert np.array_equal(order, (inside[:, 0] * 5 + inside[:, 1]) * 6 + inside[:, 2])


@pytest.mark.parametrize("grid,nb,last", [((4, 8, 8), 2, 128), ((5, 30, 52), 61, 120),
                                          ((21, 45, 80), 591, 80), ((21, 68, 120), 1339, 96)])
def test_hilbert_layout_blocks(grid, nb, last):
    lay = HilbertLayout(grid)
    assert cube_bits(grid) == max(1, int(np.ceil(np.log2(max(grid)))))
    assert lay.Nb == nb and lay.sizes[-1] == last and (lay.sizes[:-1] == 128).all()
    assert np.array_equal(np.sort(np.concatenate(lay.members)), np.arange(lay.N))    # a partition


def test_augmentation_ties_among_zero_masses_go_to_lower_rows():
    """Hand-worked: 16 query blocks all score key block j at -90 j, so every
    row's masses are e^(-90 j) / sum (normal to j = 7, denormal at j = 8,
    exactly 0 beyond).  p = 0.9 with a floor of 2 keeps j = 0, 1 in every row
    (K = 32); a budget of K + 4K adds A = 128 = 7 x 16 positive masses
    (j = 2..8 of every row) plus 16 of the 112 equal zero masses, which go to
    the lowest rows first, each row's in ascending j: rows 0 and 1 take 7,
    row 2 takes 2."""
    grid, tile = (4, 16, 16), (1, 8, 8)
    lay = BlockLayout(grid, tile)
    N = grid[0] * grid[1] * grid[2]
    q = np.zeros((1, 1, N, 128))
    k = np.zeros_like(q)
    q[..., 0] = 1.0
    for j in range(lay.Nb):
        k[0, 0, lay.members[j], 0] = -90.0 * j * np.sqrt(128.0)
    ref = routing.route(q, k, lay, 0.9, 2, ("frac", 4.0))
    hd = ref["heads"][0][0]
    assert np.all(hd["base"] == 2)
    assert 0 < hd["P"][0, 8] < np.finfo(np.float64).tiny and np.all(hd["P"][:, 9:] == 0)
    assert list(np.diff(ref["row_ptr"])) == [16, 16, 11] + [9] * 13
    cols = ref["col_idx"]
    assert list(cols[:16]) == list(range(16)) and list(cols[32:43]) == list(range(11))


# ------------------------------------------------------- non-finite inputs
def test_nonfinite_scores_keep_every_block_in_order():
    """Reading for non-finite inputs: a NaN or infinite token makes its
    block's pooled vector non-finite; every softmax row that then holds a
    non-finite score is NaN, no prefix reaches p, and the row keeps all
    blocks in block order (no augmentation candidates).  Rows untouched by
    the token keep their normal lists."""
    lay = BlockLayout((2, 8, 16), (1, 8, 8))             # 4 blocks of 64 tokens
    rng = np.random.default_rng(77)
    q = rng.normal(size=(lay.N, 16))
    k = rng.normal(size=(lay.N, 16))
    clean = routing.route_head(q, k, lay, 0.5, 1)
    q_bad = q.copy()
    q_bad[lay.members[2][5], 3] = np.nan                   # query block 2 only
    r = routing.route_head(q_bad, k, lay, 0.5, 1)
    assert r["base"][2] == lay.Nb and r["order"][2].tolist() == list(range(lay.Nb))
    for i in (0, 1, 3):
        assert r["base"][i] == clean["base"][i] and np.array_equal(r["order"][i], clean["order"][i])
    k_bad = k.copy()
    k_bad[lay.members[1][0], 0] = np.nan                    # key block 1: a NaN score in every row
    r = routing.route_head(q, k_bad, lay, 0.5, 1)
    assert np.all(r["base"] == lay.Nb)
    assert np.array_equal(r["order"], np.tile(np.arange(lay.Nb), (lay.Nb, 1)))
    # an infinite key coordinate makes a row's score +inf (a NaN row) or
    # -inf (a zero mass in an otherwise finite row), by the sign of q-bar
    k_inf = k.copy()
    k_inf[lay.members[1][0], 0] = np.inf
    r = routing.route_head(q, k_inf, lay, 0.5, 1)
    qbar0 = np.array([q[m, 0].mean() for m in lay.members])
    for i in range(lay.Nb):
        if qbar0[i] > 0:
            assert r["base"][i] == lay.Nb and r["order"][i].tolist() == list(range(lay.Nb))
        else:
            assert np.isfinite(r["P"][i]).all() and r["P"][i, 1] == 0.0
