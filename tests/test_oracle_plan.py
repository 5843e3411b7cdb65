"""Pins of the oracle plan against what the pages and plain counting fix.

Every test here is CPU-only and checks the oracle against something other
than itself: the printed six-node example, closed forms, exact integer
identities and a literal brute force of the mask definition.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.plan import dense_mask, fwd_tile_keys, bwd_tiles, por, speedup_upper
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "six_node.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_six_node_dfs_order_matches_printed_example():
    g = golden()
    p = oracle.oracle_plan(g["parent"], g["seg_len"])
    assert p.dfs_order.tolist() == g["dfs_order"]


def test_six_node_weights_match_fig4():
    g = golden()
    p = oracle.oracle_plan(g["parent"], g["seg_len"])
    assert p.n_leaves == g["n_paths"]
    for node, (num, den) in g["weights_printed"].items():
        t = int(p.node_start[int(node)])
        assert (p.g[t], p.n_leaves) == (num, den)
    per_node = [int(p.g[p.node_start[i]]) for i in range(6)]
    assert per_node == [3, 2, 1, 1, 1, 1]


def test_six_node_positions_match_section5():
    g = golden()
    p = oracle.oracle_plan(g["parent"], g["seg_len"])
    for node, (lo, hi) in g["position_ranges"].items():
        s = int(p.node_start[int(node)])
        assert p.pos[s:s + 16].tolist() == list(range(lo, hi + 1))


def test_six_node_counts():
    p = oracle.oracle_plan(*map(lambda a: a, (W.six_node_tree().parent, W.six_node_tree().seg_len)))
    assert p.n_tokens == 96
    assert p.n_flat == 144                      # three paths of 48 tokens
    # visible pairs: n0 sees a 16-triangle, depth-2 nodes 16+triangle, depth-3 32+triangle
    tri = 16 * 17 // 2
    assert p.visible_pairs == tri + 2 * (16 * 16 + tri) + 3 * (32 * 16 + tri) == 2864
    assert p.visible_pairs == int(dense_mask(p).sum())


@pytest.mark.parametrize("p_len,delta,T", [(512, 96, 44), (7, 3, 10), (0, 5, 21), (100, 1, 3)])
def test_spine_closed_forms_pure_chain(p_len, delta, T):
    """Section 2: N_flat = T p + Delta T (T+1)/2 and N_unique = p + T Delta
    (sample t is a prefix ending at spine step t: zero-length leaves)."""
    t = W.spine_tree(p_len, delta, 0, T)
    pl = oracle.oracle_plan(t.parent, t.seg_len)
    assert pl.n_leaves == T
    assert pl.n_flat == T * p_len + delta * T * (T + 1) // 2
    assert pl.n_tokens == p_len + T * delta
    assert pl.n_flat == int(pl.g.sum())


@pytest.mark.parametrize("p_len,delta,L,T", [(512, 96, 264, 44), (3, 2, 5, 7)])
def test_spine_closed_forms_with_leaves(p_len, delta, L, T):
    t = W.spine_tree(p_len, delta, L, T)
    pl = oracle.oracle_plan(t.parent, t.seg_len)
    assert pl.n_flat == T * (p_len + L) + delta * T * (T + 1) // 2
    assert pl.n_tokens == p_len + T * (delta + L)
    if (p_len, delta, L, T) == (512, 96, 264, 44):
        assert (pl.n_flat, pl.n_tokens) == (129184, 16352)


def test_compression_ratio_approaches_half_T_plus_one():
    """Section 2: with a short fixed prefix R_token -> (T+1)/2."""
    T = 43
    t = W.spine_tree(0, 10, 0, T)
    pl = oracle.oracle_plan(t.parent, t.seg_len)
    assert pl.n_flat / pl.n_tokens == pytest.approx((T + 1) / 2)


def test_por_22x():
    """Section 10: 22x fewer tokens corresponds to POR = 1 - 1/22 ~ 95.45%."""
    v = por(1, 22)
    assert round(100 * v, 2) == 95.45
    assert speedup_upper(v) == pytest.approx(22.0)


def _random_trees(n_cases=60, seed=1):
    rng = np.random.default_rng(seed)
    shapes = ["random", "chain", "star"]
    for c in range(n_cases):
        yield W.random_tree(rng, int(rng.integers(1, 14)), max_len=int(rng.integers(1, 9)),
                            p_zero=0.25, n_roots=int(rng.integers(1, 4)), shape=shapes[c % 3])


def test_path_sum_identity_exact_and_float():
    """Section 6.2: sum_k sum_{t in p_k} l_t = sum_t g_t l_t."""
    rng = np.random.default_rng(5)
    for t in _random_trees():
        pl = oracle.oracle_plan(t.parent, t.seg_len)
        assert sum(len(p) for p in pl.paths) == int(pl.g.sum()) == pl.n_flat
        ell = rng.standard_normal(pl.n_tokens)
        lhs = sum(float(ell[p].sum()) for p in pl.paths)
        assert lhs == pytest.approx(float((pl.g * ell).sum()), rel=1e-12, abs=1e-12)


def test_positions_are_path_offsets():
    """Section 5: the depth position of t equals t's index in every root-to-leaf
    path through it (what an independent per-path run would use)."""
    for t in _random_trees():
        pl = oracle.oracle_plan(t.parent, t.seg_len)
        for p in pl.paths:
            assert pl.pos[p].tolist() == list(range(len(p)))


def test_visible_pairs_and_mask_count():
    for t in _random_trees():
        pl = oracle.oracle_plan(t.parent, t.seg_len)
        if pl.n_tokens == 0:
            continue
        m = dense_mask(pl)
        assert int(m.sum()) == pl.visible_pairs
        assert (m.sum(1) == pl.pos + 1).all()        # D(t) = pos(t) + 1 keys, itself included


def test_dfs_interval_is_subtree():
    """Section 4.3: each node's subtree is one contiguous packed range."""
    for t in _random_trees():
        pl = oracle.oracle_plan(t.parent, t.seg_len)
        for a in range(pl.n_nodes):
            inside = [tok for tok in range(pl.n_tokens) if a in pl.anc[int(pl.node_of[tok])]]
            rng_ = list(range(int(pl.node_start[a]), int(pl.node_sub_end[a])))
            assert inside == rng_


def test_tile_keys_brute_force():
    for bm in (1, 3, 8):
        for t in _random_trees(30, seed=9):
            pl = oracle.oracle_plan(t.parent, t.seg_len)
            if pl.n_tokens == 0:
                continue
            m = dense_mask(pl)
            for ti, (keys, full) in enumerate(fwd_tile_keys(pl, bm)):
                rows = m[ti * bm:(ti + 1) * bm]
                assert keys.tolist() == np.nonzero(rows.any(0))[0].tolist()
                assert full.tolist() == rows[:, keys].all(0).tolist()


def test_bwd_tiles_brute_force():
    for bn in (1, 2, 5):
        for t in _random_trees(30, seed=11):
            pl = oracle.oracle_plan(t.parent, t.seg_len)
            if pl.n_tokens == 0:
                continue
            m = dense_mask(pl)
            tiles = bwd_tiles(pl, bn)
            covered = sorted(k for k0, kl, _ in tiles for k in range(k0, k0 + kl))
            assert covered == list(range(pl.n_tokens))
            for k0, kl, qe in tiles:
                assert len({int(pl.node_of[k]) for k in range(k0, k0 + kl)}) == 1
                cols = m[:, k0:k0 + kl]
                readers = np.nonzero(cols.any(1))[0]
                assert readers.min() >= k0 and readers.max() < qe
                assert cols[k0 + kl:qe].all()           # every later query in the range sees every key


def test_sibling_swap_keeps_logical_positions_and_weights():
    """Section 14.2: swapping sibling order leaves logical positions and g unchanged."""
    t = W.six_node_tree(3)
    a = oracle.oracle_plan(t.parent, t.seg_len)
    # relabel n1 <-> n2 so n2's branch is visited first
    perm = [0, 2, 1, 3, 4, 5]
    parent = [-1] * 6
    for old in range(6):
        parent[perm[old]] = -1 if t.parent[old] < 0 else perm[t.parent[old]]
    b = oracle.oracle_plan(parent, t.seg_len)
    assert b.dfs_order.tolist() != [perm[x] for x in a.dfs_order]
    for old in range(6):
        sa, sb = int(a.node_start[old]), int(b.node_start[perm[old]])
        assert a.pos[sa:sa + 3].tolist() == b.pos[sb:sb + 3].tolist()
        assert a.g[sa:sa + 3].tolist() == b.g[sb:sb + 3].tolist()


def test_forest_positions_restart():
    t = W.varlen_forest(0, n_seq=6, row_tokens=32768, max_len=300, median=40.0, p90=120.0)
    pl = oracle.oracle_plan(t.parent, t.seg_len)
    off = 0
    for n in t.seg_len:
        assert pl.pos[off:off + n].tolist() == list(range(n))
        off += n
    assert pl.n_leaves == 6 and pl.n_flat == pl.n_tokens


def test_invalid_trees_raise():
    with pytest.raises(ValueError):
        oracle.oracle_plan([1, 0], [1, 1])              # cycle, no root
    with pytest.raises(ValueError):
        oracle.oracle_plan([-1, 0, 3, 2], [1, 1, 1, 1])  # cycle beside a root
    with pytest.raises(ValueError):
        oracle.oracle_plan([-1, 5], [1, 1])
    with pytest.raises(ValueError):
        oracle.oracle_plan([-1, 0], [1, -1])


def test_zero_length_leaf_counts_as_path():
    pl = oracle.oracle_plan([-1, 0, 0], [4, 0, 2])
    assert pl.n_leaves == 2
    assert pl.g[:4].tolist() == [2, 2, 2, 2]
    assert pl.n_flat == 4 + 6
