"""The partition planner (C ABI, host only): connected subtrees under the
capacity, every token in exactly one partition, each partition's chain equal to
its root's ancestors, local plans whose packed rows map onto the whole tree's
rows with the same depth positions, and the gateway computation itself in
float64: running the oracle on every partition's local tree (chain keys only)
and relaying the chain gradients reproduces the oracle on the whole tree
(Tree Training post, sections 8.1-8.3).  Error paths return status codes."""
import numpy as np
import pytest

import oracle
import prefix_shared_masked_amd as pkg
import workloads as W


def ancestors(parent, v):
    out = []
    a = int(parent[v])
    while a >= 0:
        out.append(a)
        a = int(parent[a])
    return out[::-1]


def check_partition(tree, cap):
    parent, seg = np.asarray(tree.parent), np.asarray(tree.seg_len)
    n = len(parent)
    P = pkg.tree_partition(parent, seg, cap)
    v = P.view()
    whole = pkg.tree_plan(parent, seg)
    wv = whole.view()
    N = int(seg.sum())
    assert P.n_tokens == N and P.n_nodes == n
    part_of = v["part_of"]
    # every node in one partition, own tokens within capacity, sum of own tokens == N
    assert part_of.min() >= 0 and part_of.max() < P.n_parts
    own = np.bincount(part_of, weights=seg, minlength=P.n_parts).astype(np.int64)
    assert np.array_equal(own, v["own_tokens"])
    assert own.sum() == N and (own <= cap).all()
    assert P.n_parts >= -(-N // cap)
    naive = 0
    for p in range(P.n_parts):
        root = int(v["part_root"][p])
        assert part_of[root] == p
        # connected: every own node other than the root has its parent in the partition
        mine = np.flatnonzero(part_of == p)
        for x in mine:
            if x != root:
                assert part_of[parent[x]] == p
        # the root's parent lies in the parent partition, which precedes p
        pp = int(v["part_parent"][p])
        if parent[root] < 0:
            assert pp == -1
        else:
            assert pp == part_of[parent[root]] and 0 <= pp < p
        # local tree: the root's ancestors (root first), then the own nodes in ascending id
        l0, l1 = v["local_ptr"][p], v["local_ptr"][p + 1]
        ln, lp, ll = v["local_node"][l0:l1], v["local_parent"][l0:l1], v["local_len"][l0:l1]
        chain = ancestors(parent, root)
        nc = int(v["n_prefix"][p])
        assert nc == len(chain) and list(ln[:nc]) == chain
        assert list(ln[nc:]) == sorted(mine.tolist())
        assert np.array_equal(ll, seg[ln])
        for j in range(len(ln)):
            g = int(ln[j])
            if j < nc:
                assert lp[j] == j - 1
            else:
                assert ln[lp[j]] == parent[g] if parent[g] >= 0 else lp[j] == -1
        naive += int(seg[ln].sum())
        # the row map follows the local plan's packed order onto the whole tree's rows
        t0, t1 = v["tok_ptr"][p], v["tok_ptr"][p + 1]
        idx = v["tok_idx"][t0:t1]
        assert t1 - t0 == int(seg[ln].sum())
        pl = P.plans[p]
        if own[p] == 0:
            assert pl is None
            continue
        lv = pl.view()
        assert pl.n_tokens == t1 - t0 and pl.n_prefix_nodes == nc
        assert pl.q_start == int(seg[chain].sum()) if nc else pl.q_start == 0
        for j in range(len(ln)):
            s, L = int(lv["node_start"][j]), int(ll[j])
            assert np.array_equal(idx[s:s + L], wv["node_start"][ln[j]] + np.arange(L))
        assert np.array_equal(lv["pos"], wv["pos"][idx])  # depth positions survive the cut
    assert P.naive_tokens == naive
    # every token is an own row of exactly one partition
    own_rows = np.concatenate([v["tok_idx"][v["tok_ptr"][p] + (P.plans[p].q_start if P.plans[p] else 0):
                                            v["tok_ptr"][p + 1]] for p in range(P.n_parts)])
    assert np.array_equal(np.sort(own_rows), np.arange(N))
    return P


@pytest.mark.parametrize("seed", range(6))
def test_random_trees_many_capacities(seed):
    rng = np.random.default_rng(100 + seed)
    shape = ("random", "chain", "star")[seed % 3]
    tree = W.random_tree(rng, int(rng.integers(2, 60)), max_len=30, n_roots=1 + seed % 3, shape=shape)
    mx = max(1, int(tree.seg_len.max()))
    for cap in sorted({mx, mx + 7, 2 * mx, 64, int(tree.seg_len.sum()), int(tree.seg_len.sum()) + 5}):
        if cap >= mx:
            check_partition(tree, cap)


def test_whole_tree_fits_one_partition_per_root():
    rng = np.random.default_rng(7)
    tree = W.random_tree(rng, 40, n_roots=3, p_zero=0.0)
    P = check_partition(tree, int(tree.seg_len.sum()))
    assert P.n_parts == 3 and P.naive_tokens == P.n_tokens
    assert (P.view()["n_prefix"] == 0).all()


def test_spine_tree_counts():
    """The spine workload (root 512, 44 spine nodes of 96, a 264-token leaf on
    each): with the gateway the partitions hold N tokens in total; re-running
    every partition's ancestors would compute naive_tokens rows."""
    tree = W.spine_tree()
    for cap in (2048, 4096, 8192):
        P = check_partition(tree, cap)
        assert P.n_tokens == 16352 < P.naive_tokens
        # a partition's own rows plus its gateway chain are its local rows
        assert P.max_local_tokens == max(pl.n_tokens for pl in P.plans if pl is not None)


def test_cut_rule_on_small_examples():
    # chain 0-1-2-3 of 10 tokens each, capacity 25: post-order keeps {3,2}, cuts it at 1
    P = pkg.tree_partition([-1, 0, 1, 2], [10] * 4, 25)
    assert P.view()["part_of"].tolist() == [0, 0, 1, 1]
    # star: root 5 tokens, children 10, 20, 30; the largest children are cut first
    v = pkg.tree_partition([-1, 0, 0, 0], [5, 10, 20, 30], 40).view()
    assert v["part_of"].tolist() == [0, 0, 0, 1] and v["n_prefix"].tolist() == [0, 1]
    v = pkg.tree_partition([-1, 0, 0, 0], [5, 10, 20, 30], 30).view()
    assert v["part_of"].tolist() == [0, 0, 1, 2] and v["n_prefix"].tolist() == [0, 1, 1]
    # ties go to the smaller node id
    v = pkg.tree_partition([-1, 0, 0], [0, 10, 10], 10).view()
    assert v["part_of"].tolist() == [0, 1, 0]
    # the six-node example with capacity 2 nodes: every partition connected
    t = W.six_node_tree(16)
    check_partition(t, 32)


def test_zero_token_partition_has_no_plan():
    # a forest whose first tree holds no token: its partition gets no plan
    P = pkg.tree_partition([-1, -1, 1], [0, 10, 5], 10)
    v = P.view()
    assert P.n_parts == 3 and v["own_tokens"].tolist() == [0, 10, 5]
    assert P.plans[0] is None and P.plans[1].q_start == 0 and P.plans[2].q_start == 10


def test_errors():
    E = pkg.TreeAttnError
    with pytest.raises(E, match="status 1"):
        pkg.tree_partition([-1, 0], [5, 11], 10)          # a node longer than the capacity
    with pytest.raises(E, match="status 1"):
        pkg.tree_partition([-1, 0], [5, 5], 0)
    with pytest.raises(E, match="status 1"):
        pkg.tree_partition([-1, 5], [5, 5], 10)           # parent out of range
    with pytest.raises(E, match="status 2"):
        pkg.tree_partition([1, 0], [5, 5], 10)            # no root: a cycle
    with pytest.raises(E, match="status 2"):
        pkg.tree_partition([-1, 2, 1], [5, 5, 5], 10)


def prefix_plan_errors():
    return [([-1, 0, 0], [4, 4, 4], 1),                   # chain node with two children
            ([-1, -1, 1], [4, 4, 4], 1),                   # two roots
            ([-1, 0], [4, 0], 1)]                          # nothing below the chain


def test_prefix_plan_validation():
    for parent, seg, npre in prefix_plan_errors():
        with pytest.raises(pkg.TreeAttnError, match="status 1"):
            pkg.tree_plan(parent, seg, n_prefix_nodes=npre)
    p = pkg.tree_plan([-1, 0, 1, 2], [4, 3, 5, 6], n_prefix_nodes=2)
    assert p.q_start == 7 and p.n_tokens == 18
    # query rows are only the non-chain rows: pairs of rows >= q_start
    pos = p.view()["pos"]
    assert p.visible_pairs == int(sum(pos[i] + 1 for i in range(7, 18)))


@pytest.mark.parametrize("rope", [0.0, 10000.0])
def test_gateway_in_float64_equals_whole_tree(rope):
    """Per partition: the oracle on the local tree with the chain's upstream
    gradient zero (its rows are keys only), own rows of O/LSE/dQ written back,
    every local dK/dV row summed into the whole tree's rows.  Must equal the
    oracle on the whole tree to rounding."""
    rng = np.random.default_rng(3)
    tree = W.random_tree(rng, 30, max_len=12, n_roots=2)
    N = tree.n_tokens
    Hq, Hkv, d = 2, 1, 16
    q, k, v, do = (x.astype(np.float64) for x in W.attention_inputs(5, N, Hq, Hkv, d))
    ref = oracle.dense_mask_attention(oracle.oracle_plan(tree.parent, tree.seg_len), q, k, v,
                                      rope_base=rope, dO=do)
    for cap in (12, 20, 40):
        P = pkg.tree_partition(tree.parent, tree.seg_len, cap)
        pv = P.view()
        o, lse, dq = np.full_like(ref["o"], np.nan), np.full_like(ref["lse"], np.nan), np.full_like(q, np.nan)
        dk, dv = np.zeros_like(k), np.zeros_like(v)
        for p in range(P.n_parts):
            if P.plans[p] is None:
                continue
            l0, l1 = pv["local_ptr"][p], pv["local_ptr"][p + 1]
            idx = pv["tok_idx"][pv["tok_ptr"][p]:pv["tok_ptr"][p + 1]]
            q0 = P.plans[p].q_start
            lp = oracle.oracle_plan(pv["local_parent"][l0:l1], pv["local_len"][l0:l1])
            dol = do[idx].copy()
            dol[:q0] = 0.0
            r = oracle.dense_mask_attention(lp, q[idx], k[idx], v[idx], rope_base=rope, dO=dol)
            o[idx[q0:]] = r["o"][q0:]
            lse[:, idx[q0:]] = r["lse"][:, q0:]
            dq[idx[q0:]] = r["dq"][q0:]
            np.add.at(dk, idx, r["dk"])
            np.add.at(dv, idx, r["dv"])
        for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
            np.testing.assert_allclose(got, ref[name], rtol=0, atol=1e-11, err_msg=f"{name} cap={cap}")
