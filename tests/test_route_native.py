"""The recurrent-layer routing tables (C ABI, host only) against the oracle's
root-to-leaf paths (Tree Training post, section 9): every token's j-th path
predecessor, the chunk tree (a chunk continues its parent chunk, whose last
token is the path predecessor of its first token) and the inverse table, all
bit-exact."""
import numpy as np
import pytest

import oracle
import prefix_shared_masked_amd as pkg
import workloads as W


def check(tree, K):
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    r = pkg.tree_route(plan, K)
    v = r.view()
    N = op.n_tokens
    # path predecessors from the paths: the tokens before t on any path through t
    want = np.full((N, K - 1), -1, np.int64)
    for path in op.paths:
        path = list(path)
        for i, t in enumerate(path):
            for j in range(1, K):
                want[t, j - 1] = path[i - j] if i - j >= 0 else -1
    assert np.array_equal(v["cprev"], want)
    ch = v["chunks"]
    # chunks tile the packed tokens in order, at most `chunk` tokens, within one node
    assert ch[:, 1].sum() == N and (ch[:, 1] >= 1).all() and (ch[:, 1] <= r.chunk).all()
    assert np.array_equal(ch[:, 0], np.concatenate([[0], np.cumsum(ch[:, 1])[:-1]])[:len(ch)])
    node_of = plan.view()["node_of"]
    for s, L, p, pt in ch:
        assert (node_of[s:s + L] == node_of[s]).all()
        assert pt == (want[s, 0] if K > 1 else pt)
        if p < 0:
            assert pt == -1
        else:
            assert p < len(ch) and ch[p, 0] + ch[p, 1] - 1 == pt
    # the inverse table
    inv = {}
    for t in range(N):
        for j in range(1, K):
            q = want[t, j - 1]
            if q >= 0:
                inv.setdefault(q, []).append(t * K + j)
    sp, sc = v["succ_ptr"], v["succ"]
    for s_ in range(N):
        assert list(sc[sp[s_]:sp[s_ + 1]]) == inv.get(s_, [])
    # child chunks: exactly the chunks naming c as parent, descending
    n = len(ch)
    kp, kid = v["kid_ptr"], v["kid"]
    assert len(kp) == n + 1 and kp[0] == 0
    for c in range(n):
        assert list(kid[kp[c]:kp[c + 1]]) == [q for q in range(n - 1, -1, -1) if ch[q, 2] == c]
    # the work order: every chunk once, by depth in the chunk tree, ties ascending
    depth = np.zeros(n, np.int64)
    for c in range(n):  # a parent chunk precedes its children
        if ch[c, 2] >= 0:
            assert ch[c, 2] < c
            depth[c] = depth[ch[c, 2]] + 1
    assert list(v["order"]) == sorted(range(n), key=lambda c: (depth[c], c))


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_small_trees(K):
    rng = np.random.default_rng(K)
    check(W.six_node_tree(3), K)
    check(W.Tree(np.array([-1, 0, 1, 0]), np.array([4, 1, 3, 2]), "short_parent"), K)
    for c in range(4):
        check(W.random_tree(rng, int(rng.integers(3, 25)), max_len=9, p_zero=0.2, n_roots=1 + c % 3), K)


def test_long_nodes_are_chunked():
    t = W.Tree(np.array([-1, 0, 0]), np.array([700, 300, 256]), "long")
    check(t, 4)
    plan = pkg.tree_plan(t.parent, t.seg_len)
    r = pkg.tree_route(plan, 4)
    ch = r.view()["chunks"]
    assert r.chunk == 128
    assert ch[:, 1].tolist() == [128, 128, 128, 128, 128, 60, 128, 128, 44, 128, 128]
    assert ch[:, 2].tolist() == [-1, 0, 1, 2, 3, 4, 5, 6, 7, 5, 9]


def test_spine_tree():
    check(W.spine_tree(64, 16, 24, 6), 4)


def test_errors():
    t = W.six_node_tree(3)
    plan = pkg.tree_plan(t.parent, t.seg_len)
    for K in (0, 9):
        with pytest.raises(pkg.TreeAttnError, match="status 1"):
            pkg.tree_route(plan, K)
    pre = pkg.tree_plan([-1, 0, 1], [3, 3, 3], n_prefix_nodes=1)
    with pytest.raises(pkg.TreeAttnError, match="status 5"):
        pkg.tree_route(pre, 4)
