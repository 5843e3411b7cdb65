"""Pins of the tree-routed scan / causal-conv oracle (Tree Training post,
section 9): closed forms and torch conv1d on single sequences, finite
differences on a small tree, the post's six-node example (the DFS neighbour's
state is not the parent's), and a parent shorter than the conv window."""
import numpy as np
import pytest
import torch

import oracle
from oracle import ssm
import workloads as W


def _rand(rng, N, C):
    a = rng.uniform(0.5, 1.0, (N, C))
    b = rng.standard_normal((N, C))
    return a, b


def test_scan_closed_form():
    rng = np.random.default_rng(0)
    a, b = _rand(rng, 13, 3)
    h = ssm.scan_path(a, b)
    for t in range(13):
        ref = sum(np.prod(a[s + 1:t + 1], axis=0) * b[s] for s in range(t + 1))
        np.testing.assert_allclose(h[t], ref, rtol=1e-13)


def test_conv_matches_torch_conv1d():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((17, 5))
    w = rng.standard_normal((5, 4))
    y = ssm.conv_path(x, w)
    # torch conv1d is a cross-correlation: flip the taps so tap j multiplies x_{t-j}
    xt = torch.tensor(x.T[None])                       # [1, C, T]
    wt = torch.tensor(np.flip(w, axis=1).copy()[:, None, :])  # [C, 1, K]
    ref = torch.nn.functional.conv1d(torch.nn.functional.pad(xt, (3, 0)), wt, groups=5)[0].numpy().T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_chain_and_forest_reduce_to_sequences():
    rng = np.random.default_rng(2)
    chain = oracle.oracle_plan(np.array([-1, 0, 1]), np.array([4, 3, 5]))
    a, b = _rand(rng, 12, 2)
    np.testing.assert_allclose(ssm.tree_scan(chain, a, b)["h"], ssm.scan_path(a, b), rtol=1e-14)
    forest = oracle.oracle_plan(np.array([-1, -1]), np.array([5, 7]))
    h = ssm.tree_scan(forest, a, b)["h"]
    np.testing.assert_allclose(h[5:], ssm.scan_path(a[5:], b[5:]), rtol=1e-14)   # second root starts from 0


def test_six_node_example_routes_the_parent_state():
    """DFS n0, n1, n3, n4, n2, n5: n2's first token continues n0's end state,
    not n4's (the packed predecessor)."""
    t = W.six_node_tree(3)
    op = oracle.oracle_plan(t.parent, t.seg_len)
    assert list(op.dfs_order) == [0, 1, 3, 4, 2, 5]
    rng = np.random.default_rng(3)
    a, b = _rand(rng, op.n_tokens, 2)
    h = ssm.tree_scan(op, a, b)["h"]
    s0, s2, s4 = (int(op.node_start[n]) for n in (0, 2, 4))
    np.testing.assert_allclose(h[s2], a[s2] * h[s0 + 2] + b[s2], rtol=1e-14)
    naive = ssm.dfs_neighbour_scan(a, b)
    np.testing.assert_allclose(naive[s2], a[s2] * naive[s4 + 2] + b[s2], rtol=1e-14)
    assert not np.allclose(naive[s2], h[s2])
    path = np.r_[s0:s0 + 3, s2:s2 + 3]
    np.testing.assert_allclose(h[s2:s2 + 3], ssm.scan_path(a[path], b[path])[3:], rtol=1e-13)


def test_conv_context_crosses_a_short_parent():
    """A parent of one token is shorter than K - 1 = 3: the window of the
    child's first token reaches into the grandparent."""
    op = oracle.oracle_plan(np.array([-1, 0, 1, 0]), np.array([4, 1, 3, 2]))
    rng = np.random.default_rng(4)
    x = rng.standard_normal((op.n_tokens, 3))
    w = rng.standard_normal((3, 4))
    y = ssm.tree_conv(op, x, w)["y"]
    n0, n1, n2, n3 = (int(op.node_start[n]) for n in range(4))
    # first token of n2: taps j = 0..3 read n2[0], n1[0], n0[3], n0[2]
    ref = w[:, 0] * x[n2] + w[:, 1] * x[n1] + w[:, 2] * x[n0 + 3] + w[:, 3] * x[n0 + 2]
    np.testing.assert_allclose(y[n2], ref, rtol=1e-13)
    # first token of n3 (a sibling of n1): the context is n0's tail, not n2's
    ref3 = w[:, 0] * x[n3] + w[:, 1] * x[n0 + 3] + w[:, 2] * x[n0 + 2] + w[:, 3] * x[n0 + 1]
    np.testing.assert_allclose(y[n3], ref3, rtol=1e-13)


def test_finite_differences_on_a_tree():
    rng = np.random.default_rng(5)
    tree = W.random_tree(rng, 7, max_len=4, p_zero=0.0, n_roots=2)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    N, C = op.n_tokens, 2
    a, b = _rand(rng, N, C)
    x = rng.standard_normal((N, C))
    w = rng.standard_normal((C, 3))
    g = rng.standard_normal((N, C))
    r = ssm.tree_scan(op, a, b, g)
    rc = ssm.tree_conv(op, x, w, g)
    eps = 1e-6

    def L_scan(a_, b_):
        return float((ssm.tree_scan(op, a_, b_)["h"] * g).sum())

    def L_conv(x_, w_):
        return float((ssm.tree_conv(op, x_, w_)["y"] * g).sum())

    for idx in [(0, 0), (N // 2, 1), (N - 1, 0)]:
        for arr, grad, f, other in ((a, r["da"], lambda z: L_scan(z, b), None), (b, r["db"], lambda z: L_scan(a, z), None),
                                    (x, rc["dx"], lambda z: L_conv(z, w), None)):
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            assert (f(p) - f(m)) / (2 * eps) == pytest.approx(grad[idx], rel=1e-6, abs=1e-8)
    for idx in [(0, 0), (1, 2)]:
        p, m = w.copy(), w.copy()
        p[idx] += eps
        m[idx] -= eps
        assert (L_conv(x, p) - L_conv(x, m)) / (2 * eps) == pytest.approx(rc["dw"][idx], rel=1e-6, abs=1e-8)
