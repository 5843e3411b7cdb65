"""Oracle for tree-routed recurrent state and causal-convolution context.

Test infrastructure only (see ``oracle/__init__.py``).

Source: Tree Training post, section 9 (hybrid attention + SSM models).  In
DFS-packed order the physical predecessor of a node's first token can be the
last token of a sibling branch (the post's example: DFS n0, n1, n3, n4, n2, n5
would hand n4's state to n2).  Section 9.1: a chunk starts from its parent's
end state, h_c^(0) = h_pi(c)^(end).  Section 9.2: a causal convolution of
width K reads the parent's last K - 1 tokens as its left context,
y_c = Conv([ctx_pi(c); x_c])[K - 1:].

Readings (the post names Mamba / Gated DeltaNet layers but fixes no
recurrence): the recurrence is the diagonal gated linear one,
h_t = a_t * h_prev(t) + b_t per channel, output y_t = h_t, zero state before
a root; the convolution is depthwise, y_t = sum_{j<K} w[:, j] * x_{prev^j(t)},
where prev follows the root-to-token path (the parent's tail, and the
grandparent's when the parent is shorter than K - 1), zero past the root.

Both are defined by running every root-to-leaf path as an ordinary sequence
(the textbook sequential scan and causal conv1d) and scattering the results
back to packed order -- the equivalence the post asks for.  Backward: the
upstream gradient g_t of a token on g_t paths is split evenly over them
(as in ``attention.per_path_attention``) and the path gradients are summed,
which is the gradient of sum_t <g_t, y_t> on the tree.

Parity: pinned by the closed form of a single sequence (cumulative products),
by torch's CPU conv1d on single sequences, by finite differences on a small
tree, and by the post's six-node example, where the DFS-neighbour state
differs from the routed one (tests/test_oracle_ssm.py).
"""
from __future__ import annotations

import numpy as np


def _paths(plan):
    return plan.paths


def scan_path(a, b):
    """Textbook sequential scan h_t = a_t h_{t-1} + b_t from a zero state.
    a, b [T, C] -> h [T, C]."""
    h = np.zeros_like(b)
    s = np.zeros(b.shape[1])
    for t in range(b.shape[0]):
        s = a[t] * s + b[t]
        h[t] = s
    return h


def scan_path_bwd(a, h, g):
    """Reverse of ``scan_path`` for sum_t <g_t, h_t>: (da, db)."""
    T = g.shape[0]
    da = np.zeros_like(g)
    db = np.zeros_like(g)
    u = np.zeros(g.shape[1])
    for t in range(T - 1, -1, -1):
        u = g[t] + (a[t + 1] * u if t + 1 < T else 0.0)
        db[t] = u
        da[t] = u * (h[t - 1] if t > 0 else 0.0)
    return da, db


def tree_scan(plan, a, b, g=None):
    """Tree-routed scan over DFS-packed tokens: every root-to-leaf path run as
    its own sequence.  Returns dict(h [N, C]) and, with g, da and db."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    N = a.shape[0]
    h = np.full_like(b, np.nan)
    gcount = np.asarray(plan.g, np.float64)
    res = {}
    da = np.zeros_like(a) if g is not None else None
    db = np.zeros_like(b) if g is not None else None
    for idx in _paths(plan):
        idx = np.asarray(idx, np.int64)
        if idx.size == 0:
            continue
        hp = scan_path(a[idx], b[idx])
        seen = ~np.isnan(h[idx, 0])
        assert np.allclose(h[idx][seen], hp[seen], rtol=1e-12, atol=1e-12), "paths disagree on a shared token"
        h[idx] = hp
        if g is not None:
            gp = np.asarray(g, np.float64)[idx] / gcount[idx][:, None]
            dap, dbp = scan_path_bwd(a[idx], hp, gp)
            np.add.at(da, idx, dap)
            np.add.at(db, idx, dbp)
    assert not np.isnan(h[:N]).any()
    res["h"] = h
    if g is not None:
        res["da"] = da
        res["db"] = db
    return res


def conv_path(x, w):
    """Textbook causal depthwise conv1d: y_t = sum_{j<K} w[:, j] x_{t-j}, zero
    before the start.  x [T, C], w [C, K]."""
    T, C = x.shape
    K = w.shape[1]
    y = np.zeros_like(x)
    for j in range(K):
        y[j:] += w[:, j][None, :] * x[:T - j] if j < T else 0.0
    return y


def tree_conv(plan, x, w, g=None):
    """Tree-routed causal conv: every path as its own sequence.  Returns
    dict(y) and, with g, dx and dw."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    y = np.full_like(x, np.nan)
    gcount = np.asarray(plan.g, np.float64)
    K = w.shape[1]
    dx = np.zeros_like(x) if g is not None else None
    dw = np.zeros_like(w) if g is not None else None
    for idx in _paths(plan):
        idx = np.asarray(idx, np.int64)
        if idx.size == 0:
            continue
        yp = conv_path(x[idx], w)
        seen = ~np.isnan(y[idx, 0])
        assert np.allclose(y[idx][seen], yp[seen], rtol=1e-12, atol=1e-12), "paths disagree on a shared token"
        y[idx] = yp
        if g is not None:
            gp = np.asarray(g, np.float64)[idx] / gcount[idx][:, None]
            T = idx.size
            for j in range(min(K, T)):
                np.add.at(dx, idx[:T - j], w[:, j][None, :] * gp[j:])
                dw[:, j] += (gp[j:] * x[idx][:T - j]).sum(axis=0)
    res = dict(y=y)
    if g is not None:
        res["dx"] = dx
        res["dw"] = dw
    return res


def dfs_neighbour_scan(a, b):
    """The uncorrected form the post warns about: one sequential scan over
    the packed order, so a node's first token continues from whatever token
    precedes it in DFS order.  A negative control only."""
    return scan_path(np.asarray(a, np.float64), np.asarray(b, np.float64))
