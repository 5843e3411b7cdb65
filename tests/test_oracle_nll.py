"""Pins of the weighted-NLL oracle: torch's CPU cross_entropy and autograd in
float64, the per-path form of the "Tree Training" post (section 6.1 / 6.2,
L_tree = L_sep-avg) and the ignore-index rule of section 6.3."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _case(n=40, V=33, seed=0):
    logits, labels = W.nll_inputs(seed, n, V)
    w = np.random.default_rng(seed + 1).random(n)
    return logits, labels, w


def test_matches_torch_cross_entropy_and_autograd():
    logits, labels, w = _case()
    loss, dl, tok = oracle.weighted_nll(logits, labels, w)
    x = torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    y = torch.tensor(labels, dtype=torch.int64)
    ce = torch.nn.functional.cross_entropy(x, y, reduction="none", ignore_index=-100)
    ref = (ce * torch.tensor(w)).sum()
    ref.backward()
    assert loss == pytest.approx(ref.item(), rel=1e-13)
    np.testing.assert_allclose(tok, ce.detach().numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(dl, x.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_all_ignored_is_zero():
    logits, labels, w = _case()
    labels[:] = -100
    loss, dl, _ = oracle.weighted_nll(logits, labels, w)
    assert loss == 0.0 and not dl.any()


def test_tree_loss_equals_per_path_average():
    """Check 4 with the real loss: sum_t (g_t/K) l_t == (1/K) sum_k sum_{t in p_k} l_t."""
    rng = np.random.default_rng(2)
    for t in [W.six_node_tree(16)] + [W.random_tree(rng, 9, 7, 0.2, 2) for _ in range(8)]:
        pl = oracle.oracle_plan(t.parent, t.seg_len)
        if pl.n_tokens == 0:
            continue
        logits, labels = W.nll_inputs(5, pl.n_tokens, 17)
        w = pl.g / pl.n_leaves
        loss, _, tok = oracle.weighted_nll(logits, labels, w)
        assert loss == pytest.approx(oracle.per_path_loss(pl, tok), rel=1e-12, abs=1e-14)


def test_gradient_finite_difference():
    logits, labels, w = _case(6, 5, seed=3)
    logits = logits.astype(np.float64)
    _, dl, _ = oracle.weighted_nll(logits, labels, w)
    eps = 1e-6
    for i in range(6):
        for j in range(5):
            p, m = logits.copy(), logits.copy()
            p[i, j] += eps
            m[i, j] -= eps
            num = (oracle.weighted_nll(p, labels, w)[0] - oracle.weighted_nll(m, labels, w)[0]) / (2 * eps)
            assert dl[i, j] == pytest.approx(num, rel=1e-6, abs=1e-9)


def test_masked_logits_equal_removed_columns():
    """A logit of -inf (a masked vocabulary entry or action) is the same as
    the column being absent: loss and the remaining gradient equal those of
    the row without it, and the masked gradient is exactly zero."""
    rng = np.random.default_rng(7)
    n, V = 12, 40
    x = rng.standard_normal((n, V))
    keep = rng.random((n, V)) > 0.6
    keep[:, 0] = True
    labels = np.array([int(rng.choice(np.flatnonzero(keep[i]))) for i in range(n)])
    labels[3] = -100
    w = rng.random(n)
    xm = np.where(keep, x, -np.inf)
    loss, dl, tok = oracle.weighted_nll(xm, labels, w)
    for i in range(n):
        cols = np.flatnonzero(keep[i])
        yi = -100 if labels[i] == -100 else int(np.flatnonzero(cols == labels[i])[0])
        li, dli, toki = oracle.weighted_nll(x[i:i + 1, cols], np.array([yi]), w[i:i + 1])
        assert tok[i] == pytest.approx(toki[0], rel=1e-13, abs=1e-15)
        np.testing.assert_allclose(dl[i, cols], dli[0], rtol=1e-12, atol=1e-15)
        assert np.all(dl[i, ~keep[i]] == 0.0)
