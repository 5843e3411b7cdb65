"""Pins of the output-layer + weighted-NLL oracle (agent-rl chapter 14,
section 14.3; Tree Training post, section 6.2): torch's CPU cross_entropy over
h W^T with autograd in float64, finite differences, the closed form at h = 0,
and chunked == full."""
import numpy as np
import pytest
import torch

import oracle
from oracle.lmhead import chunked_lmhead_weighted_nll, lmhead_vocab_rows, lmhead_weighted_nll
import workloads as W


def _case(N=37, V=53, D=24, seed=0, p_ignore=0.25):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, D))
    Wt = rng.standard_normal((V, D)) / np.sqrt(D)
    labels = rng.integers(0, V, N)
    labels[rng.random(N) < p_ignore] = -100
    w = rng.random(N)
    return h, Wt, labels, w


def test_matches_torch_cross_entropy_and_autograd():
    h, Wt, labels, w = _case()
    r = lmhead_weighted_nll(h, Wt, labels, w)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(Wt, requires_grad=True)
    logits = th @ tW.T
    ce = torch.nn.functional.cross_entropy(logits, torch.tensor(labels), reduction="none", ignore_index=-100)
    ref = (ce * torch.tensor(w)).sum()
    ref.backward()
    assert r["loss"] == pytest.approx(ref.item(), rel=1e-13)
    np.testing.assert_allclose(r["token_loss"], ce.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["lse"], torch.logsumexp(logits, 1).detach().numpy(), rtol=1e-13)
    np.testing.assert_allclose(r["dh"], th.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(r["dW"], tW.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_finite_differences():
    h, Wt, labels, w = _case(N=6, V=9, D=5, seed=3, p_ignore=0.2)
    r = lmhead_weighted_nll(h, Wt, labels, w)
    eps = 1e-6
    for arr, grad in ((h, r["dh"]), (Wt, r["dW"])):
        for idx in [(0, 0), (2, 3), (arr.shape[0] - 1, arr.shape[1] - 1)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args_p = (p, Wt) if arr is h else (h, p)
            args_m = (m, Wt) if arr is h else (h, m)
            fd = (lmhead_weighted_nll(*args_p, labels, w)["loss"] - lmhead_weighted_nll(*args_m, labels, w)["loss"]) / (2 * eps)
            assert fd == pytest.approx(grad[idx], rel=1e-6, abs=1e-9)


def test_zero_hidden_closed_form():
    """h = 0 makes every logit 0: each valid token costs log V, the softmax is
    uniform, dh = sum_y w (1/V sum_v W_v - W_y), dW = 0."""
    h, Wt, labels, w = _case(N=20, V=31, D=7, seed=4)
    h[:] = 0.0
    r = lmhead_weighted_nll(h, Wt, labels, w)
    valid = labels != -100
    assert r["loss"] == pytest.approx(np.log(31) * w[valid].sum(), rel=1e-14)
    np.testing.assert_allclose(r["lse"], np.log(31), rtol=1e-15)
    assert not r["dW"].any()
    exp_dh = (w * valid)[:, None] * (Wt.mean(axis=0)[None, :] - Wt[np.where(valid, labels, 0)])
    np.testing.assert_allclose(r["dh"], exp_dh, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("chunk", [1, 7, 16, 1000])
def test_chunked_equals_full(chunk):
    h, Wt, labels, w = _case(N=45, V=40, D=16, seed=5)
    a = lmhead_weighted_nll(h, Wt, labels, w)
    b = chunked_lmhead_weighted_nll(h, Wt, labels, w, chunk=chunk)
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13)
    for k in ("lse", "token_loss", "dh", "dW"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-12, atol=1e-14, err_msg=k)


def test_tree_weights_equal_per_path_average():
    """With w = g/K from a plan, the loss is the per-path average of the
    paths' summed token losses (Tree Training post, section 6.2)."""
    t = W.six_node_tree(5)
    op = oracle.oracle_plan(t.parent, t.seg_len)
    h, Wt, labels, _ = _case(N=op.n_tokens, V=17, D=8, seed=6, p_ignore=0.0)
    r = lmhead_weighted_nll(h, Wt, labels, op.g / op.n_leaves)
    assert r["loss"] == pytest.approx(oracle.per_path_loss(op, r["token_loss"]), rel=1e-13)


@pytest.mark.parametrize("chunk", [1, 13, 2048])
def test_vocab_rows_match_torch_autograd(chunk):
    """The full-size spot-check form (lse of every token, dW on selected
    vocabulary rows, the label rows among them) against torch's CPU
    cross_entropy with autograd in float64; its magnitude sum
    sum_t |dlogits_tv| |h_t| against the same product formed from the
    absolute values of torch's per-token gradient (autograd w.r.t. the
    logits)."""
    h, Wt, labels, w = _case(N=50, V=37, D=12, seed=8)
    rows = np.unique(np.concatenate([[0, 36, 5], labels[labels >= 0][:3]]))
    r = lmhead_vocab_rows(h, Wt, labels, w, rows, chunk=chunk)
    th = torch.tensor(h)
    tW = torch.tensor(Wt, requires_grad=True)
    logits = (th @ tW.T).detach().requires_grad_(True)
    tok = torch.nn.functional.cross_entropy(logits, torch.tensor(labels, dtype=torch.int64), reduction="none",
                                            ignore_index=-100)
    (tok * torch.tensor(w)).sum().backward()
    G = logits.grad.numpy()
    np.testing.assert_allclose(r["lse"], torch.logsumexp(logits.detach(), 1).numpy(), rtol=1e-14)
    np.testing.assert_allclose(r["dW"], (G.T @ h)[rows], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["dW_abs"], (np.abs(G).T @ np.abs(h))[rows], rtol=1e-12, atol=1e-15)
