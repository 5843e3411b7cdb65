"""Oracle for the g_t/K weighted negative log-likelihood.

Test infrastructure only (see ``oracle/__init__.py``).

Source: "Tree Training" post, section 6 (per-path average loss, the swap of
sums sum_k sum_{t in p_k} l_t = sum_t g_t l_t, L_tree = sum_t (g_t/K) l_t),
section 6.3 (only supervised positions carry a loss: the ignore index marks
the rest, context tokens still pass gradient) and the loss sketch of section
12 (per-token cross entropy with ignore_index=-100, multiplied by the loss
weights and summed).

Reading: labels are per token and already aligned with the position that
predicts them (label[t] is the target predicted at t).  The sketch's
one-position shift is not applied: in DFS order the next packed token may
belong to a sibling branch, and a branching node has one next token per
child, while section 6.2 attaches exactly one l_t to each token.  The result
is a weighted SUM, not a mean over valid tokens.

Parity: pinned against torch's CPU cross_entropy and autograd in float64 and
against the per-path form (1/K) sum_k sum_{t in p_k} l_t (tests/test_oracle_nll.py).
"""
from __future__ import annotations

import numpy as np


def weighted_nll(logits, labels, w, ignore_index: int = -100):
    """loss = sum_t w_t [y_t != ignore] (logsumexp(x_t) - x_t[y_t]);
    dlogits_t = w_t [y_t != ignore] (softmax(x_t) - onehot(y_t)).
    Returns (loss, dlogits, per_token_loss) in float64."""
    x = np.asarray(logits, np.float64)
    y = np.asarray(labels, np.int64)
    w = np.asarray(w, np.float64)
    n, V = x.shape
    valid = y != ignore_index
    m = x.max(axis=1)
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    safe = np.where(valid, y, 0)
    tok = np.where(valid, lse - x[np.arange(n), safe], 0.0)
    loss = float((w * tok).sum())
    p = np.exp(x - lse[:, None])
    p[np.arange(n)[valid], y[valid]] -= 1.0
    dlogits = (w * valid)[:, None] * p
    return loss, dlogits, tok


def per_path_loss(plan, token_loss):
    """(1/K) sum over root-to-leaf paths of the sum of the path's token losses
    (the per-path average of section 6.1), from explicit path lists."""
    token_loss = np.asarray(token_loss, np.float64)
    total = sum(float(token_loss[idx].sum()) for idx in plan.paths)
    return total / plan.n_leaves
