"""Oracle for the output layer fused with the g_t/K weighted NLL.

Test infrastructure only (see ``oracle/__init__.py``).

Sources: agent-rl chapter 14, section 14.3 (the logits of N tokens over a
vocabulary of V entries are N x V numbers, 0.61 MB per token in fp32 at
V = 151,936; the fix is to cut the token axis into chunks so that only one
chunk's logits exist at a time, and to recompute each chunk's logits in the
backward instead of keeping them; the chunked-and-recomputed form returns
exactly what the full form returns), and the Tree Training post, section 6.2
(the loss is sum_t (g_t/K) l_t) and 6.3 (ignore index).

``lmhead_weighted_nll``
    The full form, by definition: logits = h W^T (a library matmul in
    float64), then ``weighted_nll`` on them; dh = dlogits W, dW = dlogits^T h.
``lmhead_vocab_rows``
    For full-size spot checks: every token's log-sum-exp over the whole
    vocabulary (chunks of tokens, torch float64 CPU products), and the rows
    dW_v = sum_t dlogits_tv h_t of selected vocabulary entries only, with
    sum_t |dlogits_tv| |h_t| beside them (the magnitude that bounds the
    rounding error of such a sum).
``chunked_lmhead_weighted_nll``
    The section 14.3 form: tokens in chunks of ``chunk``; each chunk's logits
    are formed, reduced to its weighted token losses and dropped; the
    backward forms them again from h and W for the chunk's dlogits.  Only
    one chunk's logits exist at any time.

Parity: pinned by torch's CPU cross_entropy over h W^T with autograd in
float64 (loss, dh, dW), by finite differences of the loss in h and W, by the
closed form at h = 0 (every logit 0: each valid token costs log V), and by
the agreement of the chunked and full forms (tests/test_oracle_lmhead.py).
"""
from __future__ import annotations

import numpy as np

from .nll import weighted_nll


def lmhead_weighted_nll(h, W, labels, w, ignore_index: int = -100):
    """Full form.  h [N, D], W [V, D], labels [N], w [N] ->
    dict(loss, lse [N], token_loss [N], dh [N, D], dW [V, D]) in float64."""
    h = np.asarray(h, np.float64)
    W = np.asarray(W, np.float64)
    logits = h @ W.T
    loss, dlogits, tok = weighted_nll(logits, labels, w, ignore_index)
    m = logits.max(axis=1)
    lse = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))
    return dict(loss=loss, lse=lse, token_loss=tok, dh=dlogits @ W, dW=dlogits.T @ h, dlogits=dlogits)


def chunked_lmhead_weighted_nll(h, W, labels, w, chunk: int = 1024, ignore_index: int = -100):
    """Section 14.3 form (chunks of tokens, logits recomputed for the
    backward).  Same result layout as ``lmhead_weighted_nll``."""
    h = np.asarray(h, np.float64)
    W = np.asarray(W, np.float64)
    labels = np.asarray(labels)
    w = np.asarray(w, np.float64)
    N = h.shape[0]
    loss, lse, tok = 0.0, np.zeros(N), np.zeros(N)
    # forward: one chunk's logits at a time, kept only long enough to reduce
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        x = h[s:e] @ W.T
        l_c, _, tok_c = weighted_nll(x, labels[s:e], w[s:e], ignore_index)
        m = x.max(axis=1)
        lse[s:e] = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
        tok[s:e] = tok_c
        loss += l_c
    # backward: form every chunk's logits again for its dlogits
    dh = np.zeros_like(h)
    dW = np.zeros_like(W)
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        x = h[s:e] @ W.T
        _, dx, _ = weighted_nll(x, labels[s:e], w[s:e], ignore_index)
        dh[s:e] = dx @ W
        dW += dx.T @ h[s:e]
    return dict(loss=loss, lse=lse, token_loss=tok, dh=dh, dW=dW)


def lmhead_vocab_rows(h, W, labels, w, vocab_rows, chunk: int = 2048, ignore_index: int = -100):
    """Full-form dW on selected vocabulary rows.  Each token's softmax is
    formed over the whole vocabulary (its logits h_t W^T computed whole, one
    chunk of tokens at a time); dlogits_tv = w_t [y_t != ignore]
    (softmax(x_t)_v - [y_t = v]) is kept for the selected v only.
    h [N, D], W [V, D] -> dict(lse [N], dW [R, D], dW_abs [R, D]) in float64,
    where dW_abs = sum_t |dlogits_tv| |h_t|."""
    import torch
    h = torch.from_numpy(np.asarray(h, np.float64))
    Wt = torch.from_numpy(np.asarray(W, np.float64))
    y = torch.from_numpy(np.asarray(labels, np.int64))
    wt = torch.from_numpy(np.asarray(w, np.float64))
    rows = torch.from_numpy(np.asarray(vocab_rows, np.int64))
    N, D = h.shape
    lse = torch.zeros(N, dtype=torch.float64)
    dW = torch.zeros(len(rows), D, dtype=torch.float64)
    dW_abs = torch.zeros(len(rows), D, dtype=torch.float64)
    for s in range(0, N, chunk):
        e = min(N, s + chunk)
        x = h[s:e] @ Wt.T                                                   # [c, V]
        m = x.max(dim=1).values
        l = m + torch.log(torch.exp(x - m[:, None]).sum(dim=1))
        lse[s:e] = l
        valid = (y[s:e] != ignore_index).to(torch.float64)
        dl = torch.exp(x[:, rows] - l[:, None]) - (y[s:e, None] == rows[None, :]).to(torch.float64)
        dl *= (wt[s:e] * valid)[:, None]                                    # [c, R]
        dW += dl.T @ h[s:e]
        dW_abs += dl.abs().T @ h[s:e].abs()
    return dict(lse=lse.numpy(), dW=dW.numpy(), dW_abs=dW_abs.numpy())
