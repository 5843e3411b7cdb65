"""Oracle for split-KV decode and the (max, numerator, denominator) merge.

Test infrastructure only (see ``oracle/__init__.py``).

Source: the Tree Attention notes on t6page.pages.dev -- the glossary
definition of the three mergeable quantities (running max m, numerator
n = o * e^(l - m), denominator d = e^(l - m), l the local log-sum-exp), the
associativity of max and log-sum-exp over a split A u B, and the six-step
decode algorithm (local attention per KV shard giving o_i and l_i, a global
max, n_i and d_i per shard, sums, z = n_g / d_g).

Readings: the merge of two triples uses a common maximum
M = max(m_a, m_b), n = n_a e^(m_a - M) + n_b e^(m_b - M), d likewise; the
identity is (-inf, 0, 0) and -inf - (-inf) is never evaluated.  The decode
output is z = n/d and the natural-log LSE is M + log d.

Parity: pinned by the textbook one-shot softmax, by merge results that do
not depend on the split points or on the order of merging, and by the
energy-function identity Attn = dF/dzeta at zeta = 0 (finite differences),
in tests/test_oracle_decode.py.
"""
from __future__ import annotations

import numpy as np

IDENTITY = (-np.inf, None, 0.0)


def decode_attention(q, k, v, span_ptr, spans, scale=None):
    """Single-query attention per (batch item, query head) over the KV rows
    named by the item's spans.  q [B,Hq,d]; k/v [L,Hkv,d].
    Returns o [B,Hq,d], lse [B,Hq] (float64)."""
    q = np.asarray(q, np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    grp = Hq // Hkv
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    for b in range(B):
        rows = np.concatenate([np.arange(s, s + n) for s, n in spans[span_ptr[b]:span_ptr[b + 1]]]
                              or [np.zeros(0, np.int64)]).astype(np.int64)
        for h in range(Hq):
            kk = np.asarray(k[rows, h // grp], np.float64)
            vv = np.asarray(v[rows, h // grp], np.float64)
            s = kk @ q[b, h] * scale
            mx = s.max()
            e = np.exp(s - mx)
            o[b, h] = e @ vv / e.sum()
            lse[b, h] = mx + np.log(e.sum())
    return o, lse


def partial_triple(qvec, krows, vrows, scale):
    """Local (m, n, d) of one KV shard: m = max score, n = sum e^(s-m) v,
    d = sum e^(s-m).  An empty shard gives the identity."""
    if len(krows) == 0:
        return (-np.inf, np.zeros(vrows.shape[-1]), 0.0)
    s = np.asarray(krows, np.float64) @ np.asarray(qvec, np.float64) * scale
    m = s.max()
    e = np.exp(s - m)
    return (m, e @ np.asarray(vrows, np.float64), e.sum())


def triple_from_lse(o_i, l_i, m):
    """The pages' form of a shard's triple: n_i = o_i e^(l_i - m), d_i = e^(l_i - m)
    for a global max m of the shards' log-sum-exps."""
    f = np.exp(l_i - m)
    return (m, np.asarray(o_i, np.float64) * f, f)


def merge_triples(a, b):
    ma, na, da = a
    mb, nb, db = b
    if ma == -np.inf:
        return b
    if mb == -np.inf:
        return a
    M = max(ma, mb)
    fa, fb = np.exp(ma - M), np.exp(mb - M)
    return (M, na * fa + nb * fb, da * fa + db * fb)


def finalize_triple(t):
    m, n, d = t
    return n / d, m + np.log(d)
