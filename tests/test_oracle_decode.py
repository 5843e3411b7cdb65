"""Pins of the decode oracle and the (m, n, d) merge of the Tree Attention
notes: one-shot softmax via torch's CPU routine, independence from split
points and merge order (associativity), the pages' (o_i, l_i) form of the
triple, and the energy-function derivative Attn = dF/dzeta at 0."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W


def test_decode_matches_torch_sdpa():
    B, Hq, Hkv, d = 3, 4, 2, 16
    lens = [5, 17, 1]
    span_ptr, spans, L = W.decode_spans(lens, gap=2)
    q = W.normal(0, (B, Hq, d)).astype(np.float64)
    k = W.normal(1, (L, Hkv, d)).astype(np.float64)
    v = W.normal(2, (L, Hkv, d)).astype(np.float64)
    o, lse = oracle.decode_attention(q, k, v, span_ptr, spans)
    for b in range(B):
        s, n = spans[b]
        for h in range(Hq):
            kk = torch.tensor(k[s:s + n, h // 2])[None]
            vv = torch.tensor(v[s:s + n, h // 2])[None]
            qq = torch.tensor(q[b, h])[None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)[0, 0].numpy()
            np.testing.assert_allclose(o[b, h], ref, rtol=1e-12, atol=1e-13)
            sc = (kk[0].numpy() @ q[b, h]) / np.sqrt(d)
            assert lse[b, h] == pytest.approx(np.log(np.exp(sc).sum()), rel=1e-12)


def _random_merge(parts, rng):
    parts = list(parts)
    while len(parts) > 1:
        i = int(rng.integers(len(parts) - 1))
        parts[i:i + 2] = [oracle.merge_triples(parts[i], parts[i + 1])]
    return parts[0]


def test_merge_is_order_and_split_independent():
    rng = np.random.default_rng(0)
    d = 8
    qv = rng.standard_normal(d) * 3
    kr = rng.standard_normal((200, d))
    vr = rng.standard_normal((200, d))
    direct_o, direct_l = oracle.finalize_triple(oracle.partial_triple(qv, kr, vr, 0.5))
    s = kr @ qv * 0.5
    e = np.exp(s - s.max())
    np.testing.assert_allclose(direct_o, e @ vr / e.sum(), rtol=1e-13)
    for _ in range(30):
        cuts = np.sort(rng.choice(np.arange(0, 201), size=int(rng.integers(1, 12)), replace=True))
        bounds = [0] + cuts.tolist() + [200]
        parts = [oracle.partial_triple(qv, kr[a:b], vr[a:b], 0.5) for a, b in zip(bounds[:-1], bounds[1:])]
        o, lse = oracle.finalize_triple(_random_merge(parts, rng))
        np.testing.assert_allclose(o, direct_o, rtol=1e-12, atol=1e-13)
        assert lse == pytest.approx(direct_l, rel=1e-13)


def test_pages_form_with_global_max():
    """Steps 2-6 of the decode table: local (o_i, l_i), global m = max l_i,
    n_i = o_i e^(l_i - m), d_i = e^(l_i - m), z = sum n / sum d."""
    rng = np.random.default_rng(1)
    d = 8
    qv = rng.standard_normal(d)
    kr = rng.standard_normal((64, d))
    vr = rng.standard_normal((64, d))
    shards = np.array_split(np.arange(64), 5)
    loc = [oracle.finalize_triple(oracle.partial_triple(qv, kr[i], vr[i], 1.0)) for i in shards]
    m = max(l for _, l in loc)
    tri = [oracle.triple_from_lse(o, l, m) for o, l in loc]
    z = sum(t[1] for t in tri) / sum(t[2] for t in tri)
    ref, _ = oracle.finalize_triple(oracle.partial_triple(qv, kr, vr, 1.0))
    np.testing.assert_allclose(z, ref, rtol=1e-12)


def test_energy_function_derivative():
    """F(zeta) = log sum_a exp(q.k_a + zeta.v_a); Attn = dF/dzeta at zeta = 0."""
    rng = np.random.default_rng(2)
    d = 6
    qv, kr, vr = rng.standard_normal(d), rng.standard_normal((30, d)), rng.standard_normal((30, d))
    F = lambda z: np.log(np.exp(kr @ qv + vr @ z).sum())
    eps = 1e-6
    grad = np.array([(F(eps * np.eye(d)[i]) - F(-eps * np.eye(d)[i])) / (2 * eps) for i in range(d)])
    attn, _ = oracle.finalize_triple(oracle.partial_triple(qv, kr, vr, 1.0))
    np.testing.assert_allclose(attn, grad, rtol=1e-7, atol=1e-9)


def test_identity_element():
    t = oracle.partial_triple(np.ones(4), np.ones((3, 4)), np.ones((3, 4)), 1.0)
    empty = oracle.partial_triple(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert oracle.merge_triples(empty, t) is t and oracle.merge_triples(t, empty) is t
    assert oracle.merge_triples(empty, empty)[0] == -np.inf
