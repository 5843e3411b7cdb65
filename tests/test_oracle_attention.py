"""Pins of the oracle attention (forward and backward) against what the pages
and textbook routines fix: per-path == dense mask, special cases that reduce
to torch's CPU scaled_dot_product_attention, finite differences, the leak
invariants of the "Tree Training" post (section 14.2) and negative controls
that must fail (agent-rl chapter 14, section 14.1)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.attention import per_path_attention, dense_mask_attention, rope, rope_transpose
import workloads as W


def _inputs(n, Hq, Hkv, d, seed=0):
    q, k, v, do = W.attention_inputs(seed, n, Hq, Hkv, d)
    return q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), do.astype(np.float64)


def _trees():
    rng = np.random.default_rng(3)
    yield W.six_node_tree(4)
    for c in range(10):
        yield W.random_tree(rng, int(rng.integers(1, 9)), max_len=6, p_zero=0.2,
                            n_roots=int(rng.integers(1, 3)), shape=["random", "chain", "star"][c % 3])


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2)])
def test_per_path_equals_dense_mask(rope_base, heads):
    Hq, Hkv = heads
    for t in _trees():
        pl = oracle.oracle_plan(t.parent, t.seg_len)
        if pl.n_tokens == 0:
            continue
        q, k, v, do = _inputs(pl.n_tokens, Hq, Hkv, 8)
        a = per_path_attention(pl, q, k, v, rope_base=rope_base, dO=do)
        b = dense_mask_attention(pl, q, k, v, rope_base=rope_base, dO=do, row_block=5)
        assert a["path_spread"] < 1e-12
        for key in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(a[key], b[key], rtol=1e-10, atol=1e-12, err_msg=key)


def _sdpa64(q, k, v, mask=None, causal=False):
    """torch CPU reference, float64, inputs [L,H,d]."""
    tq, tk, tv = (torch.tensor(np.transpose(x, (1, 0, 2))) for x in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=causal)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (6, 3)])
def test_single_path_is_causal_attention(Hq, Hkv):
    """A chain tree is one sequence: the tree result is plain causal attention.
    torch's enable_gqa also pins the GQA reading (query head h reads KV head
    h // (Hq/Hkv)) and the summing of KV gradients over a head group."""
    t = W.Tree(np.array([-1, 0, 1], np.int32), np.array([5, 3, 4], np.int32))
    pl = oracle.oracle_plan(t.parent, t.seg_len)
    q, k, v, do = _inputs(12, Hq, Hkv, 16)
    for res in (dense_mask_attention(pl, q, k, v, dO=do), per_path_attention(pl, q, k, v, dO=do)):
        tq, tk, tv = (torch.tensor(np.transpose(x, (1, 0, 2)), requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
        np.testing.assert_allclose(res["o"], np.transpose(out.detach().numpy(), (1, 0, 2)), rtol=1e-12, atol=1e-13)
        out.backward(torch.tensor(np.transpose(do, (1, 0, 2))))
        for key, ref in (("dq", tq), ("dk", tk), ("dv", tv)):
            np.testing.assert_allclose(res[key], np.transpose(ref.grad.numpy(), (1, 0, 2)), rtol=1e-10, atol=1e-12)


def test_forest_is_block_diagonal_varlen():
    """Several roots = varlen packing: each sequence attends causally to itself only."""
    lens = [4, 1, 7, 3]
    t = W.Tree(np.full(4, -1, np.int32), np.array(lens, np.int32))
    pl = oracle.oracle_plan(t.parent, t.seg_len)
    q, k, v, do = _inputs(sum(lens), 2, 1, 8)
    res = per_path_attention(pl, q, k, v, dO=do)
    off = 0
    for n in lens:
        sl = slice(off, off + n)
        kk = np.repeat(k[sl], 2, axis=1)
        vv = np.repeat(v[sl], 2, axis=1)
        ref = _sdpa64(q[sl], kk, vv, causal=True).numpy()
        np.testing.assert_allclose(res["o"][sl], np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-13)
        off += n


def test_tree_mask_via_torch_sdpa():
    """Dense masked attention with the literal mask, through torch's routine."""
    pl = oracle.oracle_plan(*[getattr(W.six_node_tree(3), a) for a in ("parent", "seg_len")])
    q, k, v, _ = _inputs(pl.n_tokens, 1, 1, 8)
    m = torch.tensor(oracle.dense_mask(pl))
    ref = _sdpa64(q, k, v, mask=m).numpy()
    res = dense_mask_attention(pl, q, k, v)
    np.testing.assert_allclose(res["o"], np.transpose(ref, (1, 0, 2)), rtol=1e-12, atol=1e-13)


def test_backward_finite_differences():
    pl = oracle.oracle_plan([-1, 0, 0, 1], [2, 2, 1, 2])
    rng = np.random.default_rng(0)
    q, k, v, do = _inputs(pl.n_tokens, 2, 1, 4, seed=7)
    res = per_path_attention(pl, q, k, v, rope_base=10000.0, dO=do)

    def f(q_, k_, v_):
        return float((per_path_attention(pl, q_, k_, v_, rope_base=10000.0)["o"] * do).sum())

    eps = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        for _ in range(6):
            idx = tuple(int(rng.integers(s)) for s in arr.shape)
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = dict(q_=q, k_=k, v_=v)
            args_m = dict(q_=q, k_=k, v_=v)
            key = {"dq": "q_", "dk": "k_", "dv": "v_"}[name]
            args_p[key], args_m[key] = plus, minus
            num = (f(**args_p) - f(**args_m)) / (2 * eps)
            assert res[name][idx] == pytest.approx(num, rel=1e-6, abs=1e-8), (name, idx)


def _six():
    t = W.six_node_tree(4)
    return oracle.oracle_plan(t.parent, t.seg_len)


def test_leak_sibling_edit_changes_nothing():
    """Editing n1's subtree leaves n2 and n5 bit-for-bit unchanged."""
    pl = _six()
    q, k, v, _ = _inputs(pl.n_tokens, 1, 1, 8)
    base = dense_mask_attention(pl, q, k, v, rope_base=10000.0)["o"]
    sib = [t for t in range(pl.n_tokens) if pl.node_of[t] in (1, 3, 4)]
    other = [t for t in range(pl.n_tokens) if pl.node_of[t] in (2, 5)]
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[sib] += 3.0
    v2[sib] -= 2.0
    q2[sib] *= -1
    out = dense_mask_attention(pl, q2, k2, v2, rope_base=10000.0)["o"]
    assert np.array_equal(out[other], base[other])


def test_leak_ancestor_edit_changes_all_descendants():
    pl = _six()
    q, k, v, _ = _inputs(pl.n_tokens, 1, 1, 8)
    base = per_path_attention(pl, q, k, v)["o"]
    v2 = v.copy()
    v2[int(pl.node_start[0])] += 1.0                 # first token of the root
    out = per_path_attention(pl, q, k, v2)["o"]
    assert (np.abs(out - base).max(axis=(1, 2)) > 0).all()


def test_leak_future_child_edit_leaves_ancestors():
    pl = _six()
    q, k, v, _ = _inputs(pl.n_tokens, 1, 1, 8)
    base = per_path_attention(pl, q, k, v)["o"]
    k2 = k.copy()
    kids = [t for t in range(pl.n_tokens) if pl.node_of[t] == 3]
    k2[kids] += 5.0
    out = per_path_attention(pl, q, k2, v)["o"]
    anc = [t for t in range(pl.n_tokens) if pl.node_of[t] in (0, 1)]
    assert np.array_equal(out[anc], base[anc])


def test_negative_controls_fail():
    """A plain causal mask, or DFS indices as positions, must not match the
    per-path result (agent-rl 14.1's leaky variants)."""
    import copy
    pl = _six()
    q, k, v, _ = _inputs(pl.n_tokens, 1, 1, 8)
    good = per_path_attention(pl, q, k, v, rope_base=10000.0)["o"]
    chain = oracle.oracle_plan([-1], [pl.n_tokens])     # one sequence: causal mask, running positions
    leaky = dense_mask_attention(chain, q, k, v, rope_base=10000.0)["o"]
    assert np.abs(leaky - good).max() > 0.1
    causal_depth = copy.copy(chain)                      # causal mask, depth positions
    causal_depth.pos = pl.pos
    leaky1 = dense_mask_attention(causal_depth, q, k, v, rope_base=10000.0)["o"]
    assert np.abs(leaky1 - good).max() > 0.1
    wrong = copy.copy(pl)                                # tree mask, DFS index as position
    wrong.pos = np.arange(pl.n_tokens)
    leaky2 = dense_mask_attention(wrong, q, k, v, rope_base=10000.0)["o"]
    assert np.abs(leaky2 - good).max() > 0.1


def test_rope_matches_complex_rotation():
    """Rotate-half RoPE equals multiplying x_i + i x_{i+d/2} by e^{i pos theta_i}."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 2, 8))
    pos = np.array([0, 1, 2, 5, 100, 4999, 12345])
    got = rope(x, pos, 10000.0)
    z = x[..., :4] + 1j * x[..., 4:]
    theta = 10000.0 ** (-np.arange(0, 8, 2) / 8)
    z = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    np.testing.assert_allclose(got, np.concatenate([z.real, z.imag], -1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rope_transpose(got, pos, 10000.0), x, rtol=1e-12, atol=1e-12)


def test_rope_relative_position_property():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    dots = []
    for p0 in (0, 17, 3000):
        dots.append(float((rope(q, np.array([p0 + 9]), 10000.0) * rope(k, np.array([p0]), 10000.0)).sum()))
    assert dots[0] == pytest.approx(dots[1], rel=1e-10) and dots[0] == pytest.approx(dots[2], rel=1e-9)


def test_rows_attention_grads_matches_dense():
    """The per-row / per-key gradient oracle (for full-size spot checks)
    against the dense-mask backward on a small tree with GQA and RoPE."""
    rng = np.random.default_rng(21)
    tree = W.random_tree(rng, 12, max_len=9, p_zero=0.1, n_roots=2)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    q, k, v, do = W.attention_inputs(8, op.n_tokens, 4, 2, 16)
    ref = oracle.dense_mask_attention(op, q, k, v, rope_base=10000.0, dO=do)
    rows = [0, op.n_tokens // 2, op.n_tokens - 1]
    keys = [0, op.n_tokens // 3, op.n_tokens - 1]
    dq, dk, dv = oracle.rows_attention_grads(op, q, k, v, do, rows, keys, rope_base=10000.0)
    np.testing.assert_allclose(dq, ref["dq"][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, ref["dk"][keys], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, ref["dv"][keys], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("rope_base", [0.0, 10000.0])
@pytest.mark.parametrize("heads", [(4, 2), (8, 2), (3, 3)])
def test_rows_attention_matches_dense(rope_base, heads):
    """The per-row forward oracle used for full-size spot checks, on every row
    and head of small trees (forests, chains, stars, zero-length nodes)
    against the literal dense mask of the Tree Training post (section 4.2)
    with depth positions (section 5): a wrong path slice, query position or
    GQA head would show in O or LSE."""
    Hq, Hkv = heads
    rng = np.random.default_rng(31)
    trees = [W.six_node_tree(3)] + [
        W.random_tree(rng, int(rng.integers(2, 10)), max_len=7, p_zero=0.25, n_roots=int(rng.integers(1, 4)),
                      shape=["random", "chain", "star"][c % 3]) for c in range(6)]
    for t in trees:
        op = oracle.oracle_plan(t.parent, t.seg_len)
        if op.n_tokens == 0:
            continue
        q, k, v, _ = W.attention_inputs(5, op.n_tokens, Hq, Hkv, 16)
        ref = oracle.dense_mask_attention(op, q, k, v, rope_base=rope_base)
        rows = list(range(op.n_tokens))
        o, lse = oracle.rows_attention(op, q, k, v, rows, list(range(Hq)), rope_base=rope_base)
        np.testing.assert_allclose(o, ref["o"], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse, ref["lse"], rtol=1e-10, atol=1e-12)
        # a subset of heads in a different order keeps each head's own values
        hs = [Hq - 1, 0]
        o2, lse2 = oracle.rows_attention(op, q, k, v, rows[::2], hs, rope_base=rope_base)
        np.testing.assert_allclose(o2, ref["o"][rows[::2]][:, hs], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse2, ref["lse"][hs][:, rows[::2]], rtol=1e-10, atol=1e-12)


def test_rows_attention_grads_matches_dense_everywhere():
    """rows_attention_grads on every row and key of forests with zero-length
    nodes, GQA 8/2 and RoPE on, against the dense-mask backward."""
    rng = np.random.default_rng(41)
    for c in range(3):
        tree = W.random_tree(rng, int(rng.integers(3, 9)), max_len=6, p_zero=0.25, n_roots=1 + c % 2,
                             shape=["random", "star", "chain"][c])
        op = oracle.oracle_plan(tree.parent, tree.seg_len)
        if op.n_tokens == 0:
            continue
        q, k, v, do = W.attention_inputs(9 + c, op.n_tokens, 8, 2, 8)
        ref = oracle.dense_mask_attention(op, q, k, v, rope_base=10000.0, dO=do)
        allr = list(range(op.n_tokens))
        dq, dk, dv = oracle.rows_attention_grads(op, q, k, v, do, allr, allr, rope_base=10000.0)
        np.testing.assert_allclose(dq, ref["dq"], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, ref["dk"], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, ref["dv"], rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("rope_base,heads,block", [(0.0, (4, 2), 64), (10000.0, (8, 2), 50), (10000.0, (3, 3), 1024)])
def test_causal_sequence_grads_matches_sdpa_and_dense(rope_base, heads, block):
    """The row-blocked gradient oracle of one causal sequence (for the heavy
    first keys of long varlen items) on 300 tokens: several row blocks and a
    ragged last block.  Without RoPE it equals torch's CPU
    scaled_dot_product_attention backward (causal, enable_gqa); with RoPE it
    equals the dense-mask backward of a one-node tree (the same sequence with
    depth positions 0..L-1)."""
    Hq, Hkv = heads
    L, d = 300, 16
    q, k, v, do = _inputs(L, Hq, Hkv, d, seed=13)
    rows = [0, 1, 63, 64, 150, L - 2, L - 1]
    keys = [0, 1, 2, 49, 50, 64, 200, L - 1]
    dq, dk, dv = oracle.causal_sequence_grads(q, k, v, do, rows, keys, rope_base=rope_base, block=block)
    if rope_base == 0.0:
        tq, tk, tv = (torch.tensor(np.transpose(x, (1, 0, 2)), requires_grad=True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
        out.backward(torch.tensor(np.transpose(do, (1, 0, 2))))
        ref = {n: np.transpose(t.grad.numpy(), (1, 0, 2)) for n, t in (("dq", tq), ("dk", tk), ("dv", tv))}
    else:
        op = oracle.oracle_plan(np.array([-1], np.int32), np.array([L], np.int32))
        ref = oracle.dense_mask_attention(op, q, k, v, rope_base=rope_base, dO=do)
    np.testing.assert_allclose(dq, ref["dq"][rows], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dk, ref["dk"][keys], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(dv, ref["dv"][keys], rtol=1e-9, atol=1e-12)
