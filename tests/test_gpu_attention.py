"""GPU parity of tree_attn_fwd / tree_attn_bwd against the float64 oracle.

Tolerances: fp32 path 1e-5 absolute; bf16 path |gpu - oracle| <= 2e-2 +
1e-2 |oracle| elementwise.  bf16 inputs are rounded once on the host and the
oracle sees exactly the rounded values, so input quantisation is not error.
"""
import numpy as np
import pytest
import torch

import oracle
import prefix_shared_masked_amd as pkg
import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
ATOL_BF16, RTOL_BF16, ATOL_F32 = 2e-2, 1e-2, 1e-5


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)
    return t, t.float().cpu().double().numpy()


def close(name, got, ref, dtype, where=""):
    got = got.float().cpu().double().numpy() if torch.is_tensor(got) else got
    err = np.abs(got - ref)
    if dtype == torch.float32:
        bad = err > ATOL_F32
    else:
        bad = err > ATOL_BF16 + RTOL_BF16 * np.abs(ref)
    assert not bad.any(), (f"{name}{where}: {int(bad.sum())} of {bad.size} outside tolerance, "
                           f"max err {float(err.max()):.3e}")


def run_case(tree, Hq, Hkv, d, dtype, rope, seed=0, grads=True, heads=None, recompute_dq=False):
    print(f"[case] {tree.name or 'tree'} N={tree.n_tokens} Hq={Hq} Hkv={Hkv} d={d} {dtype} rope={rope}",
          flush=True)
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    q, k, v, do = W.attention_inputs(seed, plan.n_tokens, Hq, Hkv, d)
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=rope)
    res = dict(o=o, lse=lse)
    if grads:
        dq, dk, dv = pkg.tree_attn_bwd(plan, Q, K, V, o, lse, DO, rope_base=rope, recompute_dq=recompute_dq)
        res.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.per_path_attention(op, q64, k64, v64, rope_base=rope, dO=do64 if grads else None)
    for name in res:
        close(name, res[name], ref[name], dtype)
    return plan, res, ref


def test_six_node_fp32_with_and_without_rope():
    for rope in (0.0, 10000.0):
        run_case(W.six_node_tree(16), 1, 1, 64, torch.float32, rope)


def test_fp32_random_trees_gqa():
    rng = np.random.default_rng(1)
    for c in range(4):
        t = W.random_tree(rng, int(rng.integers(3, 12)), max_len=50, p_zero=0.1, n_roots=1 + c % 2)
        run_case(t, 4, 2, 128, torch.float32, 10000.0, seed=c)


def _small_trees():
    rng = np.random.default_rng(7)
    yield W.six_node_tree(16)
    yield W.Tree(np.array([-1, 0, 0, 1], np.int32), np.array([129, 1, 15, 17], np.int32), "edges")
    yield W.Tree(np.array([-1] + [0] * 64, np.int32), np.array([40] + [7] * 64, np.int32), "star64")
    yield W.Tree(np.array([-1] * 5, np.int32), np.array([1, 64, 65, 127, 33], np.int32), "forest")
    yield W.Tree(np.array([-1] + list(range(39)), np.int32), np.array([5] * 40, np.int32), "chain40")
    yield W.spine_tree(64, 16, 24, 6)
    for c in range(3):
        yield W.random_tree(rng, int(rng.integers(5, 30)), max_len=90, p_zero=0.15, n_roots=1 + c % 3)


@pytest.mark.parametrize("heads", [(8, 2), (4, 4), (16, 2), (4, 2)])
def test_bf16_small_trees(heads):
    Hq, Hkv = heads
    for i, t in enumerate(_small_trees()):
        run_case(t, Hq, Hkv, 128, torch.bfloat16, 10000.0 if i % 2 == 0 else 0.0, seed=i)


def test_bf16_cut_key_tiles():
    """dK/dV work cut into 32-key sub-tiles over 1,024-row windows (cap 32
    blocks) and packed four to a workgroup, with partial dK/dV summed by a
    second pass: a ragged 100-key root and node 1's tiles over 2,000 rows
    cross a window, node 2's full tiles stay whole; all KV heads, with and
    without RoPE, bitwise repeatable; then the root as a key-only prefix
    (windows from q_start)."""
    tree = W.Tree(np.array([-1, 0, 1, 1], np.int32), np.array([100, 300, 900, 700], np.int32), "cut")
    for i, (Hq, Hkv) in enumerate(((8, 2), (4, 4))):
        plan, res, _ = run_case(tree, Hq, Hkv, 128, torch.bfloat16, 10000.0 if i == 0 else 0.0, seed=11 + i)
        assert plan.n_ksplit >= 4 and plan.n_kslots >= 8
    q, k, v, do = W.attention_inputs(12, tree.n_tokens, 8, 2, 128)
    Q, K, V, DO = (torch.from_numpy(x).to(DEV).bfloat16() for x in (q, k, v, do))
    o, l = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0)
    g1 = pkg.tree_attn_bwd(plan, Q, K, V, o, l, DO, rope_base=10000.0)
    g2 = pkg.tree_attn_bwd(plan, Q, K, V, o, l, DO, rope_base=10000.0)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(g1, g2))

    pe = pkg.tree_plan(tree.parent, tree.seg_len, n_prefix_nodes=1)
    q0, N = pe.q_start, pe.n_tokens
    assert q0 == 100 and pe.n_ksplit >= 1
    print(f"[case] cut prefix N={N} q0={q0}", flush=True)
    q, k, v, do = W.attention_inputs(13, N, 4, 2, 128)
    do[:q0] = 0.0
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = pkg.tree_attn_fwd(pe, Q, K, V, rope_base=10000.0)
    o[:q0] = 0
    dq, dk, dv = pkg.tree_attn_bwd(pe, Q, K, V, o, lse, DO, rope_base=10000.0)
    torch.cuda.synchronize()
    ref = oracle.dense_mask_attention(oracle.oracle_plan(tree.parent, tree.seg_len), q64, k64, v64,
                                      rope_base=10000.0, dO=do64)
    close("o", o[q0:], ref["o"][q0:], torch.bfloat16)
    close("dq", dq[q0:], ref["dq"][q0:], torch.bfloat16)
    close("dk", dk, ref["dk"], torch.bfloat16)
    close("dv", dv, ref["dv"], torch.bfloat16)


@pytest.mark.parametrize("seed", range(10))
def test_bf16_random_sweep(seed):
    """Random trees of every shape the workloads produce (chains, stars,
    forests, one-token and zero-token nodes, nodes past one 128-key tile),
    bf16 with and without RoPE, 8/2 and 32/8 heads, both backward paths,
    against the float64 per-path oracle."""
    rng = np.random.default_rng(300 + seed)
    shape = ["random", "chain", "star"][seed % 3]
    t = W.random_tree(rng, int(rng.integers(2, 40)), max_len=int(rng.integers(1, 300)), p_zero=0.1,
                      n_roots=1 + seed % 3, shape=shape)
    if t.n_tokens == 0:
        return
    Hq, Hkv = (32, 8) if seed % 2 and t.n_tokens <= 2500 else (8, 2)   # oracle time stays in seconds
    run_case(t, Hq, Hkv, 128, torch.bfloat16, 10000.0 if seed % 4 < 2 else 0.0, seed=seed,
             recompute_dq=seed % 5 == 4)


def test_bf16_recompute_dq_path():
    """The smallest backward workspace: dQ recomputes S and dP (no stored dS)
    before dK/dV; same oracle bar, on trees with short and cut key tiles."""
    trees = [W.Tree(np.array([-1, 0, 1, 1], np.int32), np.array([100, 300, 900, 700], np.int32), "cut"),
             W.spine_tree(64, 16, 24, 6), W.six_node_tree(48)]
    for i, t in enumerate(trees):
        run_case(t, 8, 2, 128, torch.bfloat16, 10000.0 if i != 1 else 0.0, seed=20 + i, recompute_dq=True)


def test_bf16_deterministic_and_sibling_leak():
    """Same inputs -> bitwise-identical gradients; editing one branch leaves
    the other branch's outputs bit-for-bit unchanged (leak test of the Tree
    Training post, section 14.2)."""
    t = W.six_node_tree(48)
    plan = pkg.tree_plan(t.parent, t.seg_len)
    view = plan.view()
    q, k, v, do = W.attention_inputs(3, plan.n_tokens, 8, 2, 128)
    Q, K, V, DO = (torch.from_numpy(x).to(DEV).bfloat16() for x in (q, k, v, do))
    o1, l1 = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0)
    g1 = pkg.tree_attn_bwd(plan, Q, K, V, o1, l1, DO, rope_base=10000.0)
    o2, l2 = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0)
    g2 = pkg.tree_attn_bwd(plan, Q, K, V, o2, l2, DO, rope_base=10000.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    node_of = view["node_of"]
    branch = torch.from_numpy(np.isin(node_of, [1, 3, 4])).to(DEV)
    other = torch.from_numpy(np.isin(node_of, [0, 2, 5])).to(DEV)
    K2, V2, Q2 = K.clone(), V.clone(), Q.clone()
    K2[branch] += 1.0
    V2[branch] -= 0.5
    Q2[branch] *= -1
    o3, l3 = pkg.tree_attn_fwd(plan, Q2, K2, V2, rope_base=10000.0)
    assert torch.equal(o3[other], o1[other]) and torch.equal(l3[:, other], l1[:, other])
    assert not torch.equal(o3[branch], o1[branch])


def _group_check(tree, seed, heads=(0, 1, 2, 3), rows_sample=64):
    """Full-size parity for one KV group (query heads 0-3 share KV head 0):
    O/LSE/dQ of those heads and dK/dV of KV head 0 against the dense-mask
    oracle restricted to those heads; O/LSE of other heads on sampled rows."""
    Hq, Hkv, d = 32, 8, 128
    print(f"[full] {tree.name} N={tree.n_tokens}", flush=True)
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    q, k, v, do = W.attention_inputs(seed, plan.n_tokens, Hq, Hkv, d)
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0)
    dq, dk, dv = pkg.tree_attn_bwd(plan, Q, K, V, o, lse, DO, rope_base=10000.0)
    torch.cuda.synchronize()
    hs = list(heads)
    ref = oracle.dense_mask_attention(op, q64, k64, v64, rope_base=10000.0, dO=do64, heads=hs)
    close("o", o[:, hs], ref["o"][:, hs], torch.bfloat16)
    close("lse", lse[hs], ref["lse"][hs], torch.bfloat16)
    close("dq", dq[:, hs], ref["dq"][:, hs], torch.bfloat16)
    close("dk", dk[:, 0], ref["dk"][:, 0], torch.bfloat16)
    close("dv", dv[:, 0], ref["dv"][:, 0], torch.bfloat16)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.integers(0, plan.n_tokens, rows_sample), [0, plan.n_tokens - 1]]))
    other = [5, 17, 31]
    ro, rl = oracle.rows_attention(op, q64, k64, v64, rows, other, rope_base=10000.0)
    close("o(sampled)", o[rows][:, other], ro, torch.bfloat16)
    close("lse(sampled)", lse[other][:, rows], rl, torch.bfloat16)


@pytest.mark.timeout(600)
def test_spine_full_size():
    _group_check(W.spine_tree(), 0)


@pytest.mark.timeout(600)
def test_random_agentic_full_size():
    _group_check(W.random_agentic_tree(0), 1)


@pytest.mark.timeout(600)
def test_varlen_forest_full_size_sampled():
    """The varlen workload at full size (64 sequences, 133K tokens, up to 16K
    each, bf16, RoPE): O and LSE of sampled (row, head) pairs, dQ of sampled
    rows (all heads) and dK/dV of keys near sequence ends (all KV heads),
    each from the per-row / per-key oracle; then, for the three longest
    sequences, dK/dV of their first four keys (each read by every row of the
    sequence) on all KV heads and dQ of their last rows (each reading the
    whole sequence) on all heads, from the row-blocked oracle of one causal
    sequence."""
    tree = W.varlen_forest(0)
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    N, Hq, Hkv, d = plan.n_tokens, 32, 8, 128
    print(f"[full] varlen N={N}", flush=True)
    q, k, v, do = W.attention_inputs(5, N, Hq, Hkv, d)
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0)
    dq, dk, dv = pkg.tree_attn_bwd(plan, Q, K, V, o, lse, DO, rope_base=10000.0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    starts = plan.view()["node_start"]
    lens = np.asarray(tree.seg_len)
    longest = np.argsort(-lens)[:3]
    rows = np.unique(np.concatenate([rng.integers(0, N, 6), starts[longest] + lens[longest] - 1]))
    heads = [0, 9, 31]
    ro, rl = oracle.rows_attention(op, q64, k64, v64, rows, heads, rope_base=10000.0)
    close("o(sampled)", o[rows][:, heads], ro, torch.bfloat16)
    close("lse(sampled)", lse[heads][:, rows], rl, torch.bfloat16)
    keys = np.unique(np.concatenate([starts[longest] + lens[longest] - 1, starts[longest] + lens[longest] - 4,
                                     starts[:2] + lens[:2] - 2]))
    gq, gk, gv = oracle.rows_attention_grads(op, q64, k64, v64, do64, rows[:4], keys, rope_base=10000.0)
    close("dq(sampled)", dq[rows[:4]], gq, torch.bfloat16)
    close("dk(sampled)", dk[keys], gk, torch.bfloat16)
    close("dv(sampled)", dv[keys], gv, torch.bfloat16)
    assert (np.asarray(tree.parent) == -1).all()          # every item is one causal sequence
    for b in longest:
        a, L = int(starts[b]), int(lens[b])
        print(f"[full] varlen heavy keys of item {b} (L={L})", flush=True)
        sl = slice(a, a + L)
        hq, hk, hv = oracle.causal_sequence_grads(q64[sl], k64[sl], v64[sl], do64[sl], [L - 2, L - 1],
                                                  [0, 1, 2, 3], rope_base=10000.0)
        close("dq(last rows)", dq[a + L - 2:a + L], hq, torch.bfloat16, f" item {b}")
        close("dk(first keys)", dk[a:a + 4], hk, torch.bfloat16, f" item {b}")
        close("dv(first keys)", dv[a:a + 4], hv, torch.bfloat16, f" item {b}")


def test_bf16_saturation_flag_and_nan_passthrough():
    """fp16 score operands: a Q or K value beyond the fp16 range is clamped
    and raises the workspace's saturation flag (forward and backward, both
    backward paths); ordinary inputs leave it clear; a NaN in one query
    element passes through to exactly that (row, head) of O and LSE and
    raises no flag, the other rows keep matching the oracle."""
    tree = W.six_node_tree(16)
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    Hq, Hkv, d = 4, 2, 128
    q, k, v, do = W.attention_inputs(3, plan.n_tokens, Hq, Hkv, d)
    (Q, q64), (K, k64), (V, v64), (DO, _) = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))

    def flags(Qx, Kx, rope):
        wf = torch.empty(pkg.attn_ws_bytes(plan, 0, 1, Hq, Hkv, d, rope), dtype=torch.uint8, device=DEV)
        pkg.clear_saturation_flag(wf)
        o, lse = pkg.tree_attn_fwd(plan, Qx, Kx, V, rope_base=rope, ws=wf)
        out = [pkg.saturation_flag(wf)]
        for op_ in (1, 2):
            wb = torch.empty(pkg.attn_ws_bytes(plan, op_, 1, Hq, Hkv, d, rope), dtype=torch.uint8, device=DEV)
            pkg.clear_saturation_flag(wb)
            pkg.tree_attn_bwd(plan, Qx, Kx, V, o, lse, DO, rope_base=rope, ws=wb, recompute_dq=op_ == 2)
            out.append(pkg.saturation_flag(wb))
        return out, o, lse

    for rope in (0.0, 10000.0):
        assert flags(Q, K, rope)[0] == [0, 0, 0]
        Qb = Q.clone()
        Qb[37, 1, 5] = 1e5
        assert flags(Qb, K, rope)[0] == [1, 1, 1]
        Kb = K.clone()
        Kb[20, 0, 100] = -1e6  # K enters fp16 times scale * log2(e) = 0.1275: beyond 65504 / 0.1275
        assert flags(Q, Kb, rope)[0] == [1, 1, 1]
    Qn = Q.clone()
    Qn[50, 2, 7] = float("nan")
    fl, o, lse = flags(Qn, K, 0.0)
    assert fl == [0, 0, 0]
    torch.cuda.synchronize()
    on, ln = o.float().cpu().numpy(), lse.cpu().numpy()
    assert np.isnan(on[50, 2]).all() and np.isnan(ln[2, 50])
    mask = np.ones(on.shape[:2], bool)
    mask[50, 2] = False
    ref = oracle.per_path_attention(op, q64, k64, v64)
    assert np.isfinite(on[mask]).all()
    close("o", on[mask], ref["o"][mask], torch.bfloat16)
    lmask = np.ones(ln.shape, bool)
    lmask[2, 50] = False
    close("lse", ln[lmask], ref["lse"][lmask], torch.bfloat16)


def test_bf16_backward_in_kv_head_rounds():
    """A backward workspace below the full dS size runs the KV heads in
    rounds of as many as fit: bitwise the same dQ/dK/dV as one round (a query
    head's dQ depends only on its own KV head's keys), and within the bar
    against the oracle; below one KV head's dS it takes the recompute path."""
    tree = W.Tree(np.array([-1, 0, 1, 1, 0], np.int32), np.array([100, 300, 500, 200, 260], np.int32), "rounds")
    Hq, Hkv, d, rope = 8, 4, 128, 10000.0
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    op = oracle.oracle_plan(tree.parent, tree.seg_len)
    q, k, v, do = W.attention_inputs(21, plan.n_tokens, Hq, Hkv, d)
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=rope)
    full = pkg.attn_ws_bytes(plan, 1, 1, Hq, Hkv, d, rope)
    one = pkg.tree_attn_bwd(plan, Q, K, V, o, lse, DO, rope_base=rope,
                            ws=torch.empty(full, dtype=torch.uint8, device=DEV))
    ref = oracle.per_path_attention(op, q64, k64, v64, rope_base=rope, dO=do64)
    for heads in (3, 2, 1):
        nbytes = None
        for budget in range(full, 0, -4096):
            nb, hh = pkg.bwd_ws_budget(plan, 1, Hq, Hkv, d, rope, budget=budget)
            if hh == heads:
                nbytes = nb
                break
        assert nbytes is not None
        print(f"[case] rounds of {heads} KV heads, ws {nbytes} of {full}", flush=True)
        got = pkg.tree_attn_bwd(plan, Q, K, V, o, lse, DO, rope_base=rope,
                                ws=torch.empty(nbytes, dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(one, got)), heads
    for name, t in zip(("dq", "dk", "dv"), one):
        close(name, t, ref[name], torch.bfloat16)
    got = pkg.tree_attn_bwd(plan, Q, K, V, o, lse, DO, rope_base=rope, ws_budget=pkg.bwd_ws_budget(
        plan, 1, Hq, Hkv, d, rope, budget=pkg.attn_ws_bytes(plan, 2, 1, Hq, Hkv, d, rope) + 1)[0])
    for name, t in zip(("dq", "dk", "dv"), got):
        close(name, t, ref[name], torch.bfloat16)
