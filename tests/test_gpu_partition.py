"""GPU parity of partitioned tree attention (Tree Training post, section 8):
tree_plan_ex's key-only prefix and tree_partition_fwd/bwd against the float64
oracle on the whole tree, and against tree_attn_fwd/bwd on the whole tree.

Tolerances as for the unpartitioned kernels (fp32 1e-5 absolute; bf16
2e-2 + 1e-2 |ref|).  In bf16 each partition's dK/dV is rounded to bf16 once
before the fp32 relay sum, which stays inside the same bound."""
import numpy as np
import pytest
import torch

import oracle
import prefix_shared_masked_amd as pkg
import workloads as W
from test_gpu_attention import DEV, close, to_dev

pytestmark = pytest.mark.gpu


def run_partitioned(tree, cap, Hq, Hkv, d, dtype, rope, seed=0):
    print(f"[part] {tree.name or 'tree'} N={tree.n_tokens} cap={cap} Hq={Hq} Hkv={Hkv} {dtype} rope={rope}",
          flush=True)
    part = pkg.tree_partition(tree.parent, tree.seg_len, cap)
    q, k, v, do = W.attention_inputs(seed, part.n_tokens, Hq, Hkv, d)
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = pkg.tree_partition_fwd(part, Q, K, V, rope_base=rope)
    dq, dk, dv = pkg.tree_partition_bwd(part, Q, K, V, o, lse, DO, rope_base=rope)
    torch.cuda.synchronize()
    ref = oracle.dense_mask_attention(oracle.oracle_plan(tree.parent, tree.seg_len), q64, k64, v64,
                                      rope_base=rope, dO=do64)
    for name, got in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        close(name, got, ref[name], dtype, f" cap={cap}")
    return part, (Q, K, V, DO), (o, lse, dq, dk, dv)


def _trees():
    rng = np.random.default_rng(11)
    yield W.six_node_tree(40)
    yield W.spine_tree(64, 16, 24, 6)
    yield W.Tree(np.array([-1] + list(range(19)), np.int32), np.array([23] * 20, np.int32), "chain20")
    yield W.Tree(np.array([-1, -1, 1, 1, 0], np.int32), np.array([0, 70, 33, 65, 40], np.int32), "forest")
    for c in range(2):
        yield W.random_tree(rng, int(rng.integers(8, 30)), max_len=80, p_zero=0.1, n_roots=1 + c)


def _caps(tree):
    mx, N = int(tree.seg_len.max()), tree.n_tokens
    return sorted({mx, max(mx, N // 3), max(mx, N // 2) + 1})


def test_fp32_partitioned_equals_oracle():
    for i, t in enumerate(_trees()):
        for cap in _caps(t):
            run_partitioned(t, cap, 4, 2, 64, torch.float32, 10000.0 if i % 2 == 0 else 0.0, seed=i)


@pytest.mark.parametrize("heads", [(8, 2), (4, 4)])
def test_bf16_partitioned_equals_oracle(heads):
    for i, t in enumerate(_trees()):
        for cap in _caps(t):
            run_partitioned(t, cap, heads[0], heads[1], 128, torch.bfloat16, 10000.0 if i % 2 else 0.0, seed=i)


def test_key_only_prefix_leaves_chain_rows_untouched():
    """tree_plan_ex: the chain's rows are keys only.  O/LSE/dQ rows of the chain
    keep whatever the caller put there; the other rows equal the oracle on the
    local tree with the chain's upstream gradient zero."""
    parent = np.array([-1, 0, 1, 2, 2, 3], np.int32)
    seg = np.array([37, 70, 29, 50, 66, 31], np.int32)
    for dtype, d in ((torch.float32, 64), (torch.bfloat16, 128)):
        plan = pkg.tree_plan(parent, seg, n_prefix_nodes=2)
        q0, N = plan.q_start, plan.n_tokens
        assert q0 == 107
        q, k, v, do = W.attention_inputs(4, N, 4, 2, d)
        do[:q0] = 0.0
        (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, dtype) for x in (q, k, v, do))
        o = torch.full((N, 4, d), 7.0, dtype=dtype, device=DEV)
        lse = torch.full((4, N), 7.0, dtype=torch.float32, device=DEV)
        dq = torch.full((N, 4, d), 7.0, dtype=dtype, device=DEV)
        pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0, o=o, lse=lse)
        o_in = o.clone()
        o_in[:q0] = 0  # the chain rows of O are never read by the backward
        _, dk, dv = pkg.tree_attn_bwd(plan, Q, K, V, o_in, lse, DO, rope_base=10000.0, dq=dq)
        torch.cuda.synchronize()
        assert bool((o[:q0] == 7.0).all()) and bool((lse[:, :q0] == 7.0).all()) and bool((dq[:q0] == 7.0).all())
        ref = oracle.dense_mask_attention(oracle.oracle_plan(parent, seg), q64, k64, v64, rope_base=10000.0,
                                          dO=do64)
        close("o", o[q0:], ref["o"][q0:], dtype)
        close("lse", lse[:, q0:], ref["lse"][:, q0:], dtype)
        close("dq", dq[q0:], ref["dq"][q0:], dtype)
        close("dk", dk, ref["dk"], dtype)
        close("dv", dv, ref["dv"], dtype)


@pytest.mark.timeout(600)
def test_spine_full_size_partitioned():
    """The spine workload (N = 16352, Hq 32, Hkv 8, d 128, bf16, RoPE) cut at
    4096 tokens: equal to the unpartitioned kernels within bf16 rounding and
    bitwise deterministic; KV group 0 against the float64 oracle."""
    tree = W.spine_tree()
    part = pkg.tree_partition(tree.parent, tree.seg_len, 4096)
    plan = pkg.tree_plan(tree.parent, tree.seg_len)
    print(f"[full-part] spine N={part.n_tokens} parts={part.n_parts}", flush=True)
    q, k, v, do = W.attention_inputs(0, part.n_tokens, 32, 8, 128)
    (Q, q64), (K, k64), (V, v64), (DO, do64) = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = pkg.tree_partition_fwd(part, Q, K, V, rope_base=10000.0)
    g = pkg.tree_partition_bwd(part, Q, K, V, o, lse, DO, rope_base=10000.0)
    o2, lse2 = pkg.tree_partition_fwd(part, Q, K, V, rope_base=10000.0)
    g2 = pkg.tree_partition_bwd(part, Q, K, V, o2, lse2, DO, rope_base=10000.0)
    assert torch.equal(o, o2) and torch.equal(lse, lse2) and all(torch.equal(a, b) for a, b in zip(g, g2))
    ow, lw = pkg.tree_attn_fwd(plan, Q, K, V, rope_base=10000.0)
    gw = pkg.tree_attn_bwd(plan, Q, K, V, ow, lw, DO, rope_base=10000.0)
    torch.cuda.synchronize()
    for name, a, b in (("o", o, ow), ("lse", lse, lw), ("dq", g[0], gw[0]), ("dk", g[1], gw[1]),
                       ("dv", g[2], gw[2])):
        close(name + "(vs whole)", a, b.float().cpu().double().numpy(), torch.bfloat16)
    hs = [0, 1, 2, 3]
    ref = oracle.dense_mask_attention(oracle.oracle_plan(tree.parent, tree.seg_len), q64, k64, v64,
                                      rope_base=10000.0, dO=do64, heads=hs)
    close("o", o[:, hs], ref["o"][:, hs], torch.bfloat16)
    close("lse", lse[hs], ref["lse"][hs], torch.bfloat16)
    close("dq", g[0][:, hs], ref["dq"][:, hs], torch.bfloat16)
    close("dk", g[1][:, 0], ref["dk"][:, 0], torch.bfloat16)
    close("dv", g[2][:, 0], ref["dv"][:, 0], torch.bfloat16)
