"""Backward workspace under a byte budget (host logic, no GPU): the dS path
stores 2 bytes per visible pair and query head, so tree_attn_bwd_ws_budget
picks the full dS workspace when it fits, else the dS blocks of as many KV
heads as fit (the backward then runs the KV heads in rounds), else the
recompute path's smallest workspace, and reports TA_ENOMEM below that."""
import pytest

import prefix_shared_masked_amd as pkg
import workloads as W

BF16 = 1


def _sizes(plan, Hq, Hkv, rope=10000.0):
    full = pkg.attn_ws_bytes(plan, 1, BF16, Hq, Hkv, 128, rope)
    small = pkg.attn_ws_bytes(plan, 2, BF16, Hq, Hkv, 128, rope)
    return full, small


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 2), (4, 4)])
def test_budget_selection_on_the_spine_tree(Hq, Hkv):
    t = W.spine_tree()
    plan = pkg.tree_plan(t.parent, t.seg_len)
    full, small = _sizes(plan, Hq, Hkv)
    per_head = plan.n_dsblk * (Hq // Hkv) * 32 * 32 * 2
    assert full - small >= Hkv * per_head          # the dS blocks of every KV head, plus a spare block
    assert pkg.bwd_ws_budget(plan, BF16, Hq, Hkv, 128, 10000.0, budget=full) == (full, Hkv)
    assert pkg.bwd_ws_budget(plan, BF16, Hq, Hkv, 128, 10000.0, budget=full * 10) == (full, Hkv)
    prev = full
    for heads in range(Hkv - 1, 0, -1):
        # the largest budget that no longer holds heads + 1 KV heads' dS
        b, h = pkg.bwd_ws_budget(plan, BF16, Hq, Hkv, 128, 10000.0, budget=prev - 1)
        assert h == heads and b < prev and b <= prev - 1
        assert b >= small + heads * per_head
        prev = b
    b, h = pkg.bwd_ws_budget(plan, BF16, Hq, Hkv, 128, 10000.0, budget=prev - 1)
    assert (b, h) == (small, 0)                    # below one KV head's dS: the recompute path
    with pytest.raises(pkg.TreeAttnError):
        pkg.bwd_ws_budget(plan, BF16, Hq, Hkv, 128, 10000.0, budget=small - 1)


def test_default_budget_bounds_the_varlen_forest():
    """The default (8 GiB) keeps the 133K-token varlen batch's backward
    workspace bounded: its full dS workspace is about 22 GB at 32/8 heads."""
    t = W.varlen_forest(0)
    plan = pkg.tree_plan(t.parent, t.seg_len)
    full, small = _sizes(plan, 32, 8)
    assert full > 16 * 2 ** 30
    b, h = pkg.bwd_ws_budget(plan, BF16, 32, 8, 128, 10000.0, budget=0)
    assert b <= 8 * 2 ** 30 and 1 <= h < 8
    assert pkg.bwd_ws_budget(plan, BF16, 32, 8, 128, 10000.0, budget=8 * 2 ** 30) == (b, h)


def test_fp32_has_no_ds_path():
    t = W.six_node_tree(16)
    plan = pkg.tree_plan(t.parent, t.seg_len)
    b, h = pkg.bwd_ws_budget(plan, 0, 1, 1, 64, 10000.0, budget=1 << 30)
    assert h == 0 and b == pkg.attn_ws_bytes(plan, 2, 0, 1, 1, 64, 10000.0)
