"""The C++ planner (through the C ABI, host only) against the oracle plan:
DFS order, positions, g_t, K, DFS intervals, ancestor chains, visible-key
sets and full flags of the forward tiles, and the backward key tiles must be
bit-exact.  Error paths return status codes."""
import ctypes

import numpy as np
import pytest

import oracle
import prefix_shared_masked_amd as pkg
from prefix_shared_masked_amd import TA_BLOCK_M, TA_BLOCK_N, TA_BLOCK_KV
import workloads as W


def expand_chunks(view, tile):
    """Keys of a query tile from the gathered chunk table, with each chunk's
    full flag repeated per key and the DFS-interval end of each key."""
    keys, full, kend = [], [], []
    for c in range(view["fq_ptr"][tile], view["fq_ptr"][tile + 1]):
        ch = view["fq_chunk"][c]
        nseg, nkeys, fl = int(ch[0]), int(ch[1]), int(ch[2])
        assert 1 <= nseg <= 4 and 1 <= nkeys <= TA_BLOCK_N
        for v in range(nkeys):
            s = max(x for x in range(4) if ch[8 + x] <= v)
            assert s < nseg
            keys.append(int(ch[4 + s] + v - ch[8 + s]))
            kend.append(int(ch[12 + s]))
            full.append(fl)
        if fl:
            assert nkeys == TA_BLOCK_N
    return np.array(keys, np.int64), np.array(full, bool), np.array(kend, np.int64)


def compare(tree):
    p = pkg.tree_plan(tree.parent, tree.seg_len)
    v = p.view()
    o = oracle.oracle_plan(tree.parent, tree.seg_len)
    assert p.n_tokens == o.n_tokens and p.n_leaves == o.n_leaves
    assert p.n_flat == o.n_flat and p.visible_pairs == o.visible_pairs
    assert v["dfs_order"].tolist() == o.dfs_order.tolist()
    assert v["node_start"].tolist() == o.node_start.tolist()
    assert v["node_sub_end"].tolist() == o.node_sub_end.tolist()
    for name in ("pos", "g", "node_of", "sub_end"):
        assert v[name].tolist() == getattr(o, name).tolist(), name
    assert p.max_pos == (int(o.pos.max()) if o.n_tokens else -1)
    for i in range(o.n_nodes):
        assert v["anc"][v["anc_ptr"][i]:v["anc_ptr"][i + 1]].tolist() == o.anc[i]
    # forward tiles: same visible keys; a chunk flagged full only if the
    # oracle says every row reads every one of its keys
    otiles = oracle.fwd_tile_keys(o, TA_BLOCK_M)
    assert p.n_qtiles == len(otiles)
    for t, (okeys, ofull) in enumerate(otiles):
        keys, full, kend = expand_chunks(v, t)
        order = np.argsort(keys, kind="stable")
        assert keys[order].tolist() == okeys.tolist(), t
        assert not (full[order] & ~ofull).any(), t
        assert kend.tolist() == o.sub_end[keys].tolist()
        # a chunk of all-full keys that is itself complete must be flagged
        for c in range(v["fq_ptr"][t], v["fq_ptr"][t + 1]):
            ch = v["fq_chunk"][c]
            ks = [int(ch[4 + s] + x) for s in range(ch[0]) for x in range(
                (ch[8 + s + 1] if s + 1 < ch[0] else ch[1]) - ch[8 + s])]
            allfull = all(ofull[np.searchsorted(okeys, kk)] for kk in ks)
            assert bool(ch[2]) == (allfull and ch[1] == TA_BLOCK_N)
    # longest chunk lists first
    counts = np.diff(v["fq_ptr"])
    assert sorted(v["fq_order"].tolist()) == list(range(p.n_qtiles))
    assert (np.diff(counts[v["fq_order"]]) <= 0).all()
    # backward key tiles
    bk = [tuple(int(x) for x in row[:3]) for row in v["bk"]]
    assert sorted(bk) == oracle.bwd_tiles(o, TA_BLOCK_KV)
    # most work first: 32-key sub-tile s reads the 32-row blocks from its own
    # diagonal block to the end of the query range
    sub = pkg.TA_KV_SUB

    def blocks(k0, kl, qe):
        nblk = -(-(qe - k0) // sub)
        return sum(nblk - s for s in range(-(-kl // sub)))
    work = [blocks(*x) for x in bk]
    assert all(a >= b for a, b in zip(work, work[1:]))
    assert p.computed_pairs_bwd == sub * sub * sum(work)
    for row in v["bk"]:
        assert o.node_of[row[0]] == row[3]
    check_pieces(p, v)
    return p, o


def check_pieces(p, v):
    """dK/dV work pieces (four wavefronts over common rows [q_lo, q_hi) on the
    query-tile grid, each owning a 32-key sub-tile and reading rows
    [max(key, r_lo), r_hi)): every sub-tile's rows [max(kw, q_start), q_end)
    are covered exactly once; a full 128-key tile spanning at most the cap's
    blocks is one piece with its four sub-tiles; every other run lies in one
    window of the cap's blocks anchored at q_start, and runs are packed only
    when the piece's span is at most one block longer than its longest run; a
    sub-tile over several windows owns consecutive slots in window order and
    a sum record; pieces are listed longest first, then by last row.  The dS
    blocks the wavefronts store are exactly the blocks the dQ lists read, each
    once, numbered 0 .. n_dsblk - 1."""
    sub, BK, KW = pkg.TA_KV_SUB, pkg.TA_BLOCK_KV, pkg.TA_KWAVE_INTS
    kp, kr, bk = v["kp"], v["kr"], v["bk"]
    q0, N = p.q_start, p.n_tokens
    assert p.n_kpieces == len(kp) and p.n_ksplit == len(kr) and kp.shape[1] == pkg.TA_KPIECE_INTS
    nb = [-(-(int(t[2]) - max(int(t[0]), q0)) // sub) for t in bk]
    cap = max(pkg.TA_KV_PIECE_MIN, -(-sum(nb) // 256))
    assert p.kv_piece_cap == cap
    W = sub * cap
    floor = lambda r: q0 + sub * ((r - q0) // sub)
    whole = {int(t[0]): int(t[2]) for t, n in zip(bk, nb) if t[1] == BK and n <= cap}
    runs, written = {}, {}
    for x in kp:
        x = [int(z) for z in x]
        qlo, qhi = x[0], x[1]
        assert x[2] == 0 and x[3] == 0 and q0 <= qlo < qhi <= N and (qlo - q0) % sub == 0
        waves = [x[4 + KW * w:4 + KW * (w + 1)] for w in range(4)]
        act = [t for t in waves if t[1] > 0]
        assert act, "a piece with no keys"
        k0 = act[0][0]
        is_whole = (k0 in whole and len(act) == 4 and all(t[4] == -1 for t in act)
                    and [t[0] for t in act] == [k0 + sub * w for w in range(4)] and act[0][3] == whole[k0]
                    and qlo == floor(max(k0, q0)))
        if is_whole:
            qe = whole.pop(k0)
            assert qhi == qe
            for t in act:
                assert t[1:5] == [sub, max(t[0], q0), qe, -1] and t[6] == 0
        else:
            lo_min, longest = min(t[2] for t in act), 0
            assert qlo == floor(lo_min)
            for kw, wk, rlo, rhi, slot, dso, z in act:
                assert 1 <= wk <= sub and qlo <= rlo < rhi <= qhi and z == 0
                win = (rhi - 1 - q0) // W
                assert (rlo - q0) // W == win and rlo == max(kw, q0, q0 + win * W)
                longest = max(longest, rhi - rlo)
            assert qhi - lo_min <= longest + sub
        for kw, wk, rlo, rhi, slot, dso, z in waves:
            if wk == 0:
                assert (rlo, rhi, slot) == (qlo, qlo, -1)
                continue
            runs.setdefault(kw, []).append((rlo, rhi, slot, wk))
            for t in range((rlo - q0) // sub, -(-(rhi - q0) // sub)):
                assert (kw, t) not in written, "a dS block stored twice"
                written[(kw, t)] = dso + t
    assert not whole, "a whole tile was not one piece"
    node_of, sub_end = v["node_of"], v["sub_end"]
    slots, cut = [], {}
    for kw, rs in runs.items():
        qe = int(sub_end[kw])
        rs.sort()
        assert rs[0][0] == max(kw, q0) and rs[-1][1] == qe, kw
        for (a0, b0, _, _), (a1, b1, _, _) in zip(rs, rs[1:]):
            assert b0 == a1
        assert len({r[3] for r in rs}) == 1 and all(node_of[kw + i] == node_of[kw] for i in range(rs[0][3]))
        if len(rs) == 1:
            assert rs[0][2] == -1
        else:
            ss = [r[2] for r in rs]
            assert ss == list(range(ss[0], ss[0] + len(rs)))
            slots += ss
            cut[kw] = (rs[0][3], ss[0], len(rs))
    assert sorted(slots) == list(range(p.n_kslots))
    assert {int(r[0]): (int(r[1]), int(r[2]), int(r[3])) for r in kr} == cut and len(cut) == len(kr)
    assert sum(r[0][3] for r in runs.values()) == N     # every key in exactly one sub-tile
    key = [(-(-(-(int(x[1]) - int(x[0])) // sub)), -int(x[1])) for x in kp]
    assert key == sorted(key)
    # dS blocks: stored once each, numbered densely, and exactly the dQ lists
    assert p.n_dsblk == len(written) and sorted(written.values()) == list(range(p.n_dsblk))
    dptr, dent, dord = v["dq_ptr"], v["dq_ent"], v["dq_order"]
    assert len(dptr) == p.n_qtiles + 1 and (np.diff(dptr) >= 1).all() and dptr[-1] == len(dent) == p.n_dsblk
    seen = {}
    for t in range(p.n_qtiles):
        ent = dent[dptr[t]:dptr[t + 1]]
        assert list(ent[:, 0]) == sorted(ent[:, 0]) and (ent[:, 3] == 0).all()
        for kw, wk, blk, _ in ent:
            seen[(int(kw), t)] = int(blk)
            assert runs[int(kw)][0][3] == wk
    assert seen == written
    cnt = np.diff(dptr)
    assert sorted(dord.tolist()) == list(range(p.n_qtiles)) and (np.diff(cnt[dord]) <= 0).all()


def test_six_node():
    p, _ = compare(W.six_node_tree(16))
    assert p.view()["dfs_order"].tolist() == [0, 1, 3, 4, 2, 5]
    assert p.visible_pairs == 2864


def test_spine_full_size():
    p, o = compare(W.spine_tree())
    assert (p.n_tokens, p.n_flat, p.n_leaves) == (16352, 129184, 44)


def test_random_agentic_tree():
    compare(W.random_agentic_tree(0))


def test_varlen_forest():
    p, o = compare(W.varlen_forest(0))
    assert p.n_leaves == 64 and p.n_flat == p.n_tokens


@pytest.mark.parametrize("seed", range(6))
def test_random_small_trees(seed):
    rng = np.random.default_rng(100 + seed)
    for c in range(40):
        shape = ["random", "chain", "star"][c % 3]
        tree = W.random_tree(rng, int(rng.integers(1, 60)), max_len=int(rng.integers(1, 140)),
                             p_zero=0.15, n_roots=int(rng.integers(1, 4)), shape=shape)
        if tree.n_tokens == 0:
            continue
        compare(tree)


def test_node_lengths_around_tile_edges():
    for L in (1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129):
        compare(W.Tree(np.array([-1, 0, 0, 1], np.int32), np.array([L, L, 3, L], np.int32)))


def test_cut_key_tiles():
    """A 100-token root over a 300-token node with 900- and 700-token
    children (2,000 rows): the tiles span 423 query blocks, so the cap is 32
    (windows of 1,024 rows); node 1's two full tiles (60 and 56 blocks) and
    its 44-key tile, and the 100-key root, are cut into 32-key sub-tiles;
    node 2's full tiles of at most 32 blocks stay whole.  With the root as a
    key-only prefix the windows start at q_start."""
    tree = W.Tree(np.array([-1, 0, 1, 1], np.int32), np.array([100, 300, 900, 700], np.int32))
    p, _ = compare(tree)
    v = p.view()
    assert p.kv_piece_cap == 32 and p.n_ksplit > 0
    # the root's four sub-tiles (32, 32, 32, 4 keys) span rows [kw, 2000): two windows each
    root = {int(r[0]): (int(r[1]), int(r[3])) for r in v["kr"] if r[0] < 100}
    assert root == {0: (32, 2), 32: (32, 2), 64: (32, 2), 96: (4, 2)}
    pe = pkg.tree_plan(tree.parent, tree.seg_len, n_prefix_nodes=1)
    check_pieces(pe, pe.view())
    assert pe.q_start == 100 and all(x[0] >= 100 for x in pe.view()["kp"])


def test_star_with_64_children_and_deep_chain():
    compare(W.Tree(np.array([-1] + [0] * 64, np.int32), np.array([40] + [7] * 64, np.int32)))
    n = 300
    compare(W.Tree(np.array([-1] + list(range(n - 1)), np.int32), np.array([3] * n, np.int32)))


def test_determinism():
    t = W.random_agentic_tree(1)
    a, b = pkg.tree_plan(t.parent, t.seg_len).view(), pkg.tree_plan(t.parent, t.seg_len).view()
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def _status(parent, seg_len, n=None, bm=0, bn=0):
    L = pkg.load_library()
    out = ctypes.c_void_p(123)
    pI32 = ctypes.POINTER(ctypes.c_int32)
    par = np.ascontiguousarray(parent, np.int32)
    sl = np.ascontiguousarray(seg_len, np.int32)
    st = L.tree_plan(par.ctypes.data_as(pI32), sl.ctypes.data_as(pI32), len(par) if n is None else n, bm, bn,
                     ctypes.byref(out))
    if st == 0:
        L.tree_plan_free(out)
    else:
        assert not out.value          # *out is NULL on error
    return st


def test_error_codes():
    assert _status([-1, 0], [1, 1]) == 0
    assert _status([1, 0], [1, 1]) == 2              # cycle without a root
    assert _status([-1, 0, 3, 2], [1, 1, 1, 1]) == 2
    assert _status([-1, 1], [1, 1]) == 2             # self-parent
    assert _status([-1, 5], [1, 1]) == 1             # parent out of range
    assert _status([-1, -2], [1, 1]) == 1
    assert _status([-1, 0], [1, -1]) == 1            # negative length
    assert _status([-1], [1], n=0) == 1
    assert _status([-1], [1], bm=16) == 5            # block sizes the kernels are not built for
    assert _status([-1], [1], bn=128) == 5
    assert _status([-1, 0], [2 ** 30, 2 ** 30]) == 3  # N overflows int32
    L = pkg.load_library()
    assert L.tree_plan(None, None, 1, 0, 0, None) == 1
    L.tree_plan_free(None)                           # NULL-safe
    with pytest.raises(pkg.TreeAttnError):
        pkg.tree_plan([0], [1])


def test_zero_token_nodes_only_between():
    compare(W.Tree(np.array([-1, 0, 1, 0, 3], np.int32), np.array([0, 5, 0, 0, 2], np.int32)))
