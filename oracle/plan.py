"""Oracle plan: what the tree packing computes, by the most direct route.

Test infrastructure only (see ``oracle/__init__.py``).

Sources ("Tree Training" post on tingdeliu.github.io):

* section 3.1: each node holds a token segment, each root-to-leaf path is one
  training sequence, K = number of paths;
* section 3.2, the X_DFS formula: a node's tokens, then each child's DFS
  serialisation in turn -- written here as a recursive visit;
* section 5, the depth-position equation: pos(t) = total length of the strict
  ancestors of node(t) + offset of t inside its node -- computed here by
  walking parent pointers;
* section 6.2: g_t = number of root-to-leaf paths through t -- computed here
  by walking from every leaf to the root and counting;
* section 4.3: the DFS interval of a node (its subtree occupies one
  contiguous range of the packed sequence);
* section 13: N_pairs = sum over tokens of the visible-context length D(t).

Readings where the pages are silent: children are visited in ascending node
id and roots in ascending id (the page's example only fixes n1 before n2, n3
before n4); several roots form a forest whose positions restart at 0
(agent-rl chapter 14, section 14.1: positions restart per packed sequence);
zero-length nodes are allowed and a zero-length leaf still counts as a path.

Parity: pinned by the printed six-node example (DFS order, Fig. 4 weights),
the closed forms of section 2 on the spine family, the path-sum identity of
section 6.2 and a dense-mask brute force (tests/test_oracle_plan.py).
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field

import numpy as np


@dataclass
class OraclePlan:
    n_nodes: int
    n_tokens: int
    dfs_order: np.ndarray          # node ids in DFS visiting order
    node_start: np.ndarray         # [n] first packed index of each node (by node id)
    node_sub_end: np.ndarray       # [n] end of each node's DFS interval
    pos: np.ndarray                # [N] depth position of each packed token
    g: np.ndarray                  # [N] number of root-to-leaf paths through the token
    node_of: np.ndarray            # [N] node id of each packed token
    sub_end: np.ndarray            # [N] node_sub_end[node_of[t]]
    n_leaves: int                  # K
    n_flat: int                    # sum over paths of the path length
    visible_pairs: int             # sum_t (pos(t) + 1)
    anc: list = field(default_factory=list)    # [n] ancestor-or-self node ids, root first
    paths: list = field(default_factory=list)  # per leaf (DFS order): packed token indices root->leaf
    seg_len: np.ndarray = None
    parent: np.ndarray = None


def oracle_plan(parent, seg_len) -> OraclePlan:
    parent = [int(p) for p in parent]
    seg_len = [int(s) for s in seg_len]
    n = len(parent)
    if n <= 0 or len(seg_len) != n:
        raise ValueError("need n_nodes > 0 and one length per node")
    for i in range(n):
        if seg_len[i] < 0:
            raise ValueError(f"node {i} has negative length")
        if parent[i] < -1 or parent[i] >= n:
            raise ValueError(f"node {i} has parent {parent[i]} out of range")

    children = [[] for _ in range(n)]
    roots = []
    for i in range(n):                       # ascending id => children and roots ascending
        (roots if parent[i] == -1 else children[parent[i]]).append(i)

    order, start, sub_end = [], [0] * n, [0] * n
    cursor = 0
    old_limit = sys.getrecursionlimit()
    sys.setrecursionlimit(max(old_limit, 4 * n + 100))

    def visit(node):
        nonlocal cursor
        order.append(node)
        start[node] = cursor
        cursor += seg_len[node]
        for c in children[node]:
            visit(c)
        sub_end[node] = cursor

    try:
        for r in roots:
            visit(r)
    finally:
        sys.setrecursionlimit(old_limit)
    if len(order) != n:
        raise ValueError("parent pointers contain a cycle")

    # ancestor-or-self chain of every node, by walking parent pointers
    anc = []
    for i in range(n):
        chain, a = [], i
        while a != -1:
            chain.append(a)
            a = parent[a]
        anc.append(chain[::-1])

    N = cursor
    node_of = np.empty(N, np.int64)
    pos = np.empty(N, np.int64)
    for node in range(n):
        base = sum(seg_len[a] for a in anc[node][:-1])     # strict ancestors' lengths
        for j in range(seg_len[node]):
            node_of[start[node] + j] = node
            pos[start[node] + j] = base + j

    # g: walk up from every leaf and count
    count = [0] * n
    leaves = [i for i in order if not children[i]]
    for leaf in leaves:
        for a in anc[leaf]:
            count[a] += 1
    g = np.array([count[node_of[t]] for t in range(N)], np.int64)

    paths = []
    for leaf in leaves:
        idx = [start[a] + j for a in anc[leaf] for j in range(seg_len[a])]
        paths.append(np.array(idx, np.int64))
    n_flat = int(sum(len(p) for p in paths))

    node_sub_end = np.array(sub_end, np.int64)
    return OraclePlan(
        n_nodes=n, n_tokens=N, dfs_order=np.array(order, np.int64),
        node_start=np.array(start, np.int64), node_sub_end=node_sub_end,
        pos=pos, g=g, node_of=node_of, sub_end=node_sub_end[node_of] if N else np.zeros(0, np.int64),
        n_leaves=len(leaves), n_flat=n_flat, visible_pairs=int((pos + 1).sum()),
        anc=anc, paths=paths, seg_len=np.array(seg_len, np.int64), parent=np.array(parent, np.int64))


def fwd_tile_keys(plan: OraclePlan, block_m: int):
    """For each query tile [q0, q0+block_m): the sorted keys visible to at least
    one row of the tile, and for each such key whether every row of the tile
    sees it.

    Enumerates node pairs: for every node b owning rows of the tile and every
    ancestor-or-self a of b, the keys of a that some row of b may read (all of
    a's tokens for a strict ancestor, tokens of b up to b's last row in the
    tile).  The visibility rule is the tree mask of section 4.2: key j is
    visible to row i iff j <= i and node(j) is an ancestor-or-self of node(i).
    """
    N = plan.n_tokens
    out = []
    for q0 in range(0, N, block_m):
        q1 = min(N, q0 + block_m)
        nodes = {}
        for i in range(q0, q1):
            nodes[int(plan.node_of[i])] = i          # last row of node b inside the tile
        keys = []
        anc_sets = []
        for b, last_row in nodes.items():
            anc_sets.append(set(plan.anc[b]))
            for a in plan.anc[b]:
                s = int(plan.node_start[a])
                e = s + int(plan.seg_len[a]) if a != b else last_row + 1
                keys.append(np.arange(s, e, dtype=np.int64))
        keys = np.unique(np.concatenate(keys)) if keys else np.zeros(0, np.int64)
        common = set.intersection(*anc_sets) if anc_sets else set()
        full = np.array([(k <= q0) and (int(plan.node_of[k]) in common) for k in keys], bool)
        out.append((keys, full))
    return out


def bwd_tiles(plan: OraclePlan, block_n: int):
    """Key tiles of at most block_n keys that never cross a node boundary, with
    the query range that reads them: every query in [k0, node_sub_end) lies in
    the node's subtree (the node's DFS interval, section 4.3)."""
    tiles = []
    for a in range(plan.n_nodes):
        s = int(plan.node_start[a])
        e = s + int(plan.seg_len[a])
        for k0 in range(s, e, block_n):
            tiles.append((k0, min(block_n, e - k0), int(plan.node_sub_end[a])))
    return sorted(tiles)


def dense_mask(plan: OraclePlan, rows=None) -> np.ndarray:
    """The N x N tree mask written literally from the mask prototype of
    section 12: key k is allowed for query q iff k <= q and node(k) is an
    ancestor (or the node itself) of node(q), found by walking parent
    pointers from node(q).  ``rows`` restricts to a subset of queries."""
    N = plan.n_tokens
    rows = range(N) if rows is None else rows
    rows = list(rows)
    m = np.zeros((len(rows), N), bool)
    for r, qi in enumerate(rows):
        qn = int(plan.node_of[qi])
        chain = set()
        a = qn
        while a != -1:
            chain.add(a)
            a = int(plan.parent[a])
        for kj in range(qi + 1):
            if int(plan.node_of[kj]) in chain:
                m[r, kj] = True
    return m


def por(n_tree: int, n_flat: int) -> float:
    """Potential overlap ratio of section 10: 1 - N_tree / N_flat."""
    return 1.0 - n_tree / n_flat


def speedup_upper(por_value: float) -> float:
    """Upper bound on token/compute reuse of section 10: N_flat / N_tree = 1 / (1 - POR)."""
    return 1.0 / (1.0 - por_value)
