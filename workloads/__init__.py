"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only builds inputs: tree shapes (``parent``/``seg_len`` arrays),
random tensors, labels and decode batches.  It holds none of the method's
arithmetic (no DFS, no positions, no path counts, no attention), so both the
oracle and the HIP path can consume its output without sharing code.

Tree shapes follow the pages' workloads:

* the six-node example tree of "Tree Training" (Fig. 2 of the tingdeliu.github.io
  post, section 3.2): n0 -> {n1, n2}, n1 -> {n3, n4}, n2 -> {n5};
* the navigation-episode "spine": a shared prompt root, T history nodes
  H_t chained one after another, each with a leaf L_t holding the step's
  observation and action-query tokens (post, sections 2 and 11.1);
* a random agentic rollout tree (branching 1-4, depth <= 8, lognormal node
  lengths);
* varlen packing: lognormal sequence lengths, first-fit-decreasing into fixed
  rows, every sequence its own root (agent-rl chapter 14, section 14.1);
* split-KV decode batches (Tree Attention notes, decode algorithm table).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Tree",
    "six_node_tree",
    "spine_tree",
    "random_agentic_tree",
    "varlen_forest",
    "random_tree",
    "normal",
    "nll_inputs",
    "decode_spans",
]


@dataclass
class Tree:
    """A prefix tree as two int32 arrays indexed by node id.

    ``parent[i] == -1`` marks a root; several roots form a forest.
    ``seg_len[i]`` is the number of tokens node i holds (may be 0).
    """

    parent: np.ndarray
    seg_len: np.ndarray
    name: str = ""

    @property
    def n_nodes(self) -> int:
        return int(self.parent.shape[0])

    @property
    def n_tokens(self) -> int:
        return int(self.seg_len.sum())


def _tree(parent, seg_len, name=""):
    return Tree(np.asarray(parent, dtype=np.int32), np.asarray(seg_len, dtype=np.int32), name)


def six_node_tree(seg: int = 16) -> Tree:
    """The pages' six-node example: n0 root, n1/n2 children of n0, n3/n4 of n1, n5 of n2."""
    return _tree([-1, 0, 0, 1, 1, 2], [seg] * 6, "six_node")


def spine_tree(p: int = 512, delta: int = 96, leaf_len: int = 264, T: int = 44) -> Tree:
    """Navigation-episode spine: root of p tokens, H_t (id 2t-1, delta tokens)
    chained under H_{t-1} (H_1 under the root), leaf L_t (id 2t, leaf_len
    tokens) under H_t, for t = 1..T.  leaf_len = 0 gives the pages' pure
    prefix chain, where sample t ends at spine node t."""
    n = 2 * T + 1
    parent = np.empty(n, np.int32)
    seg = np.empty(n, np.int32)
    parent[0], seg[0] = -1, p
    for t in range(1, T + 1):
        h, leaf = 2 * t - 1, 2 * t
        parent[h] = 0 if t == 1 else 2 * (t - 1) - 1
        seg[h] = delta
        parent[leaf] = h
        seg[leaf] = leaf_len
    return Tree(parent, seg, f"spine_p{p}_d{delta}_l{leaf_len}_T{T}")


def random_agentic_tree(seed: int = 0, target_tokens: int = 32768, max_depth: int = 8,
                        branch=(1, 4), median: float = 256.0, sigma: float = 0.8,
                        clip=(32, 4096)) -> Tree:
    """Random rollout tree grown until it holds at least ``target_tokens``.

    The root sits at depth 1.  Each round picks a uniformly random node that
    has not been expanded yet; below ``max_depth`` it gets b ~ U{branch}
    children whose lengths are round(median * exp(sigma * z)) clipped to
    ``clip``; a node at ``max_depth`` is retired without children.  Node ids
    follow creation order.
    """
    rng = np.random.default_rng(seed)

    def draw_len():
        return int(np.clip(round(median * math.exp(sigma * rng.standard_normal())), clip[0], clip[1]))

    parent, seg, depth = [-1], [draw_len()], [1]
    frontier = [0]
    total = seg[0]
    while total < target_tokens and frontier:
        idx = int(rng.integers(len(frontier)))
        node = frontier[idx]
        frontier[idx] = frontier[-1]
        frontier.pop()
        if depth[node] >= max_depth:
            continue
        b = int(rng.integers(branch[0], branch[1] + 1))
        for _ in range(b):
            parent.append(node)
            seg.append(draw_len())
            depth.append(depth[node] + 1)
            frontier.append(len(parent) - 1)
            total += seg[-1]
    return _tree(parent, seg, f"random_agentic_s{seed}")


def varlen_lengths(seed: int = 0, n_seq: int = 64, median: float = 1024.0,
                   p90: float = 5120.0, max_len: int = 16384) -> np.ndarray:
    """Lognormal sequence lengths with the given median and 90th percentile,
    clipped to [1, max_len]."""
    rng = np.random.default_rng(seed)
    sigma = math.log(p90 / median) / 1.2815515655446004  # z of the 90th percentile
    z = rng.standard_normal(n_seq)
    return np.clip(np.rint(median * np.exp(sigma * z)), 1, max_len).astype(np.int64)


def ffd_rows(lengths, row_tokens: int):
    """First-fit decreasing: longest first (ties keep the lower index), each
    sequence into the first row with room.  Raises if one does not fit."""
    order = sorted(range(len(lengths)), key=lambda i: -int(lengths[i]))
    rows, used = [], []
    for i in order:
        n = int(lengths[i])
        if n > row_tokens:
            raise ValueError(f"sequence of {n} tokens does not fit a row of {row_tokens}")
        for r, u in enumerate(used):
            if u + n <= row_tokens:
                rows[r].append(i)
                used[r] += n
                break
        else:
            rows.append([i])
            used.append(n)
    return rows


def varlen_forest(seed: int = 0, n_seq: int = 64, row_tokens: int = 32768, **kw) -> Tree:
    """Varlen packing as a forest: each sequence is a root node; node ids follow
    the packed order (rows one after another, members in FFD order)."""
    lengths = varlen_lengths(seed, n_seq, **kw)
    rows = ffd_rows(lengths, row_tokens)
    order = [i for r in rows for i in r]
    t = _tree([-1] * len(order), [int(lengths[i]) for i in order], f"varlen_s{seed}")
    t.rows = rows
    return t


def random_tree(rng: np.random.Generator, n_nodes: int, max_len: int = 40, p_zero: float = 0.1,
                n_roots: int = 1, shuffle_ids: bool = True, shape: str = "random") -> Tree:
    """Small random trees for property tests: random attachment (or a chain or
    a star), optional zero-length nodes, several roots, and node ids that need
    not be in topological order."""
    n_roots = max(1, min(n_roots, n_nodes))
    parent = np.full(n_nodes, -1, np.int64)
    for i in range(n_roots, n_nodes):
        if shape == "chain":
            parent[i] = i - 1
        elif shape == "star":
            parent[i] = 0
        else:
            parent[i] = rng.integers(0, i)
    seg = rng.integers(1, max_len + 1, n_nodes)
    seg[rng.random(n_nodes) < p_zero] = 0
    if shuffle_ids:
        perm = rng.permutation(n_nodes)          # old id -> new id
        new_parent = np.full(n_nodes, -1, np.int64)
        new_seg = np.empty(n_nodes, np.int64)
        for old in range(n_nodes):
            new_parent[perm[old]] = -1 if parent[old] < 0 else perm[parent[old]]
            new_seg[perm[old]] = seg[old]
        parent, seg = new_parent, new_seg
    return _tree(parent, seg, f"random_{shape}_{n_nodes}")


def normal(seed: int, shape, dtype=np.float32) -> np.ndarray:
    """Standard-normal array from a seeded PCG64 stream."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32).astype(dtype, copy=False)


def attention_inputs(seed: int, n_tokens: int, Hq: int, Hkv: int, d: int):
    """q [N,Hq,d], k/v [N,Hkv,d] and an upstream gradient dO [N,Hq,d], all N(0,1) fp32."""
    return (normal(seed, (n_tokens, Hq, d)), normal(seed + 1, (n_tokens, Hkv, d)),
            normal(seed + 2, (n_tokens, Hkv, d)), normal(seed + 3, (n_tokens, Hq, d)))


def nll_inputs(seed: int, n_tokens: int, vocab: int, p_ignore: float = 0.25, ignore_index: int = -100):
    """Random logits N(0,1) [N,V] fp32 and uniform labels in [0,V), with a seeded
    fraction set to ``ignore_index`` (unsupervised positions)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((n_tokens, vocab), dtype=np.float32)
    labels = rng.integers(0, vocab, n_tokens).astype(np.int32)
    labels[rng.random(n_tokens) < p_ignore] = ignore_index
    return logits, labels


def decode_spans(lengths, gap: int = 0):
    """One contiguous KV span per batch item, items laid out one after another
    (``gap`` unused rows between them).  Returns (span_ptr [B+1], spans [B,2]
    as (start, len), total rows)."""
    lengths = [int(x) for x in lengths]
    span_ptr = np.arange(len(lengths) + 1, dtype=np.int32)
    spans = np.zeros((len(lengths), 2), np.int32)
    off = 0
    for b, n in enumerate(lengths):
        spans[b] = (off, n)
        off += n + gap
    return span_ptr, spans, off
