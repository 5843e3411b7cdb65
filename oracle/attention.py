"""Oracle attention: the tree-packed result by its plain definitions, float64.

Test infrastructure only (see ``oracle/__init__.py``).

Two independent routes to the same numbers:

``per_path_attention``
    The equivalence the "Tree Training" post states for its tree mask
    (section 4.2: every token's visible context is exactly that of the
    independent root-to-leaf run; section 14.1: compare against running every
    path on its own).  Every root-to-leaf path is run as an ordinary causal
    sequence with positions 0..L-1, with textbook softmax attention
    softmax(Q K^T * scale + causal) V.  Outputs are scattered back to packed
    order.  For the backward, the loss identity of section 6.2
    (L_tree = sum_t g_t/K l_t = (1/K) sum_k sum_{t in p_k} l_t) means the
    packed upstream gradient dO_t is shared by the g_t paths through t: path k
    receives dO_t / g_t and the path gradients are summed into packed order
    (shared ancestors accumulate the gradients of all descendants, section 7).

``dense_mask_attention``
    The mask equation of section 4.2 / the mask prototype of section 12
    written literally (key j allowed for query i iff j <= i and node(j) is an
    ancestor-or-self of node(i)), with depth positions (section 5), masked
    softmax attention and the textbook dense backward
    (dP = dO V^T, dS = P * (dP - rowsum(dO * O)), dQ = dS K s, dK = dS^T Q s,
    dV = P^T dO).  Query rows are evaluated a group at a time only to bound
    memory; every row's softmax is computed whole.

RoPE reading (the pages only say positions are tree depth; the rotary base
10000 is the workload's): rotate-half pairing (i, i + d/2), angle
pos * base^(-2i/d).  GQA reading: query head h uses KV head h // (Hq / Hkv).
LSE is the natural log of sum_j exp(scale * q.k_j).

``rows_attention``, ``rows_attention_grads``, ``causal_sequence_grads``
    Spot-check forms for full sizes: outputs of selected rows from each row's
    own path, and gradients of selected rows and keys (per row, or per block
    of rows of one causal sequence) from the dense backward's definitions.

Parity: pinned by the dense/per-path agreement, by single-path and forest
special cases against torch's CPU scaled_dot_product_attention, by finite
differences of the backward and by the leak invariants of section 14.2
(tests/test_oracle_attention.py).
"""
from __future__ import annotations

import numpy as np


def rope(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate x [T, H, d] by angles pos[t] * base^(-2i/d) on pairs (i, i+d/2)."""
    if not base:
        return x
    d = x.shape[-1]
    half = d // 2
    inv = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rope_transpose(dy: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Apply the transposed rotation (the gradient of ``rope`` w.r.t. x)."""
    if not base:
        return dy
    d = dy.shape[-1]
    half = d // 2
    inv = base ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    d1, d2 = dy[..., :half], dy[..., half:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def _kv_head(Hq: int, Hkv: int) -> np.ndarray:
    return np.arange(Hq) // (Hq // Hkv)


def _causal_attention(q, k, v, scale, dO=None):
    """Textbook causal attention of one sequence.  q [L,H,d], k/v [L,H,d] (KV
    already expanded per query head).  Returns O [L,H,d], LSE [H,L] and, if
    dO is given, (dq, dk, dv) per query head."""
    L = q.shape[0]
    qh, kh, vh = (np.transpose(a, (1, 0, 2)) for a in (q, k, v))     # [H, L, d]
    S = qh @ np.transpose(kh, (0, 2, 1)) * scale                      # [H, L, L]
    S = np.where(np.tril(np.ones((L, L), bool))[None], S, -np.inf)
    m = S.max(-1, keepdims=True)
    E = np.exp(S - m)
    den = E.sum(-1, keepdims=True)
    P = E / den
    O = P @ vh
    lse = (m + np.log(den))[..., 0]
    out = np.transpose(O, (1, 0, 2))
    if dO is None:
        return out, lse, None
    dOh = np.transpose(dO, (1, 0, 2))
    dP = dOh @ np.transpose(vh, (0, 2, 1))
    Drow = (dOh * O).sum(-1, keepdims=True)
    dS = P * (dP - Drow)
    dq = dS @ kh * scale
    dk = np.transpose(dS, (0, 2, 1)) @ qh * scale
    dv = np.transpose(P, (0, 2, 1)) @ dOh
    return out, lse, tuple(np.transpose(a, (1, 0, 2)) for a in (dq, dk, dv))


def per_path_attention(plan, q, k, v, scale=None, rope_base=0.0, dO=None, heads=None,
                       check_consistency=True):
    """Tree attention by running each root-to-leaf path as its own sequence.

    q [N,Hq,d], k/v [N,Hkv,d] (any float dtype, computed in float64).
    ``heads`` restricts the work to a subset of query heads (the other heads'
    outputs stay zero); KV gradients then hold only those heads' share.
    Returns dict(o, lse, dq, dk, dv, path_spread) where path_spread is the
    largest disagreement between two paths' outputs for a shared token."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    kvh = _kv_head(Hq, Hkv)[heads]
    o = np.zeros((N, Hq, d))
    lse = np.zeros((Hq, N))
    seen = np.zeros(N, bool)
    spread = 0.0
    grads = dO is not None
    if grads:
        dO = np.asarray(dO, np.float64)
        dq = np.zeros((N, Hq, d))
        dk = np.zeros((N, Hkv, d))
        dv = np.zeros((N, Hkv, d))
        g = plan.g.astype(np.float64)
    for idx in plan.paths:
        L = len(idx)
        if L == 0:
            continue
        p = np.arange(L)
        qp = rope(q[idx][:, heads], p, rope_base)
        kr = rope(k[idx], p, rope_base)
        kp = kr[:, kvh]
        vp = v[idx][:, kvh]
        dOp = dO[idx][:, heads] / g[idx][:, None, None] if grads else None
        op, lp, gr = _causal_attention(qp, kp, vp, scale, dOp)
        if check_consistency and seen[idx].any():
            sh = seen[idx]
            spread = max(spread, float(np.abs(o[idx[sh]][:, heads] - op[sh]).max(initial=0.0)),
                         float(np.abs(lse[heads][:, idx[sh]] - lp[:, sh]).max(initial=0.0)))
        o[np.ix_(idx, heads)] = op
        lse[np.ix_(heads, idx)] = lp
        seen[idx] = True
        if grads:
            gq, gk, gv = gr
            dq[np.ix_(idx, heads)] += rope_transpose(gq, p, rope_base)
            gk = rope_transpose(gk, p, rope_base)
            for hi, kh in enumerate(kvh):
                dk[idx, kh] += gk[:, hi]
                dv[idx, kh] += gv[:, hi]
    res = dict(o=o, lse=lse, path_spread=spread)
    if grads:
        res.update(dq=dq, dk=dk, dv=dv)
    return res


def _mask_rows(plan, r0, r1, n_keys):
    """Rows [r0, r1) of the tree mask over keys [0, n_keys): key j allowed for
    query i iff j <= i and node(j) is on the parent chain of node(i)."""
    node_of = plan.node_of
    keys = np.arange(n_keys)
    m = np.zeros((r1 - r0, n_keys), bool)
    cache = {}
    for i in range(r0, r1):
        b = int(node_of[i])
        if b not in cache:
            chain, a = [], b
            while a != -1:
                chain.append(a)
                a = int(plan.parent[a])
            cache[b] = np.isin(node_of[:n_keys], chain)
        m[i - r0] = cache[b] & (keys <= i)
    return m


def dense_mask_attention(plan, q, k, v, scale=None, rope_base=0.0, dO=None, heads=None,
                         row_block=1024):
    """Tree attention from the dense N x N mask and depth positions.
    Same arguments and result layout as ``per_path_attention``."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    kvh = _kv_head(Hq, Hkv)[heads]
    qr = rope(q[:, heads], plan.pos, rope_base)                     # [N, h, d]
    kr = rope(k, plan.pos, rope_base)[:, kvh]                       # [N, h, d]
    vr = v[:, kvh]
    qh, kh, vh = (np.transpose(a, (1, 0, 2)) for a in (qr, kr, vr))  # [h, N, d]
    o = np.zeros((N, Hq, d))
    lse = np.zeros((Hq, N))
    grads = dO is not None
    if grads:
        dOh = np.transpose(np.asarray(dO, np.float64)[:, heads], (1, 0, 2))
        dqh = np.zeros_like(qh)
        dkh = np.zeros_like(kh)
        dvh = np.zeros_like(vh)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        mask = _mask_rows(plan, r0, r1, r1)                          # keys > r1-1 never visible
        S = qh[:, r0:r1] @ np.transpose(kh[:, :r1], (0, 2, 1)) * scale
        S = np.where(mask[None], S, -np.inf)
        m = S.max(-1, keepdims=True)
        E = np.exp(S - m)
        den = E.sum(-1, keepdims=True)
        P = E / den
        O = P @ vh[:, :r1]
        o[r0:r1][:, heads] = np.transpose(O, (1, 0, 2))
        lse[heads, r0:r1] = (m + np.log(den))[..., 0]
        if grads:
            g = dOh[:, r0:r1]
            dP = g @ np.transpose(vh[:, :r1], (0, 2, 1))
            Drow = (g * O).sum(-1, keepdims=True)
            dS = P * (dP - Drow)
            dqh[:, r0:r1] += dS @ kh[:, :r1] * scale
            dkh[:, :r1] += np.transpose(dS, (0, 2, 1)) @ qh[:, r0:r1] * scale
            dvh[:, :r1] += np.transpose(P, (0, 2, 1)) @ g
    res = dict(o=o, lse=lse)
    if grads:
        dq = np.zeros((N, Hq, d))
        dq[:, heads] = rope_transpose(np.transpose(dqh, (1, 0, 2)), plan.pos, rope_base)
        dk = np.zeros((N, Hkv, d))
        dv = np.zeros((N, Hkv, d))
        gk = rope_transpose(np.transpose(dkh, (1, 0, 2)), plan.pos, rope_base)
        gv = np.transpose(dvh, (1, 0, 2))
        for hi, kh_ in enumerate(kvh):
            dk[:, kh_] += gk[:, hi]
            dv[:, kh_] += gv[:, hi]
        res.update(dq=dq, dk=dk, dv=dv)
    return res


def rows_attention(plan, q, k, v, rows, heads, scale=None, rope_base=0.0):
    """Forward output and LSE of selected (row, head) pairs only, each from the
    row's own root-to-node path (the independent-run definition), for spot
    checks at sizes where whole-tree oracles are too slow.
    Returns o [len(rows), len(heads), d], lse [len(heads), len(rows)]."""
    q = np.asarray(q)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    kvh = _kv_head(Hq, Hkv)
    o = np.zeros((len(rows), len(heads), d))
    lse = np.zeros((len(heads), len(rows)))
    for ri, i in enumerate(rows):
        b = int(plan.node_of[i])
        idx = np.concatenate([np.arange(plan.node_start[a], plan.node_start[a] + plan.seg_len[a])
                              for a in plan.anc[b][:-1]] +
                             [np.arange(plan.node_start[b], i + 1)]).astype(np.int64)
        p = np.arange(len(idx))
        for hi, h in enumerate(heads):
            qi = rope(np.asarray(q[i:i + 1, h:h + 1], np.float64), p[-1:], rope_base)[0, 0]
            kk = rope(np.asarray(k[idx][:, kvh[h]:kvh[h] + 1], np.float64), p, rope_base)[:, 0]
            vv = np.asarray(v[idx][:, kvh[h]], np.float64)
            s = kk @ qi * scale
            mx = s.max()
            e = np.exp(s - mx)
            o[ri, hi] = e @ vv / e.sum()
            lse[hi, ri] = mx + np.log(e.sum())
    return o, lse


def _row_path(plan, i):
    b = int(plan.node_of[i])
    return np.concatenate([np.arange(plan.node_start[a], plan.node_start[a] + plan.seg_len[a])
                           for a in plan.anc[b][:-1]] + [np.arange(plan.node_start[b], i + 1)]).astype(np.int64)


def rows_attention_grads(plan, q, k, v, dO, rows, keys, scale=None, rope_base=0.0):
    """Gradients of selected rows and keys only, from the definitions of the
    dense backward (dP = dO V^T, D = rowsum(dO * O), dS = P (dP - D),
    dQ = dS K s, dK = dS^T Q s, dV = P^T dO) restricted to what each output
    needs: dq of query row i over i's own path; dk, dv of key j over every
    query that reads j (the rows [j, sub_end(j)) of the packed order, each
    with its own full-path softmax), all query heads of j's KV group summed.
    For spot checks at sizes where whole-tree oracles are too slow.
    Returns dq [len(rows), Hq, d], dk [len(keys), Hkv, d], dv [len(keys), Hkv, d]."""
    q = np.asarray(q)
    N, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    cache = {}

    def row(i, h):
        """Everything of query row i, head h: path, rotated keys, P, D."""
        if (i, h) in cache:
            return cache[(i, h)]
        idx = _row_path(plan, i)
        p = np.arange(len(idx))
        g = h // G
        qi = rope(np.asarray(q[i:i + 1, h:h + 1], np.float64), p[-1:], rope_base)[0, 0]
        kk = rope(np.asarray(k[idx][:, g:g + 1], np.float64), p, rope_base)[:, 0]
        vv = np.asarray(v[idx][:, g], np.float64)
        s = kk @ qi * scale
        P = np.exp(s - s.max())
        P /= P.sum()
        o = P @ vv
        do = np.asarray(dO[i, h], np.float64)
        D = float(do @ o)
        dS = P * (vv @ do - D)
        cache[(i, h)] = (idx, qi, kk, P, dS, do)
        return cache[(i, h)]

    dq = np.zeros((len(rows), Hq, d))
    for ri, i in enumerate(rows):
        for h in range(Hq):
            idx, qi, kk, P, dS, do = row(i, h)
            g_rot = dS @ kk * scale                       # gradient w.r.t. the rotated q_i
            dq[ri, h] = rope_transpose(g_rot[None, None, :], np.array([plan.pos[i]]), rope_base)[0, 0]
    dk = np.zeros((len(keys), Hkv, d))
    dv = np.zeros((len(keys), Hkv, d))
    for kj, j in enumerate(keys):
        for i in range(int(j), int(plan.sub_end[j])):
            for h in range(Hq):
                idx, qi, kk, P, dS, do = row(i, h)
                at = int(np.flatnonzero(idx == j)[0])
                g = h // G
                dk[kj, g] += dS[at] * qi * scale
                dv[kj, g] += P[at] * do
        dk[kj] = rope_transpose(dk[kj][None], np.array([plan.pos[j]]), rope_base)[0]
    return dq, dk, dv


def causal_sequence_grads(q, k, v, dO, rows, keys, scale=None, rope_base=0.0, block=1024):
    """Gradients of selected query rows and keys of ONE causal sequence (a
    single root-to-leaf path, or one item of a varlen forest) with positions
    0..L-1, from the dense backward's definitions (dP = dO V^T,
    D = rowsum(dO * O), dS = P (dP - D), dQ = dS K s, dK = dS^T Q s,
    dV = P^T dO).  A key early in a long sequence is read by thousands of
    rows, each needing its own whole-row softmax; the rows are therefore taken
    a block at a time (each row's softmax, O and D still formed over its full
    row of keys), and only the selected columns of dS and P are kept.
    Products and exponentials run as torch float64 CPU ops.
    q, dO [L, Hq, d]; k, v [L, Hkv, d]; rows, keys: indices into 0..L-1.
    Returns dq [len(rows), Hq, d], dk [len(keys), Hkv, d], dv [len(keys), Hkv, d]."""
    import torch
    q = np.asarray(q, np.float64)
    L, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if not scale else float(scale)
    pos = np.arange(L)
    rows = np.asarray(rows, np.int64)
    keys = np.asarray(keys, np.int64)
    qr = torch.from_numpy(rope(q, pos, rope_base))
    kr = torch.from_numpy(rope(np.asarray(k, np.float64), pos, rope_base))
    vv = torch.from_numpy(np.asarray(v, np.float64))
    do = torch.from_numpy(np.asarray(dO, np.float64))
    kidx = torch.from_numpy(keys)
    dq_rot = torch.zeros(len(rows), Hq, d, dtype=torch.float64)
    dk_rot = torch.zeros(len(keys), Hkv, d, dtype=torch.float64)
    dv = torch.zeros(len(keys), Hkv, d, dtype=torch.float64)
    for r0 in range(0, L, block):
        r1 = min(L, r0 + block)
        causal = torch.arange(r1)[None, :] <= torch.arange(r0, r1)[:, None]          # [rows, keys]
        sel_rows = [(ri, int(i) - r0) for ri, i in enumerate(rows) if r0 <= i < r1]
        for h in range(Hq):
            g = h // G
            S = (qr[r0:r1, h] @ kr[:r1, g].T) * scale
            S = S.masked_fill(~causal, float("-inf"))
            P = torch.exp(S - S.max(dim=1, keepdim=True).values)
            P /= P.sum(dim=1, keepdim=True)
            O = P @ vv[:r1, g]
            Drow = (do[r0:r1, h] * O).sum(dim=1)                                     # [rows]
            seen = torch.nonzero(kidx < r1).flatten()                                 # keys these rows can read
            if len(seen):
                kj = kidx[seen]
                Pk = P[:, kj]                                                        # [rows, keys]
                dSk = Pk * (do[r0:r1, h] @ vv[kj, g].T - Drow[:, None])
                dk_rot[seen, g] += (dSk.T @ qr[r0:r1, h]) * scale
                dv[seen, g] += Pk.T @ do[r0:r1, h]
            for ri, li in sel_rows:
                dS = P[li] * (vv[:r1, g] @ do[r0 + li, h] - Drow[li])
                dq_rot[ri, h] = (dS @ kr[:r1, g]) * scale
    dq = rope_transpose(dq_rot.numpy(), pos[rows], rope_base)
    dk = rope_transpose(dk_rot.numpy(), pos[keys], rope_base)
    return dq, dk, dv.numpy()
