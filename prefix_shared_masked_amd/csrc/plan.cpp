// Host planner for tree attention over a DFS-packed prefix tree.
//
// Builds, from parent[] and seg_len[], everything the kernels need:
//  - the DFS serialisation (Tree Training post, section 3.2) with children and
//    roots in ascending node id, done with an explicit stack;
//  - depth positions (section 5): a node's first position is its parent's
//    first position plus the parent's length, propagated top-down;
//  - g_t (section 6.2) as the leaf count of node(t)'s subtree, accumulated
//    bottom-up over the reversed visiting order, and K = number of leaves;
//  - the DFS interval [node_start, node_sub_end) of every node (section 4.3);
//  - the forward "ancestor block table" (section 4.3): for each query tile
//    of TA_BLOCK_M rows, the keys some row may read, as node segments packed
//    into gathered chunks of TA_BLOCK_N key slots, flagged when every row
//    reads every key so the kernel can skip the element mask;
//  - the backward key tiles: at most TA_BLOCK_KV keys inside one node, read
//    by the contiguous query range [k0, node_sub_end) (a key's readers are
//    exactly the later tokens of its node's subtree).
// Integer-only and deterministic.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <limits>
#include <new>
#include <numeric>
#include <vector>

#include "tree_attn.h"
#include "plan_internal.h"

namespace {

constexpr int64_t kI32Max = std::numeric_limits<int32_t>::max();

struct Segment {
  int32_t k0, k1, kend;  // keys [k0, k1) of one node; row i reads key j iff j <= i < kend
  bool full;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

ta_status build(const int32_t* parent, const int32_t* seg_len, int32_t n, int32_t n_prefix, ta_plan* p) {
  p->n_nodes = n;
  p->n_prefix_nodes = n_prefix;
  p->block_m = TA_BLOCK_M;
  p->block_n = TA_BLOCK_N;
  p->block_kv = TA_BLOCK_KV;

  // children in ascending id via a counting sort on the parent
  std::vector<int32_t> child_ptr(n + 1, 0), child(n), roots;
  for (int32_t i = 0; i < n; ++i) {
    if (parent[i] < 0) roots.push_back(i);
    else child_ptr[parent[i] + 1]++;
  }
  for (int32_t i = 0; i < n; ++i) child_ptr[i + 1] += child_ptr[i];
  {
    std::vector<int32_t> fill(child_ptr.begin(), child_ptr.end() - 1);
    for (int32_t i = 0; i < n; ++i)
      if (parent[i] >= 0) child[fill[parent[i]]++] = i;
  }

  // preorder with an explicit stack: pushing in reverse pops in ascending id
  p->dfs_order.reserve(n);
  p->node_start.assign(n, 0);
  std::vector<int64_t> pos0(n, 0);
  std::vector<int32_t> stack;
  stack.reserve(n);
  for (auto it = roots.rbegin(); it != roots.rend(); ++it) stack.push_back(*it);
  int64_t cursor = 0;
  while (!stack.empty()) {
    int32_t node = stack.back();
    stack.pop_back();
    p->dfs_order.push_back(node);
    p->node_start[node] = static_cast<int32_t>(cursor);
    pos0[node] = parent[node] < 0 ? 0 : pos0[parent[node]] + seg_len[parent[node]];
    cursor += seg_len[node];
    if (cursor > kI32Max) return TA_ERANGE;
    for (int32_t c = child_ptr[node + 1] - 1; c >= child_ptr[node]; --c) stack.push_back(child[c]);
  }
  if (static_cast<int32_t>(p->dfs_order.size()) != n) return TA_ECYCLE;
  const int32_t N = static_cast<int32_t>(cursor);
  p->n_tokens = N;

  // Key-only prefix: nodes 0..n_prefix-1 form a chain from the only root (node
  // i's parent is i - 1, and each has exactly one child, the next chain node
  // or, for the last one, the root of everything else).  The chain is then
  // visited first, so its tokens are [0, q_start).
  if (n_prefix > 0) {
    if (roots.size() != 1 || roots[0] != 0) return TA_EINVAL;
    for (int32_t i = 0; i < n_prefix; ++i) {
      if (i > 0 && parent[i] != i - 1) return TA_EINVAL;
      if (i + 1 < n_prefix && (child_ptr[i + 1] - child_ptr[i] != 1 || child[child_ptr[i]] != i + 1))
        return TA_EINVAL;
      if (i + 1 == n_prefix && child_ptr[i + 1] - child_ptr[i] > 1) return TA_EINVAL;
    }
    p->q_start = p->node_start[n_prefix - 1] + seg_len[n_prefix - 1];
    if (p->q_start == N) return TA_EINVAL;  // the nodes below the chain hold no token
  }
  const int32_t Q0 = p->q_start;

  // bottom-up: subtree token counts and leaf counts
  std::vector<int64_t> sub_tok(n, 0), leaves(n, 0);
  for (int32_t r = n - 1; r >= 0; --r) {
    int32_t node = p->dfs_order[r];
    sub_tok[node] += seg_len[node];
    if (child_ptr[node + 1] == child_ptr[node]) leaves[node] = 1;
    if (parent[node] >= 0) {
      sub_tok[parent[node]] += sub_tok[node];
      leaves[parent[node]] += leaves[node];
    }
  }
  p->node_sub_end.assign(n, 0);
  int64_t K = 0;
  for (int32_t i = 0; i < n; ++i) {
    p->node_sub_end[i] = static_cast<int32_t>(p->node_start[i] + sub_tok[i]);
    if (parent[i] < 0) K += leaves[i];
  }
  p->n_leaves = static_cast<int32_t>(K);

  // per-token arrays
  p->pos.resize(N);
  p->g.resize(N);
  p->node_of.resize(N);
  p->sub_end.resize(N);
  int64_t n_flat = 0, pairs = 0, max_pos = -1;
  for (int32_t node : p->dfs_order) {
    int32_t s = p->node_start[node];
    for (int32_t j = 0; j < seg_len[node]; ++j) {
      int64_t ps = pos0[node] + j;
      p->pos[s + j] = static_cast<int32_t>(ps);
      p->g[s + j] = static_cast<int32_t>(leaves[node]);
      p->node_of[s + j] = node;
      p->sub_end[s + j] = p->node_sub_end[node];
      n_flat += leaves[node];
      if (s + j >= Q0) pairs += ps + 1;  // pairs whose query is a real (non-prefix) row
      max_pos = std::max(max_pos, ps);
    }
  }
  p->n_flat = n_flat;
  p->visible_pairs = pairs;
  p->max_pos = static_cast<int32_t>(max_pos);

  // ancestor-or-self chains, root first (depth = chain length)
  std::vector<int32_t> depth(n, 0);
  for (int32_t node : p->dfs_order) depth[node] = parent[node] < 0 ? 1 : depth[parent[node]] + 1;
  p->anc_ptr.assign(n + 1, 0);
  for (int32_t i = 0; i < n; ++i) {
    int64_t next = int64_t(p->anc_ptr[i]) + depth[i];
    if (next > kI32Max) return TA_ERANGE;
    p->anc_ptr[i + 1] = static_cast<int32_t>(next);
  }
  p->anc.resize(p->anc_ptr[n]);
  for (int32_t i = 0; i < n; ++i) {
    int32_t w = p->anc_ptr[i + 1];
    for (int32_t a = i; a >= 0; a = parent[a]) p->anc[--w] = a;
  }

  // forward tiles: union of visible node segments, packed into key chunks
  const int32_t BM = p->block_m, BN = p->block_n;
  const int32_t n_qt = (N - Q0 + BM - 1) / BM;  // query tiles cover rows [q_start, N)
  p->n_qtiles = n_qt;
  p->fq_ptr.assign(n_qt + 1, 0);
  std::vector<int32_t> stamp(n, -1);
  std::vector<Segment> segs;
  int64_t comp_fwd = 0;
  for (int32_t t = 0; t < n_qt; ++t) {
    const int32_t q0 = Q0 + t * BM, q1 = std::min(N, q0 + BM);
    segs.clear();
    for (int32_t i = q0; i < q1;) {
      const int32_t b = p->node_of[i];
      const int32_t b_end = p->node_start[b] + seg_len[b];
      const int32_t last = std::min(b_end, q1);  // rows [i, last) belong to b
      for (int32_t a = b; a >= 0 && stamp[a] != t; a = parent[a]) {
        stamp[a] = t;
        const int32_t k0 = p->node_start[a];
        const int32_t k1 = (a == b) ? last : k0 + seg_len[a];
        if (k1 > k0) {
          // keys <= q0 of a node whose DFS interval holds every row of the tile
          // are read by every row; the rest needs the element mask
          const int32_t kend = p->node_sub_end[a];
          const int32_t split = (q1 <= kend) ? std::min(k1, q0 + 1) : k0;
          if (split > k0) segs.push_back({k0, split, kend, true});
          if (k1 > split) segs.push_back({std::max(k0, split), k1, kend, false});
        }
      }
      i = last;
    }
    std::sort(segs.begin(), segs.end(), [](const Segment& x, const Segment& y) { return x.k0 < y.k0; });

    int32_t ch[TA_CHUNK_INTS];
    int32_t nseg = 0, nkeys = 0;
    bool full = true;
    auto reset = [&]() {
      nseg = 0;
      nkeys = 0;
      full = true;
      for (int s = 0; s < TA_CHUNK_MAX_SEG; ++s) {
        ch[4 + s] = 0;
        ch[8 + s] = BN;
        ch[12 + s] = 0;
      }
    };
    auto flush = [&]() {
      if (nkeys == 0) return;
      ch[0] = nseg;
      ch[1] = nkeys;
      ch[2] = (full && nkeys == BN) ? 1 : 0;
      ch[3] = 0;
      if (nseg < TA_CHUNK_MAX_SEG) {
        for (int s = nseg; s < TA_CHUNK_MAX_SEG; ++s) ch[4 + s] = ch[4];
      }
      p->fq_chunk.insert(p->fq_chunk.end(), ch, ch + TA_CHUNK_INTS);
      comp_fwd += int64_t(q1 - q0) * BN;
      reset();
    };
    reset();
    for (const Segment& sg : segs) {
      int32_t k = sg.k0;
      while (k < sg.k1) {
        if (nkeys == BN || nseg == TA_CHUNK_MAX_SEG) flush();
        const int32_t take = std::min(sg.k1 - k, BN - nkeys);
        ch[4 + nseg] = k;
        ch[8 + nseg] = nkeys;
        ch[12 + nseg] = sg.kend;
        full = full && sg.full;
        ++nseg;
        nkeys += take;
        k += take;
      }
    }
    flush();
    const int64_t nch = int64_t(p->fq_chunk.size()) / TA_CHUNK_INTS;
    if (nch * TA_CHUNK_INTS > kI32Max) return TA_ERANGE;
    p->fq_ptr[t + 1] = static_cast<int32_t>(nch);
  }
  p->n_chunks = p->fq_ptr[n_qt];
  p->computed_pairs_fwd = comp_fwd;

  // longest chunk lists first (stable), so the tail of the grid is short work
  p->fq_order.resize(n_qt);
  std::iota(p->fq_order.begin(), p->fq_order.end(), 0);
  std::stable_sort(p->fq_order.begin(), p->fq_order.end(), [&](int32_t x, int32_t y) {
    return (p->fq_ptr[x + 1] - p->fq_ptr[x]) > (p->fq_ptr[y + 1] - p->fq_ptr[y]);
  });

  // backward key tiles, most work first.  A tile holds up to TA_BLOCK_KV keys
  // of one node; its queries are the rows [max(k0, q_start), q_end) (the key-
  // only prefix has no query rows); the kernel runs 32-key sub-tiles against
  // 32-row query blocks.
  const int32_t BK = p->block_kv, SUB = TA_KV_SUB;
  struct KT {
    int32_t k0, klen, qe, node;
    int64_t work;
  };
  std::vector<KT> kts;
  int64_t comp_bwd = 0;
  for (int32_t node : p->dfs_order) {
    const int32_t s = p->node_start[node], e = s + seg_len[node], qe = p->node_sub_end[node];
    for (int32_t k0 = s; k0 < e; k0 += BK) {
      const int32_t kl = std::min(BK, e - k0), qs = std::max(k0, Q0);
      // every tile has a query row: its own first key, or (a chain key) the
      // rows below the chain, whose DFS interval it spans; the dK/dV kernel
      // relies on it
      if (qe <= qs) return TA_EINVAL;
      const int64_t nblk = (int64_t(std::max(qe - qs, 0)) + SUB - 1) / SUB;
      int64_t blocks = 0;
      for (int32_t sub = 0; sub * SUB < kl; ++sub) blocks += std::max<int64_t>(nblk - (qs == k0 ? sub : 0), 0);
      kts.push_back({k0, kl, qe, node, blocks});
      comp_bwd += blocks * SUB * SUB;
    }
  }
  std::stable_sort(kts.begin(), kts.end(), [](const KT& x, const KT& y) { return x.work > y.work; });
  if (int64_t(kts.size()) * 4 > kI32Max) return TA_ERANGE;
  p->n_ktiles = static_cast<int32_t>(kts.size());
  p->bk.resize(kts.size() * 4);
  for (size_t i = 0; i < kts.size(); ++i) {
    p->bk[4 * i + 0] = kts[i].k0;
    p->bk[4 * i + 1] = kts[i].klen;
    p->bk[4 * i + 2] = kts[i].qe;
    p->bk[4 * i + 3] = kts[i].node;
  }
  p->computed_pairs_bwd = comp_bwd;

  // dK/dV work pieces.  A dK/dV workgroup works four sub-tiles (a pair of
  // wavefronts each), each owning the dK/dV of up to 32 keys of one node
  // over a common run of
  // 32-row query blocks [q_lo, q_hi) staged once in LDS; blocks lie on the
  // query-tile grid q_start + 32t, so each (block, sub-tile) is one dS block
  // the dQ pass reads back.  Two things make whole tiles a poor unit: the
  // root's keys are read by every query, so one workgroup can carry far more
  // than an average CU's share, and a node shorter than 128 keys leaves
  // wavefronts idle (the 96-token history nodes of a navigation episode: a
  // quarter of the work).  So a full 128-key tile whose range spans at most
  // `cap` blocks stays one piece; every other tile is split into its 32-key
  // sub-tiles, each cut at the windows of a grid of `cap` blocks anchored at
  // q_start, and the sub-tile runs of one window are packed four to a piece
  // when their row spans nest (a run joins only if the piece's span grows by
  // at most one block over its longest run).  A sub-tile cut over several
  // windows writes fp32 partial dK/dV to one slot per window (consecutive, in
  // window order) that a second pass sums in slot order; one run in one
  // window stores directly.  cap = max(TA_KV_PIECE_MIN, ceil(total blocks /
  // 256)): about 256 CUs' worth for any number of KV heads.  Pieces are listed
  // longest first, then by their last row (the workgroups resident at one
  // time stream the same rows through L2).
  {
    int64_t total = 0;
    std::vector<int32_t> tb(kts.size());
    for (size_t i = 0; i < kts.size(); ++i) {
      tb[i] = (kts[i].qe - std::max(kts[i].k0, Q0) + SUB - 1) / SUB;
      total += tb[i];
    }
    const int32_t cap = static_cast<int32_t>(std::max<int64_t>(TA_KV_PIECE_MIN, (total + 255) / 256));
    const int64_t W = int64_t(SUB) * cap;  // rows per window
    auto grid_floor = [&](int32_t r) { return Q0 + SUB * ((r - Q0) / SUB); };

    // sub-tiles: keys [kw, kw + wk) of one node, query tiles [t_lo, t_hi),
    // dS blocks ds0 .. ds0 + t_hi - t_lo - 1
    struct Sub {
      int32_t kw, wk, qe, t_lo, t_hi;
      int64_t ds0;
    };
    std::vector<Sub> subs;
    std::vector<int32_t> first_sub(kts.size());
    int64_t nds = 0;
    for (size_t i = 0; i < kts.size(); ++i) {
      first_sub[i] = static_cast<int32_t>(subs.size());
      for (int32_t kw = kts[i].k0; kw < kts[i].k0 + kts[i].klen; kw += SUB) {
        Sub x;
        x.kw = kw;
        x.wk = std::min(SUB, kts[i].k0 + kts[i].klen - kw);
        x.qe = kts[i].qe;
        x.t_lo = (std::max(kw, Q0) - Q0) / SUB;
        x.t_hi = (x.qe - Q0 + SUB - 1) / SUB;
        x.ds0 = nds;
        nds += x.t_hi - x.t_lo;
        subs.push_back(x);
      }
    }
    if (nds > kI32Max) return TA_ERANGE;
    p->n_dsblk = nds;

    struct Run {
      int32_t lo, hi, sub, slot, seq;  // rows [lo, hi) of sub-tile `sub`
    };
    struct KP {
      int32_t rec[TA_KPIECE_INTS];
      int32_t blocks, seq;
    };
    auto wave_rec = [&](int32_t* t, const Sub& x, int32_t lo, int32_t hi, int32_t slot) {
      t[0] = x.kw;
      t[1] = x.wk;
      t[2] = lo;
      t[3] = hi;
      t[4] = slot;
      t[5] = static_cast<int32_t>(x.ds0 - x.t_lo);
      t[6] = 0;
    };
    std::vector<KP> kps;
    std::vector<std::vector<Run>> win;  // runs by window
    int32_t slots = 0, seq = 0;
    for (size_t i = 0; i < kts.size(); ++i) {
      const int32_t kl = kts[i].klen, qe = kts[i].qe, qs = std::max(kts[i].k0, Q0);
      if (kl == BK && tb[i] <= cap) {
        KP x{};
        x.rec[0] = grid_floor(qs);
        x.rec[1] = qe;
        for (int w = 0; w < 4; ++w) {
          const Sub& su = subs[first_sub[i] + w];
          wave_rec(x.rec + 4 + TA_KWAVE_INTS * w, su, std::max(su.kw, Q0), qe, -1);
        }
        x.blocks = (qe - x.rec[0] + SUB - 1) / SUB;
        x.seq = seq++;
        kps.push_back(x);
        continue;
      }
      const int32_t sub_end = i + 1 < kts.size() ? first_sub[i + 1] : static_cast<int32_t>(subs.size());
      for (int32_t si = first_sub[i]; si < sub_end; ++si) {
        const Sub& su = subs[si];
        const int32_t lo = std::max(su.kw, Q0);
        const int64_t m0 = (lo - Q0) / W, m1 = (qe - 1 - Q0) / W;
        const int32_t nw = static_cast<int32_t>(m1 - m0 + 1);
        if (nw > 1) p->kr.insert(p->kr.end(), {su.kw, su.wk, slots, nw});
        for (int64_t m = m0; m <= m1; ++m) {
          if (win.size() <= size_t(m)) win.resize(m + 1);
          const int32_t a = static_cast<int32_t>(std::max<int64_t>(lo, Q0 + m * W));
          const int32_t b = static_cast<int32_t>(std::min<int64_t>(qe, Q0 + (m + 1) * W));
          win[m].push_back({a, b, si, nw > 1 ? slots + static_cast<int32_t>(m - m0) : -1, seq++});
        }
        if (nw > 1) slots += nw;
      }
    }
    for (std::vector<Run>& rs : win) {
      std::stable_sort(rs.begin(), rs.end(),
                       [](const Run& x, const Run& y) { return x.lo != y.lo ? x.lo < y.lo : x.hi < y.hi; });
      size_t j = 0;
      while (j < rs.size()) {
        int32_t lo = rs[j].lo, hi = rs[j].hi, longest = hi - lo;
        size_t e = j + 1;
        while (e < rs.size() && e - j < 4) {
          const int32_t l2 = std::min(lo, rs[e].lo), h2 = std::max(hi, rs[e].hi);
          const int32_t m2 = std::max(longest, rs[e].hi - rs[e].lo);
          if (h2 - l2 > m2 + SUB) break;
          lo = l2;
          hi = h2;
          longest = m2;
          ++e;
        }
        KP x{};
        x.rec[0] = grid_floor(lo);
        x.rec[1] = hi;
        for (int w = 0; w < 4; ++w) {
          int32_t* t = x.rec + 4 + TA_KWAVE_INTS * w;
          if (j + w < e) {
            const Run& r = rs[j + w];
            wave_rec(t, subs[r.sub], r.lo, r.hi, r.slot);
          } else {  // idle wavefront: no keys, no rows (its loads read key 0, nothing is stored)
            t[0] = 0;
            t[1] = 0;
            t[2] = x.rec[0];
            t[3] = x.rec[0];
            t[4] = -1;
            t[5] = 0;
            t[6] = 0;
          }
        }
        x.blocks = (hi - x.rec[0] + SUB - 1) / SUB;
        x.seq = rs[j].seq;
        kps.push_back(x);
        j = e;
      }
    }
    std::stable_sort(kps.begin(), kps.end(), [](const KP& x, const KP& y) {
      if (x.blocks != y.blocks) return x.blocks > y.blocks;
      if (x.rec[1] != y.rec[1]) return x.rec[1] > y.rec[1];
      return x.seq < y.seq;
    });
    if (int64_t(kps.size()) * TA_KPIECE_INTS > kI32Max) return TA_ERANGE;
    p->kp.reserve(kps.size() * TA_KPIECE_INTS);
    for (const KP& x : kps) p->kp.insert(p->kp.end(), x.rec, x.rec + TA_KPIECE_INTS);
    p->n_kpieces = static_cast<int32_t>(kps.size());
    p->n_ksplit = static_cast<int32_t>(p->kr.size() / 4);
    p->n_kslots = slots;
    p->kv_piece_cap = cap;

    // dQ lists: per query tile, the sub-tiles some of its rows read, by first
    // key, each with its dS block (kw, wk, block, 0); tiles with the most
    // entries first
    std::vector<int32_t> cnt(n_qt + 1, 0);
    for (const Sub& x : subs)
      for (int32_t t = x.t_lo; t < x.t_hi; ++t) ++cnt[t + 1];
    p->dq_ptr.assign(n_qt + 1, 0);
    for (int32_t t = 0; t < n_qt; ++t) p->dq_ptr[t + 1] = p->dq_ptr[t] + cnt[t + 1];
    if (int64_t(p->dq_ptr[n_qt]) * 4 > kI32Max) return TA_ERANGE;
    std::vector<int32_t> order(subs.size());
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) { return subs[x].kw < subs[y].kw; });
    std::vector<int32_t> fill(p->dq_ptr.begin(), p->dq_ptr.end() - 1);
    p->dq_ent.assign(size_t(p->dq_ptr[n_qt]) * 4, 0);
    for (int32_t si : order) {
      const Sub& x = subs[si];
      for (int32_t t = x.t_lo; t < x.t_hi; ++t) {
        int32_t* e = p->dq_ent.data() + size_t(fill[t]++) * 4;
        e[0] = x.kw;
        e[1] = x.wk;
        e[2] = static_cast<int32_t>(x.ds0 + t - x.t_lo);
      }
    }
    p->dq_order.resize(n_qt);
    std::iota(p->dq_order.begin(), p->dq_order.end(), 0);
    std::stable_sort(p->dq_order.begin(), p->dq_order.end(), [&](int32_t x, int32_t y) {
      return (p->dq_ptr[x + 1] - p->dq_ptr[x]) > (p->dq_ptr[y + 1] - p->dq_ptr[y]);
    });
  }

  // device image: pos | fq_ptr | fq_chunk | fq_order | bk | kp | kr | dq_ptr | dq_ent | dq_order,
  // each 256-aligned
  size_t off = 0;
  p->off_pos = off;
  off = align256(off + sizeof(int32_t) * size_t(std::max(N, 1)));
  p->off_fq_ptr = off;
  off = align256(off + sizeof(int32_t) * p->fq_ptr.size());
  p->off_fq_chunk = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->fq_chunk.size(), 1));
  p->off_fq_order = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->fq_order.size(), 1));
  p->off_bk = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->bk.size(), 1));
  p->off_kp = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->kp.size(), 1));
  p->off_kr = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->kr.size(), 1));
  p->off_dq_ptr = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->dq_ptr.size(), 1));
  p->off_dq_ent = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->dq_ent.size(), 1));
  p->off_dq_order = off;
  off = align256(off + sizeof(int32_t) * std::max<size_t>(p->dq_order.size(), 1));
  p->device_bytes = off;
  return TA_OK;
}

}  // namespace

extern "C" ta_status tree_plan(const int32_t* parent, const int32_t* seg_len, int32_t n_nodes,
                               int32_t block_m, int32_t block_n, ta_plan** out) {
  return tree_plan_ex(parent, seg_len, n_nodes, 0, block_m, block_n, out);
}

extern "C" ta_status tree_plan_ex(const int32_t* parent, const int32_t* seg_len, int32_t n_nodes,
                                  int32_t n_prefix_nodes, int32_t block_m, int32_t block_n, ta_plan** out) {
  if (!out) return TA_EINVAL;
  *out = nullptr;
  if (!parent || !seg_len || n_nodes <= 0 || n_prefix_nodes < 0 || n_prefix_nodes > n_nodes) return TA_EINVAL;
  if ((block_m != 0 && block_m != TA_BLOCK_M) || (block_n != 0 && block_n != TA_BLOCK_N))
    return TA_EUNSUPPORTED;
  for (int32_t i = 0; i < n_nodes; ++i) {
    if (seg_len[i] < 0 || parent[i] < -1 || parent[i] >= n_nodes) return TA_EINVAL;
    if (parent[i] == i) return TA_ECYCLE;
  }
  ta_plan* p = new (std::nothrow) ta_plan();
  if (!p) return TA_ENOMEM;
  ta_status st;
  try {
    st = build(parent, seg_len, n_nodes, n_prefix_nodes, p);
  } catch (const std::bad_alloc&) {
    st = TA_ENOMEM;
  }
  if (st != TA_OK) {
    delete p;
    return st;
  }
  *out = p;
  return TA_OK;
}

extern "C" ta_status tree_plan_view(const ta_plan* p, ta_plan_view* v) {
  if (!p || !v) return TA_EINVAL;
  std::memset(v, 0, sizeof(*v));
  v->n_nodes = p->n_nodes;
  v->n_tokens = p->n_tokens;
  v->n_leaves = p->n_leaves;
  v->max_pos = p->max_pos;
  v->block_m = p->block_m;
  v->block_n = p->block_n;
  v->block_kv = p->block_kv;
  v->n_qtiles = p->n_qtiles;
  v->n_chunks = p->n_chunks;
  v->n_ktiles = p->n_ktiles;
  v->n_flat = p->n_flat;
  v->visible_pairs = p->visible_pairs;
  v->computed_pairs_fwd = p->computed_pairs_fwd;
  v->computed_pairs_bwd = p->computed_pairs_bwd;
  v->dfs_order = p->dfs_order.data();
  v->node_start = p->node_start.data();
  v->node_sub_end = p->node_sub_end.data();
  v->pos = p->pos.data();
  v->g = p->g.data();
  v->node_of = p->node_of.data();
  v->sub_end = p->sub_end.data();
  v->anc_ptr = p->anc_ptr.data();
  v->anc = p->anc.data();
  v->fq_ptr = p->fq_ptr.data();
  v->fq_chunk = p->fq_chunk.data();
  v->fq_order = p->fq_order.data();
  v->bk = p->bk.data();
  v->n_prefix_nodes = p->n_prefix_nodes;
  v->q_start = p->q_start;
  v->n_kpieces = p->n_kpieces;
  v->n_ksplit = p->n_ksplit;
  v->n_kslots = p->n_kslots;
  v->kv_piece_cap = p->kv_piece_cap;
  v->kp = p->kp.data();
  v->kr = p->kr.data();
  v->n_dsblk = p->n_dsblk;
  v->dq_ptr = p->dq_ptr.data();
  v->dq_ent = p->dq_ent.data();
  v->dq_order = p->dq_order.data();
  return TA_OK;
}

extern "C" ta_status tree_plan_device_bytes(const ta_plan* p, size_t* bytes) {
  if (!p || !bytes) return TA_EINVAL;
  *bytes = p->device_bytes;
  return TA_OK;
}

extern "C" void tree_plan_free(ta_plan* p) { delete p; }

extern "C" const char* ta_status_string(ta_status s) {
  switch (s) {
    case TA_OK: return "ok";
    case TA_EINVAL: return "invalid argument";
    case TA_ECYCLE: return "parent pointers contain a cycle";
    case TA_ERANGE: return "size exceeds the int32 index range";
    case TA_ENOMEM: return "out of memory or buffer too small";
    case TA_EUNSUPPORTED: return "unsupported configuration";
    case TA_EHIP: return "HIP error";
  }
  return "unknown status";
}
