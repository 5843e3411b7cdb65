// Redundancy-free tree partitioning (Tree Training post, section 8): a tree
// whose unique tokens exceed one device's capacity is cut along node
// boundaries into connected subtrees (8.3), so the partition dependency graph
// is again a tree and every token belongs to exactly one partition (8.1: the
// unique work stays N).  A child partition reads the K/V of its root's
// ancestor chain from the partitions above it instead of recomputing them
// (8.2, the gateway), which tree_plan_ex expresses as a key-only prefix.
//
// The cut rule is this library's (the post fixes only the constraints): a
// post-order pass keeps, at every node, its own tokens plus the still-open
// subtrees of its children; while that exceeds the capacity, the largest
// open child (ties: smaller id) is cut off as a partition of its own.
#include <algorithm>
#include <new>
#include <vector>

#include "tree_attn.h"

#include "partition_internal.h"
#include "plan_internal.h"

namespace {

ta_status build_partition(const int32_t* parent, const int32_t* seg_len, int32_t n, int64_t cap, ta_partition* P) {
  P->n_nodes = n;
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
  // preorder (children in ascending id), packed token starts
  std::vector<int32_t> order, node_start(n, 0), stack;
  order.reserve(n);
  for (auto it = roots.rbegin(); it != roots.rend(); ++it) stack.push_back(*it);
  int64_t cursor = 0;
  while (!stack.empty()) {
    const int32_t v = stack.back();
    stack.pop_back();
    order.push_back(v);
    node_start[v] = static_cast<int32_t>(cursor);
    cursor += seg_len[v];
    if (cursor > INT32_MAX) return TA_ERANGE;
    for (int32_t c = child_ptr[v + 1] - 1; c >= child_ptr[v]; --c) stack.push_back(child[c]);
  }
  if (static_cast<int32_t>(order.size()) != n) return TA_ECYCLE;

  // post-order cut
  std::vector<int64_t> open(n, 0);
  std::vector<char> is_root(n, 0);
  std::vector<int32_t> kids;
  for (int32_t r = n - 1; r >= 0; --r) {
    const int32_t v = order[r];
    int64_t tot = seg_len[v];
    kids.clear();
    for (int32_t c = child_ptr[v]; c < child_ptr[v + 1]; ++c) {
      tot += open[child[c]];
      kids.push_back(child[c]);
    }
    if (tot > cap) {
      std::sort(kids.begin(), kids.end(), [&](int32_t a, int32_t b) {
        return open[a] != open[b] ? open[a] > open[b] : a < b;
      });
      for (int32_t c : kids) {
        if (tot <= cap) break;
        is_root[c] = 1;
        tot -= open[c];
      }
    }
    open[v] = tot;
    if (parent[v] < 0) is_root[v] = 1;
  }

  // partitions numbered in preorder of their roots (parents first)
  P->part_of.assign(n, -1);
  for (int32_t v : order) {
    if (is_root[v]) {
      P->part_of[v] = P->n_parts++;
      P->part_root.push_back(v);
    } else {
      P->part_of[v] = P->part_of[parent[v]];
    }
  }
  const int32_t np = P->n_parts;
  P->part_parent.resize(np);
  P->n_prefix.resize(np);
  P->own_tokens.assign(np, 0);
  for (int32_t v = 0; v < n; ++v) P->own_tokens[P->part_of[v]] += seg_len[v];
  // own nodes of each partition in ascending id, and in preorder
  std::vector<std::vector<int32_t>> own(np), own_pre(np);
  for (int32_t v = 0; v < n; ++v) own[P->part_of[v]].push_back(v);
  for (int32_t v : order) own_pre[P->part_of[v]].push_back(v);

  std::vector<int32_t> lid(n, -1), chain;
  P->local_ptr.assign(np + 1, 0);
  P->tok_ptr.assign(np + 1, 0);
  for (int32_t p = 0; p < np; ++p) {
    const int32_t root = P->part_root[p];
    P->part_parent[p] = parent[root] < 0 ? -1 : P->part_of[parent[root]];
    chain.clear();
    for (int32_t a = parent[root]; a >= 0; a = parent[a]) chain.push_back(a);
    std::reverse(chain.begin(), chain.end());
    const int32_t nc = static_cast<int32_t>(chain.size());
    P->n_prefix[p] = nc;
    int32_t k = 0;
    for (int32_t a : chain) {
      lid[a] = k;
      P->local_node.push_back(a);
      P->local_parent.push_back(k - 1);
      P->local_len.push_back(seg_len[a]);
      ++k;
    }
    for (int32_t v : own[p]) lid[v] = k++;
    for (int32_t v : own[p]) {
      P->local_node.push_back(v);
      P->local_parent.push_back(v == root ? nc - 1 : lid[parent[v]]);
      P->local_len.push_back(seg_len[v]);
    }
    P->local_ptr[p + 1] = static_cast<int32_t>(P->local_node.size());
    // local tokens in the local plan's order: the chain, then the own nodes in
    // preorder (ascending local ids keep the siblings' order)
    for (int32_t a : chain)
      for (int32_t j = 0; j < seg_len[a]; ++j) P->tok_idx.push_back(node_start[a] + j);
    for (int32_t v : own_pre[p])
      for (int32_t j = 0; j < seg_len[v]; ++j) P->tok_idx.push_back(node_start[v] + j);
    if (P->tok_idx.size() > size_t(INT32_MAX)) return TA_ERANGE;
    P->tok_ptr[p + 1] = static_cast<int32_t>(P->tok_idx.size());
    for (int32_t a : chain) lid[a] = -1;
    for (int32_t v : own[p]) lid[v] = -1;
  }
  P->n_tokens = cursor;
  P->naive_tokens = static_cast<int64_t>(P->tok_idx.size());
  return TA_OK;
}

// Local plans (tree_plan_ex with the chain as key-only prefix) and the layout
// of the device image: per partition its plan tables, then its row map.
ta_status build_local_plans(ta_partition* P, int32_t block_m, int32_t block_n) {
  const int32_t np = P->n_parts;
  P->plans.assign(np, nullptr);
  P->off_plan.assign(np, 0);
  P->off_idx.assign(np, 0);
  size_t off = 0;
  for (int32_t p = 0; p < np; ++p) {
    const int32_t l0 = P->local_ptr[p], nl = P->local_ptr[p + 1] - l0;
    const int32_t rows = P->tok_ptr[p + 1] - P->tok_ptr[p];
    P->max_local = std::max(P->max_local, rows);
    if (P->own_tokens[p] == 0) continue;  // nothing to compute: no plan
    ta_status st = tree_plan_ex(P->local_parent.data() + l0, P->local_len.data() + l0, nl, P->n_prefix[p],
                                block_m, block_n, &P->plans[p]);
    if (st != TA_OK) return st;
    P->off_plan[p] = off;
    off += (P->plans[p]->device_bytes + 255) & ~size_t(255);
    P->off_idx[p] = off;
    off += (size_t(rows) * sizeof(int32_t) + 255) & ~size_t(255);
  }
  P->device_bytes = off;
  return TA_OK;
}

}  // namespace

extern "C" ta_status tree_partition(const int32_t* parent, const int32_t* seg_len, int32_t n_nodes,
                                    int64_t capacity, int32_t block_m, int32_t block_n, ta_partition** out) {
  if (!out) return TA_EINVAL;
  *out = nullptr;
  if (!parent || !seg_len || n_nodes <= 0 || capacity < 1) return TA_EINVAL;
  for (int32_t i = 0; i < n_nodes; ++i) {
    if (seg_len[i] < 0 || seg_len[i] > capacity || parent[i] < -1 || parent[i] >= n_nodes) return TA_EINVAL;
    if (parent[i] == i) return TA_ECYCLE;
  }
  ta_partition* P = new (std::nothrow) ta_partition();
  if (!P) return TA_ENOMEM;
  ta_status st;
  try {
    st = build_partition(parent, seg_len, n_nodes, capacity, P);
    if (st == TA_OK) st = build_local_plans(P, block_m, block_n);
  } catch (const std::bad_alloc&) {
    st = TA_ENOMEM;
  }
  if (st != TA_OK) {
    delete P;
    return st;
  }
  *out = P;
  return TA_OK;
}

extern "C" ta_status tree_partition_view(const ta_partition* P, ta_partition_view* v) {
  if (!P || !v) return TA_EINVAL;
  v->n_nodes = P->n_nodes;
  v->n_parts = P->n_parts;
  v->max_local_tokens = P->max_local;
  v->reserved = 0;
  v->n_tokens = P->n_tokens;
  v->naive_tokens = P->naive_tokens;
  v->part_of = P->part_of.data();
  v->part_root = P->part_root.data();
  v->part_parent = P->part_parent.data();
  v->n_prefix = P->n_prefix.data();
  v->own_tokens = P->own_tokens.data();
  v->local_ptr = P->local_ptr.data();
  v->local_node = P->local_node.data();
  v->local_parent = P->local_parent.data();
  v->local_len = P->local_len.data();
  v->tok_ptr = P->tok_ptr.data();
  v->tok_idx = P->tok_idx.data();
  return TA_OK;
}

extern "C" ta_status tree_partition_plan(const ta_partition* P, int32_t i, const ta_plan** plan) {
  if (!P || !plan || i < 0 || i >= P->n_parts) return TA_EINVAL;
  *plan = P->plans[i];
  return TA_OK;
}

extern "C" ta_status tree_partition_device_bytes(const ta_partition* P, size_t* bytes) {
  if (!P || !bytes) return TA_EINVAL;
  *bytes = P->device_bytes;
  return TA_OK;
}

extern "C" void tree_partition_free(ta_partition* P) { delete P; }
