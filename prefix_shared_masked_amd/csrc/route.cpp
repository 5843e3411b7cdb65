// Routing tables for recurrent layers over a DFS-packed tree (Tree Training
// post, section 9): which state a chunk starts from (9.1: its parent's end
// state, not its packed predecessor's) and which tokens a causal convolution
// reads as left context (9.2: the parent's last K - 1 tokens, continuing up
// the path when the parent is shorter).
#include <algorithm>
#include <new>

#include "plan_internal.h"
#include "route_internal.h"
#include "tree_attn.h"

namespace {

constexpr int32_t kChunk = 128;  // tokens per scan chunk (256: 10% slower scans on the spine tree, 64: the walk dominates)

ta_status build_route(const ta_plan* p, int32_t K, ta_route* R) {
  const int32_t n = p->n_nodes, N = p->n_tokens;
  R->n_tokens = N;
  R->chunk = kChunk;
  R->conv_k = K;
  // parent of each node from its ancestor chain (root .. self)
  std::vector<int32_t> parent(n, -1), seg(n);
  for (int32_t v = 0; v < n; ++v) {
    const int32_t a0 = p->anc_ptr[v], a1 = p->anc_ptr[v + 1];
    parent[v] = a1 - a0 >= 2 ? p->anc[a1 - 2] : -1;
  }
  // seg_len from the DFS layout: node_sub_end is the end of the subtree; the
  // node's own tokens are those whose node_of is v
  std::fill(seg.begin(), seg.end(), 0);
  for (int32_t t = 0; t < N; ++t) seg[p->node_of[t]]++;
  // last chunk and last token of each node (for its children), resolved
  // through zero-length ancestors
  std::vector<int32_t> last_chunk(n, -1), last_tok(n, -1);
  for (int32_t v : p->dfs_order) {
    int32_t pc = -1, pt = -1;
    if (parent[v] >= 0) {
      pc = last_chunk[parent[v]];
      pt = last_tok[parent[v]];
    }
    const int32_t s = p->node_start[v], L = seg[v];
    for (int32_t o = 0; o < L; o += kChunk) {
      const int32_t len = std::min(kChunk, L - o);
      R->chunks.insert(R->chunks.end(), {s + o, len, pc, pt});
      pc = static_cast<int32_t>(R->chunks.size() / 4) - 1;
      pt = s + o + len - 1;
    }
    last_chunk[v] = pc;  // the node's own last chunk, or its parent's when it holds no token
    last_tok[v] = pt;
  }
  R->n_chunks = static_cast<int32_t>(R->chunks.size() / 4);
  // child chunks, CSR, descending
  R->kid_ptr.assign(R->n_chunks + 1, 0);
  for (int32_t c = 0; c < R->n_chunks; ++c)
    if (R->chunks[4 * c + 2] >= 0) R->kid_ptr[R->chunks[4 * c + 2] + 1]++;
  for (int32_t c = 0; c < R->n_chunks; ++c) R->kid_ptr[c + 1] += R->kid_ptr[c];
  R->kid.assign(R->kid_ptr[R->n_chunks], 0);
  {
    std::vector<int32_t> fill(R->kid_ptr.begin(), R->kid_ptr.end() - 1);
    for (int32_t c = R->n_chunks - 1; c >= 0; --c)
      if (R->chunks[4 * c + 2] >= 0) R->kid[fill[R->chunks[4 * c + 2]]++] = c;
  }
  {  // chunk depths (a parent precedes its children), then a stable sort by depth
    std::vector<int32_t> depth(R->n_chunks, 0);
    for (int32_t c = 0; c < R->n_chunks; ++c)
      if (R->chunks[4 * c + 2] >= 0) depth[c] = depth[R->chunks[4 * c + 2]] + 1;
    R->order.resize(R->n_chunks);
    for (int32_t c = 0; c < R->n_chunks; ++c) R->order[c] = c;
    std::stable_sort(R->order.begin(), R->order.end(), [&](int32_t x, int32_t y) { return depth[x] < depth[y]; });
  }
  // path predecessor of every token, then its powers
  std::vector<int32_t> prev(N, -1);
  for (int32_t c = 0; c < R->n_chunks; ++c) {
    const int32_t s = R->chunks[4 * c], len = R->chunks[4 * c + 1];
    prev[s] = R->chunks[4 * c + 3];
    for (int32_t i = 1; i < len; ++i) prev[s + i] = s + i - 1;
  }
  const int32_t KM = K - 1;
  R->cprev.assign((size_t)N * std::max(KM, 0), -1);
  std::vector<int32_t> cnt(N, 0);
  for (int32_t t = 0; t < N; ++t) {
    int32_t q = t;
    for (int32_t j = 1; j <= KM; ++j) {
      q = q >= 0 ? prev[q] : -1;
      R->cprev[(size_t)t * KM + (j - 1)] = q;
      if (q >= 0) cnt[q]++;
    }
  }
  R->succ_ptr.assign(N + 1, 0);
  for (int32_t s = 0; s < N; ++s) R->succ_ptr[s + 1] = R->succ_ptr[s] + cnt[s];
  R->succ.assign(R->succ_ptr[N], 0);
  std::vector<int32_t> fill(R->succ_ptr.begin(), R->succ_ptr.end() - 1);
  for (int32_t t = 0; t < N; ++t)  // ascending t: each list comes out ordered
    for (int32_t j = 1; j <= KM; ++j) {
      const int32_t q = R->cprev[(size_t)t * KM + (j - 1)];
      if (q >= 0) R->succ[fill[q]++] = t * K + j;
    }
  auto a256 = [](size_t x) { return (x + 255) & ~size_t(255); };
  size_t off = 0;
  R->off_chunks = off;
  off += a256(R->chunks.size() * 4);
  R->off_cprev = off;
  off += a256(R->cprev.size() * 4);
  R->off_succ_ptr = off;
  off += a256(R->succ_ptr.size() * 4);
  R->off_succ = off;
  off += a256(R->succ.size() * 4);
  R->off_kid_ptr = off;
  off += a256(R->kid_ptr.size() * 4);
  R->off_kid = off;
  off += a256(R->kid.size() * 4);
  R->off_order = off;
  off += a256(R->order.size() * 4);
  R->device_bytes = std::max<size_t>(off, 256);
  return TA_OK;
}

}  // namespace

extern "C" ta_status tree_route(const ta_plan* plan, int32_t conv_k, ta_route** out) {
  if (!out) return TA_EINVAL;
  *out = nullptr;
  if (!plan || conv_k < 1 || conv_k > 8) return TA_EINVAL;
  if (plan->n_prefix_nodes != 0) return TA_EUNSUPPORTED;
  if ((int64_t)plan->n_tokens * conv_k > INT32_MAX) return TA_ERANGE;
  ta_route* R = new (std::nothrow) ta_route();
  if (!R) return TA_ENOMEM;
  ta_status st;
  try {
    st = build_route(plan, conv_k, R);
  } catch (const std::bad_alloc&) {
    st = TA_ENOMEM;
  }
  if (st != TA_OK) {
    delete R;
    return st;
  }
  *out = R;
  return TA_OK;
}

extern "C" ta_status tree_route_view(const ta_route* R, ta_route_view* v) {
  if (!R || !v) return TA_EINVAL;
  v->n_tokens = R->n_tokens;
  v->n_chunks = R->n_chunks;
  v->chunk = R->chunk;
  v->conv_k = R->conv_k;
  v->chunks = R->chunks.data();
  v->cprev = R->cprev.data();
  v->succ_ptr = R->succ_ptr.data();
  v->succ = R->succ.data();
  v->kid_ptr = R->kid_ptr.data();
  v->kid = R->kid.data();
  v->order = R->order.data();
  return TA_OK;
}

extern "C" ta_status tree_route_device_bytes(const ta_route* R, size_t* bytes) {
  if (!R || !bytes) return TA_EINVAL;
  *bytes = R->device_bytes;
  return TA_OK;
}

extern "C" void tree_route_free(ta_route* R) { delete R; }
