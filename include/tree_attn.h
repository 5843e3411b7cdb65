/*
 * tree_attn.h -- C ABI of the tree-attention library (gfx950 / MI355X).
 *
 * The library computes exact softmax attention over a prefix tree that is
 * packed in depth-first order, the g_t/K weighted negative log-likelihood of
 * the packed tokens, and single-query decode over split KV with an
 * associative (max, numerator, denominator) merge.
 *
 * Definitions the calls follow (page titles and sections):
 *  - "Tree Training" post (tingdeliu.github.io, tree-training-prefix-reuse):
 *      3.1  a node holds a token segment; each root-to-leaf path is one
 *           training sequence; K = number of paths.
 *      3.2  DFS serialisation: a node's tokens, then each child's
 *           serialisation, so every node appears once.
 *      4.2  the tree mask: packed token i reads key j iff j <= i and node(j)
 *           is an ancestor-or-self of node(i); attention is
 *           softmax(Q K^T / sqrt(d) + M) V.
 *      4.3  production kernels must not build a dense N x N mask: they use the
 *           DFS interval, parent, depth and an ancestor block table and skip
 *           invisible blocks.
 *      5    positions are tree depth: summed length of the strict ancestors
 *           plus the offset inside the node.
 *      6.2  g_t = number of root-to-leaf paths through t; the tree loss is
 *           sum_t (g_t / K) l_t.
 *      12   the TreeNode record and the packing outputs (packed order,
 *           position ids, loss weights).
 *  - Tree Attention notes (t6page.pages.dev, tree-attention): the three
 *    mergeable quantities m, n = o e^(l-m), d = e^(l-m) and the decode
 *    algorithm (local attention per KV shard, global max, sums, z = n/d).
 *  - agent-rl tutorial chapter 14, section 14.1: sequence packing with a
 *    block-diagonal causal mask and positions that restart per sequence;
 *    here that is a forest (every sequence a root).
 *
 * Conventions for every call:
 *  - All tensors are caller-owned, contiguous, and live in device memory
 *    unless stated otherwise.  The library never allocates device memory; a
 *    call that needs scratch space takes a caller-provided workspace whose
 *    size the matching *_ws_bytes query returns.
 *  - Kernel calls are asynchronous on the given HIP stream.  Validation
 *    errors are returned before anything is launched; a failed launch
 *    returns TA_EHIP.
 *  - Plans are immutable after tree_plan returns and may be shared between
 *    threads.  The library's only global mutable state is the scratch array
 *    of tree_decode_splitkv_noalloc (one per device) with the table of its
 *    per-device addresses and that table's mutex, kept until the process
 *    ends; every other call keeps nothing between calls.  Every kernel is
 *    the library's own (no vendor library is called).
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum ta_status {
  TA_OK = 0,
  TA_EINVAL = 1,       /* null pointer, bad size, parent out of range, negative length, bad layout */
  TA_ECYCLE = 2,       /* parent pointers do not form a forest */
  TA_ERANGE = 3,       /* a count overflows the int32 index space of the kernels */
  TA_ENOMEM = 4,       /* host allocation failed, or a caller buffer is too small */
  TA_EUNSUPPORTED = 5, /* valid request the kernels are not built for (head dim, block sizes, dtype) */
  TA_EHIP = 6          /* a HIP call or kernel launch failed */
} ta_status;

typedef enum ta_dtype { TA_F32 = 0, TA_BF16 = 1 } ta_dtype;

/* Tile sizes the kernels are built for.  tree_plan accepts 0 (default) or
 * exactly these values. */
#define TA_BLOCK_M 32   /* query rows per forward tile */
#define TA_BLOCK_N 64   /* key slots per gathered key chunk */
#define TA_BLOCK_KV 128 /* keys per backward key tile (never crosses a node) */
#define TA_KV_SUB 32    /* backward sub-tile: 32 keys against 32-row query blocks */
#define TA_KV_PIECE_MIN 32 /* dK/dV pieces span at least this many 32-row query blocks */
#define TA_KPIECE_INTS 32 /* (q_lo, q_hi, 0, 0) + 4 x TA_KWAVE_INTS */
#define TA_KWAVE_INTS 7
#define TA_CHUNK_INTS 16
#define TA_CHUNK_MAX_SEG 4

/* Layout of one gathered key chunk (TA_CHUNK_INTS int32):
 *   [0] nseg      number of key segments (1..TA_CHUNK_MAX_SEG)
 *   [1] nkeys     key slots in use (1..TA_BLOCK_N); slots >= nkeys are padding
 *   [2] full      1 iff every row of the query tile reads every key of the chunk
 *   [3] reserved
 *   [4..7]   kstart[s]  first packed key index of segment s
 *   [8..11]  vstart[s]  first slot of segment s (unused segments hold TA_BLOCK_N)
 *   [12..15] kend[s]    end of the DFS interval of the node segment s lies in:
 *                        row i reads key j of segment s iff j <= i < kend[s]. */

typedef struct ta_plan ta_plan;

/* Read-only view of a plan.  Every pointer is host memory owned by the plan
 * and stays valid until tree_plan_free. */
typedef struct ta_plan_view {
  int32_t n_nodes;
  int32_t n_tokens;          /* N: unique tokens */
  int32_t n_leaves;          /* K: root-to-leaf paths (zero-length leaves count) */
  int32_t max_pos;           /* largest depth position, -1 if N == 0 */
  int32_t block_m, block_n, block_kv;
  int32_t n_qtiles, n_chunks, n_ktiles;
  int64_t n_flat;            /* sum over paths of the path length = sum_t g_t */
  int64_t visible_pairs;     /* sum over query rows t >= q_start of (pos(t) + 1): (i, j) pairs the
                                mask allows, per head */
  int64_t computed_pairs_fwd;/* pairs the forward tiles compute, per head (>= visible_pairs) */
  int64_t computed_pairs_bwd;/* pairs the backward key tiles compute, per head */
  const int32_t* dfs_order;  /* [n_nodes] node ids in visiting order */
  const int32_t* node_start; /* [n_nodes] first packed index, by node id */
  const int32_t* node_sub_end;/* [n_nodes] end of the node's DFS interval */
  const int32_t* pos;        /* [N] depth position */
  const int32_t* g;          /* [N] paths through the token */
  const int32_t* node_of;    /* [N] owning node */
  const int32_t* sub_end;    /* [N] node_sub_end[node_of[t]] */
  const int32_t* anc_ptr;    /* [n_nodes + 1] CSR offsets into anc */
  const int32_t* anc;        /* ancestor-or-self chains, root first, per node id */
  const int32_t* fq_ptr;     /* [n_qtiles + 1] chunk range of each query tile */
  const int32_t* fq_chunk;   /* [n_chunks * TA_CHUNK_INTS] gathered key chunks (layout above) */
  const int32_t* fq_order;   /* [n_qtiles] query tiles, most chunks first */
  const int32_t* bk;         /* [n_ktiles * 4] (k0, klen, q_end, node), most work first; every
                                query in [max(k0, q_start), q_end) lies in the node's subtree */
  int32_t n_prefix_nodes;    /* key-only chain prefix (tree_plan_ex), 0 for tree_plan */
  int32_t q_start;           /* its tokens [0, q_start) are keys only: no query tiles, no outputs */
  /* dK/dV work pieces (bf16 backward).  A piece is one workgroup: four
   * wavefronts, each owning the dK/dV of up to 32 keys of one node (a
   * sub-tile), over a common run of query rows [q_lo, q_hi) staged once;
   * q_lo lies on the query-tile grid q_start + 32t.  A full 128-key tile of
   * bk whose query range [max(k0, q_start), q_end) spans at most
   * kv_piece_cap 32-row blocks is one piece; the other tiles are cut into
   * sub-tiles, each cut at the windows of kv_piece_cap blocks anchored at
   * q_start, and the runs of one window are packed up to four to a piece.
   * A sub-tile cut over several windows writes fp32 partial dK/dV to one
   * workspace slot per window (consecutive, in window order), summed in slot
   * order by a second pass, so the result stays deterministic. */
  int32_t n_kpieces;         /* pieces */
  int32_t n_ksplit;          /* sub-tiles cut over several windows */
  int32_t n_kslots;          /* partial slots: sum of n_windows over cut sub-tiles */
  int32_t kv_piece_cap;      /* max(TA_KV_PIECE_MIN, ceil(total query blocks of all tiles / 256)) */
  const int32_t* kp;         /* [n_kpieces * TA_KPIECE_INTS] (q_lo, q_hi, 0, 0, then per wavefront
                                (kw, wk, r_lo, r_hi, slot, ds_off, 0)): wavefront w owns keys
                                [kw, kw + wk) (wk = 0: idle) and reads rows [max(key, r_lo), r_hi),
                                q_lo <= r_lo, r_hi <= q_hi; slot -1 stores dK/dV directly; its dS
                                block of query tile t is ds_off + t; longest first */
  const int32_t* kr;         /* [n_ksplit * 4] (kw, wk, first slot, n_windows) of each cut sub-tile */
  /* dS blocks: one per (query tile t, sub-tile) such that a row of t reads
   * the sub-tile, numbered sub-tile by sub-tile; dq lists them per tile. */
  int64_t n_dsblk;           /* dS blocks per query head */
  const int32_t* dq_ptr;     /* [n_qtiles + 1] entry range of each query tile */
  const int32_t* dq_ent;     /* [dq_ptr[n_qtiles] * 4] (kw, wk, dS block, 0), by first key */
  const int32_t* dq_order;   /* [n_qtiles] query tiles, most entries first */
} ta_plan_view;

/* Build the plan of a prefix tree (host only, synchronous, deterministic).
 * parent[i] = -1 marks a root (several roots: a forest, e.g. varlen packing);
 * seg_len[i] >= 0 tokens in node i.  Children are serialised in ascending
 * node id, roots in ascending id.  block_m / block_n: 0 or TA_BLOCK_M /
 * TA_BLOCK_N.  On success *out owns all tables; free with tree_plan_free.
 * Errors: TA_EINVAL (null pointer, n_nodes <= 0, negative length, parent out
 * of range), TA_ECYCLE, TA_ERANGE (N, a table or sum_t depth does not fit
 * int32), TA_EUNSUPPORTED (other block sizes), TA_ENOMEM.  On error *out is
 * set to NULL. */
ta_status tree_plan(const int32_t* parent, const int32_t* seg_len, int32_t n_nodes,
                    int32_t block_m, int32_t block_n, ta_plan** out);

/* tree_plan with a key-only prefix: the subtree of one partition of a tree
 * too large for one device, planned below the ancestor chain of its root
 * (the "gateway" of the Tree Training post, sections 8.1-8.2: a child
 * partition reads its ancestors' K/V instead of recomputing them).  Nodes
 * 0..n_prefix_nodes-1 are that chain: node 0 is the only root, node i's
 * parent is i - 1, and each chain node has exactly one child (the next chain
 * node; for the last one, the partition's root).  The chain's tokens
 * [0, q_start) serve as keys only: the forward and dQ kernels form no query
 * tiles for them and leave their O, LSE and dQ rows untouched, and dK/dV of
 * a chain key sums over the partition's queries only (the gradient the
 * partition relays to its parent).  Depth positions count the chain, so they
 * equal the positions in the whole tree.  n_prefix_nodes = 0 is tree_plan.
 * Errors as tree_plan, plus TA_EINVAL when the chain rules do not hold. */
ta_status tree_plan_ex(const int32_t* parent, const int32_t* seg_len, int32_t n_nodes,
                       int32_t n_prefix_nodes, int32_t block_m, int32_t block_n, ta_plan** out);

ta_status tree_plan_view(const ta_plan* plan, ta_plan_view* view);

/* Device copy of the tables the kernels read.  The caller allocates
 * tree_plan_device_bytes bytes of device memory (256-byte aligned) and
 * tree_plan_upload copies the tables in, asynchronously on the stream, from
 * host memory owned by the plan (the plan must outlive the copy).  The
 * kernels take that buffer as `dplan`; keep it alive while they run. */
ta_status tree_plan_device_bytes(const ta_plan* plan, size_t* bytes);
ta_status tree_plan_upload(const ta_plan* plan, void* dplan, size_t bytes, hipStream_t stream);

/* NULL-safe. */
void tree_plan_free(ta_plan* plan);

/* Workspace bytes of tree_attn_fwd (op = 0) or tree_attn_bwd (op = 1: the
 * full backward; op = 2: the smallest backward workspace) for this plan and
 * shape; 0 when none is needed.  For TA_BF16, op 1 includes the dS blocks
 * (2 * n_dsblk * 1024 bytes per query head) that let dQ read dS instead of
 * recomputing S and dP; with op 2's size dQ recomputes them. */
ta_status tree_attn_ws_bytes(const ta_plan* plan, int32_t op, ta_dtype dt, int32_t Hq, int32_t Hkv,
                             int32_t d, float rope_base, size_t* bytes);

/* Forward tree attention (Tree Training post, sections 4.2, 4.3 and 5).
 * q, o: [N, Hq, d]; k, v: [N, Hkv, d] in dtype dt (TA_BF16: bf16 inputs,
 * fp32 accumulation; TA_F32: fp32 throughout).  lse: [Hq, N] fp32, natural
 * log of sum_j exp(scale q_i . k_j) over the visible keys.  Query head h
 * reads KV head h / (Hq / Hkv).  d must be 64 or 128 (TA_BF16: 128).
 * scale <= 0 selects 1/sqrt(d).  rope_base > 0 rotates q and k by depth
 * position (rotate-half pairs (i, i + d/2), angle pos * base^(-2i/d));
 * 0 disables it.  ws: tree_attn_ws_bytes(op = 0) bytes of device memory.
 * Precision of the bf16 path: scores use fp16 copies of (rotated) Q and K,
 * which hold every bf16 value of magnitude <= 65504 exactly and rotated
 * values with 8x finer rounding than bf16; P is rounded to bf16 for P V;
 * accumulation is fp32 throughout.
 * Saturation flag (TA_BF16): the first int32 of ws.  A (rotated, scaled) Q
 * or K value beyond the fp16 range is clamped to +-65504 and the call stores
 * 1 there; NaN inputs pass through unclamped (and reach the outputs as NaN).
 * The library never clears the flag: the caller zeroes it and reads it back
 * when it wants to know (tree_attn_bwd uses the same word of its workspace,
 * the partition calls the first word of theirs).
 * A plan without tokens returns TA_OK after checking plan, heads, d and dt,
 * without touching any tensor pointer (empty tensors may be null); the same
 * holds for tree_attn_bwd, and for the scan and conv calls on a route
 * without tokens (tree_conv_bwd then zeroes dw).
 * Errors: TA_EINVAL, TA_EUNSUPPORTED, TA_ENOMEM (ws too small), TA_EHIP. */
ta_status tree_attn_fwd(const ta_plan* plan, const void* dplan, ta_dtype dt, const void* q,
                        const void* k, const void* v, int32_t Hq, int32_t Hkv, int32_t d,
                        float scale, float rope_base, void* o, float* lse, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* Backward of tree_attn_fwd for upstream gradient dO [N, Hq, d].  o and lse
 * are the forward's outputs.  dq [N, Hq, d], dk and dv [N, Hkv, d] are
 * overwritten (not accumulated), in dtype dt.  The gradient of a shared key
 * is the sum over every descendant query that reads it (section 7: shared
 * prefixes receive the gradients of all branches).  Deterministic: the same
 * inputs give bitwise-identical outputs (no atomics).
 * ws: tree_attn_ws_bytes(op = 1) bytes, or at least op = 2 bytes.  TA_BF16
 * with the op-1 size: the dK/dV kernel stores the fp16 dS of every (query
 * tile, 32-key sub-tile) block and dQ = scale * dS K reads it back (one
 * product).  With less, the call uses what fits: when the dS blocks of at
 * least one KV head fit, the KV heads run in rounds of as many as fit (a
 * query head's dQ depends on its own KV head's keys only, so the results are
 * bitwise the same); below that, dQ recomputes S and dP (three products)
 * before dK/dV.  tree_attn_bwd_ws_budget picks the size for a byte budget.
 * Errors as tree_attn_fwd (TA_ENOMEM below the op-2 size). */
ta_status tree_attn_bwd(const ta_plan* plan, const void* dplan, ta_dtype dt, const void* q,
                        const void* k, const void* v, const void* o, const float* lse,
                        const void* dO, int32_t Hq, int32_t Hkv, int32_t d, float scale,
                        float rope_base, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* The dS workspace grows with the visible pairs (2 bytes per pair and query
 * head: 2.8 GB for the 16K-token spine tree at 32 query heads, 22 GB for a
 * 133K-token varlen batch), so callers bound it.  tree_attn_bwd_ws_budget
 * returns in *bytes the largest tree_attn_bwd workspace within `budget`
 * bytes (0 selects TA_BWD_WS_BUDGET_DEFAULT) and in *kv_heads_per_round how
 * many KV heads' dS blocks it holds: Hkv = one round (the op-1 size), fewer =
 * rounds over the KV heads, 0 = the recompute path (the op-2 size).  Returns
 * TA_ENOMEM, with *bytes = the op-2 size, when even that exceeds the budget. */
#define TA_BWD_WS_BUDGET_DEFAULT ((size_t)8 << 30) /* 8 GiB */
ta_status tree_attn_bwd_ws_budget(const ta_plan* plan, ta_dtype dt, int32_t Hq, int32_t Hkv,
                                  int32_t d, float rope_base, size_t budget, size_t* bytes,
                                  int32_t* kv_heads_per_round);

/* Stage timing.  The *_ex variants behave exactly like the plain calls and,
 * when events is not NULL, also record events[i] (created by the caller with
 * hipEventCreate) on the stream at the stage boundaries listed below; at most
 * n_events are recorded.  Nothing else changes, so callers can time each
 * kernel with hipEventElapsedTime.
 *   tree_attn_fwd_ex:       [0] start, [1] after the K conversion/RoPE pass,
 *                           [2] after the attention kernel.
 *   tree_attn_bwd_ex:       [0] start, [1] after the preparation passes;
 *                           bf16 with the dS workspace: [2] after the dK/dV
 *                           kernel and its partial sum (of the first round of
 *                           KV heads), [3] after the (last) dQ kernel;
 *                           otherwise [2] after the dQ kernel, [3] after
 *                           dK/dV.
 *   tree_decode_splitkv_ex: [0] start, [1] after the partial kernel,
 *                           [2] after the merge kernel. */
typedef struct ihipEvent_t* hipEvent_t;
ta_status tree_attn_fwd_ex(const ta_plan* plan, const void* dplan, ta_dtype dt, const void* q,
                           const void* k, const void* v, int32_t Hq, int32_t Hkv, int32_t d,
                           float scale, float rope_base, void* o, float* lse, void* ws,
                           size_t ws_bytes, hipEvent_t* events, int32_t n_events,
                           hipStream_t stream);
ta_status tree_attn_bwd_ex(const ta_plan* plan, const void* dplan, ta_dtype dt, const void* q,
                           const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, int32_t Hq, int32_t Hkv, int32_t d, float scale,
                           float rope_base, void* dq, void* dk, void* dv, void* ws,
                           size_t ws_bytes, hipEvent_t* events, int32_t n_events,
                           hipStream_t stream);

/* Workspace bytes of tree_weighted_nll for N rows. */
ta_status tree_nll_ws_bytes(int32_t N, int32_t V, size_t* bytes);

/* g_t/K weighted negative log-likelihood (Tree Training post, sections 6.2,
 * 6.3 and 12): loss = sum_t w_t [y_t != ignore_index] (logsumexp(x_t) -
 * x_t[y_t]) -- a weighted SUM.  Labels are per packed token and already
 * aligned with the position that predicts them (no shift).
 * logits: [N, V] fp32 (dt must be TA_F32); labels: [N] int32; w: [N] fp32
 * (normally g_t / K).  loss: one device fp32.  dlogits: [N, V] fp32
 * w_t valid_t (softmax(x_t) - onehot(y_t)), or NULL for loss only.
 * err_flag: device int32 or NULL; set to 1 when a label is neither
 * ignore_index nor in [0, V) (that row then contributes 0).
 * Errors: TA_EINVAL, TA_EUNSUPPORTED, TA_ENOMEM, TA_EHIP. */
ta_status tree_weighted_nll(ta_dtype dt, const void* logits, const int32_t* labels, const float* w,
                            int32_t N, int32_t V, int32_t ignore_index, float* loss, void* dlogits,
                            int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Output layer fused with the weighted NLL (agent-rl chapter 14, section
 * 14.3; Tree Training post, sections 6.2 and 6.3) ----------------------------
 * loss = sum_t w_t [y_t valid] (logsumexp_v(h_t . W_v) - h_t . W_{y_t}) for
 * hidden states h [N, Dm] and output weights W [V, Dm] (bf16, row-major),
 * without ever holding the N x V logits: the forward reduces 256 x 256 logit
 * tiles to per-token (max, sum) partials on the matrix cores; the backward
 * recomputes the logits one vocabulary chunk at a time (section 14.3's
 * recompute), forms dS = w [valid] (softmax - onehot(y)) in bf16 for that
 * chunk only and accumulates dh += dS W_chunk (fp32) and dW_chunk = dS^T h.
 * labels [N] int32 (ignore_index marks unsupervised tokens; another label
 * outside [0, V) contributes 0 and sets *err_flag = 1 when err_flag is not
 * NULL); w [N] fp32 (g_t/K for a tree).  loss: device fp32 scalar (a fixed-
 * order sum: bitwise reproducible).  lse: optional [N] fp32 output (natural
 * log).  dh [N, Dm] and dW [V, Dm] (bf16, overwritten): both NULL for the
 * forward only, else both set.  vocab_chunk: vocabulary rows per backward
 * chunk (0 picks about 512 MB of dS; rounded down to whole 256-row tiles).
 * Dm must be a multiple of 32.  ws: tree_lmhead_nll_ws_bytes bytes.
 * Precision: products of bf16 values accumulate in fp32; dS is rounded to
 * bf16 for the two backward products.
 * Errors: TA_EINVAL, TA_EUNSUPPORTED, TA_ERANGE, TA_ENOMEM, TA_EHIP. */
ta_status tree_lmhead_nll_ws_bytes(int32_t N, int32_t V, int32_t Dm, int32_t need_grad,
                                   int32_t vocab_chunk, size_t* bytes);
ta_status tree_lmhead_nll(ta_dtype dt, const void* h, const void* W, const int32_t* labels,
                          const float* w, int32_t N, int32_t V, int32_t Dm, int32_t ignore_index,
                          int32_t vocab_chunk, float* loss, float* lse, void* dh, void* dW,
                          int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes of tree_decode_splitkv; *n_splits_out receives the split
 * count it will use (n_splits = 0 picks one from the longest item). */
ta_status tree_decode_ws_bytes(int32_t B, int32_t Hq, int32_t d, int32_t max_len, int32_t n_splits,
                               size_t* bytes, int32_t* n_splits_out);

/* Split-KV single-query decode (Tree Attention notes, decode algorithm):
 * every workgroup attends one query token per (batch item, query head) to
 * its slice of the item's KV rows and emits (m, n, d); a log-depth pairwise
 * merge across the slices gives z = n/d and lse = m + log d.
 * q, o: [B, Hq, d]; k, v: [L_total, Hkv, d]; lse: [B, Hq] fp32.
 * span_ptr [B + 1] and spans [.., 2] (device int32): item b reads the rows
 * spans[s] = (start, len) for s in [span_ptr[b], span_ptr[b+1]) in order
 * (plain decode: one span; tree decode: the ancestor chain of a leaf).  The
 * call does not know the K/V row count and does not read the span tables on
 * the host: the caller guarantees every span lies inside k / v and every
 * item's total length is at most max_len (the Python binding checks both on
 * the host unless asked not to).
 * max_len bounds every item's total length.  dt: TA_BF16, d = 128.
 * Precision: q.k products of bf16 values accumulate exactly in fp32; the
 * probabilities are rounded to bf16 for the P V product (fp32 accumulation);
 * the softmax sums and the merge are fp32.
 * Errors: TA_EINVAL, TA_EUNSUPPORTED, TA_ENOMEM, TA_EHIP. */
ta_status tree_decode_splitkv(ta_dtype dt, const void* q, const void* k, const void* v,
                              const int32_t* span_ptr, const int32_t* spans, int32_t B,
                              int32_t Hq, int32_t Hkv, int32_t d, int32_t max_len, float scale,
                              int32_t n_splits, void* o, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Allocation-free tree_decode_splitkv, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and arguments without a workspace; the
 * per-slice partials go to a fixed device array of TA_DECODE_SCRATCH_BYTES
 * inside the library (one per GPU, resolved on the first call on that GPU
 * and held until the process ends).  The call allocates nothing.  Calls whose
 * partials (tree_decode_ws_bytes) exceed the array return TA_ENOMEM before
 * launching anything.  Every call on a GPU uses that GPU's one array, so calls
 * that overlap on one GPU (other streams, other threads) race: serialise them.
 * Nothing in the array needs clearing between calls (every partial a call
 * reads it writes first).  Errors as tree_decode_splitkv. */
#define TA_DECODE_SCRATCH_BYTES ((size_t)16 << 20) /* 16 MiB: e.g. B = 8, 32 heads, 64 slices */
ta_status tree_decode_splitkv_noalloc(ta_dtype dt, const void* q, const void* k, const void* v,
                                      const int32_t* span_ptr, const int32_t* spans, int32_t B,
                                      int32_t Hq, int32_t Hkv, int32_t d, int32_t max_len,
                                      float scale, int32_t n_splits, void* o, float* lse,
                                      hipStream_t stream);

ta_status tree_decode_splitkv_ex(ta_dtype dt, const void* q, const void* k, const void* v,
                                 const int32_t* span_ptr, const int32_t* spans, int32_t B,
                                 int32_t Hq, int32_t Hkv, int32_t d, int32_t max_len, float scale,
                                 int32_t n_splits, void* o, float* lse, void* ws, size_t ws_bytes,
                                 hipEvent_t* events, int32_t n_events, hipStream_t stream);

/* ---- Partitioning a tree too large for one device (Tree Training post,
 * section 8) ----------------------------------------------------------------
 * tree_partition cuts a tree (or forest) along node boundaries into connected
 * subtrees whose own tokens fit `capacity` (section 8.3: each partition is a
 * connected subtree, so the partitions form a tree and each has one parent
 * partition).  Every token belongs to exactly one partition, so the unique
 * work stays N (section 8.1).  A partition's local tree is the ancestor chain
 * of its root (key-only, as in tree_plan_ex: the gateway K/V its parent
 * partitions export, section 8.2) followed by its own nodes in ascending
 * global id; the chain and the own nodes keep their depth positions.
 * Cut rule (the post fixes only the constraints): a post-order pass keeps at
 * each node its own tokens plus the open subtrees of its children and, while
 * that exceeds capacity, cuts off the largest open child subtree (ties: the
 * smaller node id).  Partitions are numbered in preorder of their roots, so a
 * parent partition precedes its children.
 * parent / seg_len as for tree_plan; capacity >= every seg_len (a node is
 * never split); block_m / block_n as for tree_plan (used for the local plans).
 * Errors: TA_EINVAL (null pointer, n_nodes <= 0, capacity < 1, a node longer
 * than capacity, bad parent), TA_ECYCLE, TA_ERANGE, TA_EUNSUPPORTED,
 * TA_ENOMEM.  On error *out is NULL. */
typedef struct ta_partition ta_partition;

typedef struct ta_partition_view {
  int32_t n_nodes, n_parts;
  int32_t max_local_tokens;     /* largest chain + own row count of a partition */
  int32_t reserved;
  int64_t n_tokens;             /* N = sum of own tokens over the partitions */
  int64_t naive_tokens;         /* sum of (chain + own) tokens: the rows a partition
                                   scheme that re-runs the ancestors would compute */
  const int32_t* part_of;       /* [n_nodes] partition of each node */
  const int32_t* part_root;     /* [n_parts] global node id of each partition's root */
  const int32_t* part_parent;   /* [n_parts] parent partition, -1 for a tree's root */
  const int32_t* n_prefix;      /* [n_parts] chain nodes of the local tree */
  const int64_t* own_tokens;    /* [n_parts] */
  const int32_t* local_ptr;     /* [n_parts + 1] CSR over local nodes */
  const int32_t* local_node;    /* global node id of each local node */
  const int32_t* local_parent;  /* local parent id (-1 for local node 0) */
  const int32_t* local_len;     /* seg_len of each local node */
  const int32_t* tok_ptr;       /* [n_parts + 1] CSR over local rows */
  const int32_t* tok_idx;       /* global packed row of each local row, in the
                                   local plan's packed order */
} ta_partition_view;

ta_status tree_partition(const int32_t* parent, const int32_t* seg_len, int32_t n_nodes,
                         int64_t capacity, int32_t block_m, int32_t block_n, ta_partition** out);
ta_status tree_partition_view(const ta_partition* part, ta_partition_view* view);
/* The local plan of partition i (owned by the partition object). */
ta_status tree_partition_plan(const ta_partition* part, int32_t i, const ta_plan** plan);
/* Device image of every local plan and row map, as tree_plan_device_bytes /
 * tree_plan_upload (the partition must outlive the asynchronous copy). */
ta_status tree_partition_device_bytes(const ta_partition* part, size_t* bytes);
ta_status tree_partition_upload(const ta_partition* part, void* dpart, size_t bytes,
                                hipStream_t stream);
/* NULL-safe. */
void tree_partition_free(ta_partition* part);

/* Workspace bytes of tree_partition_fwd (op = 0) / tree_partition_bwd (op = 1). */
ta_status tree_partition_ws_bytes(const ta_partition* part, int32_t op, ta_dtype dt, int32_t Hq,
                                  int32_t Hkv, int32_t d, float rope_base, size_t* bytes);

/* Tree attention run one partition at a time through the gateway (section
 * 8.2), with the whole tree's tensors in the layouts of tree_attn_fwd/bwd.
 * Each partition gathers its rows (the chain's K/V are the gateway leaves it
 * reads from its ancestors; the chain's Q, O and dO rows are zero-filled and
 * never read), runs tree_attn_fwd/bwd on its local plan and writes back its
 * own rows of O, LSE and dQ.  The backward relays every local dK/dV row,
 * chain rows included, into an fp32 accumulator per global row (the fp32
 * accumulator of section 8.2 for cut nodes shared by several children;
 * partitions are visited in a fixed order, so results are deterministic),
 * which is finally written to dk/dv in dt.  On one device the partitions run
 * in sequence; each one is the work a separate device would do.  The results
 * equal tree_attn_fwd/bwd on the whole tree up to rounding order (in bf16,
 * each partition's dK/dV is rounded to bf16 once before the fp32 sum).
 * Errors as tree_attn_fwd/bwd. */
ta_status tree_partition_fwd(const ta_partition* part, const void* dpart, ta_dtype dt,
                             const void* q, const void* k, const void* v, int32_t Hq, int32_t Hkv,
                             int32_t d, float scale, float rope_base, void* o, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);
ta_status tree_partition_bwd(const ta_partition* part, const void* dpart, ta_dtype dt,
                             const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dO, int32_t Hq, int32_t Hkv, int32_t d,
                             float scale, float rope_base, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* ---- Recurrent layers over the packed tree (Tree Training post, section 9) --
 * In DFS-packed order the token before a node's first token can belong to a
 * sibling branch; recurrent layers must instead continue from the parent.
 * tree_route builds, from a plan (tree_plan, no key-only prefix), the tables
 * for: (9.1) a linear recurrence h_t = a_t * h_prev(t) + b_t per channel
 * whose chunks start from their parent's end state -- every node is cut into
 * chunks of up to `chunk` tokens, a chunk's parent being the previous chunk
 * of its node or the last chunk of the nearest ancestor that holds tokens,
 * zero state before a root -- and (9.2) a causal depthwise convolution of
 * width conv_k (1..8) whose window runs back along the root-to-token path
 * (the parent's last conv_k - 1 tokens, continuing into the grandparent when
 * the parent is shorter; zero past the root).  chunks are in DFS order, so a
 * parent chunk precedes its children.  Errors: TA_EINVAL, TA_EUNSUPPORTED
 * (a plan with a key-only prefix), TA_ERANGE, TA_ENOMEM. */
typedef struct ta_route ta_route;
typedef struct ta_route_view {
  int32_t n_tokens, n_chunks, chunk, conv_k;
  const int32_t* chunks;    /* [n_chunks][4]: first token, length, parent chunk or -1, the token
                               before the first one on the path or -1 */
  const int32_t* cprev;     /* [N][conv_k - 1]: the j-th path predecessor of t (j = 1..), -1 past the root */
  const int32_t* succ_ptr;  /* [N + 1] CSR: the (t, j) whose j-th predecessor is s, */
  const int32_t* succ;      /* encoded t * conv_k + j, ascending t */
  const int32_t* kid_ptr;   /* [n_chunks + 1] CSR: the child chunks of each chunk (those whose */
  const int32_t* kid;       /* parent it is), each list in descending chunk order */
  const int32_t* order;     /* [n_chunks]: the chunks by depth in the chunk tree, ties in DFS order
                               (the scan's work order; parents before children) */
} ta_route_view;
ta_status tree_route(const ta_plan* plan, int32_t conv_k, ta_route** out);
ta_status tree_route_view(const ta_route* route, ta_route_view* view);
ta_status tree_route_device_bytes(const ta_route* route, size_t* bytes);
ta_status tree_route_upload(const ta_route* route, void* droute, size_t bytes, hipStream_t stream);
void tree_route_free(ta_route* route); /* NULL-safe */

/* Tree-routed scan.  a, b, h: [N, C] fp32 (token-major, channels contiguous),
 * h = the recurrence's states (the layer's output).  Backward: given the
 * forward's h and the upstream gradient dh [N, C], writes da = dh_total *
 * h_prev and db = dh_total, where dh_total of a node's last token sums the
 * contributions of every child branch.  One pass per direction: the
 * workgroup of a chunk waits for the end state of its parent chunk
 * (forward), or the outgoing gradients of its child chunks (backward),
 * which other workgroups of the same launch publish through ws.
 * Deterministic: every sum and composition has a fixed order whatever the
 * timing.  ws: tree_scan_ws_bytes, cleared by the call itself; its 32-bit
 * word 1 is set to nonzero if a wait for a published value ran out (bounded
 * waits; the workgroups' ticket order rules this out), in which case the
 * outputs are not valid.  Calls that share a ws must not overlap.  Errors:
 * TA_EINVAL, TA_ERANGE, TA_ENOMEM, TA_EUNSUPPORTED, TA_EHIP. */
ta_status tree_scan_ws_bytes(const ta_route* route, int32_t C, size_t* bytes);
ta_status tree_scan_fwd(const ta_route* route, const void* droute, const float* a, const float* b,
                        int32_t C, float* h, void* ws, size_t ws_bytes, hipStream_t stream);
ta_status tree_scan_bwd(const ta_route* route, const void* droute, const float* a, const float* h,
                        const float* dh, int32_t C, float* da, float* db, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Tree-routed causal conv.  x, y, dy, dx: [N, C] fp32; w, dw: [C, conv_k]
 * fp32, tap j multiplying the j-th path predecessor (j = 0: the token itself).
 * dx and dw are overwritten; deterministic.  ws (backward only):
 * tree_conv_ws_bytes.  Errors as tree_scan_fwd. */
ta_status tree_conv_ws_bytes(const ta_route* route, int32_t C, size_t* bytes);
ta_status tree_conv_fwd(const ta_route* route, const void* droute, const float* x, const float* w,
                        int32_t C, float* y, hipStream_t stream);
ta_status tree_conv_bwd(const ta_route* route, const void* droute, const float* x, const float* w,
                        const float* dy, int32_t C, float* dx, float* dw, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* Static text for a status code. */
const char* ta_status_string(ta_status s);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
