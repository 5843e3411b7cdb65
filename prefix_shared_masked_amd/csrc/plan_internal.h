// Internal definition of the opaque plan (host side).
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

struct ta_plan {
  int32_t n_nodes = 0, n_tokens = 0, n_leaves = 0, max_pos = -1;
  int32_t n_prefix_nodes = 0, q_start = 0;  // key-only chain prefix: tokens [0, q_start)
  int32_t block_m = 0, block_n = 0, block_kv = 0;
  int32_t n_qtiles = 0, n_chunks = 0, n_ktiles = 0;
  int32_t n_kpieces = 0, n_ksplit = 0, n_kslots = 0, kv_piece_cap = 0;  // dK/dV work pieces
  int64_t n_dsblk = 0;  // dS blocks per query head (query tile x 32-key sub-tile pairs)
  int64_t n_flat = 0, visible_pairs = 0, computed_pairs_fwd = 0, computed_pairs_bwd = 0;
  std::vector<int32_t> dfs_order, node_start, node_sub_end;
  std::vector<int32_t> pos, g, node_of, sub_end;
  std::vector<int32_t> anc_ptr, anc;
  std::vector<int32_t> fq_ptr, fq_chunk, fq_order, bk, kp, kr, dq_ptr, dq_ent, dq_order;
  // byte offsets of each table inside the device image
  size_t off_pos = 0, off_fq_ptr = 0, off_fq_chunk = 0, off_fq_order = 0, off_bk = 0, off_kp = 0, off_kr = 0;
  size_t off_dq_ptr = 0, off_dq_ent = 0, off_dq_order = 0;
  size_t device_bytes = 0;
};
