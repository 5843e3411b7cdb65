// Internal definition of the opaque partition object (host side).
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

#include "tree_attn.h"

struct ta_partition {
  int32_t n_nodes = 0, n_parts = 0, max_local = 0;
  int64_t n_tokens = 0, naive_tokens = 0;
  std::vector<int32_t> part_of, part_root, part_parent, n_prefix;
  std::vector<int64_t> own_tokens;
  std::vector<int32_t> local_ptr, local_node, local_parent, local_len;
  std::vector<int32_t> tok_ptr, tok_idx;
  // local plan of each partition (nullptr when it owns no token) and the byte
  // offsets of its plan image and row map inside the device image
  std::vector<ta_plan*> plans;
  std::vector<size_t> off_plan, off_idx;
  size_t device_bytes = 0;
  ~ta_partition() {
    for (ta_plan* p : plans) tree_plan_free(p);
  }
};
