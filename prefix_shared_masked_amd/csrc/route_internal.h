// Internal definition of the opaque routing object (host side).
#pragma once
#include <cstddef>
#include <cstdint>
#include <vector>

struct ta_route {
  int32_t n_tokens = 0, n_chunks = 0, chunk = 0, conv_k = 0;
  // chunks in DFS order (a parent chunk precedes its children):
  // [start, len, parent chunk or -1, token before the first one on the path or -1]
  std::vector<int32_t> chunks;  // 4 per chunk
  // child chunks of each chunk (those whose parent it is), CSR, each list in
  // descending chunk order (the order the backward sums their gradients in)
  std::vector<int32_t> kid_ptr, kid;
  // the chunks by depth in the chunk tree (ties in DFS order): the order the
  // scan takes them in (parents first; reversed for the backward), which
  // puts the chunks of one depth -- the next link of a long chain and the
  // branches hanging off earlier links -- side by side
  std::vector<int32_t> order;
  // conv: prev^j(t) for j = 1..conv_k-1, [N][conv_k - 1], -1 past the root
  std::vector<int32_t> cprev;
  // inverse of cprev: for token s the (t, j) with prev^j(t) = s, encoded t * conv_k + j, CSR
  std::vector<int32_t> succ_ptr, succ;
  size_t off_chunks = 0, off_cprev = 0, off_succ_ptr = 0, off_succ = 0, off_kid_ptr = 0, off_kid = 0, off_order = 0,
         device_bytes = 0;
};
