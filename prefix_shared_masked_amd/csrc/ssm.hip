// Tree-routed linear recurrence and causal convolution over DFS-packed tokens
// (Tree Training post, section 9).  Rows are tokens, C channels per row, fp32.
//
// Scan h_t = a_t h_prev(t) + b_t, prev(t) following the root-to-token path
// (section 9.1: a chunk starts from its parent's end state).  Chunks of up to
// 128 tokens form a tree (parent = the previous chunk of the node, or the
// last chunk of the nearest ancestor holding tokens).  Three passes, all with
// consecutive lanes on consecutive channels, so every row access is
// coalesced:
//   reduce: per (chunk, channel) the chunk's decay A = prod a and its end
//           state H from a zero start;
//   walk:   per channel, chunks in DFS order: start = end of the parent chunk,
//           end = A start + H (a few hundred dependent steps, their inputs
//           fetched in batches ahead of the chain);
//   apply:  per (chunk, channel) the scan again from its start, writing h.
// The backward runs the mirror image: a reverse local scan per chunk, a walk
// in reverse DFS order that adds every chunk's outgoing gradient a_first dh_first
// into its parent (the sum over branches a shared prefix receives), and a
// reverse scan per chunk writing da = dh h_prev and db = dh.
//
// Causal conv y_t = sum_j w[c][j] x_{prev^j(t)} (section 9.2: the window runs
// back along the path into the parent's tail): a gather over the planner's
// predecessor table; its backward gathers over the inverse table (dx) and
// reduces over tokens in a fixed order (dw), so no atomics.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "route_internal.h"

namespace ta {
namespace ssm {

constexpr int TH = 256;

__global__ __launch_bounds__(TH) void scan_reduce(const int4* __restrict__ ch, const float* __restrict__ a,
                                                  const float* __restrict__ b, int C, float* __restrict__ A,
                                                  float* __restrict__ H) {
  const int c = blockIdx.x, k = blockIdx.y * TH + threadIdx.x;
  if (k >= C) return;
  const int4 r = ch[c];
  float da = 1.f, h = 0.f;
  const float* ap = a + (size_t)r.x * C + k;
  const float* bp = b + (size_t)r.x * C + k;
#pragma unroll 8
  for (int i = 0; i < r.y; ++i) {
    const float x = ap[(size_t)i * C], y = bp[(size_t)i * C];
    h = fmaf(x, h, y);
    da *= x;
  }
  A[(size_t)c * C + k] = da;
  H[(size_t)c * C + k] = h;
}

// Chunks in DFS order; a chunk's parent precedes it.  The end state of the
// previous chunk is kept in a register (the parent of most chunks), others
// come back from memory.  Inputs of 8 chunks are fetched before their chain.
__global__ __launch_bounds__(TH) void scan_walk(const int4* __restrict__ ch, int n_chunks, const float* __restrict__ A,
                                                const float* __restrict__ H, int C, float* __restrict__ hin,
                                                float* __restrict__ hend) {
  const int k = blockIdx.x * TH + threadIdx.x;
  if (k >= C) return;
  float prev_end = 0.f;
  for (int c0 = 0; c0 < n_chunks; c0 += 8) {
    float av[8], hv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(c0 + u, n_chunks - 1);
      av[u] = A[(size_t)c * C + k];
      hv[u] = H[(size_t)c * C + k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u;
      if (c >= n_chunks) break;
      const int p = ch[c].z;
      const float s = p < 0 ? 0.f : (p == c - 1 ? prev_end : hend[(size_t)p * C + k]);
      prev_end = fmaf(av[u], s, hv[u]);
      hin[(size_t)c * C + k] = s;
      hend[(size_t)c * C + k] = prev_end;
    }
  }
}

__global__ __launch_bounds__(TH) void scan_apply(const int4* __restrict__ ch, const float* __restrict__ a,
                                                 const float* __restrict__ b, int C, const float* __restrict__ hin,
                                                 float* __restrict__ h) {
  const int c = blockIdx.x, k = blockIdx.y * TH + threadIdx.x;
  if (k >= C) return;
  const int4 r = ch[c];
  float s = hin[(size_t)c * C + k];
  const size_t o = (size_t)r.x * C + k;
#pragma unroll 8
  for (int i = 0; i < r.y; ++i) {
    s = fmaf(a[o + (size_t)i * C], s, b[o + (size_t)i * C]);
    h[o + (size_t)i * C] = s;
  }
}

// Backward, local pass: u = g_t + a_{t+1} u from the chunk's end with nothing
// coming in; U = u at the first token, B = prod_{t > first} a_t.
__global__ __launch_bounds__(TH) void scan_reduce_bwd(const int4* __restrict__ ch, const float* __restrict__ a,
                                                      const float* __restrict__ g, int C, float* __restrict__ U,
                                                      float* __restrict__ B) {
  const int c = blockIdx.x, k = blockIdx.y * TH + threadIdx.x;
  if (k >= C) return;
  const int4 r = ch[c];
  const size_t o = (size_t)r.x * C + k;
  float u = 0.f, dec = 1.f, an = 0.f;  // an: a of the token after the current one
#pragma unroll 8
  for (int i = r.y - 1; i >= 0; --i) {
    u = fmaf(an, u, g[o + (size_t)i * C]);
    if (i + 1 < r.y) dec *= an;
    an = a[o + (size_t)i * C];
  }
  U[(size_t)c * C + k] = u;
  B[(size_t)c * C + k] = dec;
}

// Reverse DFS order: every successor of a chunk has a larger index, so a
// chunk's incoming gradient is complete when the walk reaches it.
__global__ __launch_bounds__(TH) void scan_walk_bwd(const int4* __restrict__ ch, int n_chunks, const float* __restrict__ a,
                                                    const float* __restrict__ U, const float* __restrict__ B, int C,
                                                    float* __restrict__ gin) {
  const int k = blockIdx.x * TH + threadIdx.x;
  if (k >= C) return;
  for (int c = 0; c < n_chunks; ++c) gin[(size_t)c * C + k] = 0.f;
  for (int c1 = n_chunks - 1; c1 >= 0; c1 -= 8) {
    float uv[8], bv[8], af[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = max(c1 - u, 0);
      uv[u] = U[(size_t)c * C + k];
      bv[u] = B[(size_t)c * C + k];
      af[u] = a[(size_t)ch[c].x * C + k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c1 - u;
      if (c < 0) break;
      const int p = ch[c].z;
      if (p < 0) continue;
      const float dh0 = fmaf(bv[u], gin[(size_t)c * C + k], uv[u]);
      gin[(size_t)p * C + k] += af[u] * dh0;
    }
  }
}

// The two walks with the per-chunk state of a workgroup's channels kept in
// LDS: one wavefront per WC channels, column `lane` of an [n_chunks][WC]
// array, so a chunk whose parent is not the previous one reads the parent's
// end state (forward) or adds into the parent's incoming gradient (backward)
// without a round trip to memory.  Each lane touches only its own column (no
// barrier); the arithmetic and its order are those of scan_walk /
// scan_walk_bwd.  Used while n_chunks * WC floats fit in LDS_WALK_MAX bytes.
constexpr int WC = 64;
constexpr size_t LDS_WALK_MAX = 64 * 1024;

__global__ __launch_bounds__(WC) void scan_walk_lds(const int4* __restrict__ ch, int n_chunks, const float* __restrict__ A,
                                                    const float* __restrict__ H, int C, float* __restrict__ hin,
                                                    float* __restrict__ hend) {
  extern __shared__ float se[];  // [n_chunks][WC] end states
  const int lane = threadIdx.x, k0 = blockIdx.x * WC + lane;
  const bool live = k0 < C;
  const int k = live ? k0 : C - 1;
  // inputs of the next group of 8 chunks are fetched while this group's chain runs
  float prev_end = 0.f, av[8], hv[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = min(u, n_chunks - 1);
    av[u] = A[(size_t)c * C + k];
    hv[u] = H[(size_t)c * C + k];
  }
  for (int c0 = 0; c0 < n_chunks; c0 += 8) {
    float an[8], hn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(c0 + 8 + u, n_chunks - 1);
      an[u] = A[(size_t)c * C + k];
      hn[u] = H[(size_t)c * C + k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u;
      if (c >= n_chunks) break;
      const int p = ch[c].z;
      const float s = p < 0 ? 0.f : (p == c - 1 ? prev_end : se[p * WC + lane]);
      prev_end = fmaf(av[u], s, hv[u]);
      se[c * WC + lane] = prev_end;
      if (live) {
        hin[(size_t)c * C + k] = s;
        hend[(size_t)c * C + k] = prev_end;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      av[u] = an[u];
      hv[u] = hn[u];
    }
  }
}

__global__ __launch_bounds__(WC) void scan_walk_bwd_lds(const int4* __restrict__ ch, int n_chunks,
                                                        const float* __restrict__ a, const float* __restrict__ U,
                                                        const float* __restrict__ B, int C, float* __restrict__ gin) {
  extern __shared__ float sg[];  // [n_chunks][WC] incoming gradients
  const int lane = threadIdx.x, k0 = blockIdx.x * WC + lane;
  const bool live = k0 < C;
  const int k = live ? k0 : C - 1;
  for (int c = 0; c < n_chunks; ++c) sg[c * WC + lane] = 0.f;
  // inputs of the next group of 8 chunks are fetched while this group's chain runs
  float uv[8], bv[8], af[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = max(n_chunks - 1 - u, 0);
    uv[u] = U[(size_t)c * C + k];
    bv[u] = B[(size_t)c * C + k];
    af[u] = a[(size_t)ch[c].x * C + k];
  }
  for (int c1 = n_chunks - 1; c1 >= 0; c1 -= 8) {
    float un[8], bn[8], fn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = max(c1 - 8 - u, 0);
      un[u] = U[(size_t)c * C + k];
      bn[u] = B[(size_t)c * C + k];
      fn[u] = a[(size_t)ch[c].x * C + k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c1 - u;
      if (c < 0) break;
      const int p = ch[c].z;
      if (p < 0) continue;
      const float dh0 = fmaf(bv[u], sg[c * WC + lane], uv[u]);
      sg[p * WC + lane] += af[u] * dh0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      uv[u] = un[u];
      bv[u] = bn[u];
      af[u] = fn[u];
    }
  }
  if (live)
    for (int c = 0; c < n_chunks; ++c) gin[(size_t)c * C + k] = sg[c * WC + lane];
}

__global__ __launch_bounds__(TH) void scan_apply_bwd(const int4* __restrict__ ch, const float* __restrict__ a,
                                                     const float* __restrict__ h, const float* __restrict__ g, int C,
                                                     const float* __restrict__ gin, float* __restrict__ da,
                                                     float* __restrict__ db) {
  const int c = blockIdx.x, k = blockIdx.y * TH + threadIdx.x;
  if (k >= C) return;
  const int4 r = ch[c];
  const size_t o = (size_t)r.x * C + k;
  float u = gin[(size_t)c * C + k], an = 1.f;  // u carries a_{t+1} dh_{t+1} (the incoming sum at the end)
#pragma unroll 4
  for (int i = r.y - 1; i >= 0; --i) {
    const float dh = g[o + (size_t)i * C] + an * u;
    const float hp = i > 0 ? h[o + (size_t)(i - 1) * C] : (r.w >= 0 ? h[(size_t)r.w * C + k] : 0.f);
    db[o + (size_t)i * C] = dh;
    da[o + (size_t)i * C] = dh * hp;
    u = dh;
    an = a[o + (size_t)i * C];
  }
}

// Causal conv over the path: y[t][k] = sum_j w[k][j] x[prev^j(t)][k].  VW
// consecutive channels per lane (VW = 4: 16-byte accesses when C % 4 == 0).
template <int VW>
struct Vec;
template <>
struct Vec<1> {
  typedef float T;
  static __device__ __forceinline__ float get(const T& v, int) { return v; }
  static __device__ __forceinline__ void set(T& v, int, float x) { v = x; }
};
template <>
struct Vec<4> {
  typedef f32x4 T;
  static __device__ __forceinline__ float get(const T& v, int i) { return v[i]; }
  static __device__ __forceinline__ void set(T& v, int i, float x) { v[i] = x; }
};

// A block covers TG tokens x (TH * VW) channels; each lane holds its
// channels' taps in registers for all TG tokens.
constexpr int TG = 8;
template <int VW>
__device__ __forceinline__ void load_taps(const float* __restrict__ w, int k, int K, float (&wr)[8][VW]) {
#pragma unroll
  for (int e = 0; e < VW; ++e)
#pragma unroll
    for (int j = 0; j < 8; ++j) wr[j][e] = j < K ? w[(size_t)(k + e) * K + j] : 0.f;
}

// Within a node (and from a parent into its first child, which follows it in
// DFS order) the j-th path predecessor of token t is the packed row t - j.
// A group of TG tokens whose taps all follow that pattern -- checked on the
// table by the lanes of each wavefront, the same answer in every wavefront
// of the block -- reads its TG + K - 1 rows once into registers; other groups
// gather through the table.  KT: the compile-time width for the register
// window (2..4), or 0: gather only.  Lanes past the channels clamp their
// loads and skip their stores, so every lane takes part in the vote.
template <int KT>
__device__ __forceinline__ bool window_prev(const int32_t* __restrict__ cprev, int N, int t0) {
  const int lane = threadIdx.x & 63;
  bool ok = t0 + TG <= N;
  if (lane < TG * (KT - 1) && ok) {
    const int t = t0 + lane / (KT - 1), j = lane % (KT - 1) + 1;
    // (t - j >= 0: the table marks a missing predecessor with -1, which t - j = -1 would match)
    ok = t - j >= 0 && cprev[(size_t)t0 * (KT - 1) + lane] == t - j;
  }
  return __all(ok);
}

template <int VW, int KT>
__global__ __launch_bounds__(TH) void conv_fwd(const int32_t* __restrict__ cprev, int N, int K, const float* __restrict__ x,
                                               const float* __restrict__ w, int C, float* __restrict__ y) {
  typedef typename Vec<VW>::T V;
  const int k0 = (blockIdx.y * TH + threadIdx.x) * VW;
  const bool live = k0 < C;
  const int k = live ? k0 : C - VW;
  float wr[8][VW];
  load_taps<VW>(w, k, K, wr);
  const int t0 = blockIdx.x * TG;
  if (KT > 1 && window_prev<KT>(cprev, N, t0)) {
    V r[TG + KT - 1];  // rows t0 - KT + 1 .. t0 + TG - 1 (all >= 0: every tap has a predecessor)
#pragma unroll
    for (int i = 0; i < TG + KT - 1; ++i) r[i] = *(const V*)(x + (size_t)(t0 - (KT - 1) + i) * C + k);
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      V s;
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        float acc = wr[0][e] * Vec<VW>::get(r[tt + KT - 1], e);
#pragma unroll
        for (int j = 1; j < KT; ++j) acc = fmaf(wr[j][e], Vec<VW>::get(r[tt + KT - 1 - j], e), acc);
        Vec<VW>::set(s, e, acc);
      }
      if (live) *(V*)(y + (size_t)(t0 + tt) * C + k) = s;
    }
    return;
  }
  const int t1 = min(N, t0 + TG);
  for (int t = t0; t < t1; ++t) {
    const V x0 = *(const V*)(x + (size_t)t * C + k);
    V s;
#pragma unroll
    for (int e = 0; e < VW; ++e) Vec<VW>::set(s, e, wr[0][e] * Vec<VW>::get(x0, e));
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      if (j >= K) break;
      // no branch on the table: a tap past the root loads the token's own row
      // and contributes zero, so every load of the token can issue at once
      const int q = cprev[(size_t)t * (K - 1) + (j - 1)];  // uniform over the block
      const V xv = *(const V*)(x + (size_t)(q >= 0 ? q : t) * C + k);
#pragma unroll
      for (int e = 0; e < VW; ++e)
        Vec<VW>::set(s, e, fmaf(wr[j][e], q >= 0 ? Vec<VW>::get(xv, e) : 0.f, Vec<VW>::get(s, e)));
    }
    if (live) *(V*)(y + (size_t)t * C + k) = s;
  }
}

// dx[s] = sum_j w[j] dy[t] over the (t, j) with prev^j(t) = s (the inverse
// table: sp / sc, codes t*K + j ordered by t).  Window: every token s of the
// group has exactly the K - 1 successors s + 1 .. s + K - 1 (prev^j(s + j)
// = s and no other), so dx[s] = sum_j w[j] dy[s + j] from TG + K - 1 rows.
template <int KT>
__device__ __forceinline__ bool window_succ(const int32_t* __restrict__ cprev, const int32_t* __restrict__ sp, int N,
                                            int s0) {
  const int lane = threadIdx.x & 63;
  bool ok = s0 + TG + KT - 1 <= N;
  if (ok && lane < TG * (KT - 1)) {
    const int s = s0 + lane / (KT - 1), j = lane % (KT - 1) + 1;
    ok = cprev[(size_t)(s + j) * (KT - 1) + (j - 1)] == s;
  }
  if (ok && lane < TG) ok = sp[s0 + lane + 1] - sp[s0 + lane] == KT - 1;
  return __all(ok);
}

// dx of one group of TG tokens s0.. for this lane's channels.
template <int VW, int KT>
__device__ __forceinline__ void conv_dx_group(const int32_t* __restrict__ cprev, const int32_t* __restrict__ sp,
                                              const int32_t* __restrict__ sc, int N, int K,
                                              const float* __restrict__ dy, const float (&wr)[8][VW], int C, int k,
                                              bool live, int s0, float* __restrict__ dx) {
  typedef typename Vec<VW>::T V;
  if (KT > 1 && window_succ<KT>(cprev, sp, N, s0)) {
    V r[TG + KT - 1];  // rows s0 .. s0 + TG + KT - 2
#pragma unroll
    for (int i = 0; i < TG + KT - 1; ++i) r[i] = *(const V*)(dy + (size_t)(s0 + i) * C + k);
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      V v;
#pragma unroll
      for (int e = 0; e < VW; ++e) {
        float acc = wr[0][e] * Vec<VW>::get(r[tt], e);
#pragma unroll
        for (int j = 1; j < KT; ++j) acc = fmaf(wr[j][e], Vec<VW>::get(r[tt + j], e), acc);
        Vec<VW>::set(v, e, acc);
      }
      if (live) *(V*)(dx + (size_t)(s0 + tt) * C + k) = v;
    }
    return;
  }
  const int s1 = min(N, s0 + TG);
  for (int s = s0; s < s1; ++s) {
    const V g0 = *(const V*)(dy + (size_t)s * C + k);
    V v;
#pragma unroll
    for (int e = 0; e < VW; ++e) Vec<VW>::set(v, e, wr[0][e] * Vec<VW>::get(g0, e));
    for (int i = sp[s]; i < sp[s + 1]; ++i) {
      const int code = sc[i], t = code / K, j = code - t * K;
      const V g = *(const V*)(dy + (size_t)t * C + k);
#pragma unroll
      for (int jj = 1; jj < 8; ++jj)
        if (jj == j) {
#pragma unroll
          for (int e = 0; e < VW; ++e) Vec<VW>::set(v, e, fmaf(wr[jj][e], Vec<VW>::get(g, e), Vec<VW>::get(v, e)));
        }
    }
    if (live) *(V*)(dx + (size_t)s * C + k) = v;
  }
}

// dw terms of one group of tokens t0 .. min(t0 + TG, tend) - 1: acc[j] +=
// dy[t] x[prev^j(t)] in token order.
template <int VW, int KT>
__device__ __forceinline__ void conv_dw_group(const int32_t* __restrict__ cprev, int N, int K,
                                              const float* __restrict__ x, const float* __restrict__ dy, int C, int k,
                                              int t0, int tend, float (&acc)[8][VW]) {
  typedef typename Vec<VW>::T V;
  if (KT > 1 && t0 + TG <= tend && window_prev<KT>(cprev, N, t0)) {
    V r[TG + KT - 1], g[TG];
#pragma unroll
    for (int i = 0; i < TG + KT - 1; ++i) r[i] = *(const V*)(x + (size_t)(t0 - (KT - 1) + i) * C + k);
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) g[tt] = *(const V*)(dy + (size_t)(t0 + tt) * C + k);
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int j = 0; j < KT; ++j)
#pragma unroll
        for (int e = 0; e < VW; ++e)
          acc[j][e] = fmaf(Vec<VW>::get(g[tt], e), Vec<VW>::get(r[tt + KT - 1 - j], e), acc[j][e]);
    return;
  }
  const int t1 = min(tend, t0 + TG);
  for (int t = t0; t < t1; ++t) {
    const V g = *(const V*)(dy + (size_t)t * C + k);
    const V x0 = *(const V*)(x + (size_t)t * C + k);
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[0][e] = fmaf(Vec<VW>::get(g, e), Vec<VW>::get(x0, e), acc[0][e]);
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      if (j >= K) break;
      const int q = cprev[(size_t)t * (K - 1) + (j - 1)];
      const V xq = *(const V*)(x + (size_t)(q >= 0 ? q : t) * C + k);
#pragma unroll
      for (int e = 0; e < VW; ++e)
        acc[j][e] = fmaf(Vec<VW>::get(g, e), q >= 0 ? Vec<VW>::get(xq, e) : 0.f, acc[j][e]);
    }
  }
}

// The conv backward in one pass over x and dy.  dx[s] = sum_j w[j] dy[t] over
// the (t, j) with prev^j(t) = s (the inverse table: sp / sc, codes t*K + j
// ordered by t); window: every token s of a group has exactly the K - 1
// successors s + 1 .. s + K - 1 (prev^j(s + j) = s and no other), so dx[s] =
// sum_j w[j] dy[s + j] from TG + K - 1 rows.  dw partials: per block of TOKB
// tokens and channel, sum_t dy[t] x[prev^j(t)] in token order (fixed).  A
// block walks its TOKB tokens group by group, each group's dx and then its
// dw terms, so the dy rows the two read are fetched from HBM once.
constexpr int TOKB = 256;
template <int VW, int KT>
__global__ __launch_bounds__(TH) void conv_bwd(const int32_t* __restrict__ cprev, const int32_t* __restrict__ sp,
                                               const int32_t* __restrict__ sc, int N, int K,
                                               const float* __restrict__ x, const float* __restrict__ dy,
                                               const float* __restrict__ w, int C, float* __restrict__ dx,
                                               float* __restrict__ part) {
  const int k0 = (blockIdx.y * TH + threadIdx.x) * VW, tb = blockIdx.x;
  const bool live = k0 < C;
  const int k = live ? k0 : C - VW;
  float wr[8][VW];
  load_taps<VW>(w, k, K, wr);
  float acc[8][VW];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < VW; ++e) acc[j][e] = 0.f;
  const int tend = min(N, (tb + 1) * TOKB);
  for (int t0 = tb * TOKB; t0 < tend; t0 += TG) {
    conv_dx_group<VW, KT>(cprev, sp, sc, N, K, dy, wr, C, k, live, t0, dx);
    conv_dw_group<VW, KT>(cprev, N, K, x, dy, C, k, t0, tend, acc);
  }
  if (!live) return;
#pragma unroll
  for (int e = 0; e < VW; ++e)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < K) part[((size_t)tb * C + k + e) * K + j] = acc[j][e];
}

__global__ __launch_bounds__(TH) void conv_dw_sum(const float* __restrict__ part, int nb, int C, int K,
                                                  float* __restrict__ dw) {
  const int i = blockIdx.x * TH + threadIdx.x;  // k * K + j
  if (i >= C * K) return;
  float s = 0.f;
  for (int b = 0; b < nb; ++b) s += part[(size_t)b * C * K + i];
  dw[i] = s;
}

}  // namespace ssm
}  // namespace ta

using namespace ta;

namespace {
struct RouteDev {
  const int4* ch;
  const int32_t *cprev, *succ_ptr, *succ;
};
RouteDev dev_tables(const ta_route* R, const void* d) {
  const char* b = (const char*)d;
  return {(const int4*)(b + R->off_chunks), (const int32_t*)(b + R->off_cprev), (const int32_t*)(b + R->off_succ_ptr),
          (const int32_t*)(b + R->off_succ)};
}
size_t scan_ws(const ta_route* R, int C) { return align256((size_t)R->n_chunks * C * sizeof(float)) * 4; }
size_t conv_ws(const ta_route* R, int C) {
  return align256((size_t)((R->n_tokens + ssm::TOKB - 1) / ssm::TOKB) * C * R->conv_k * sizeof(float));
}
}  // namespace

extern "C" ta_status tree_route_upload(const ta_route* R, void* droute, size_t bytes, hipStream_t stream) {
  if (!R || !droute) return TA_EINVAL;
  if (bytes < R->device_bytes) return TA_ENOMEM;
  char* b = (char*)droute;
  struct Part {
    size_t off;
    const std::vector<int32_t>* v;
  } parts[] = {{R->off_chunks, &R->chunks}, {R->off_cprev, &R->cprev}, {R->off_succ_ptr, &R->succ_ptr},
               {R->off_succ, &R->succ}};
  for (const Part& x : parts) {
    if (x.v->empty()) continue;
    if (hipMemcpyAsync(b + x.off, x.v->data(), x.v->size() * 4, hipMemcpyHostToDevice, stream) != hipSuccess)
      return TA_EHIP;
  }
  return TA_OK;
}

extern "C" ta_status tree_scan_ws_bytes(const ta_route* R, int32_t C, size_t* bytes) {
  if (!R || !bytes || C <= 0) return TA_EINVAL;
  *bytes = scan_ws(R, C);
  return TA_OK;
}

extern "C" ta_status tree_conv_ws_bytes(const ta_route* R, int32_t C, size_t* bytes) {
  if (!R || !bytes || C <= 0) return TA_EINVAL;
  *bytes = conv_ws(R, C);
  return TA_OK;
}

extern "C" ta_status tree_scan_fwd(const ta_route* R, const void* droute, const float* a, const float* b, int32_t C,
                                   float* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!R || !droute || !a || !b || !h || C <= 0) return TA_EINVAL;
  if ((int64_t)R->n_tokens * C > ((int64_t)1 << 40)) return TA_ERANGE;
  if (R->n_chunks == 0) return TA_OK;
  const size_t need = scan_ws(R, C);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  const RouteDev d = dev_tables(R, droute);
  const size_t seg = need / 4;
  float* A = (float*)ws;
  float* H = (float*)((char*)ws + seg);
  float* hin = (float*)((char*)ws + 2 * seg);
  float* hend = (float*)((char*)ws + 3 * seg);
  const int cb = (C + ssm::TH - 1) / ssm::TH;
  hipLaunchKernelGGL(ssm::scan_reduce, dim3(R->n_chunks, cb), dim3(ssm::TH), 0, stream, d.ch, a, b, C, A, H);
  TA_LAUNCH_CHECK();
  const size_t lds = (size_t)R->n_chunks * ssm::WC * sizeof(float);
  if (lds <= ssm::LDS_WALK_MAX)
    hipLaunchKernelGGL(ssm::scan_walk_lds, dim3((C + ssm::WC - 1) / ssm::WC), dim3(ssm::WC), lds, stream, d.ch,
                       R->n_chunks, (const float*)A, (const float*)H, C, hin, hend);
  else
    hipLaunchKernelGGL(ssm::scan_walk, dim3(cb), dim3(ssm::TH), 0, stream, d.ch, R->n_chunks, (const float*)A,
                       (const float*)H, C, hin, hend);
  TA_LAUNCH_CHECK();
  hipLaunchKernelGGL(ssm::scan_apply, dim3(R->n_chunks, cb), dim3(ssm::TH), 0, stream, d.ch, a, b, C,
                     (const float*)hin, h);
  TA_LAUNCH_CHECK();
  return TA_OK;
}

extern "C" ta_status tree_scan_bwd(const ta_route* R, const void* droute, const float* a, const float* h,
                                   const float* dh, int32_t C, float* da, float* db, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!R || !droute || !a || !h || !dh || !da || !db || C <= 0) return TA_EINVAL;
  if ((int64_t)R->n_tokens * C > ((int64_t)1 << 40)) return TA_ERANGE;
  if (R->n_chunks == 0) return TA_OK;
  const size_t need = scan_ws(R, C);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  const RouteDev d = dev_tables(R, droute);
  const size_t seg = need / 4;
  float* U = (float*)ws;
  float* B = (float*)((char*)ws + seg);
  float* gin = (float*)((char*)ws + 2 * seg);
  const int cb = (C + ssm::TH - 1) / ssm::TH;
  hipLaunchKernelGGL(ssm::scan_reduce_bwd, dim3(R->n_chunks, cb), dim3(ssm::TH), 0, stream, d.ch, a, dh, C, U, B);
  TA_LAUNCH_CHECK();
  const size_t lds = (size_t)R->n_chunks * ssm::WC * sizeof(float);
  if (lds <= ssm::LDS_WALK_MAX)
    hipLaunchKernelGGL(ssm::scan_walk_bwd_lds, dim3((C + ssm::WC - 1) / ssm::WC), dim3(ssm::WC), lds, stream, d.ch,
                       R->n_chunks, a, (const float*)U, (const float*)B, C, gin);
  else
    hipLaunchKernelGGL(ssm::scan_walk_bwd, dim3(cb), dim3(ssm::TH), 0, stream, d.ch, R->n_chunks, a,
                       (const float*)U, (const float*)B, C, gin);
  TA_LAUNCH_CHECK();
  hipLaunchKernelGGL(ssm::scan_apply_bwd, dim3(R->n_chunks, cb), dim3(ssm::TH), 0, stream, d.ch, a, h, dh, C,
                     (const float*)gin, da, db);
  TA_LAUNCH_CHECK();
  return TA_OK;
}

namespace {

// The conv launches for channel width VW and register-window width KT
// (conv_k when it is 2..4, else 0: gather only).
template <int VW, int KT>
void launch_conv_fwd(const ta_route* R, const RouteDev& d, const float* x, const float* w, int C, float* y,
                     hipStream_t st) {
  const int cb = (C / VW + ssm::TH - 1) / ssm::TH;
  hipLaunchKernelGGL((ssm::conv_fwd<VW, KT>), dim3((R->n_tokens + ssm::TG - 1) / ssm::TG, cb), dim3(ssm::TH), 0, st,
                     d.cprev, R->n_tokens, R->conv_k, x, w, C, y);
}

template <int VW, int KT>
void launch_conv_bwd(const ta_route* R, const RouteDev& d, const float* x, const float* w, const float* dy, int C,
                     float* dx, float* part, hipStream_t st) {
  const int cb = (C / VW + ssm::TH - 1) / ssm::TH;
  const int nb = (R->n_tokens + ssm::TOKB - 1) / ssm::TOKB;
  hipLaunchKernelGGL((ssm::conv_bwd<VW, KT>), dim3(nb, cb), dim3(ssm::TH), 0, st, d.cprev, d.succ_ptr, d.succ,
                     R->n_tokens, R->conv_k, x, dy, w, C, dx, part);
}

template <int VW>
void conv_fwd_k(const ta_route* R, const RouteDev& d, const float* x, const float* w, int C, float* y,
                hipStream_t st) {
  switch (R->conv_k) {
    case 2: launch_conv_fwd<VW, 2>(R, d, x, w, C, y, st); break;
    case 3: launch_conv_fwd<VW, 3>(R, d, x, w, C, y, st); break;
    case 4: launch_conv_fwd<VW, 4>(R, d, x, w, C, y, st); break;
    default: launch_conv_fwd<VW, 0>(R, d, x, w, C, y, st); break;
  }
}

template <int VW>
void conv_bwd_k(const ta_route* R, const RouteDev& d, const float* x, const float* w, const float* dy, int C,
                float* dx, float* part, hipStream_t st) {
  switch (R->conv_k) {
    case 2: launch_conv_bwd<VW, 2>(R, d, x, w, dy, C, dx, part, st); break;
    case 3: launch_conv_bwd<VW, 3>(R, d, x, w, dy, C, dx, part, st); break;
    case 4: launch_conv_bwd<VW, 4>(R, d, x, w, dy, C, dx, part, st); break;
    default: launch_conv_bwd<VW, 0>(R, d, x, w, dy, C, dx, part, st); break;
  }
}

}  // namespace

extern "C" ta_status tree_conv_fwd(const ta_route* R, const void* droute, const float* x, const float* w, int32_t C,
                                   float* y, hipStream_t stream) {
  if (!R || !droute || !x || !w || !y || C <= 0) return TA_EINVAL;
  if (R->n_tokens == 0) return TA_OK;
  const RouteDev d = dev_tables(R, droute);
  if (C % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)y % 16 == 0)
    conv_fwd_k<4>(R, d, x, w, C, y, stream);
  else
    conv_fwd_k<1>(R, d, x, w, C, y, stream);
  TA_LAUNCH_CHECK();
  return TA_OK;
}

extern "C" ta_status tree_conv_bwd(const ta_route* R, const void* droute, const float* x, const float* w,
                                   const float* dy, int32_t C, float* dx, float* dw, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!R || !droute || !x || !w || !dy || !dx || !dw || C <= 0) return TA_EINVAL;
  if (R->n_tokens == 0) return TA_OK;
  const size_t need = conv_ws(R, C);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  const RouteDev d = dev_tables(R, droute);
  const int nb = (R->n_tokens + ssm::TOKB - 1) / ssm::TOKB;
  if (C % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)dy % 16 == 0 && (uintptr_t)dx % 16 == 0)
    conv_bwd_k<4>(R, d, x, w, dy, C, dx, (float*)ws, stream);
  else
    conv_bwd_k<1>(R, d, x, w, dy, C, dx, (float*)ws, stream);
  TA_LAUNCH_CHECK();
  hipLaunchKernelGGL(ssm::conv_dw_sum, dim3((C * R->conv_k + ssm::TH - 1) / ssm::TH), dim3(ssm::TH), 0, stream,
                     (const float*)ws, nb, C, R->conv_k, dw);
  TA_LAUNCH_CHECK();
  return TA_OK;
}
