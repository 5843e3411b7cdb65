// Tree-routed linear recurrence and causal convolution over DFS-packed tokens
// (Tree Training post, section 9).  Rows are tokens, C channels per row, fp32.
//
// Scan h_t = a_t h_prev(t) + b_t, prev(t) following the root-to-token path
// (section 9.1: a chunk starts from its parent's end state).  Chunks of up to
// 128 tokens form a tree (parent = the previous chunk of the node, or the
// last chunk of the nearest ancestor holding tokens).  One pass per
// direction: a workgroup per (chunk, channel block) scans its chunk from
// registers once the parent chunk's end state (forward) or the child chunks'
// outgoing gradients (backward: the sum over branches a shared prefix
// receives) have been published, so each element is read and written once
// (see the kernels below).
//
// Causal conv y_t = sum_j w[c][j] x_{prev^j(t)} (section 9.2: the window runs
// back along the path into the parent's tail): a gather over the planner's
// predecessor table; its backward gathers over the inverse table (dx) and
// reduces over tokens in a fixed order (dw), so no atomics.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>

#include "common.h"
#include "route_internal.h"

namespace ta {
namespace ssm {

constexpr int TH = 256;

// VW consecutive channels per lane (VW = 4: 16-byte accesses when C % 4 == 0).
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

// Single pass.  One workgroup per (chunk, 64 VW channels): 128 / SG
// wavefronts of SG tokens each cover a chunk (at most 128 tokens), lane l
// holds channels VW l .. VW l + VW - 1 of the block.  The workgroups take
// their (chunk, channel block) from a ticket counter in the route's chunk
// order (parents first; reversed for the backward), so a chunk waits only on
// chunks whose workgroups took a smaller ticket and are already running or
// done: every wait ends.  Each wavefront keeps its segment's inputs in
// registers, so every element is read once and written once:
//   forward:  per segment the decay A = prod a and the end state H from a
//             zero start; the chunk's start state is its parent chunk's end
//             state, published by the parent's workgroup; segment starts
//             follow by composing the segments before (s <- A s + H, in
//             segment order); the scan from there writes h, and the chunk's
//             last state is published for its children.
//   backward: per segment the local reverse scan from the segment's end with
//             nothing coming in (U = dh at its first token, B = prod of a
//             after it); the chunk's incoming gradient is the sum over its
//             child chunks (in the route's fixed order) of a_first dh_first,
//             published by the children's workgroups -- the sum over branches
//             a shared prefix receives; segment incomings follow from the
//             last segment down; the reverse scan writes da = dh h_prev and
//             db = dh, and the chunk publishes a_first dh_first.
// A published value is one 64-bit word per (chunk, channel): flag in the high
// half, the fp32 value in the low half, written and polled with agent-scope
// atomics, so value and flag arrive together on every XCD.  Every result is
// a fixed sequence of operations whatever the timing: bitwise repeatable.
// The waits are bounded (SPIN_MAX polls); a wait that runs out (which the
// ticket order rules out) sets the workspace's timeout word and goes on with
// zero, so the kernel always exits.
constexpr int SCAN_CHUNK = 128;  // most tokens a route chunk holds
constexpr int SPIN_MAX = 1 << 22;  // polls of at least ~100 cycles each: seconds, far past any real wait

// The sum, in list order, of the VW-channel values published at
// p + idx[e] * stride for e in [e0, e1) (idx null: the single index e0);
// up to four of them are polled together.
template <int VW>
__device__ __forceinline__ void wait_sum(const uint64_t* p, const int32_t* idx, int e0, int e1, size_t stride,
                                         uint32_t* timeout, float (&sum)[VW]) {
#pragma unroll
  for (int x = 0; x < VW; ++x) sum[x] = 0.f;
  for (int e = e0; e < e1; e += 4) {
    const int m = min(4, e1 - e);
    const uint64_t* q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = p + (size_t)(idx ? idx[e + min(j, m - 1)] : e0) * stride;
    uint64_t v[4][VW];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int x = 0; x < VW; ++x) v[j][x] = 0;
    bool all = false;
    for (int it = 0; it < SPIN_MAX && !all; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int x = 0; x < VW; ++x)
          if (j < m && !(v[j][x] >> 32)) v[j][x] = __hip_atomic_load(q[j] + x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      all = true;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int x = 0; x < VW; ++x) all = all && (j >= m || (v[j][x] >> 32));
      if (!all) __builtin_amdgcn_s_sleep(2);
    }
    if (!all) __hip_atomic_store(timeout, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int x = 0; x < VW; ++x)
        if (j < m) sum[x] += __uint_as_float((uint32_t)v[j][x]);
  }
}
__device__ __forceinline__ void publish(uint64_t* p, float x) {
  __hip_atomic_store(p, (1ull << 32) | __float_as_uint(x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Clears the workspace header (ticket counter, timeout word) and the
// published words before a pass (a kernel, not a memset: callers may capture
// the calls in a graph).
__global__ __launch_bounds__(TH) void scan_clear(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * TH + threadIdx.x; i < n16; i += (size_t)gridDim.x * TH) p[i] = uint4{0, 0, 0, 0};
}

template <int VW, int SG>
__global__ __launch_bounds__(64 * (SCAN_CHUNK / SG)) void scan_fwd(const int4* __restrict__ ch,
                                                                   const int32_t* __restrict__ order, int nkb,
                                                                   const float* __restrict__ a,
                                                                   const float* __restrict__ b, int C,
                                                                   float* __restrict__ h, uint32_t* hdr, uint64_t* pub) {
  constexpr int NW = SCAN_CHUNK / SG;
  typedef Vec<VW> VV;
  typedef typename VV::T V;
  __shared__ int s_ticket;
  __shared__ V sA[NW][64], sH[NW][64], s0[64];
  if (threadIdx.x == 0) s_ticket = (int)atomicAdd(hdr, 1u);
  __syncthreads();
  const int t = s_ticket, q = t / nkb, kb = t - q * nkb, c = order[q];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k0 = (kb * 64 + lane) * VW;
  const bool live = k0 < C;
  const int k = live ? k0 : C - VW;
  const int4 r = ch[c];
  const int i0 = w * SG, n = max(0, min(SG, r.y - i0));
  const size_t o = (size_t)(r.x + i0) * C + k;
  // (rows past the segment's end repeat its last row: loads without branches)
  V av[SG], bv[SG];
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < SG; ++i) {
      const size_t oi = o + (size_t)min(i, n - 1) * C;
      av[i] = *(const V*)(a + oi);
      bv[i] = *(const V*)(b + oi);
    }
  }
  V A, H;
#pragma unroll
  for (int x = 0; x < VW; ++x) {
    float pa = 1.f, ph = 0.f;
#pragma unroll
    for (int i = 0; i < SG; ++i)
      if (i < n) {
        ph = fmaf(VV::get(av[i], x), ph, VV::get(bv[i], x));
        pa *= VV::get(av[i], x);
      }
    VV::set(A, x, pa);
    VV::set(H, x, ph);
  }
  sA[w][lane] = A;
  sH[w][lane] = H;
  if (w == 0) {
    float st[VW];
    if (r.z >= 0) {
      wait_sum<VW>(pub + k, nullptr, r.z, r.z + 1, (size_t)C, hdr + 1, st);
    } else {
#pragma unroll
      for (int x = 0; x < VW; ++x) st[x] = 0.f;
    }
    V sv;
#pragma unroll
    for (int x = 0; x < VW; ++x) VV::set(sv, x, st[x]);
    s0[lane] = sv;
  }
  __syncthreads();
  if (n == 0) return;
  float s[VW];
#pragma unroll
  for (int x = 0; x < VW; ++x) s[x] = VV::get(s0[lane], x);
  for (int u = 0; u < w; ++u) {
    const V pa = sA[u][lane], ph = sH[u][lane];
#pragma unroll
    for (int x = 0; x < VW; ++x) s[x] = fmaf(VV::get(pa, x), s[x], VV::get(ph, x));
  }
#pragma unroll
  for (int i = 0; i < SG; ++i)
    if (i < n) {
      V y;
#pragma unroll
      for (int x = 0; x < VW; ++x) {
        s[x] = fmaf(VV::get(av[i], x), s[x], VV::get(bv[i], x));
        VV::set(y, x, s[x]);
      }
      if (live) *(V*)(h + o + (size_t)i * C) = y;
    }
  if (live && i0 + n == r.y)
#pragma unroll
    for (int x = 0; x < VW; ++x) publish(pub + (size_t)c * C + k + x, s[x]);
}

template <int VW, int SG>
__global__ __launch_bounds__(64 * (SCAN_CHUNK / SG)) void scan_bwd(
    const int4* __restrict__ ch, const int32_t* __restrict__ order, const int32_t* __restrict__ kid_ptr,
    const int32_t* __restrict__ kid, int n_chunks, int nkb, const float* __restrict__ a, const float* __restrict__ h,
    const float* __restrict__ g, int C, float* __restrict__ da, float* __restrict__ db, uint32_t* hdr,
    uint64_t* pub) {
  constexpr int NW = SCAN_CHUNK / SG;
  typedef Vec<VW> VV;
  typedef typename VV::T V;
  __shared__ int s_ticket;
  __shared__ V sU[NW][64], sB[NW][64], sF[NW][64], sG[64];
  if (threadIdx.x == 0) s_ticket = (int)atomicAdd(hdr, 1u);
  __syncthreads();
  const int t = s_ticket, q = t / nkb, kb = t - q * nkb, c = order[n_chunks - 1 - q];
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int k0 = (kb * 64 + lane) * VW;
  const bool live = k0 < C;
  const int k = live ? k0 : C - VW;
  const int4 r = ch[c];
  const int i0 = w * SG, n = max(0, min(SG, r.y - i0));
  const size_t o = (size_t)(r.x + i0) * C + k;
  // a, dh and h_prev of the segment's tokens (h_prev of the chunk's first
  // token: the token before it on the path, or zero at a root)
  V av[SG], gv[SG], hv[SG];
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < SG; ++i) {
      const int ii = min(i, n - 1);
      const size_t oi = o + (size_t)ii * C;
      av[i] = *(const V*)(a + oi);
      gv[i] = *(const V*)(g + oi);
      if (i0 + ii > 0) {
        hv[i] = *(const V*)(h + (size_t)(r.x + i0 + ii - 1) * C + k);
      } else if (r.w >= 0) {
        hv[i] = *(const V*)(h + (size_t)r.w * C + k);
      } else {
#pragma unroll
        for (int x = 0; x < VW; ++x) VV::set(hv[i], x, 0.f);
      }
    }
  }
  // local reverse scan: u = g_i + a_{i+1} u from the segment's end
  V U, B, F;
#pragma unroll
  for (int x = 0; x < VW; ++x) {
    float u = 0.f, dec = 1.f, an = 0.f;
#pragma unroll
    for (int i = SG - 1; i >= 0; --i)
      if (i < n) {
        u = fmaf(an, u, VV::get(gv[i], x));
        if (i + 1 < n) dec *= an;
        an = VV::get(av[i], x);
      }
    VV::set(U, x, u);
    VV::set(B, x, dec);
    VV::set(F, x, n > 0 ? VV::get(av[0], x) : 0.f);
  }
  sU[w][lane] = U;
  sB[w][lane] = B;
  sF[w][lane] = F;
  if (w == 0) {
    float gin[VW];
    wait_sum<VW>(pub + k, kid, kid_ptr[c], kid_ptr[c + 1], (size_t)C, hdr + 1, gin);
    V gv0;
#pragma unroll
    for (int x = 0; x < VW; ++x) VV::set(gv0, x, gin[x]);
    sG[lane] = gv0;
  }
  __syncthreads();
  if (n == 0) return;
  // the gradient arriving at this segment's last token from after it
  const int last = (r.y - 1) / SG;
  float dh[VW];
#pragma unroll
  for (int x = 0; x < VW; ++x) dh[x] = VV::get(sG[lane], x);
  for (int v = last; v > w; --v) {
    const V f = sF[v][lane], bb = sB[v][lane], uu = sU[v][lane];
#pragma unroll
    for (int x = 0; x < VW; ++x) dh[x] = VV::get(f, x) * fmaf(VV::get(bb, x), dh[x], VV::get(uu, x));
  }
  float an[VW];
#pragma unroll
  for (int x = 0; x < VW; ++x) an[x] = 1.f;
#pragma unroll
  for (int i = SG - 1; i >= 0; --i)
    if (i < n) {
      V vb, va;
#pragma unroll
      for (int x = 0; x < VW; ++x) {
        dh[x] = fmaf(an[x], dh[x], VV::get(gv[i], x));
        VV::set(vb, x, dh[x]);
        VV::set(va, x, dh[x] * VV::get(hv[i], x));
        an[x] = VV::get(av[i], x);
      }
      if (live) {
        *(V*)(db + o + (size_t)i * C) = vb;
        *(V*)(da + o + (size_t)i * C) = va;
      }
    }
  if (live && w == 0)
#pragma unroll
    for (int x = 0; x < VW; ++x) publish(pub + (size_t)c * C + k + x, VV::get(av[0], x) * dh[x]);
}

// Causal conv over the path: y[t][k] = sum_j w[k][j] x[prev^j(t)][k].  VW
// consecutive channels per lane (VW = 4: 16-byte accesses when C % 4 == 0).

// A block covers TG tokens x (TH * VW) channels; each lane holds its
// channels' taps in registers for all TG tokens.
constexpr int TG = 8;  // (4 or 16 tokens per forward block: 39% and 1% slower)
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
                                               const float* __restrict__ w, int C, int cb, float* __restrict__ y) {
  typedef typename Vec<VW>::T V;
  // channel blocks innermost: consecutive blocks cover one token group's whole rows
  const int tg = blockIdx.x / cb, kb = blockIdx.x - tg * cb;
  const int k0 = (kb * TH + threadIdx.x) * VW;
  const bool live = k0 < C;
  const int k = live ? k0 : C - VW;
  float wr[8][VW];
  load_taps<VW>(w, k, K, wr);
  const int t0 = tg * TG;
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
constexpr int TOKB = 256;  // (64 or 128: 37% and 22% slower, most of it in summing the partials)
template <int VW, int KT>
__global__ __launch_bounds__(TH) void conv_bwd(const int32_t* __restrict__ cprev, const int32_t* __restrict__ sp,
                                               const int32_t* __restrict__ sc, int N, int K,
                                               const float* __restrict__ x, const float* __restrict__ dy,
                                               const float* __restrict__ w, int C, float* __restrict__ dx,
                                               int cb, float* __restrict__ part) {
  const int tb = blockIdx.x / cb, kb = blockIdx.x - tb * cb;  // channel blocks innermost
  const int k0 = (kb * TH + threadIdx.x) * VW;
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
  const int32_t *cprev, *succ_ptr, *succ, *kid_ptr, *kid, *order;
};
RouteDev dev_tables(const ta_route* R, const void* d) {
  const char* b = (const char*)d;
  return {(const int4*)(b + R->off_chunks),    (const int32_t*)(b + R->off_cprev), (const int32_t*)(b + R->off_succ_ptr),
          (const int32_t*)(b + R->off_succ),   (const int32_t*)(b + R->off_kid_ptr),
          (const int32_t*)(b + R->off_kid),    (const int32_t*)(b + R->off_order)};
}
// scan workspace: a 256-byte header (ticket counter, timeout word), then one
// published 64-bit word per (chunk, channel)
constexpr size_t SCAN_HDR = 256;
size_t scan_ws(const ta_route* R, int C) { return SCAN_HDR + align256((size_t)R->n_chunks * C * sizeof(uint64_t)); }
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
  } parts[] = {{R->off_chunks, &R->chunks},   {R->off_cprev, &R->cprev}, {R->off_succ_ptr, &R->succ_ptr},
               {R->off_succ, &R->succ},       {R->off_kid_ptr, &R->kid_ptr}, {R->off_kid, &R->kid},
               {R->off_order, &R->order}};
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

namespace {
// Clears the scan workspace and returns its header and published words.
ta_status scan_prepare(const ta_route* R, int C, void* ws, size_t ws_bytes, hipStream_t stream, uint32_t** hdr,
                       uint64_t** pub) {
  const size_t need = scan_ws(R, C);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  if (R->chunk > ssm::SCAN_CHUNK) return TA_EUNSUPPORTED;
  const size_t n16 = need / 16;
  hipLaunchKernelGGL(ssm::scan_clear, dim3((unsigned)std::min<size_t>((n16 + ssm::TH - 1) / ssm::TH, 2048)),
                     dim3(ssm::TH), 0, stream, (uint4*)ws, n16);
  TA_LAUNCH_CHECK();
  *hdr = (uint32_t*)ws;
  *pub = (uint64_t*)((char*)ws + SCAN_HDR);
  return TA_OK;
}

// 16-byte channel vectors (VW = 4) when every row is 16-byte aligned, with
// SG = 16 tokens per wavefront: a 512-thread workgroup covers a chunk x 256
// channels and each row access is one contiguous KiB (8-token segments with
// 1,024 threads ran the forward 2% slower; the backward, holding three inputs
// per token, would spill there); else one channel per lane, SG = 32.
constexpr int SCAN_SG4 = 16, SCAN_SG1 = 32;
bool scan_vec4(int C, std::initializer_list<const void*> ptrs) {
  if (C % 4) return false;
  for (const void* p : ptrs)
    if ((uintptr_t)p % 16) return false;
  return true;
}
// A launch's work-items (blocks x threads) must stay below 2^32.
bool grid_fits(uint64_t blocks, int threads) { return blocks * (uint64_t)threads < (1ull << 32); }
int scan_blocks(const ta_route* R, int C, int vw, unsigned* grid) {
  const int nkb = (C + 64 * vw - 1) / (64 * vw);
  if (!grid_fits((uint64_t)R->n_chunks * nkb, 64 * (ssm::SCAN_CHUNK / SCAN_SG4))) return -1;
  *grid = (unsigned)(R->n_chunks * nkb);
  return nkb;
}
}  // namespace

extern "C" ta_status tree_scan_fwd(const ta_route* R, const void* droute, const float* a, const float* b, int32_t C,
                                   float* h, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!R || !droute || C <= 0) return TA_EINVAL;
  if (R->n_chunks == 0) return TA_OK;  // no tokens: nothing to read or write
  if (!a || !b || !h) return TA_EINVAL;
  if ((int64_t)R->n_tokens * C > ((int64_t)1 << 40)) return TA_ERANGE;
  const bool v4 = scan_vec4(C, {a, b, h});
  unsigned grid;
  const int nkb = scan_blocks(R, C, v4 ? 4 : 1, &grid);
  if (nkb < 0) return TA_ERANGE;
  uint32_t* hdr;
  uint64_t* pub;
  const ta_status st = scan_prepare(R, C, ws, ws_bytes, stream, &hdr, &pub);
  if (st != TA_OK) return st;
  const RouteDev d = dev_tables(R, droute);
  if (v4)
    hipLaunchKernelGGL((ssm::scan_fwd<4, SCAN_SG4>), dim3(grid), dim3(64 * (ssm::SCAN_CHUNK / SCAN_SG4)), 0, stream,
                       d.ch, d.order, nkb, a, b, C, h, hdr, pub);
  else
    hipLaunchKernelGGL((ssm::scan_fwd<1, SCAN_SG1>), dim3(grid), dim3(64 * (ssm::SCAN_CHUNK / SCAN_SG1)), 0, stream,
                       d.ch, d.order, nkb, a, b, C, h, hdr, pub);
  TA_LAUNCH_CHECK();
  return TA_OK;
}

extern "C" ta_status tree_scan_bwd(const ta_route* R, const void* droute, const float* a, const float* h,
                                   const float* dh, int32_t C, float* da, float* db, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  if (!R || !droute || C <= 0) return TA_EINVAL;
  if (R->n_chunks == 0) return TA_OK;  // no tokens: nothing to read or write
  if (!a || !h || !dh || !da || !db) return TA_EINVAL;
  if ((int64_t)R->n_tokens * C > ((int64_t)1 << 40)) return TA_ERANGE;
  const bool v4 = scan_vec4(C, {a, h, dh, da, db});
  unsigned grid;
  const int nkb = scan_blocks(R, C, v4 ? 4 : 1, &grid);
  if (nkb < 0) return TA_ERANGE;
  uint32_t* hdr;
  uint64_t* pub;
  const ta_status st = scan_prepare(R, C, ws, ws_bytes, stream, &hdr, &pub);
  if (st != TA_OK) return st;
  const RouteDev d = dev_tables(R, droute);
  if (v4)
    hipLaunchKernelGGL((ssm::scan_bwd<4, SCAN_SG4>), dim3(grid), dim3(64 * (ssm::SCAN_CHUNK / SCAN_SG4)), 0, stream,
                       d.ch, d.order, d.kid_ptr, d.kid, R->n_chunks, nkb, a, h, dh, C, da, db, hdr, pub);
  else
    hipLaunchKernelGGL((ssm::scan_bwd<1, SCAN_SG1>), dim3(grid), dim3(64 * (ssm::SCAN_CHUNK / SCAN_SG1)), 0, stream,
                       d.ch, d.order, d.kid_ptr, d.kid, R->n_chunks, nkb, a, h, dh, C, da, db, hdr, pub);
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
  const unsigned ntg = (unsigned)((R->n_tokens + ssm::TG - 1) / ssm::TG);
  hipLaunchKernelGGL((ssm::conv_fwd<VW, KT>), dim3(ntg * cb), dim3(ssm::TH), 0, st, d.cprev, R->n_tokens,
                     R->conv_k, x, w, C, cb, y);
}

template <int VW, int KT>
void launch_conv_bwd(const ta_route* R, const RouteDev& d, const float* x, const float* w, const float* dy, int C,
                     float* dx, float* part, hipStream_t st) {
  const int cb = (C / VW + ssm::TH - 1) / ssm::TH;
  const int nb = (R->n_tokens + ssm::TOKB - 1) / ssm::TOKB;
  hipLaunchKernelGGL((ssm::conv_bwd<VW, KT>), dim3((unsigned)nb * cb), dim3(ssm::TH), 0, st, d.cprev, d.succ_ptr,
                     d.succ, R->n_tokens, R->conv_k, x, dy, w, C, dx, cb, part);
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
  if (!R || !droute || C <= 0) return TA_EINVAL;
  if (R->n_tokens == 0) return TA_OK;  // nothing to read or write
  if (!x || !w || !y) return TA_EINVAL;
  if (!grid_fits((uint64_t)((R->n_tokens + ssm::TG - 1) / ssm::TG) * ((C + ssm::TH - 1) / ssm::TH), ssm::TH))
    return TA_ERANGE;
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
  if (!R || !droute || C <= 0) return TA_EINVAL;
  if (R->n_tokens == 0) {  // no tokens: dw = 0, nothing else to read or write
    if (!dw) return TA_EINVAL;
    hipLaunchKernelGGL(ssm::conv_dw_sum, dim3((C * R->conv_k + ssm::TH - 1) / ssm::TH), dim3(ssm::TH), 0, stream,
                       (const float*)nullptr, 0, C, R->conv_k, dw);
    TA_LAUNCH_CHECK();
    return TA_OK;
  }
  if (!x || !w || !dy || !dx || !dw) return TA_EINVAL;
  const int nb = (R->n_tokens + ssm::TOKB - 1) / ssm::TOKB;
  if (!grid_fits((uint64_t)nb * ((C + ssm::TH - 1) / ssm::TH), ssm::TH)) return TA_ERANGE;
  const size_t need = conv_ws(R, C);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  const RouteDev d = dev_tables(R, droute);
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
