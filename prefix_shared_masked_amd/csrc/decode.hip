// Split-KV single-query decode with a log-depth (max, numerator, denominator)
// merge (Tree Attention notes: the three mergeable quantities, their
// associativity, and the decode algorithm -- local attention per KV shard,
// global max, rescaled sums, z = n/d).  On one GPU the shards are KV slices
// handled by different workgroups, and the "AllReduce" is a pairwise merge
// tree of depth ceil(log2 S) over the S slices.
//
// Partial kernel: one workgroup per (slice, KV head x group of <= 4 query
// heads, batch item).  Decode is HBM-bound (each KV byte is used for a
// handful of FLOPs), so the kernel is a streaming loop: eight lanes cover a
// 256-byte K or V row with 32-byte loads, a wavefront walks 32 rows per
// step, scores are reduced across the eight lanes and the running
// (m, l, o) is updated once per block of four keys per lane group.
// Merge kernel: one workgroup per (batch item, query head); round r merges
// slice pairs (i, i + 2^r) in parallel over the head dimension.
#include "common.h"

namespace ta {
namespace dec {

constexpr int D = 128;
constexpr int HG = 4;   // query heads per workgroup
constexpr int KB = 4;   // keys per lane group per step
constexpr int MAX_SPLITS = 120;  // merge keeps S x (2 + D) floats in 64 KB of LDS

__device__ __forceinline__ void bf16x16_to_f32(const uint4& a, const uint4& b, float* f) {
  const uint32_t u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = __uint_as_float(u[i] << 16);
    f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

struct Params {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const int32_t* span_ptr;
  const int32_t* spans;
  float* part;  // [B, Hq, S] x (2 + D): m (log2 units), l, o[D]
  int B, Hq, Hkv, G, S;
  float scale_log2;
};

__global__ __launch_bounds__(256) void partial_kernel(Params P) {
  __shared__ float sh_m[4][HG], sh_l[4][HG], sh_o[4][HG][D];
  const int split = blockIdx.x;
  const int kvh = blockIdx.y % P.Hkv, hgrp = blockIdx.y / P.Hkv;
  const int b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int kl = lane >> 3, dp = lane & 7;
  const int nh = min(HG, P.G - hgrp * HG);
  const int h0 = kvh * P.G + hgrp * HG;

  // this item's total length and this workgroup's slice of it
  const int sp0 = P.span_ptr[b], sp1 = P.span_ptr[b + 1];
  int L = 0;
  for (int s = sp0; s < sp1; ++s) L += P.spans[2 * s + 1];
  const int per = (((L + P.S - 1) / P.S) + 31) & ~31;
  const int vs = min(L, split * per), ve = min(L, vs + per);

  float qv[HG][16];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    const int h = hh < nh ? h0 + hh : h0;
    const bf16* qr = P.q + ((size_t)b * P.Hq + h) * D + dp * 16;
    const uint4 a = *(const uint4*)qr, c = *(const uint4*)(qr + 8);
    bf16x16_to_f32(a, c, qv[hh]);
#pragma unroll
    for (int e = 0; e < 16; ++e) qv[hh][e] *= P.scale_log2;
  }
  float m[HG], l[HG], o[HG][16];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[hh][e] = 0.f;
  }

  // walk the spans that overlap [vs, ve) in virtual order
  int base = 0;
  for (int s = sp0; s < sp1 && base < ve; ++s) {
    const int st = P.spans[2 * s], len = P.spans[2 * s + 1];
    const int lo = max(vs, base), hi = min(ve, base + len);
    for (int v0 = lo + wave * (8 * KB); v0 < hi; v0 += 4 * 8 * KB) {
      float sc[KB][HG];
      int rows[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int vv = v0 + u * 8 + kl;
        rows[u] = vv < hi ? st + (vv - base) : -1;
        float kf[16];
        if (rows[u] >= 0) {
          const bf16* kr = P.k + ((size_t)rows[u] * P.Hkv + kvh) * D + dp * 16;
          bf16x16_to_f32(*(const uint4*)kr, *(const uint4*)(kr + 8), kf);
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) kf[e] = 0.f;
        }
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) a = fmaf(qv[hh][e], kf[e], a);
          sc[u][hh] = a;
        }
      }
#pragma unroll
      for (int u = 0; u < KB; ++u)
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          float a = sc[u][hh];
          a += __shfl_xor(a, 1);
          a += __shfl_xor(a, 2);
          a += __shfl_xor(a, 4);
          sc[u][hh] = rows[u] >= 0 ? a : -INFINITY;
        }
#pragma unroll
      for (int hh = 0; hh < HG; ++hh) {
        float mx = m[hh];
#pragma unroll
        for (int u = 0; u < KB; ++u) mx = fmaxf(mx, sc[u][hh]);
        const float muse = mx == -INFINITY ? 0.f : mx;
        const float a = exp2f_fast(m[hh] - muse);
        l[hh] *= a;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[hh][e] *= a;
        m[hh] = mx;
#pragma unroll
        for (int u = 0; u < KB; ++u) sc[u][hh] = exp2f_fast(sc[u][hh] - muse);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        if (rows[u] < 0) continue;
        float vf[16];
        const bf16* vr = P.v + ((size_t)rows[u] * P.Hkv + kvh) * D + dp * 16;
        bf16x16_to_f32(*(const uint4*)vr, *(const uint4*)(vr + 8), vf);
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          l[hh] += sc[u][hh];
#pragma unroll
          for (int e = 0; e < 16; ++e) o[hh][e] = fmaf(sc[u][hh], vf[e], o[hh][e]);
        }
      }
    }
    base += len;
  }

  // merge the eight lane groups of the wavefront (lanes with equal dp)
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const float m2 = __shfl_xor(m[hh], off), l2 = __shfl_xor(l[hh], off);
      const float M = fmaxf(m[hh], m2);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float fa = exp2f_fast(m[hh] - Mu), fb = exp2f_fast(m2 - Mu);
      l[hh] = l[hh] * fa + l2 * fb;
#pragma unroll
      for (int e = 0; e < 16; ++e) o[hh][e] = o[hh][e] * fa + __shfl_xor(o[hh][e], off) * fb;
      m[hh] = M;
    }
  }
  if (kl == 0) {
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      if (dp == 0) {
        sh_m[wave][hh] = m[hh];
        sh_l[wave][hh] = l[hh];
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) sh_o[wave][hh][dp * 16 + e] = o[hh][e];
    }
  }
  __syncthreads();
  // merge the four wavefronts: thread -> (head, d)
  for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh_m[w][hh]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float lt = 0.f, ot = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f_fast(sh_m[w][hh] - Mu);
      lt += sh_l[w][hh] * f;
      ot += sh_o[w][hh][d] * f;
    }
    float* dst = P.part + (((size_t)b * P.Hq + h0 + hh) * P.S + split) * (2 + D);
    if (d == 0) {
      dst[0] = M;
      dst[1] = lt;
    }
    dst[2 + d] = ot;
  }
}

// Log-depth merge: round r combines slices i and i + 2^r for every i that is a
// multiple of 2^(r+1); identity (-inf, 0, 0) never evaluates -inf - -inf.
__global__ __launch_bounds__(1024) void merge_kernel(const float* __restrict__ part, int S, bf16* __restrict__ o,
                                                     float* __restrict__ lse) {
  extern __shared__ float smem[];
  float* sm = smem;          // [S]
  float* sl = sm + S;        // [S]
  float* so = sl + S;        // [S][D]
  const int bh = blockIdx.x;
  const float* src = part + (size_t)bh * S * (2 + D);
  for (int i = threadIdx.x; i < S * D; i += blockDim.x) so[i] = src[(i / D) * (2 + D) + 2 + (i % D)];
  for (int i = threadIdx.x; i < S; i += blockDim.x) {
    sm[i] = src[i * (2 + D)];
    sl[i] = src[i * (2 + D) + 1];
  }
  __syncthreads();
  for (int stride = 1; stride < S; stride <<= 1) {
    const int pairs = (S + 2 * stride - 1) / (2 * stride);
    // numerators of every pair, from the maxima of the previous round
    for (int it = threadIdx.x; it < pairs * D; it += blockDim.x) {
      const int i = (it / D) * 2 * stride, d = it % D, j = i + stride;
      if (j >= S) continue;
      const float M = fmaxf(sm[i], sm[j]);
      const float Mu = M == -INFINITY ? 0.f : M;
      so[i * D + d] = so[i * D + d] * exp2f_fast(sm[i] - Mu) + so[j * D + d] * exp2f_fast(sm[j] - Mu);
    }
    __syncthreads();
    // then the maxima and denominators
    for (int p = threadIdx.x; p < pairs; p += blockDim.x) {
      const int i = p * 2 * stride, j = i + stride;
      if (j >= S) continue;
      const float M = fmaxf(sm[i], sm[j]);
      const float Mu = M == -INFINITY ? 0.f : M;
      sl[i] = sl[i] * exp2f_fast(sm[i] - Mu) + sl[j] * exp2f_fast(sm[j] - Mu);
      sm[i] = M;
    }
    __syncthreads();
  }
  const float l0 = sl[0];
  const float inv = l0 > 0.f ? 1.f / l0 : 0.f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) o[(size_t)bh * D + d] = (bf16)(so[d] * inv);
  if (threadIdx.x == 0) lse[bh] = sm[0] * TA_LN2 + logf(l0);
}

}  // namespace dec
}  // namespace ta

using namespace ta;

namespace {
int32_t pick_splits(int32_t max_len, int32_t n_splits) {
  if (n_splits > 0) return n_splits;
  int32_t s = (max_len + 2047) / 2048;
  return s < 1 ? 1 : (s > dec::MAX_SPLITS ? dec::MAX_SPLITS : s);
}
}  // namespace

extern "C" ta_status tree_decode_ws_bytes(int32_t B, int32_t Hq, int32_t d, int32_t max_len, int32_t n_splits,
                                          size_t* bytes, int32_t* n_splits_out) {
  if (!bytes || B <= 0 || Hq <= 0 || d <= 0 || max_len < 0 || n_splits < 0) return TA_EINVAL;
  const int32_t S = pick_splits(max_len, n_splits);
  if (S > dec::MAX_SPLITS) return TA_EUNSUPPORTED;
  *bytes = align256((size_t)B * Hq * S * (2 + d) * sizeof(float));
  if (n_splits_out) *n_splits_out = S;
  return TA_OK;
}

extern "C" ta_status tree_decode_splitkv(ta_dtype dt, const void* q, const void* k, const void* v,
                                         const int32_t* span_ptr, const int32_t* spans, int32_t B, int32_t Hq,
                                         int32_t Hkv, int32_t d, int32_t max_len, float scale, int32_t n_splits,
                                         void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return tree_decode_splitkv_ex(dt, q, k, v, span_ptr, spans, B, Hq, Hkv, d, max_len, scale, n_splits, o, lse, ws,
                                ws_bytes, nullptr, 0, stream);
}

extern "C" ta_status tree_decode_splitkv_ex(ta_dtype dt, const void* q, const void* k, const void* v,
                                            const int32_t* span_ptr, const int32_t* spans, int32_t B, int32_t Hq,
                                            int32_t Hkv, int32_t d, int32_t max_len, float scale, int32_t n_splits,
                                            void* o, float* lse, void* ws, size_t ws_bytes, hipEvent_t* ev,
                                            int32_t nev, hipStream_t stream) {
  if (dt != TA_BF16 || d != dec::D) return TA_EUNSUPPORTED;
  if (!q || !k || !v || !span_ptr || !spans || !o || !lse) return TA_EINVAL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_len < 0 || n_splits < 0) return TA_EINVAL;
  size_t need;
  int32_t S;
  ta_status st = tree_decode_ws_bytes(B, Hq, d, max_len, n_splits, &need, &S);
  if (st != TA_OK) return st;
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  if (scale <= 0.f) scale = 1.f / sqrtf((float)d);
  dec::Params P;
  P.q = (const bf16*)q;
  P.k = (const bf16*)k;
  P.v = (const bf16*)v;
  P.span_ptr = span_ptr;
  P.spans = spans;
  P.part = (float*)ws;
  P.B = B;
  P.Hq = Hq;
  P.Hkv = Hkv;
  P.G = Hq / Hkv;
  P.S = S;
  P.scale_log2 = scale * TA_LOG2E;
  const int hgroups = (P.G + dec::HG - 1) / dec::HG;
  mark(ev, nev, 0, stream);
  hipLaunchKernelGGL(dec::partial_kernel, dim3(S, Hkv * hgroups, B), dim3(256), 0, stream, P);
  TA_LAUNCH_CHECK();
  mark(ev, nev, 1, stream);
  const size_t shmem = (size_t)S * (2 + d) * sizeof(float);
  hipLaunchKernelGGL(dec::merge_kernel, dim3(B * Hq), dim3(1024), shmem, stream, (const float*)ws, S, (bf16*)o, lse);
  TA_LAUNCH_CHECK();
  mark(ev, nev, 2, stream);
  return TA_OK;
}
