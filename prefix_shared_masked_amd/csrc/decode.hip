// Split-KV single-query decode with a log-depth (max, numerator, denominator)
// merge (Tree Attention notes: the three mergeable quantities, their
// associativity, and the decode algorithm -- local attention per KV shard,
// global max, rescaled sums, z = n/d).  On one GPU the shards are KV slices
// handled by different workgroups, and the "AllReduce" is a pairwise merge
// tree of depth ceil(log2 S) over the S slices.
//
// Decode is HBM-bound: each K/V byte feeds a few FLOPs per query head.  The
// partial kernel therefore keeps as many bytes in flight as the LDS holds
// (direct global-to-LDS copies into a per-wavefront ring) and leaves the
// arithmetic to the matrix cores, so the vector ALU does only the softmax.
// Merge kernel: one workgroup per (batch item, query head); round r merges
// slice pairs (i, i + 2^r) in parallel over the head dimension.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace ta {
namespace dec {

constexpr int D = 128;
constexpr int MAX_SPLITS = 120;  // merge keeps S x (2 + D) floats in 64 KB of LDS
constexpr int AUTO_SPLITS = 32;  // default cap on the slice count

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

// ---------------------------------------------------------------------------
// Matrix-core partial kernel.  One workgroup per (slice, KV head x group of
// up to 32 query heads, batch item); the slice is cut into four contiguous
// parts, one per wavefront, so each wavefront streams its own keys through a
// private two-stage LDS ring with direct global-to-LDS copies (non-temporal:
// every K/V byte is read once) and needs no workgroup barrier in its loop.
// Per 32-key block: S^T = K q^T on 32x32x16 bf16 MFMA (keys on the rows, the
// query heads on the 32 columns, so each lane owns one head and the running
// max / sum stay in registers plus one exchange with the lane 32 away), then
// O^T += V^T P^T with V^T from the LDS transpose read.  The products of bf16
// values are exact in the fp32 accumulators, so no conversion work is left
// on the vector ALU.  The four wavefronts' (m, l, o) are merged in LDS.
constexpr int KS = 32;               // keys per block (one MFMA row tile)
constexpr int WV = 4;                // wavefronts per workgroup
constexpr int HC = 32;               // query heads per workgroup (MFMA columns)
constexpr int STAGE = 2 * KS * D;    // bf16 elements per ring stage: K rows, then V rows

struct Blk {
  int row, n;  // physical first row, valid keys (1..KS)
};

// The KS-key blocks of the virtual range [pos, end) of one item's spans, in
// order; wavefront-uniform (the span table is read with scalar loads).
struct SpanWalk {
  cint_ptr spans;
  int s, s1, base, pos, end;
  __device__ __forceinline__ bool next(Blk& out) {
    while (s < s1 && pos < end) {
      const int st = spans[2 * s], len = spans[2 * s + 1];
      const int hi = min(end, base + len);
      if (pos < hi) {
        out.row = st + (pos - base);
        out.n = min(KS, hi - pos);
        pos += out.n;
        return true;
      }
      base += len;
      ++s;
      pos = max(pos, base);
    }
    return false;
  }
};


// Copies block b's K and V rows into one ring stage (swizzled 256-byte rows;
// rows past the block's valid keys repeat its last key and are masked).
// Copy i fills rows 4i..4i+3: lane l writes row 4i + l/16, piece l%16.
__device__ __forceinline__ void stage_block(const Params& P, const Blk& b, int kvh, bf16* sb) {
  const int l = threadIdx.x & 63, sub = l >> 4;
#pragma unroll
  for (int i = 0; i < KS / 4; ++i) {
    const int r = 4 * i + sub;
    const int poff = ((l & 15) ^ swz(r & 15)) << 3;
    const size_t off = ((size_t)(b.row + min(r, b.n - 1)) * P.Hkv + kvh) * D + poff;
    copy16_to_lds_nt(P.k + off, sb + 4 * i * D);
    copy16_to_lds_nt(P.v + off, sb + KS * D + 4 * i * D);
  }
}

__global__ __launch_bounds__(256, 1) void partial_kernel(Params P) {
  __shared__ __attribute__((aligned(1024))) bf16 ring[WV][2][STAGE];
  const int split = blockIdx.x;
  const int kvh = blockIdx.y % P.Hkv, hgrp = blockIdx.y / P.Hkv;
  const int b = blockIdx.z;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int nh = min(HC, P.G - hgrp * HC);
  const bool hvalid = col < nh;
  const int h = kvh * P.G + hgrp * HC + (hvalid ? col : 0);

  // this item's length, this workgroup's slice and this wavefront's part
  const cint_ptr sp = as_const(P.spans);
  const int sp0 = as_const(P.span_ptr)[b], sp1 = as_const(P.span_ptr)[b + 1];
  int L = 0;
  for (int s = sp0; s < sp1; ++s) L += sp[2 * s + 1];
  const int per = (((L + P.S - 1) / P.S) + KS - 1) & ~(KS - 1);
  const int vs = min(L, split * per), ve = min(L, vs + per);
  const int wper = (((ve - vs + WV - 1) / WV) + KS - 1) & ~(KS - 1);
  SpanWalk walk{sp, sp0, sp1, 0, min(ve, vs + w * wper), min(ve, vs + (w + 1) * wper)};

  // q as the B operand: lane = head column, k-slots 16 s + 8 half + e
  bf16x8 qf[8];
  {
    const bf16* qr = P.q + ((size_t)b * P.Hq + h) * D + half * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = hvalid ? *(const bf16x8*)(qr + 16 * s) : bf16x8{};
  }
  // the q loads must land before the ring copies start counting on vmcnt
  asm volatile("s_waitcnt vmcnt(0)" ::"v"(qf[0]), "v"(qf[7]) : "memory");

  int koff[8], voff[4][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = col * D + (((2 * s + half) ^ swz(col & 15)) << 3);
  {
    const int trow = half * 4 + ((lane & 15) >> 2);
    const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int r = trow + 8 * x;
        voff[dt][x] = r * D + (((4 * dt + (tcol >> 3)) ^ swz(r)) << 3) + (tcol & 7);
      }
  }

  float m = -INFINITY, l = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  auto compute = [&](const bf16* sb, int n) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) sc = mfma32(*(const bf16x8*)(sb + koff[s]), qf[s], sc);
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] *= P.scale_log2;
    if (n < KS) {  // uniform: only a span's last block is ragged
      // register r <-> key slot 8 (r / 4) + 4 half + r % 4
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * half + (r & 3) >= n) sc[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, sc[r]);
    mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32));
    // lazy rescaling as in the forward kernel: the reference moves only when
    // the block max exceeds it by more than 8 (log2 units)
    if (__builtin_amdgcn_ballot_w64(mx > m + 8.f)) {
      const float mnew = __builtin_elementwise_maximum(m, mx);
      const float alpha = exp2f_fast(m - ((mnew == -INFINITY) ? 0.f : mnew));
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      m = mnew;
    }
    const float muse = (m == -INFINITY) ? 0.f : m;
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2f_fast(sc[r] - muse);
      l += p;
      pb[r >> 3][r & 7] = (bf16)p;
    }
    const bf16* vb = sb + KS * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x4 t0 = lds_read_tr(vb + kk * 16 * D + voff[dt][0]);
        const bf16x4 t1 = lds_read_tr(vb + kk * 16 * D + voff[dt][1]);
        acc[dt] = mfma32(cat(t0, t1), pb[kk], acc[dt]);
      }
    // every LDS read of this stage has returned before it is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  bf16* const r0 = ring[w][0];
  bf16* const r1 = ring[w][1];
  Blk b0, b1;
  bool h0 = walk.next(b0);
  if (h0) stage_block(P, b0, kvh, r0);
  bool h1 = h0 && walk.next(b1);
  if (h1) stage_block(P, b1, kvh, r1);
  while (h0) {
    // a stage is 2 * KS / 4 = 16 copies; the other stage may still be in flight
    if (h1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(r0, b0.n);
    h0 = h1 && walk.next(b0);
    if (h0) stage_block(P, b0, kvh, r0);
    if (!h1) break;
    if (h0) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(r1, b1.n);
    h1 = h0 && walk.next(b1);
    if (h1) stage_block(P, b1, kvh, r1);
  }
  lds_copies_wait();
  __syncthreads();  // every wavefront is done with its ring: reuse it for the merge

  // per wavefront: m (log2 units), l and o of each head
  float* sm = (float*)&ring[0][0][0];      // [WV][HC]
  float* sl = sm + WV * HC;                // [WV][HC]
  float* so = sl + WV * HC;                // [WV][HC][D]
  const float lt = l + __shfl_xor(l, 32);
  if (hvalid) {
    if (half == 0) {
      sm[w * HC + col] = m;
      sl[w * HC + col] = lt;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        so[(w * HC + col) * D + dt * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = acc[dt][r];
  }
  __syncthreads();
  const int h0g = kvh * P.G + hgrp * HC;
  for (int idx = threadIdx.x; idx < nh * D; idx += 256) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < WV; ++x) M = __builtin_elementwise_maximum(M, sm[x * HC + hh]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float ls = 0.f, os = 0.f;
#pragma unroll
    for (int x = 0; x < WV; ++x) {
      const float f = exp2f_fast(sm[x * HC + hh] - Mu);
      ls += sl[x * HC + hh] * f;
      os += so[(x * HC + hh) * D + d] * f;
    }
    float* dst = P.part + (((size_t)b * P.Hq + h0g + hh) * P.S + split) * (2 + D);
    if (d == 0) {
      dst[0] = M;
      dst[1] = ls;
    }
    dst[2 + d] = os;
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

// Scratch of the allocation-free decode entry point: the per-slice partials
// live in this file-scope device array (one copy per GPU the library runs
// on, held until the process ends) instead of a caller workspace.  Host code
// never uses the array's name as an address: each device's copy is resolved
// once with hipGetSymbolAddress and that pointer is what the kernels get.
static __device__ __align__(256) unsigned char scratch[TA_DECODE_SCRATCH_BYTES];

using namespace ta;

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device id -> its copy of scratch, resolved on first use

ta_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return TA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return TA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TA_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TA_OK;
}

int32_t pick_splits(int32_t max_len, int32_t n_splits) {
  if (n_splits > 0) return n_splits;
  // about 8K keys (2K per wavefront) per workgroup up to 32K keys, otherwise
  // about 2K per workgroup up to AUTO_SPLITS slices.  At B = 8 and 8 KV heads
  // this picks 4 / 32 / 32 / 32 slices at 32K / 64K / 128K / 256K keys: one
  // round of 256 workgroups at 32K, and the best or within noise of the best
  // of 4 to 64 slices in a sweep of every length on one box (two rounds of
  // 512 workgroups were the worst shape at every length)
  if (max_len <= 32768) return std::max<int32_t>(1, (max_len + 8191) / 8192);
  return std::min<int32_t>(dec::AUTO_SPLITS, (max_len + 2047) / 2048);
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
  const int hgroups = (P.G + dec::HC - 1) / dec::HC;
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

extern "C" ta_status tree_decode_splitkv_noalloc(ta_dtype dt, const void* q, const void* k, const void* v,
                                                 const int32_t* span_ptr, const int32_t* spans, int32_t B,
                                                 int32_t Hq, int32_t Hkv, int32_t d, int32_t max_len, float scale,
                                                 int32_t n_splits, void* o, float* lse, hipStream_t stream) {
  if (dt != TA_BF16 || d != dec::D) return TA_EUNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_len < 0 || n_splits < 0) return TA_EINVAL;
  size_t need;
  int32_t S;
  ta_status st = tree_decode_ws_bytes(B, Hq, d, max_len, n_splits, &need, &S);
  if (st != TA_OK) return st;
  if (need > TA_DECODE_SCRATCH_BYTES) return TA_ENOMEM;  // the partials do not fit the fixed scratch
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != TA_OK) return st;
  return tree_decode_splitkv_ex(dt, q, k, v, span_ptr, spans, B, Hq, Hkv, d, max_len, scale, n_splits, o, lse, ws,
                                TA_DECODE_SCRATCH_BYTES, nullptr, 0, stream);
}
