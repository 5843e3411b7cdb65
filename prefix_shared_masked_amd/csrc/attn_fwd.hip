// Tree-attention forward on gfx950.
//
// Semantics (Tree Training post): packed token i reads key j iff j <= i and
// node(j) is an ancestor-or-self of node(i) (section 4.2), which in DFS order
// is j <= i < kend(j) with kend the end of node(j)'s DFS interval (section
// 4.3); positions are tree depth (section 5).  O = softmax(scale Q K^T + M) V
// and LSE = log sum_j exp(scale q_i . k_j).
//
// bf16 kernel layout, one workgroup = one 32-row query tile x up to four query
// heads that share a KV head (one wavefront per head):
//  - the tile's keys come from the plan's gathered chunk list (the ancestor
//    block table): only keys some row may read are ever loaded, so invisible
//    sibling subtrees cost nothing (section 4.3, "skip, do not mask");
//  - each chunk of 64 key rows is gathered from HBM straight into LDS with
//    16-byte global-to-LDS copies (double-buffered: the next chunk's copies
//    are in flight while the current chunk is computed);
//  - S^T = K Q^T on 32x32x16 bf16 MFMA with Q resident in registers, so each
//    lane owns one query column: the row max and row sum are in-register plus
//    a single exchange with the lane 32 away;
//  - the element mask j <= i < kend is evaluated only on chunks the plan did
//    not flag as fully visible;
//  - O^T += V^T P^T on MFMA, V^T read from LDS with the transpose read, P^T
//    straight from the S^T accumulators;
//  - the XCD round-robin of workgroups puts consecutive block ids on
//    different XCDs, so blockIdx % Hkv picks the KV head and every XCD keeps
//    re-reading the same KV head's ancestors in its own L2.
#include <algorithm>
#include <cstring>

#include "common.h"
#include "plan_internal.h"

namespace ta {

// ---------------------------------------------------------------------------
// RoPE by depth position and/or dtype conversion: y[t, h, :] = mul R(pos[t])
// x[t, h, :] (transpose=1 gives R^T; base <= 0 converts only), and when y2 is
// given also y2[t, h, :] = R(pos[t]) x[t, h, :] in bf16.  Rotate-half pairs
// (i, i + d/2), angle pos * base^(-2i/d).  A thread takes one token and four
// consecutive pairs (i, i + d/2) .. (i + 3, i + 3 + d/2): the sines and
// cosines are computed once and applied to all H heads, and every access is
// a 4-element vector (consecutive threads take consecutive groups of four,
// so each load and store of a wavefront is one contiguous run per token).
template <typename T>
__device__ __forceinline__ void ld4(const T* p, float (&v)[4]) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  const T4 x = *(const T4*)p;
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = (float)x[u];
}
template <typename T>
__device__ __forceinline__ void st4(T* p, const float (&v)[4], bool&) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  T4 x;
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = (T)v[u];
  *(T4*)p = x;
}
template <>
__device__ __forceinline__ void st4<f16>(f16* p, const float (&v)[4], bool& sat) {
  typedef f16 T4 __attribute__((ext_vector_type(4)));
  T4 x;
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = to_f16_sat(v[u], sat);
  *(T4*)p = x;
}

template <typename Ti, typename To>
__global__ void rope_kernel(const Ti* x, To* y, bf16* y2, const int32_t* __restrict__ pos,  // x may alias y
                            int N, int H, int d, float base, int transpose, float mul, int32_t* sat_flag) {
  bool sat = false;
  const int half = d / 2, groups = half / 4;
  const size_t total = (size_t)N * groups;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int i = 4 * (int)(idx % groups);
    const int t = (int)(idx / groups);
    float s[4], c[4];
    const int pt = base > 0.f ? pos[t] : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s[u] = 0.f;
      c[u] = 1.f;
      if (base > 0.f) rope_sincos(pt, i + u, d, base, &s[u], &c[u]);
      if (transpose) s[u] = -s[u];
    }
    // Each thread reads and writes only its own elements, so the loads of a
    // batch of heads may all be issued before any store, also in place: one
    // memory round trip per batch instead of one per head.  The loads are
    // unconditional so that none waits for another.
    constexpr int HB = 8;
    for (int h0 = 0; h0 < H; h0 += HB) {
      float x1[HB][4], x2[HB][4];
#pragma unroll
      for (int b = 0; b < HB; ++b) {  // unconditional (a head past H re-reads head H - 1)
        const size_t row = ((size_t)t * H + min(h0 + b, H - 1)) * d;
        ld4(x + row + i, x1[b]);
        ld4(x + row + i + half, x2[b]);
      }
#pragma unroll
      for (int b = 0; b < HB; ++b)
        if (h0 + b < H) {
          const size_t row = ((size_t)t * H + h0 + b) * d;
          float r1[4], r2[4], o1[4], o2[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            r1[u] = x1[b][u] * c[u] - x2[b][u] * s[u];
            r2[u] = x2[b][u] * c[u] + x1[b][u] * s[u];
            o1[u] = mul * r1[u];
            o2[u] = mul * r2[u];
          }
          st4(y + row + i, o1, sat);
          st4(y + row + i + half, o2, sat);
          if (y2) {
            st4(y2 + row + i, r1, sat);
            st4(y2 + row + i + half, r2, sat);
          }
        }
    }
  }
  report_sat(sat_flag, sat);
}

template <typename Ti, typename To>
hipError_t launch_rope(const Ti* x, To* y, const int32_t* pos, int N, int H, int d, float base, int transpose,
                       hipStream_t st, float mul, bf16* y2, int32_t* sat_flag) {
  const size_t total = (size_t)N * (d / 8);  // a thread per (token, four pairs)
  if (total == 0) return hipSuccess;
  const int blocks = (int)std::min<size_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL((rope_kernel<Ti, To>), dim3(blocks), dim3(256), 0, st, x, y, y2, pos, N, H, d, base, transpose,
                     mul, sat_flag);
  return hipGetLastError();
}

template hipError_t launch_rope<float, float>(const float*, float*, const int32_t*, int, int, int, float, int,
                                              hipStream_t, float, bf16*, int32_t*);
template hipError_t launch_rope<bf16, f16>(const bf16*, f16*, const int32_t*, int, int, int, float, int,
                                           hipStream_t, float, bf16*, int32_t*);

namespace fwd {

constexpr int D = 128;
constexpr int BM = TA_BLOCK_M;
constexpr int BN = TA_BLOCK_N;

struct Params {
  const bf16* q;
  const f16* k;   // fp16 copy of K (rotated when RoPE is on) times scale * log2(e)
  const bf16* v;
  bf16* o;
  float* lse;
  const int32_t* pos;
  const int32_t* fq_ptr;
  const int32_t* fq_chunk;
  const int32_t* fq_order;
  int32_t* sat;  // saturation flag (fp16 conversion of Q clamped), may be null
  int N, Hq, Hkv, G;
  int q0;  // first query row (rows below are a key-only prefix)
  float rope_base;
};

// The two halves of a wavefront (lanes l and l + 32) hold the same query
// column; v_permlane32_swap with x in both operands leaves x[l % 32] in the
// first and x[32 + l % 32] in the second, in every lane, so one instruction
// combines both halves.  It is issued from inline asm: when both results of
// the compiler builtin feed one arithmetic instruction, this compiler reads
// the first result register twice (checked in the generated code: r0 + r1
// became v_add v2, v3, v3).  s_nop 1: a VALU write of an operand needs two
// wait states before the swap reads it.
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}
__device__ __forceinline__ float halves_max(float x) {
  float a, b;
  halves(x, a, b);
  return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float halves_sum(float x) {
  float a, b;
  halves(x, a, b);
  return a + b;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(Params P) {
  __shared__ __attribute__((aligned(1024))) f16 sK[2][BN * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][BN * D];
  __shared__ __attribute__((aligned(16))) int sJ[2][BN];
  __shared__ __attribute__((aligned(16))) int sE[2][BN];
  __shared__ double sInv[D / 2];

  const int kvh = blockIdx.x % P.Hkv;
  const int tile = as_const(P.fq_order)[blockIdx.x / P.Hkv];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int hsub = blockIdx.y * 4 + wave;
  const bool active = hsub < P.G;  // wave-uniform
  rope_inv_table(sInv, D / 2, D, P.rope_base);
  __syncthreads();
  const int h = kvh * P.G + (active ? hsub : 0);
  const int qi = P.q0 + tile * BM + col;
  const bool qvalid = qi < P.N;

  // Q (rotated by depth position, fp16) as the B operand: lane = query
  // column, k-slots s*16 + half*8 + e.
  f16x8 qf[8];
  {
    bool sat = false;
    const bf16* qrow = P.q + ((size_t)(qvalid ? qi : 0) * P.Hq + h) * D + half * 8;
    const bool rot = P.rope_base > 0.f && qvalid;
    const int p = qvalid ? P.pos[qi] : 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 t1 = *(const bf16x8*)(qrow + s * 16);
      const bf16x8 t2 = *(const bf16x8*)(qrow + (s + 4) * 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x1 = qvalid ? (float)t1[e] : 0.f, x2 = qvalid ? (float)t2[e] : 0.f;
        if (rot) {
          float sn, cs;
          rope_sincos_at(p, sInv[s * 16 + half * 8 + e], &sn, &cs);
          const float y1 = x1 * cs - x2 * sn;
          x2 = x2 * cs + x1 * sn;
          x1 = y1;
        }
        qf[s][e] = to_f16_sat(x1, sat);
        qf[s + 4][e] = to_f16_sat(x2, sat);
      }
    }
    report_sat(P.sat, sat && active);
  }

  // Staging.  Copy k (k = 0..3) of wavefront w fills rows 4(w + 4k) + l/16
  // of a chunk's K and V tiles (a swizzled 16-byte piece per lane).  A chunk
  // of one 64-key segment (most chunks) holds keys delta .. delta + 63, so
  // its copies take a scalar base and fixed per-lane offsets; other chunks
  // gather their rows per lane.  The key indices and interval ends of the
  // slots go to sJ / sE only for chunks that need the element mask.
  const int t = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(wave);
  const int sub = lane >> 4;
  const uint32_t kvrow = (uint32_t)P.Hkv * (D * 2);  // bytes between consecutive tokens
  const uint32_t piece = (uint32_t)(((lane & 15) ^ swz((4 * w + sub) & 15)) << 4);
  uint32_t voff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) voff[k] = (uint32_t)(4 * (w + 4 * k) + sub) * kvrow + piece;
  const uint32_t ldsK = lds_addr(&sK[0][0]), ldsV = lds_addr(&sV[0][0]);
  // copies chunk c into buffer b; returns the chunk's "fully visible" flag
  auto stage = [&](int c, int b) -> int {
    const ChunkRec ch = load_chunk(as_const(P.fq_chunk) + (size_t)c * TA_CHUNK_INTS);
    const int full = ch.h[2];
    if (ch.h[0] == 1 && ch.h[1] == BN) {
      const int delta = ch.ks[0] - ch.ko[0];
      const size_t off = ((size_t)delta * P.Hkv + kvh) * (D * 2);
      const char* kb = (const char*)P.k + off;
      const char* vb = (const char*)P.v + off;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t r = (uint32_t)(4 * (w + 4 * k)) * (D * 2);
        copy16_to_lds_s(kb, voff[k], ldsK + b * (BN * D * 2) + r);
        copy16_to_lds_s(vb, voff[k], ldsV + b * (BN * D * 2) + r);
      }
      if (!full && t < BN) {
        sJ[b][t] = t + delta;
        sE[b][t] = ch.ke[0];
      }
    } else {
      const int poff = (int)(piece >> 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = w + 4 * k;
        int j, e;
        chunk_slot(ch, 4 * i + sub, j, e);
        const size_t off = ((size_t)j * P.Hkv + kvh) * D + poff;
        copy16_to_lds(P.k + off, sK[b] + 4 * i * D);
        copy16_to_lds(P.v + off, sV[b] + 4 * i * D);
      }
      if (!full) {
        int j, e;
        chunk_slot(ch, lane, j, e);
        if (t < BN) {
          sJ[b][t] = j;
          sE[b][t] = e;
        }
      }
    }
    return full;
  };

  // Swizzled LDS offsets (in elements), fixed per lane: koff[s] for the
  // 16-byte K row read of k-group s (rows col and col + 32 share them);
  // voff_t[dt][x] for the V transpose read of d-tile dt, rows trow + 8x of
  // each 16-row group.
  const int trow = half * 4 + ((lane & 15) >> 2);
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int koff[8], vto[4][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = col * D + (((2 * s + half) ^ swz(col & 15)) << 3);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = trow + 8 * x;
      vto[dt][x] = r * D + (((4 * dt + (tcol >> 3)) ^ swz(r)) << 3) + (tcol & 7);
    }

  // Online softmax with a lazily moved reference.  The score accumulators
  // start from -mref (the MFMA's C operand), so S - mref comes out of the
  // matrix unit and the exponentials need no subtraction.  mref moves (and
  // O, l are rescaled) only when some lane's max over a 32-key half exceeds
  // it by more than 8 (log2 units), or at the lane's first half with a
  // visible key; otherwise the stale reference keeps P <= 2^8, and O / l and
  // LSE = mref + log2(l) do not depend on it.
  float mref = 0.f, l = 0.f;
  bool has = false;  // a visible key has been seen (mref is then a max reference)
  f32x16 seed;
#pragma unroll
  for (int r = 0; r < 16; ++r) seed[r] = 0.f;
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  const bf16x2 ones = {(bf16)1.f, (bf16)1.f};
  auto fence = []() { __builtin_amdgcn_sched_barrier(0); };

  // Softmax of one 32-key half (S^T register r <-> key slot
  // kt*32 + 8*(r/4) + 4*half + r%4, in log2 units, minus the reference the
  // accumulators were seeded with; `shift` is how far mref has moved since):
  // element mask on partial chunks, max, lazy rescale, P = exp2 in bf16, and
  // the row sum of the rounded P that enters P V.
  auto softmax_half = [&](f32x16& s, int b, int kt, int full, float& shift, bf16x8& p0, bf16x8& p1) {
    if (!full) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int v0 = kt * 32 + r4 * 8 + half * 4;
        const int4 J = *(const int4*)&sJ[b][v0], E = *(const int4*)&sE[b][v0];
        const int j[4] = {J.x, J.y, J.z, J.w}, e[4] = {E.x, E.y, E.z, E.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (!(j[u] <= qi && qi < e[u])) s[r4 * 4 + u] = -INFINITY;
      }
    }
    // max relative to the current mref, NaN-propagating (v_maximum3)
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[r], s[r + 1]));
    mx = halves_max(mx) - shift;
    const bool need = (!has || mx > 8.f) && mx != -INFINITY;
    if (__builtin_amdgcn_ballot_w64(need || shift != 0.f)) {
      const float delta = need ? mx : 0.f;
      const float alpha = exp2f_fast(-delta);
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
      mref += delta;
      has = has || need;
      const float sub = shift + delta;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] -= sub;
      shift += delta;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p0[e] = (bf16)exp2f_fast(s[e]);
      p1[e] = (bf16)exp2f_fast(s[8 + e]);
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[e], p0[e + 1]}, ones, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[e], p1[e + 1]}, ones, l, false);
    }
    asm volatile("" : "+v"(p0), "+v"(p1), "+v"(l));
  };

  // One chunk from buffer b (static after unrolling), as two 32-key halves
  // so the matrix unit has queued work while the VALU runs: score MFMAs of
  // both halves (K rows read two k-groups ahead), softmax of half 0 while
  // half 1's score MFMAs run, P V of half 0, softmax of half 1 while those
  // run, P V of half 1.  The source order is the issue order (scheduling
  // fences; empty asm statements pin the softmax results in place).
  auto compute = [&](int b, int full) {
    const f16* kb = sK[b];
    const bf16* vb = sV[b];
    f32x16 st[2];
    f16x8 ka[16];
    ka[0] = *(const f16x8*)(kb + koff[0]);
    ka[1] = *(const f16x8*)(kb + koff[1]);
    fence();
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // i = kt * 8 + s
      if (i + 2 < 16) ka[i + 2] = *(const f16x8*)(kb + ((i + 2) >> 3) * 32 * D + koff[(i + 2) & 7]);
      const int kt = i >> 3, s = i & 7;
      st[kt] = mfma32h(ka[i], qf[s], s == 0 ? seed : st[kt]);
      fence();
    }
    float shift = 0.f;
    bf16x8 pb[4];
    // transpose-read operands of half 0's P V, then its softmax
    bf16x8 vt[4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        vt[dt][kk] = cat(lds_read_tr(vb + kk * 16 * D + vto[dt][0]), lds_read_tr(vb + kk * 16 * D + vto[dt][1]));
    softmax_half(st[0], b, 0, full, shift, pb[0], pb[1]);
    fence();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc[dt] = mfma32(vt[dt][kk], pb[kk], acc[dt]);
    fence();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        vt[dt][kk] =
            cat(lds_read_tr(vb + (kk + 2) * 16 * D + vto[dt][0]), lds_read_tr(vb + (kk + 2) * 16 * D + vto[dt][1]));
    softmax_half(st[1], b, 1, full, shift, pb[2], pb[3]);
    fence();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) acc[dt] = mfma32(vt[dt][kk], pb[kk + 2], acc[dt]);
    if (__builtin_amdgcn_ballot_w64(shift != 0.f)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) seed[r] = -mref;
    }
  };

  const int c0 = as_const(P.fq_ptr)[tile], c1 = as_const(P.fq_ptr)[tile + 1];
  int full = stage(c0, 0);
  lds_copies_wait();
  __syncthreads();
  // Double buffer, unrolled by two so each buffer's LDS offsets are
  // immediates: the next chunk's copies go into the other buffer while this
  // one is computed (the last chunk copies itself again, into the buffer
  // nobody reads).  Wavefronts without a head (fewer than four heads per KV
  // head) stage and wait but compute nothing.
  for (int c = c0; c < c1; c += 2) {
    {
      const int fn = stage(c + 1 < c1 ? c + 1 : c, 1);
      if (active) compute(0, full);
      full = fn;
      lds_copies_wait();
      __syncthreads();
    }
    if (c + 1 < c1) {
      const int fn = stage(c + 2 < c1 ? c + 2 : c + 1, 0);
      if (active) compute(1, full);
      full = fn;
      lds_copies_wait();
      __syncthreads();
    }
  }

  const float lt = halves_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (active && qvalid) {
    bf16* orow = P.o + ((size_t)qi * P.Hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 wv;
#pragma unroll
        for (int u = 0; u < 4; ++u) wv[u] = (bf16)(acc[dt][r4 * 4 + u] * inv);
        *(bf16x4*)(orow + dt * 32 + r4 * 8 + half * 4) = wv;
      }
    if (half == 0) P.lse[(size_t)h * P.N + qi] = (has ? mref + log2f(lt) : -INFINITY) * TA_LN2;
  }
}

}  // namespace fwd

// ---------------------------------------------------------------------------
// fp32 path: one thread per (query row, head), walking the same gathered
// chunks; exact fp32 arithmetic for small problems and for checking.
template <int D>
__global__ __launch_bounds__(TA_BLOCK_M) void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                              const float* __restrict__ v, float* __restrict__ o,
                                                              float* __restrict__ lse, const int32_t* __restrict__ fq_ptr,
                                                              const int32_t* __restrict__ fq_chunk, int N, int Hq, int Hkv,
                                                              float scale, int q0) {
  const int tile = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, kvh = h / G;
  const int i = q0 + tile * TA_BLOCK_M + threadIdx.x;
  if (i >= N) return;
  float qv[D], acc[D];
  for (int x = 0; x < D; ++x) {
    qv[x] = q[((size_t)i * Hq + h) * D + x];
    acc[x] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int c = fq_ptr[tile]; c < fq_ptr[tile + 1]; ++c) {
    const int32_t* ch = fq_chunk + (size_t)c * TA_CHUNK_INTS;
    for (int slot = 0; slot < ch[1]; ++slot) {
      int j, kend;
      chunk_slot(ch, slot, j, kend);
      if (!(j <= i && i < kend)) continue;
      const float* kr = k + ((size_t)j * Hkv + kvh) * D;
      const float* vr = v + ((size_t)j * Hkv + kvh) * D;
      float s = 0.f;
      for (int x = 0; x < D; ++x) s = fmaf(qv[x], kr[x], s);
      s *= scale;
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn), p = expf(s - mn);
      l = l * a + p;
      for (int x = 0; x < D; ++x) acc[x] = acc[x] * a + p * vr[x];
      m = mn;
    }
  }
  for (int x = 0; x < D; ++x) o[((size_t)i * Hq + h) * D + x] = acc[x] / l;
  lse[(size_t)h * N + i] = m + logf(l);
}

}  // namespace ta

using namespace ta;

extern "C" ta_status tree_plan_upload(const ta_plan* p, void* dplan, size_t bytes, hipStream_t stream) {
  if (!p || !dplan) return TA_EINVAL;
  if (bytes < p->device_bytes) return TA_ENOMEM;
  char* base = (char*)dplan;
  struct Part {
    size_t off;
    const std::vector<int32_t>* vec;
  } parts[] = {{p->off_pos, &p->pos},
               {p->off_fq_ptr, &p->fq_ptr},
               {p->off_fq_chunk, &p->fq_chunk},
               {p->off_fq_order, &p->fq_order},
               {p->off_bk, &p->bk},
               {p->off_kp, &p->kp},
               {p->off_kr, &p->kr},
               {p->off_dq_ptr, &p->dq_ptr},
               {p->off_dq_ent, &p->dq_ent},
               {p->off_dq_order, &p->dq_order}};
  for (const Part& x : parts) {
    if (x.vec->empty()) continue;
    if (hipMemcpyAsync(base + x.off, x.vec->data(), x.vec->size() * sizeof(int32_t), hipMemcpyHostToDevice,
                       stream) != hipSuccess)
      return TA_EHIP;
  }
  return TA_OK;
}

namespace {

ta_status check_common(const ta_plan* p, const void* dplan, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d) {
  if (!p || !dplan) return TA_EINVAL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return TA_EINVAL;
  if (dt == TA_BF16) {
    if (d != 128) return TA_EUNSUPPORTED;
  } else if (dt == TA_F32) {
    if (d != 64 && d != 128) return TA_EUNSUPPORTED;
  } else {
    return TA_EUNSUPPORTED;
  }
  if ((int64_t)p->n_tokens * Hq * d > ((int64_t)1 << 40)) return TA_ERANGE;
  return TA_OK;
}

size_t fwd_ws(const ta_plan* p, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d, float rope_base) {
  const size_t N = p->n_tokens;
  if (dt == TA_BF16) return TA_WS_FLAG_BYTES + align256(N * Hkv * d * sizeof(f16));  // flag, fp16 (rotated) K
  if (rope_base <= 0.f) return 0;
  return align256(N * Hq * d * sizeof(float)) + align256(N * Hkv * d * sizeof(float));
}

}  // namespace

// Backward workspace (defined in attn_bwd.hip).
size_t ta_bwd_ws(const ta_plan* p, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d, float rope_base, bool with_ds);

extern "C" ta_status tree_attn_ws_bytes(const ta_plan* p, int32_t op, ta_dtype dt, int32_t Hq, int32_t Hkv,
                                        int32_t d, float rope_base, size_t* bytes) {
  if (!p || !bytes || op < 0 || op > 2) return TA_EINVAL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return TA_EINVAL;
  *bytes = op == 0 ? fwd_ws(p, dt, Hq, Hkv, d, rope_base) : ta_bwd_ws(p, dt, Hq, Hkv, d, rope_base, op == 1);
  return TA_OK;
}

extern "C" ta_status tree_attn_fwd(const ta_plan* p, const void* dplan, ta_dtype dt, const void* q, const void* k,
                                   const void* v, int32_t Hq, int32_t Hkv, int32_t d, float scale, float rope_base,
                                   void* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  return tree_attn_fwd_ex(p, dplan, dt, q, k, v, Hq, Hkv, d, scale, rope_base, o, lse, ws, ws_bytes, nullptr, 0,
                          stream);
}

extern "C" ta_status tree_attn_fwd_ex(const ta_plan* p, const void* dplan, ta_dtype dt, const void* q, const void* k,
                                      const void* v, int32_t Hq, int32_t Hkv, int32_t d, float scale, float rope_base,
                                      void* o, float* lse, void* ws, size_t ws_bytes, hipEvent_t* ev, int32_t nev,
                                      hipStream_t stream) {
  ta_status st = check_common(p, dplan, dt, Hq, Hkv, d);
  if (st != TA_OK) return st;
  const int N = p->n_tokens;
  if (N == 0) return TA_OK;  // nothing to read or write (empty tensors may be null)
  if (!q || !k || !v || !o || !lse) return TA_EINVAL;
  const size_t need = fwd_ws(p, dt, Hq, Hkv, d, rope_base);
  if (need && (!ws || ws_bytes < need)) return TA_ENOMEM;
  if (scale <= 0.f) scale = 1.f / sqrtf((float)d);
  const char* base = (const char*)dplan;
  const int32_t* pos = (const int32_t*)(base + p->off_pos);
  const int32_t* fq_ptr = (const int32_t*)(base + p->off_fq_ptr);
  const int32_t* fq_chunk = (const int32_t*)(base + p->off_fq_chunk);
  const int32_t* fq_order = (const int32_t*)(base + p->off_fq_order);

  mark(ev, nev, 0, stream);
  if (dt == TA_BF16) {
    int32_t* sat = (int32_t*)ws;
    f16* kk = (f16*)((char*)ws + TA_WS_FLAG_BYTES);
    if (launch_rope<bf16, f16>((const bf16*)k, kk, pos, N, Hkv, d, rope_base, 0, stream, scale * TA_LOG2E, nullptr,
                               sat) != hipSuccess)
      return TA_EHIP;
    mark(ev, nev, 1, stream);
    fwd::Params P;
    P.q = (const bf16*)q;
    P.k = kk;
    P.v = (const bf16*)v;
    P.o = (bf16*)o;
    P.lse = lse;
    P.pos = pos;
    P.fq_ptr = fq_ptr;
    P.fq_chunk = fq_chunk;
    P.fq_order = fq_order;
    P.sat = sat;
    P.N = N;
    P.Hq = Hq;
    P.Hkv = Hkv;
    P.G = Hq / Hkv;
    P.q0 = p->q_start;
    P.rope_base = rope_base;
    dim3 grid(p->n_qtiles * Hkv, (P.G + 3) / 4);
    hipLaunchKernelGGL(fwd::fwd_bf16_kernel, grid, dim3(256), 0, stream, P);
    TA_LAUNCH_CHECK();
    mark(ev, nev, 2, stream);
    return TA_OK;
  }

  const float* qq = (const float*)q;
  const float* kk = (const float*)k;
  if (rope_base > 0.f) {
    float* qr = (float*)ws;
    float* kr = (float*)((char*)ws + align256((size_t)N * Hq * d * sizeof(float)));
    if (launch_rope<float, float>(qq, qr, pos, N, Hq, d, rope_base, 0, stream) != hipSuccess) return TA_EHIP;
    if (launch_rope<float, float>(kk, kr, pos, N, Hkv, d, rope_base, 0, stream) != hipSuccess) return TA_EHIP;
    qq = qr;
    kk = kr;
  }
  mark(ev, nev, 1, stream);
  dim3 grid(p->n_qtiles, Hq);
  if (d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(TA_BLOCK_M), 0, stream, qq, kk, (const float*)v, (float*)o, lse,
                       fq_ptr, fq_chunk, N, Hq, Hkv, scale, p->q_start);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(TA_BLOCK_M), 0, stream, qq, kk, (const float*)v, (float*)o,
                       lse, fq_ptr, fq_chunk, N, Hq, Hkv, scale, p->q_start);
  TA_LAUNCH_CHECK();
  mark(ev, nev, 2, stream);
  return TA_OK;
}
