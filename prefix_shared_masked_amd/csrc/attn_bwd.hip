// Tree-attention backward on gfx950.
//
// With P = softmax(scale Q K^T + M) and upstream dO, the gradients are
//   D_i = sum_c dO_ic O_ic,  dS = P * (dO V^T - D),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
// and with depth RoPE the rotated-space dQ/dK are rotated back by R^T.  The
// gradient of a shared key sums over every descendant query that reads it
// (Tree Training post, sections 6.2 and 7: one forward of the shared prefix,
// the branches' gradients add up at the ancestors).
//
// Three launches on one stream, no atomics, bitwise deterministic:
//  1. fp16 copy of K (rotated with RoPE) and, with RoPE, a rotated bf16 K;
//  2. dQ, query-stationary: one workgroup per (32-row query tile, KV head),
//     one wavefront per query head, walking the forward's gathered key
//     chunks.  P is recomputed from LSE; S^T, dP^T and dQ^T are MFMA tiles
//     with the query on the lane, K^T read with the LDS transpose read.  It
//     also writes D and an fp16 copy of the rotated Q for step 3;
//  3. dK/dV, key-stationary: one workgroup per (node-aligned tile of at most
//     128 keys, KV head), one wavefront per 32 keys.  Every query in
//     [k0, kend) of the node's DFS interval reads every key of the tile
//     (only a wavefront's diagonal block needs the causal compare), so Q and
//     dO stream as contiguous 32-row blocks with no gather; each block is
//     staged in LDS once and shared by the four wavefronts, and the loop runs
//     over every query head of the GQA group, so the group's sum stays in
//     registers.  Scores use the fp16 copies of rotated Q and K (finer
//     rounding than bf16 for rotated values; same MFMA rate), so P matches
//     the forward's.  K and V stay in registers; dV += P^T dO and
//     dK += dS^T Q use the LDS transpose read of the staged blocks.
#include "common.h"
#include "plan_internal.h"

namespace ta {
namespace bwd {

constexpr int D = 128;
constexpr int BM = TA_BLOCK_M;
constexpr int BN = TA_BLOCK_N;
constexpr int PK = D + 8;   // row-read friendly pitch
constexpr int PT = D + 16;  // transpose-read friendly pitch

// ---------------------------------------------------------------------------
struct DQParams {
  const bf16* q;
  const bf16* k;  // rotated when RoPE is on
  const bf16* v;
  const bf16* o;
  const bf16* dO;
  const float* lse;
  bf16* dq;
  float* Dd;    // [Hq, N] out
  f16* qs;      // [N, Hq, d] out: fp16 copy of Q (rotated when RoPE is on)
  const int32_t* pos;
  const int32_t* fq_ptr;
  const int32_t* fq_chunk;
  const int32_t* fq_order;
  int N, Hq, Hkv, G;
  float scale, scale_log2, rope_base;
};

// Copies chunk c's 64 K and V rows into one LDS buffer (swizzled 256-byte
// rows, see swz) and its key indices / DFS-interval ends into sJ / sE.  Copy
// instruction i of a tile fills rows 4i..4i+3; wavefront w issues i = w + 4k.
__device__ __forceinline__ void stage_chunk(const DQParams& P, int c, int kvh, bf16* sKb, bf16* sVb, int* sJb,
                                            int* sEb) {
  const ChunkRec ch = load_chunk(as_const(P.fq_chunk) + (size_t)c * TA_CHUNK_INTS);
  const int t = threadIdx.x, l = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = w + 4 * k;
    const int row = 4 * i + (l >> 4);
    int j, e;
    chunk_slot(ch, row, j, e);
    const int piece = (l & 15) ^ swz(row & 15);
    const size_t off = ((size_t)j * P.Hkv + kvh) * D + piece * 8;
    copy16_to_lds(P.k + off, sKb + 4 * i * D);
    copy16_to_lds(P.v + off, sVb + 4 * i * D);
  }
  int j, e;
  chunk_slot(ch, l, j, e);
  if (t < BN) {
    sJb[t] = j;
    sEb[t] = e;
  }
}

__global__ __launch_bounds__(256, 1) void dq_bf16_kernel(DQParams P) {
  __shared__ __attribute__((aligned(1024))) bf16 sK[2][BN * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][BN * D];
  __shared__ __attribute__((aligned(16))) int sJ[2][BN];
  __shared__ __attribute__((aligned(16))) int sE[2][BN];

  const int kvh = blockIdx.x % P.Hkv;
  const int tile = as_const(P.fq_order)[blockIdx.x / P.Hkv];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int hsub = blockIdx.y * 4 + wave;
  const bool active = hsub < P.G;
  const int h = kvh * P.G + (active ? hsub : 0);
  const int qi = tile * BM + col;
  const bool qvalid = qi < P.N;
  const size_t rowoff = ((size_t)(qvalid ? qi : 0) * P.Hq + h) * D;

  // Q (rotated) and dO as B operands; D_i = dO_i . O_i
  bf16x8 qf[8], df[8];
  float Di, lse_i;
  {
    const bool rot = P.rope_base > 0.f && qvalid;
    const int p = qvalid ? P.pos[qi] : 0;
    float dsum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 t1 = *(const bf16x8*)(P.q + rowoff + s * 16 + half * 8);
      const bf16x8 t2 = *(const bf16x8*)(P.q + rowoff + (s + 4) * 16 + half * 8);
      f16x8 qh1, qh2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x1 = qvalid ? (float)t1[e] : 0.f, x2 = qvalid ? (float)t2[e] : 0.f;
        if (rot) {
          float sn, cs;
          rope_sincos(p, s * 16 + half * 8 + e, D, P.rope_base, &sn, &cs);
          const float y1 = x1 * cs - x2 * sn;
          x2 = x2 * cs + x1 * sn;
          x1 = y1;
        }
        qf[s][e] = (bf16)x1;
        qf[s + 4][e] = (bf16)x2;
        qh1[e] = to_f16_sat(x1);
        qh2[e] = to_f16_sat(x2);
      }
      if (active && qvalid) {
        *(f16x8*)(P.qs + rowoff + s * 16 + half * 8) = qh1;
        *(f16x8*)(P.qs + rowoff + (s + 4) * 16 + half * 8) = qh2;
      }
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 td = *(const bf16x8*)(P.dO + rowoff + s * 16 + half * 8);
      const bf16x8 to = *(const bf16x8*)(P.o + rowoff + s * 16 + half * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        df[s][e] = qvalid ? td[e] : (bf16)0.f;
        dsum += (float)td[e] * (float)to[e];
      }
    }
    Di = dsum + __shfl_xor(dsum, 32);
    if (!qvalid) Di = 0.f;
    lse_i = qvalid ? P.lse[(size_t)h * P.N + qi] * TA_LOG2E : 0.f;
    if (active && qvalid) {
      if (half == 0) P.Dd[(size_t)h * P.N + qi] = Di;
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  const int c0 = as_const(P.fq_ptr)[tile], c1 = as_const(P.fq_ptr)[tile + 1];
  stage_chunk(P, c0, kvh, sK[0], sV[0], sJ[0], sE[0]);
  lds_copies_wait();
  __syncthreads();

  // Swizzled LDS offsets (in elements), fixed per lane: koff[s] for the
  // 16-byte row reads of k-group s (K for S^T, V for dP^T; rows col and
  // col + 32 share them), toff[dt][x] for the K transpose read of d-tile dt,
  // rows trow + 8x of each 16-row group.
  const int trow = half * 4 + ((lane & 15) >> 2);
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int koff[8], toff[4][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = col * D + (((2 * s + half) ^ swz(col & 15)) << 3);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = trow + 8 * x;
      toff[dt][x] = r * D + (((4 * dt + (tcol >> 3)) ^ swz(r)) << 3) + (tcol & 7);
    }

  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) & 1;
    // copy the next chunk into the other buffer (the last iteration copies
    // its own chunk again, into the buffer nobody reads)
    stage_chunk(P, c + 1 < c1 ? c + 1 : c, kvh, sK[buf ^ 1], sV[buf ^ 1], sJ[buf ^ 1], sE[buf ^ 1]);
    if (active) {
      const bf16* kb = sK[buf];
      const bf16* vb = sV[buf];
      f32x16 s0 = f32x16{}, s1 = f32x16{}, p0 = f32x16{}, p1 = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a0 = *(const bf16x8*)(kb + koff[s]);
        const bf16x8 a1 = *(const bf16x8*)(kb + 32 * D + koff[s]);
        s0 = mfma32(a0, qf[s], s0);
        s1 = mfma32(a1, qf[s], s1);
        const bf16x8 b0 = *(const bf16x8*)(vb + koff[s]);
        const bf16x8 b1 = *(const bf16x8*)(vb + 32 * D + koff[s]);
        p0 = mfma32(b0, df[s], p0);
        p1 = mfma32(b1, df[s], p1);
      }
      const int full = as_const(P.fq_chunk)[(size_t)c * TA_CHUNK_INTS + 2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] = exp2f_fast(s0[r] * P.scale_log2 - lse_i);
        s1[r] = exp2f_fast(s1[r] * P.scale_log2 - lse_i);
      }
      if (!full) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int v0 = r4 * 8 + half * 4;
          const int4 J0 = *(const int4*)&sJ[buf][v0], E0 = *(const int4*)&sE[buf][v0];
          const int4 J1 = *(const int4*)&sJ[buf][32 + v0], E1 = *(const int4*)&sE[buf][32 + v0];
          const int j0[4] = {J0.x, J0.y, J0.z, J0.w}, e0[4] = {E0.x, E0.y, E0.z, E0.w};
          const int j1[4] = {J1.x, J1.y, J1.z, J1.w}, e1[4] = {E1.x, E1.y, E1.z, E1.w};
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (!(j0[u] <= qi && qi < e0[u])) s0[r4 * 4 + u] = 0.f;
            if (!(j1[u] <= qi && qi < e1[u])) s1[r4 * 4 + u] = 0.f;
          }
        }
      }
      bf16x8 db[4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        db[0][e] = (bf16)(s0[e] * (p0[e] - Di));
        db[1][e] = (bf16)(s0[8 + e] * (p0[8 + e] - Di));
        db[2][e] = (bf16)(s1[e] * (p1[e] - Di));
        db[3][e] = (bf16)(s1[8 + e] * (p1[8 + e] - Di));
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x4 t0 = lds_read_tr(kb + kk * 16 * D + toff[dt][0]);
          const bf16x4 t1 = lds_read_tr(kb + kk * 16 * D + toff[dt][1]);
          acc[dt] = mfma32(cat(t0, t1), db[kk], acc[dt]);
        }
    }
    lds_copies_wait();
    __syncthreads();
  }

  if (active && qvalid) {
    // dQ^T register r of tile dt <-> d = dt*32 + 8*(r/4) + 4*half + r%4;
    // the rotate-half partner d + 64 sits in tile dt + 2 of the same lane.
    float g[4][16];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) g[dt][r] = acc[dt][r] * P.scale;
    if (P.rope_base > 0.f) {
      const int p = P.pos[qi];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sn, cs;
          rope_sincos(p, dt * 32 + 8 * (r >> 2) + 4 * half + (r & 3), D, P.rope_base, &sn, &cs);
          const float y1 = g[dt][r], y2 = g[dt + 2][r];
          g[dt][r] = y1 * cs + y2 * sn;
          g[dt + 2][r] = y2 * cs - y1 * sn;
        }
    }
    bf16* out = P.dq + rowoff;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = (bf16)g[dt][r4 * 4 + u];
        *(bf16x4*)(out + dt * 32 + r4 * 8 + half * 4) = w;
      }
  }
}

// ---------------------------------------------------------------------------
struct KVParams {
  const f16* q;   // fp16 copy of Q (rotated when RoPE is on)
  const f16* k;   // fp16 copy of K (rotated when RoPE is on)
  const bf16* v;
  const bf16* dO;
  const float* lse;
  const float* Dd;
  bf16* dk;
  bf16* dv;
  const int32_t* pos;
  const int32_t* bk;
  int N, Hq, Hkv, G;
  float scale, scale_log2, rope_base;
};

constexpr int SUB = TA_KV_SUB;  // keys per wavefront = rows per query block

// One staged query block in LDS: fp16 Q rows (scores, and the transpose-read
// operand of dK), bf16 dO rows (dP, and the transpose-read operand of dV),
// and the rows' LSE and D.
struct KVStageLayout {
  static constexpr int Q16 = 0;                                 // f16 [SUB][PK]
  static constexpr int DO = Q16 + SUB * PK * 2;                 // bf16 [SUB][PT]
  static constexpr int LS = DO + SUB * PT * 2;                  // float [SUB]
  static constexpr int DD = LS + SUB * 4;                       // float [SUB]
  static constexpr int BYTES = DD + SUB * 4;
};

struct KVLoad {
  u32x4 q[2], d[2];
  float x;
};

__global__ __launch_bounds__(256, 1) void dkv_bf16_kernel(KVParams P) {
  using L = KVStageLayout;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::BYTES];

  const int kvh = blockIdx.x % P.Hkv;
  const cint_ptr tl = as_const(P.bk) + (size_t)(blockIdx.x / P.Hkv) * 4;
  const int k0 = tl[0], klen = tl[1], qe = tl[2];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int col = lane & 31, half = lane >> 5;
  const int kw = k0 + SUB * wave;                 // this wavefront's first key
  const int wkeys = max(0, min(SUB, klen - SUB * wave));
  const bool kvalid = col < wkeys;
  const int key = kw + col;

  // K (fp16) and V as B operands held in registers: lane = key column,
  // k-slots s*16 + half*8 + e; keys past the tile are zero.
  f16x8 kf[8];
  bf16x8 vf[8];
  {
    const size_t off = ((size_t)(kvalid ? key : k0) * P.Hkv + kvh) * D + half * 8;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 a0 = *(const u32x4*)(P.k + off + s * 16), c0 = *(const u32x4*)(P.v + off + s * 16);
      const u32x4 a = kvalid ? a0 : z, c = kvalid ? c0 : z;
      kf[s] = __builtin_bit_cast(f16x8, a);
      vf[s] = __builtin_bit_cast(bf16x8, c);
    }
  }
  // dK and dV accumulate in AGPRs for the whole loop
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  agpr_fence8(dk, dv);
  const int trow = half * 4 + ((lane & 15) >> 2);
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);

  // Items are (query head, 32-row block); all four wavefronts share each
  // staged block.  Thread t loads 32 bytes of Q and of dO of row t/8 and, for
  // t < 64, one LSE (t < 32) or D value.  Rows past the query range stage as
  // zeros (LSE = D = 0), so they contribute exactly nothing.
  const int nblk = (qe - k0 + SUB - 1) / SUB;
  const int nitem = P.G * nblk;
  const int lrow = t >> 3, lpart = (t & 7) * 16;
  // fetch() only issues loads (from always-valid rows); everything that
  // consumes the loaded values, the zero-select for rows past the range
  // included, happens in stage(), so the loads stay in flight until then.
  auto fetch = [&](int it, KVLoad& ld) {
    const int h = kvh * P.G + it / nblk;
    const int qb = k0 + SUB * (it % nblk);
    const int row = min(qb + lrow, qe - 1);
    const size_t roff = ((size_t)row * P.Hq + h) * D + lpart;
    ld.q[0] = *(const u32x4*)(P.q + roff);
    ld.q[1] = *(const u32x4*)(P.q + roff + 8);
    ld.d[0] = *(const u32x4*)(P.dO + roff);
    ld.d[1] = *(const u32x4*)(P.dO + roff + 8);
    ld.x = 0.f;
    if (t < 2 * SUB) {
      const int r = qb + (t & (SUB - 1));
      if (r < qe) ld.x = t < SUB ? P.lse[(size_t)h * P.N + r] : P.Dd[(size_t)h * P.N + r];
    }
  };
  auto stage = [&](int it, const KVLoad& ld, char* base) {
    const bool rv = k0 + SUB * (it % nblk) + lrow < qe;
    const u32x4 z = {0u, 0u, 0u, 0u};
    f16* q16 = (f16*)(base + L::Q16);
    bf16* dob = (bf16*)(base + L::DO);
    *(u32x4*)(q16 + lrow * PK + lpart) = rv ? ld.q[0] : z;
    *(u32x4*)(q16 + lrow * PK + lpart + 8) = rv ? ld.q[1] : z;
    *(u32x4*)(dob + lrow * PT + lpart) = rv ? ld.d[0] : z;
    *(u32x4*)(dob + lrow * PT + lpart + 8) = rv ? ld.d[1] : z;
    if (t < 2 * SUB) ((float*)(base + (t < SUB ? L::LS : L::DD)))[t & (SUB - 1)] = t < SUB ? ld.x * TA_LOG2E : ld.x;
  };
  // One staged block: S and dP, then P and dS in registers, then
  // dV += P^T dO (bf16) and dK += dS^T Q (fp16).  Every wavefront runs every
  // block: blocks that end before its first key are fully masked by the
  // causal compare, and keys past the tile are never stored.  (Keeping the
  // accumulating MFMAs unconditional lets the accumulators stay in AGPRs.)
  auto compute = [&](int it, const char* base) {
    const int qb = k0 + SUB * (it % nblk);
    const f16* q16 = (const f16*)(base + L::Q16);
    const bf16* dob = (const bf16*)(base + L::DO);
    const float* ls = (const float*)(base + L::LS);
    const float* dd = (const float*)(base + L::DD);
    f32x16 S = f32x16{}, dP = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const f16x8 a = *(const f16x8*)(q16 + col * PK + s * 16 + half * 8);
      const bf16x8 c = *(const bf16x8*)(dob + col * PT + s * 16 + half * 8);
      S = mfma32h(a, kf[s], S);
      dP = mfma32(c, vf[s], dP);
    }
    // register r <-> query row qb + 8*(r/4) + 4*half + r%4, key kw + col;
    // each group of four rows takes its LSE and D as one float4 from LDS
    const bool diag = qb <= kw;  // diagonal or earlier: key <= row needed
    bf16x8 pa[2];
    float ds[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 l4 = *(const float4*)(ls + 8 * r4 + 4 * half);
      const float4 d4 = *(const float4*)(dd + 8 * r4 + 4 * half);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * r4 + u;
        float p = exp2f_fast(S[r] * P.scale_log2 - lv[u]);
        if (diag && key > qb + 8 * r4 + 4 * half + u) p = 0.f;
        pa[r >> 3][r & 7] = (bf16)p;
        ds[r] = p * (dP[r] - dv4[u]);
      }
    }
    const f16x8 sa[2] = {pack_f16_rtz(ds), pack_f16_rtz(ds + 8)};
    // all transpose reads of a d-tile are issued before its four MFMAs
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      bf16x8 od[2];
      f16x8 oq[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        od[qs] = cat(lds_read_tr(dob + (qs * 16 + trow) * PT + dt * 32 + tcol),
                     lds_read_tr(dob + (qs * 16 + 8 + trow) * PT + dt * 32 + tcol));
        oq[qs] = cat(lds_read_tr(q16 + (qs * 16 + trow) * PK + dt * 32 + tcol),
                     lds_read_tr(q16 + (qs * 16 + 8 + trow) * PK + dt * 32 + tcol));
      }
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        mfma32_acc(dv[dt], pa[qs], od[qs]);
        mfma32h_acc(dk[dt], sa[qs], oq[qs]);
      }
    }
  };

  // Block b sits in LDS buffer b & 1.  Its global loads are issued two
  // blocks ahead (two register sets, alternating), so their latency hides
  // behind two blocks of compute.  Fetches and stages run unconditionally
  // (past the last item they reload it and fill a buffer nobody reads), which
  // keeps the staging registers free of control flow.  nitem >= 1: a tile's
  // query range holds at least its own first key.
  const int last = nitem - 1;
  KVLoad la, lb;
  fetch(0, la);
  stage(0, la, smem);
  fetch(min(1, last), la);
  fetch(min(2, last), lb);
  __syncthreads();
  for (int it = 0; it < nitem; it += 2) {
    compute(it, smem);
    stage(min(it + 1, last), la, smem + L::BYTES);
    fetch(min(it + 3, last), la);
    __syncthreads();
    if (it + 1 >= nitem) break;
    compute(it + 1, smem + L::BYTES);
    stage(min(it + 2, last), lb, smem);
    fetch(min(it + 4, last), lb);
    __syncthreads();
  }

  agpr_fence8(dk, dv);
  // Each wavefront owns its keys: scale and rotate dK back, store dK and dV.
  // Accumulator register r of tile dt <-> key kw + 8*(r/4) + 4*half + r%4,
  // d = dt*32 + col; the rotate-half partner d + 64 is tile dt + 2.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kr = 8 * (r >> 2) + 4 * half + (r & 3);
    if (kr >= wkeys) continue;
    const size_t o = ((size_t)(kw + kr) * P.Hkv + kvh) * D;
    float g[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) g[dt] = dk[dt][r] * P.scale;
    if (P.rope_base > 0.f) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        float sn, cs;
        rope_sincos(P.pos[kw + kr], dt * 32 + col, D, P.rope_base, &sn, &cs);
        const float y1 = g[dt], y2 = g[dt + 2];
        g[dt] = y1 * cs + y2 * sn;
        g[dt + 2] = y2 * cs - y1 * sn;
      }
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      P.dk[o + dt * 32 + col] = (bf16)g[dt];
      P.dv[o + dt * 32 + col] = (bf16)dv[dt][r];
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path.
template <int D_>
__global__ __launch_bounds__(TA_BLOCK_M) void dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                             const float* __restrict__ v, const float* __restrict__ o,
                                                             const float* __restrict__ dO, const float* __restrict__ lse,
                                                             float* __restrict__ dq, float* __restrict__ Dd,
                                                             const int32_t* __restrict__ fq_ptr,
                                                             const int32_t* __restrict__ fq_chunk, int N, int Hq,
                                                             int Hkv, float scale) {
  const int tile = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, kvh = h / G;
  const int i = tile * TA_BLOCK_M + threadIdx.x;
  if (i >= N) return;
  const size_t ro = ((size_t)i * Hq + h) * D_;
  float Di = 0.f;
  for (int x = 0; x < D_; ++x) Di = fmaf(dO[ro + x], o[ro + x], Di);
  Dd[(size_t)h * N + i] = Di;
  const float li = lse[(size_t)h * N + i];
  float acc[D_];
  for (int x = 0; x < D_; ++x) acc[x] = 0.f;
  for (int c = fq_ptr[tile]; c < fq_ptr[tile + 1]; ++c) {
    const int32_t* ch = fq_chunk + (size_t)c * TA_CHUNK_INTS;
    for (int slot = 0; slot < ch[1]; ++slot) {
      int j, kend;
      chunk_slot(ch, slot, j, kend);
      if (!(j <= i && i < kend)) continue;
      const float* kr = k + ((size_t)j * Hkv + kvh) * D_;
      const float* vr = v + ((size_t)j * Hkv + kvh) * D_;
      float s = 0.f, dp = 0.f;
      for (int x = 0; x < D_; ++x) {
        s = fmaf(q[ro + x], kr[x], s);
        dp = fmaf(dO[ro + x], vr[x], dp);
      }
      const float p = expf(s * scale - li);
      const float ds = p * (dp - Di) * scale;
      for (int x = 0; x < D_; ++x) acc[x] = fmaf(ds, kr[x], acc[x]);
    }
  }
  for (int x = 0; x < D_; ++x) dq[ro + x] = acc[x];
}

template <int D_>
__global__ __launch_bounds__(TA_BLOCK_KV) void dkv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                               const float* __restrict__ v, const float* __restrict__ dO,
                                                               const float* __restrict__ lse, const float* __restrict__ Dd,
                                                               float* __restrict__ dk, float* __restrict__ dv,
                                                               const int32_t* __restrict__ bk, int N, int Hq, int Hkv,
                                                               float scale) {
  const int32_t* tl = bk + (size_t)blockIdx.x * 4;
  const int kvh = blockIdx.y, G = Hq / Hkv;
  if ((int)threadIdx.x >= tl[1]) return;
  const int j = tl[0] + threadIdx.x, qe = tl[2];
  const size_t ko = ((size_t)j * Hkv + kvh) * D_;
  float gk[D_], gv[D_];
  for (int x = 0; x < D_; ++x) gk[x] = gv[x] = 0.f;
  for (int hs = 0; hs < G; ++hs) {
    const int h = kvh * G + hs;
    for (int i = j; i < qe; ++i) {
      const size_t ro = ((size_t)i * Hq + h) * D_;
      float s = 0.f, dp = 0.f;
      for (int x = 0; x < D_; ++x) {
        s = fmaf(q[ro + x], k[ko + x], s);
        dp = fmaf(dO[ro + x], v[ko + x], dp);
      }
      const float p = expf(s * scale - lse[(size_t)h * N + i]);
      const float ds = p * (dp - Dd[(size_t)h * N + i]) * scale;
      for (int x = 0; x < D_; ++x) {
        gv[x] = fmaf(p, dO[ro + x], gv[x]);
        gk[x] = fmaf(ds, q[ro + x], gk[x]);
      }
    }
  }
  for (int x = 0; x < D_; ++x) {
    dk[ko + x] = gk[x];
    dv[ko + x] = gv[x];
  }
}

}  // namespace bwd
}  // namespace ta

using namespace ta;

size_t ta_bwd_ws(const ta_plan* p, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d, float rope_base) {
  const size_t N = p->n_tokens;
  size_t b = align256(N * Hq * sizeof(float));  // D
  if (dt == TA_BF16) {
    b += align256(N * Hq * d * sizeof(f16)) + align256(N * Hkv * d * sizeof(f16));  // fp16 Q, K
    if (rope_base > 0.f) b += align256(N * Hkv * d * sizeof(bf16));                 // rotated bf16 K
  } else if (rope_base > 0.f) {
    b += align256(N * Hq * d * sizeof(float)) + align256(N * Hkv * d * sizeof(float));
  }
  return b;
}

extern "C" ta_status tree_attn_bwd(const ta_plan* p, const void* dplan, ta_dtype dt, const void* q, const void* k,
                                   const void* v, const void* o, const float* lse, const void* dO, int32_t Hq,
                                   int32_t Hkv, int32_t d, float scale, float rope_base, void* dq, void* dk, void* dv,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  return tree_attn_bwd_ex(p, dplan, dt, q, k, v, o, lse, dO, Hq, Hkv, d, scale, rope_base, dq, dk, dv, ws, ws_bytes,
                          nullptr, 0, stream);
}

extern "C" ta_status tree_attn_bwd_ex(const ta_plan* p, const void* dplan, ta_dtype dt, const void* q, const void* k,
                                      const void* v, const void* o, const float* lse, const void* dO, int32_t Hq,
                                      int32_t Hkv, int32_t d, float scale, float rope_base, void* dq, void* dk,
                                      void* dv, void* ws, size_t ws_bytes, hipEvent_t* ev, int32_t nev,
                                      hipStream_t stream) {
  if (!p || !dplan) return TA_EINVAL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return TA_EINVAL;
  if (dt == TA_BF16 ? d != 128 : (dt != TA_F32 || (d != 64 && d != 128))) return TA_EUNSUPPORTED;
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return TA_EINVAL;
  const size_t need = ta_bwd_ws(p, dt, Hq, Hkv, d, rope_base);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  const int N = p->n_tokens;
  if (N == 0) return TA_OK;
  if (scale <= 0.f) scale = 1.f / sqrtf((float)d);
  const char* base = (const char*)dplan;
  const int32_t* pos = (const int32_t*)(base + p->off_pos);
  const int32_t* fq_ptr = (const int32_t*)(base + p->off_fq_ptr);
  const int32_t* fq_chunk = (const int32_t*)(base + p->off_fq_chunk);
  const int32_t* fq_order = (const int32_t*)(base + p->off_fq_order);
  const int32_t* bk = (const int32_t*)(base + p->off_bk);
  const bool rope = rope_base > 0.f;
  char* w = (char*)ws;
  float* Dd = (float*)w;
  w += align256((size_t)N * Hq * sizeof(float));

  if (dt == TA_BF16) {
    f16* qs = (f16*)w;
    w += align256((size_t)N * Hq * d * sizeof(f16));
    f16* ks = (f16*)w;
    w += align256((size_t)N * Hkv * d * sizeof(f16));
    mark(ev, nev, 0, stream);
    const bf16* kb = (const bf16*)k;
    if (launch_rope<bf16, f16>((const bf16*)k, ks, pos, N, Hkv, d, rope_base, 0, stream) != hipSuccess)
      return TA_EHIP;
    if (rope) {
      if (launch_rope<bf16, bf16>((const bf16*)k, (bf16*)w, pos, N, Hkv, d, rope_base, 0, stream) != hipSuccess)
        return TA_EHIP;
      kb = (const bf16*)w;
    }
    mark(ev, nev, 1, stream);
    bwd::DQParams A;
    A.q = (const bf16*)q;
    A.k = kb;
    A.v = (const bf16*)v;
    A.o = (const bf16*)o;
    A.dO = (const bf16*)dO;
    A.lse = lse;
    A.dq = (bf16*)dq;
    A.Dd = Dd;
    A.qs = qs;
    A.pos = pos;
    A.fq_ptr = fq_ptr;
    A.fq_chunk = fq_chunk;
    A.fq_order = fq_order;
    A.N = N;
    A.Hq = Hq;
    A.Hkv = Hkv;
    A.G = Hq / Hkv;
    A.scale = scale;
    A.scale_log2 = scale * TA_LOG2E;
    A.rope_base = rope_base;
    hipLaunchKernelGGL(bwd::dq_bf16_kernel, dim3(p->n_qtiles * Hkv, (A.G + 3) / 4), dim3(256), 0, stream, A);
    TA_LAUNCH_CHECK();
    mark(ev, nev, 2, stream);

    bwd::KVParams B;
    B.q = qs;
    B.k = ks;
    B.v = (const bf16*)v;
    B.dO = (const bf16*)dO;
    B.lse = lse;
    B.Dd = Dd;
    B.dk = (bf16*)dk;
    B.dv = (bf16*)dv;
    B.pos = pos;
    B.bk = bk;
    B.N = N;
    B.Hq = Hq;
    B.Hkv = Hkv;
    B.G = Hq / Hkv;
    B.scale = scale;
    B.scale_log2 = scale * TA_LOG2E;
    B.rope_base = rope_base;
    hipLaunchKernelGGL(bwd::dkv_bf16_kernel, dim3(p->n_ktiles * Hkv), dim3(256), 0, stream, B);
    TA_LAUNCH_CHECK();
    mark(ev, nev, 3, stream);
    return TA_OK;
  }

  void* qrot = rope ? (void*)w : nullptr;
  if (rope) w += align256((size_t)N * Hq * d * sizeof(float));
  void* krot = rope ? (void*)w : nullptr;
  const float* qq = (const float*)q;
  const float* kk = (const float*)k;
  if (rope) {
    if (launch_rope<float, float>(qq, (float*)qrot, pos, N, Hq, d, rope_base, 0, stream) != hipSuccess) return TA_EHIP;
    if (launch_rope<float, float>(kk, (float*)krot, pos, N, Hkv, d, rope_base, 0, stream) != hipSuccess) return TA_EHIP;
    qq = (const float*)qrot;
    kk = (const float*)krot;
  }
  dim3 g1(p->n_qtiles, Hq), g2(p->n_ktiles, Hkv);
  if (d == 64) {
    hipLaunchKernelGGL(bwd::dq_f32_kernel<64>, g1, dim3(TA_BLOCK_M), 0, stream, qq, kk, (const float*)v,
                       (const float*)o, (const float*)dO, lse, (float*)dq, Dd, fq_ptr, fq_chunk, N, Hq, Hkv, scale);
    hipLaunchKernelGGL(bwd::dkv_f32_kernel<64>, g2, dim3(TA_BLOCK_KV), 0, stream, qq, kk, (const float*)v,
                       (const float*)dO, lse, Dd, (float*)dk, (float*)dv, bk, N, Hq, Hkv, scale);
  } else {
    hipLaunchKernelGGL(bwd::dq_f32_kernel<128>, g1, dim3(TA_BLOCK_M), 0, stream, qq, kk, (const float*)v,
                       (const float*)o, (const float*)dO, lse, (float*)dq, Dd, fq_ptr, fq_chunk, N, Hq, Hkv, scale);
    hipLaunchKernelGGL(bwd::dkv_f32_kernel<128>, g2, dim3(TA_BLOCK_KV), 0, stream, qq, kk, (const float*)v,
                       (const float*)dO, lse, Dd, (float*)dk, (float*)dv, bk, N, Hq, Hkv, scale);
  }
  TA_LAUNCH_CHECK();
  if (rope) {
    if (launch_rope<float, float>((const float*)dq, (float*)dq, pos, N, Hq, d, rope_base, 1, stream) != hipSuccess)
      return TA_EHIP;
    if (launch_rope<float, float>((const float*)dk, (float*)dk, pos, N, Hkv, d, rope_base, 1, stream) != hipSuccess)
      return TA_EHIP;
  }
  return TA_OK;
}
