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
// On one stream, no atomics, bitwise deterministic.  bf16 with the full
// workspace (the dS path):
//  1. preparation: fp16 copy of K times scale * log2(e) (rotated with RoPE);
//     prep_kernel: fp16 copy of the rotated Q, -D and -LSE * log2(e);
//  2. dK/dV, key-stationary, over the planner's work pieces: up to four
//     32-key sub-tiles of one node per workgroup, each worked by two
//     wavefronts on one SIMD (one holds K and forms S, P and dV; the other
//     holds V and forms dP, dS and dK, taking P from the first through LDS),
//     over a common run of 32-row query blocks on the query-tile grid.  Every
//     query of a node's DFS interval reads every key of the node, so Q and dO
//     stream as contiguous blocks with no gather; each block is staged in LDS
//     once for the eight wavefronts, and the loop runs over every query head
//     of the GQA group, so the group's sum stays in registers.  Scores use
//     the fp16 copies of rotated Q and K (finer rounding than bf16 for
//     rotated values; same MFMA rate), so P matches the forward's.  dV += P^T
//     dO and dK += dS^T Q use the LDS transpose read of the staged blocks.
//     The fp16 dS of every (query tile, sub-tile) block is stored for step 3,
//     and sub-tiles cut over several query windows leave fp32 partials that
//     dkv_sum_kernel adds in a fixed order;
//  3. dQ = scale dS K from the stored dS (dq_ds_kernel), query-stationary
//     over each query tile's list of sub-tiles.
// With the smallest workspace the dQ kernel (dq_bf16_kernel) runs before
// dK/dV instead, walks the forward's gathered key chunks and recomputes P
// from LSE and dP (S^T, dP^T and dQ^T as MFMA tiles with the query on the
// lane, K^T from the LDS transpose read); it also writes the fp16 rotated Q,
// -D and -LSE * log2(e) that dK/dV reads.  The fp32 path keeps plain
// reference kernels (a thread per query row / key).
#include <algorithm>

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
  float* nld;   // [Hq][nqb][64] out: per 32-row query block, -LSE * log2(e) of its rows, then -D
  f16* qs;      // [N, Hq, d] out: fp16 copy of Q (rotated when RoPE is on)
  int32_t* sat;  // saturation flag (fp16 conversion of Q clamped)
  const int32_t* pos;
  const int32_t* fq_ptr;
  const int32_t* fq_chunk;
  const int32_t* fq_order;
  int N, Hq, Hkv, G, nqb;
  int q0;  // first query row (rows below are a key-only prefix)
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
  // this lane's row within each 4-row copy and its swizzled 16-byte piece
  // (rows 4i + l/16 with i = w + 4k share their low four bits)
  const int sub = l >> 4;
  const int poff = ((l & 15) ^ swz((4 * w + sub) & 15)) << 3;
  if (ch.h[0] == 1 && ch.h[1] == BN) {
    // one segment filling all 64 slots: slot v holds key v + delta
    const int delta = ch.ks[0] - ch.ko[0];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = w + 4 * k;
      const size_t off = ((size_t)(4 * i + sub + delta) * P.Hkv + kvh) * D + poff;
      copy16_to_lds(P.k + off, sKb + 4 * i * D);
      copy16_to_lds(P.v + off, sVb + 4 * i * D);
    }
    if (t < BN) {
      sJb[t] = t + delta;
      sEb[t] = ch.ke[0];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = w + 4 * k;
      int j, e;
      chunk_slot(ch, 4 * i + sub, j, e);
      const size_t off = ((size_t)j * P.Hkv + kvh) * D + poff;
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
}

__global__ __launch_bounds__(256, 2) void dq_bf16_kernel(DQParams P) {
  __shared__ __attribute__((aligned(1024))) bf16 sK[2][BN * D];
  __shared__ __attribute__((aligned(1024))) bf16 sV[2][BN * D];
  __shared__ __attribute__((aligned(16))) int sJ[2][BN];
  __shared__ __attribute__((aligned(16))) int sE[2][BN];
  __shared__ double sInv[D / 2];

  const int kvh = blockIdx.x % P.Hkv;
  const int tile = as_const(P.fq_order)[blockIdx.x / P.Hkv];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int hsub = blockIdx.y * 4 + wave;
  rope_inv_table(sInv, D / 2, D, P.rope_base);
  __syncthreads();
  const bool active = hsub < P.G;
  const int h = kvh * P.G + (active ? hsub : 0);
  const int qi = P.q0 + tile * BM + col;
  const bool qvalid = qi < P.N;
  const size_t rowoff = ((size_t)(qvalid ? qi : 0) * P.Hq + h) * D;

  // Q (rotated) and dO as B operands; D_i = dO_i . O_i
  bf16x8 qf[8], df[8];
  float Di, lse_i;
  {
    bool sat = false;
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
          rope_sincos_at(p, sInv[s * 16 + half * 8 + e], &sn, &cs);
          const float y1 = x1 * cs - x2 * sn;
          x2 = x2 * cs + x1 * sn;
          x1 = y1;
        }
        qf[s][e] = (bf16)x1;
        qf[s + 4][e] = (bf16)x2;
        qh1[e] = to_f16_sat(x1, sat);
        qh2[e] = to_f16_sat(x2, sat);
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
    report_sat(P.sat, sat && active);
    Di = dsum + __shfl_xor(dsum, 32);
    if (!qvalid) Di = 0.f;
    lse_i = qvalid ? P.lse[(size_t)h * P.N + qi] * TA_LOG2E : 0.f;
    // rows past the last token get zeros: the dK/dV kernel stages whole
    // 32-row blocks and masks those rows, and 0 * (finite) stays 0
    if (active && half == 0) {
      float* rec = P.nld + ((size_t)h * P.nqb + tile) * (2 * BM);
      rec[col] = qvalid ? -lse_i : 0.f;
      rec[BM + col] = qvalid ? -Di : 0.f;
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
    // The chunk is processed as two halves of 32 keys, which keeps S^T and
    // dP^T at 16 registers each (the kernel fits two workgroups per CU).
    // Wavefronts without a head (fewer than four heads per KV head) compute
    // too and never store.
    {
      const int full = as_const(P.fq_chunk)[(size_t)c * TA_CHUNK_INTS + 2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16* kb = sK[buf] + kh * 32 * D;
        const bf16* vb = sV[buf] + kh * 32 * D;
        f32x16 sc = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          sc = mfma32(*(const bf16x8*)(kb + koff[s]), qf[s], sc);
          dp = mfma32(*(const bf16x8*)(vb + koff[s]), df[s], dp);
        }
        // S^T register r <-> key slot kh*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = exp2f_fast(sc[r] * P.scale_log2 - lse_i);
        if (!full) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int v0 = kh * 32 + r4 * 8 + half * 4;
            const int4 J = *(const int4*)&sJ[buf][v0], E = *(const int4*)&sE[buf][v0];
            const int jj[4] = {J.x, J.y, J.z, J.w}, ee[4] = {E.x, E.y, E.z, E.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (!(jj[u] <= qi && qi < ee[u])) sc[r4 * 4 + u] = 0.f;
          }
        }
        bf16x8 db[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          db[0][e] = (bf16)(sc[e] * (dp[e] - Di));
          db[1][e] = (bf16)(sc[8 + e] * (dp[8 + e] - Di));
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const bf16x4 t0 = lds_read_tr(kb + kk * 16 * D + toff[dt][0]);
            const bf16x4 t1 = lds_read_tr(kb + kk * 16 * D + toff[dt][1]);
            acc[dt] = mfma32(cat(t0, t1), db[kk], acc[dt]);
          }
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
          rope_sincos_at(p, sInv[dt * 32 + 8 * (r >> 2) + 4 * half + (r & 3)], &sn, &cs);
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
// A dS block holds the fp16 dS of 32 keys x 32 positions (position
// half*16 + r is accumulator register r of the dK/dV lanes of half `half`,
// i.e. query row 8*(r/4) + 4*half + r%4 of the block) in the dK/dV lanes'
// register order: plane i = r/8 holds, for lane l = key + 32*half, the
// eight values r%8 = 0..7 as one 16-byte unit, at unit l in plane 0 and
// unit l^4 in plane 1.  Each plane is one contiguous 1 KiB store of the
// producing wavefront; the XOR keeps the two planes' units of a transpose
// read on different LDS banks.  Element offset (in f16 units):
__device__ __forceinline__ constexpr int ds_elem(int key, int pos) {
  return ((pos >> 3) & 1) * 512 + ((key + 32 * (pos >> 4)) ^ (4 * ((pos >> 3) & 1))) * 8 + (pos & 7);
}

struct KVParams {
  const f16* q;   // fp16 copy of Q (rotated when RoPE is on)
  const f16* k;   // fp16 copy of K (rotated when RoPE is on) times scale * log2(e)
  const bf16* v;
  const bf16* dO;
  const float* nld;  // [Hq][nqb][64]: per 32-row query block, -LSE * log2(e) of its rows, then -D
  bf16* dk;
  bf16* dv;
  const int32_t* pos;
  const int32_t* kp;  // work pieces, TA_KPIECE_INTS each
  const int32_t* kr;  // cut sub-tiles: (kw, wk, first slot, n_windows)
  float* part;        // partial dK/dV slots (PART_WAVE floats per slot and KV head)
  f16* ds;            // dS blocks [nkv][n_dsblk][G] of 32 keys x 32 positions (ds_elem) of this round's KV heads (dS path only)
  f16* ds_spare;      // a 32 x 32 block that absorbs the stores of blocks a wavefront does not own
  int n_sum;          // cut sub-tiles
  int n_dsblk;
  int kv0, nkv;       // this launch's KV heads: kv0 .. kv0 + nkv - 1 (the backward may run them in rounds)
  int nqb;            // 32-row query blocks from q0 (the plan's query tiles)
  int N, Hq, Hkv, G;
  int q0;  // first query row (rows below are a key-only prefix)
  float scale, scale_log2, rope_base;
};

constexpr int SUB = TA_KV_SUB;  // keys per wavefront = rows per query block

// A partial slot holds one wavefront's raw dK and dV accumulators for one
// KV head in register order: [dK | dV] each [tile dt 4][r/4 4][lane 64]
// [r%4 4] floats, so the wavefront writes and reads 1 KiB contiguous runs
// (register r of tile dt of lane l <-> key 8*(r/4) + 4*(l/32) + r%4 of its
// 32, dimension dt*32 + l%32).
constexpr int PART_WAVE = 2 * 4 * 16 * 64;

// dK of one key (scaled, rotated back by -pos) and dV of one key, in bf16,
// dimensions dt*32 + col for dt = 0..3 (the rotate-half partner of d is tile
// dt + 2).  inv: the inverse frequencies of dimensions col and 32 + col.
__device__ __forceinline__ void store_k(const KVParams& P, int kvh, int key, int col, const double (&inv)[2],
                                        float (&g)[4]) {
  const size_t o = ((size_t)key * P.Hkv + kvh) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) g[dt] *= P.scale;
  if (P.rope_base > 0.f) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      float sn, cs;
      rope_sincos_at(P.pos[key], inv[dt], &sn, &cs);
      const float y1 = g[dt], y2 = g[dt + 2];
      g[dt] = y1 * cs + y2 * sn;
      g[dt + 2] = y2 * cs - y1 * sn;
    }
  }
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) P.dk[o + dt * 32 + col] = (bf16)g[dt];
}
__device__ __forceinline__ void store_v(const KVParams& P, int kvh, int key, int col, const float (&v)[4]) {
  const size_t o = ((size_t)key * P.Hkv + kvh) * D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) P.dv[o + dt * 32 + col] = (bf16)v[dt];
}

// One staged query block in LDS: fp16 Q rows (scores, and the transpose-read
// operand of dK), bf16 dO rows (dP, and the transpose-read operand of dV),
// both as swizzled 256-byte rows (see swz), and the rows' -LSE * log2(e) and
// -D, which seed the S and dP accumulators.
struct KVStageLayout {
  static constexpr int Q16 = 0;                  // f16 [SUB][D]
  static constexpr int DO = Q16 + SUB * D * 2;   // bf16 [SUB][D]
  static constexpr int LS = DO + SUB * D * 2;    // float [SUB]
  static constexpr int DD = LS + SUB * 4;        // float [SUB]
  static constexpr int BYTES = DD + SUB * 4;
};
static_assert(KVStageLayout::BYTES % 16 == 0, "stage buffers stay 16-byte aligned");
constexpr int KV_NBUF = 7;           // staged blocks: copies run five items ahead, a block lives three steps
constexpr int KV_XCH = 2 * 64 * 16;  // one sub-tile's P block in fp16: [register half 2][lane 64][16 bytes]

// Two wavefronts per 32-key sub-tile, one of each role, eight per workgroup
// (wavefronts w and w + 4 share sub-tile w; with eight wavefronts on four
// SIMDs every SIMD holds two, so one's MFMAs can run while the other
// waits, whichever pairing the dispatcher makes):
//  role A (w < 4) holds the sub-tile's K, computes S = Q K^T - LSE, P and
//    dV += P^T dO, and hands P (fp16) to its partner through LDS;
//  role B (w >= 4) holds V, computes dP = dO V^T - D, dS = P dP (with the P
//    of the previous step) and dK += dS^T Q, and stores the fp16 dS blocks.
// Each role keeps 64 accumulators instead of 128, so two wavefronts fit on
// every SIMD and one's MFMAs run while the other waits on its exponentials,
// LDS reads or conversions.  All eight share the staged blocks; a block is
// read by A one step before its item (scores), by both during it, and by B
// one step after (dK); seven buffers rotate and copies run five items
// ahead, so a copy has three steps to land.  Items are (32-row block, query head) of the piece's rows
// [qlo, qhi), blocks from the end down and the heads of the group innermost:
// the workgroups resident on an XCD share a KV head and mostly the same
// rows, so one fetch serves them from L2.  Rows past qhi (and past the last
// token, clamped to it) are masked to P = 0, like every row outside a
// sub-tile's [key, rhi), so they contribute nothing.
// DS: also store the fp16 dS blocks for the dQ pass (the dS path).
template <bool DS>
__global__ __launch_bounds__(512, 1) void dkv_bf16_kernel(KVParams P) {
  using L = KVStageLayout;
  __shared__ __attribute__((aligned(1024))) char smem[KV_NBUF * L::BYTES + 2 * 4 * KV_XCH];

  const int kvr = blockIdx.x % P.nkv, kvh = P.kv0 + kvr;
  const cint_ptr tl = as_const(P.kp) + (size_t)(blockIdx.x / P.nkv) * TA_KPIECE_INTS;
  const int qlo = tl[0], qhi = tl[1];
  const int lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = wv & 3;
  const bool roleB = wv >= 4;
  // sub-tile w: keys [kw, kw + wkeys) (0: idle), rows [rlo, rhi) within
  // [qlo, qhi) (each key reads rows [max(key, rlo), rhi)), partial slot or
  // -1, and the dS block of query tile t: dsoff + t
  const cint_ptr tw = tl + 4 + TA_KWAVE_INTS * w;
  const int kw = tw[0], wkeys = tw[1], rlo = tw[2], rhi = tw[3], slot = tw[4], dsoff = tw[5];
  const bool kvalid = col < wkeys;
  const int key = kw + col;

  // K (fp16, role A) or V (bf16, role B) as the B operand of the score
  // MFMAs, held in registers: lane = key column, k-slots s*16 + half*8 + e;
  // keys past the tile are zero.
  u32x4 fr[8];
  {
    const char* src = roleB ? (const char*)P.v : (const char*)P.k;
    const size_t off = (((size_t)(kvalid ? key : kw) * P.Hkv + kvh) * D + half * 8) * 2;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 a = *(const u32x4*)(src + off + s * 32);
      fr[s] = kvalid ? a : z;
    }
  }
  // dV (role A) or dK (role B) accumulates in registers for the whole loop
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};
  acc_fence4(acc);

  // Swizzled LDS offsets (in bytes), fixed per lane: koff[s] for the 16-byte
  // row reads of k-group s (Q for S, dO for dP), toff[dt][x] for the
  // transpose reads of d-tile dt, rows trow + 8x of each 16-row group.
  const int trow = half * 4 + ((lane & 15) >> 2);
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int koff[8], toff[4][2];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff[s] = 2 * (col * D + (((2 * s + half) ^ swz(col & 15)) << 3));
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = trow + 8 * x;
      toff[dt][x] = 2 * (r * D + (((4 * dt + (tcol >> 3)) ^ swz(r)) << 3) + (tcol & 7));
    }

  const int G = P.G;
  const int nblk = (qhi - qlo + SUB - 1) / SUB;   // >= 1: the plan gives every piece a query row
  const int nitem = G * nblk;
  // Staging: wavefront wv copies rows 4 wv + lane/16 of the block's fp16 Q
  // and bf16 dO (a swizzled 16-byte piece per lane), and wavefront 0 also
  // the block's 32 -LSE * log2(e) and 32 -D values (one 256-byte record).
  // The per-lane offsets inside a block are fixed, so only the scalar base
  // (block, head) changes from item to item.  The staging cursor (sbi, sg)
  // walks the items without divisions (past the last item it repeats the
  // last one, into the buffer nobody reads); sbuf is the buffer it fills.
  const int rowA = 4 * wv + (lane >> 4);
  const uint32_t piece = (uint32_t)(((lane & 15) ^ swz(rowA & 15)) << 4);
  const uint32_t rstride = (uint32_t)P.Hq * (D * 2);
  const uint32_t lds0 = lds_addr(smem);
  int sbi = nblk - 1, sg = 0, sbuf = 0;
  auto stage_next = [&]() {
    const int qb = qlo + SUB * sbi;
    const int h = kvh * G + sg;
    const uint32_t v = (uint32_t)min(rowA, P.N - 1 - qb) * rstride + piece;
    const size_t off = ((size_t)qb * P.Hq + h) * (D * 2);
    const uint32_t lb = lds0 + sbuf * L::BYTES;
    copy16_to_lds_s((const char*)P.q + off, v, lb + L::Q16 + wv * 1024);
    copy16_to_lds_s((const char*)P.dO + off, v, lb + L::DO + wv * 1024);
    if (wv == 0) copy4_to_lds_s(P.nld + ((size_t)h * P.nqb + ((qb - P.q0) >> 5)) * (2 * SUB), lane * 4, lb + L::LS);
    if (sg + 1 < G) {
      ++sg;
    } else if (sbi > 0) {
      sg = 0;
      --sbi;
    }
    sbuf = sbuf + 1 == KV_NBUF ? 0 : sbuf + 1;
  };
  // Each wavefront issues two copies per step (wavefront 0 three), role B
  // two dS stores after them.  Vector memory operations complete in issue
  // order.  At the end of step j the items up to j + 3 must have landed (the
  // next step reads item j + 3 ahead, see end_step_a): role A allows four
  // outstanding operations (the copies of items j + 4 and j + 5; wavefront 0
  // six).  Role B allows six: this step's copies and stores and the stores of
  // step j - 1, so its copies of j + 4 and everything before them (the
  // stores of step j - 2 included) have completed.
  auto end_step = []() {
    asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __syncthreads();
  };
  auto buf = [&](int b) { return smem + b * L::BYTES; };
  auto next_buf = [](int b) { return b + 1 == KV_NBUF ? 0 : b + 1; };
  auto fence = []() { __builtin_amdgcn_sched_barrier(0); };
  // an item cursor (block bi, head g), advanced like the staging cursor
  auto adv = [&](int& bi, int& g) {
    if (g + 1 < G) {
      ++g;
    } else {
      g = 0;
      --bi;
    }
  };
  char* const xch = smem + KV_NBUF * L::BYTES + w * KV_XCH + lane * 16;  // this lane's P slot, parity 0

#pragma unroll
  for (int i = 0; i < 5; ++i) stage_next();
  asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // items 0, 1 and 2 landed
  __syncthreads();

  if (!roleB) {
    // ---- role A: S, P, dV ------------------------------------------------
    // element mask limit: key <= row < rhi is (row - key) < lim; keys past a
    // short sub-tile read no rows, so their P is exactly zero
    const unsigned lim = kvalid ? (unsigned)max(rhi - key, 0) : 0u;
    auto seed = [&](const char* b, f32x16& S) {  // register r <-> row 8*(r/4) + 4*half + r%4
      const float* ls = (const float*)(b + L::LS);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 l4 = *(const float4*)(ls + 8 * r4 + 4 * half);
        S[4 * r4 + 0] = l4.x;
        S[4 * r4 + 1] = l4.y;
        S[4 * r4 + 2] = l4.z;
        S[4 * r4 + 3] = l4.w;
      }
    };
    int cb = 0, ibi = nblk - 1, ig = 0;  // item j: buffer, block, head
    f32x16 Sa, Sb;
    {
      const char* b0 = buf(0);
      seed(b0, Sa);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        Sa = mfma32h(*(const f16x8*)(b0 + L::Q16 + koff[s]), __builtin_bit_cast(f16x8, fr[s]), Sa);
    }
    f16x8 qn0, qn1;  // the first two Q operands of the next step's score MFMAs
    {
      const char* b1 = buf(1);
      seed(b1, Sb);
      qn0 = *(const f16x8*)(b1 + L::Q16 + koff[0]);
      qn1 = *(const f16x8*)(b1 + L::Q16 + koff[1]);
    }
    // At the end of step j every wavefront has waited for its copies of the
    // items up to j + 3 (role A: four copies of items j + 4, j + 5 may be
    // outstanding, six for wavefront 0, which also copies the seed records;
    // role B: six, see below), so after the barrier the items up to j + 3 are
    // in LDS and step j + 1 may read item j + 3 ahead of its own barrier.
    auto end_step_a = [&]() {
      if (wv == 0)
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      __syncthreads();
    };
    // One step per item j, in two runs of eight MFMAs.  The score MFMAs of
    // item j + 1 (a dependent chain) carry the element mask's result and the
    // exponentials of S(j) (computed in the previous step) between them, so
    // the VALU work of a step runs while this wavefront's own MFMAs do; then
    // the dV += P(j)^T dO(j) MFMAs (d-tiles innermost, so consecutive ones are
    // independent), with P(j) handed to role B through LDS among them.  The
    // copies of item j + 5 go out in the first run.  LDS operands are read two
    // MFMAs ahead; the seed and first two operands of the next step's score
    // MFMAs (item j + 2) are read at the end of the second run, so the next
    // step's first MFMA waits for no LDS read.  The source order is the issue
    // order.
    auto step = [&](int j, f32x16& Sg, f32x16& Sn) {
      const char* gb = buf(cb);
      const char* nb = buf(next_buf(cb));
      const char* nnb = buf(next_buf(next_buf(cb)));  // item j + 2
      const int qb = qlo + SUB * ibi;
      f16x8 qa[8];
      bf16x8 od[8];  // transpose reads of dO(j): MFMA m = 2 dt + qs
      auto read_od = [&](int m) {
        const char* o = gb + L::DO + (m & 1) * 16 * D * 2;
        od[m] = cat(lds_read_tr((const bf16*)(o + toff[m >> 1][0])), lds_read_tr((const bf16*)(o + toff[m >> 1][1])));
      };
      qa[0] = qn0;  // Sn already holds its seed
      qa[1] = qn1;
      if (qb < kw + SUB || qb + SUB > rhi || wkeys < SUB) {
        const int d0 = qb + 4 * half - key;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((unsigned)(d0 + 8 * (r >> 2) + (r & 3)) >= lim) Sg[r] = -INFINITY;
      }
      fence();
      // score MFMAs of item j + 1 with the exponentials of item j between them
      float p[16];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < 6) qa[s + 2] = *(const f16x8*)(nb + L::Q16 + koff[s + 2]);
        if (s >= 6) read_od(2 * (s - 6));
        Sn = mfma32h(qa[s], __builtin_bit_cast(f16x8, fr[s]), Sn);
        p[2 * s] = exp2f_fast(Sg[2 * s]);
        p[2 * s + 1] = exp2f_fast(Sg[2 * s + 1]);
        if (s == 1) stage_next();
        fence();
      }
      bf16x8 pa[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) pa[hh][e] = (bf16)p[8 * hh + e];
      fence();
      char* const xp = xch + (j & 1) * (4 * KV_XCH);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = 2 * (u & 3) + (u >> 2);  // d-tiles innermost: consecutive MFMAs are independent
        if (u < 6) read_od(2 * ((u + 2) & 3) + ((u + 2) >> 2));
        acc[s >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa[s & 1], od[s], acc[s >> 1], 0, 0, 0);
        if (u == 2) *(f16x8*)xp = pack_f16_rte(p);
        if (u == 3) *(f16x8*)(xp + 1024) = pack_f16_rte(p + 8);
        if (u == 6) seed(nnb, Sg);  // S(j) is spent: it becomes S(j + 2)'s seed
        if (u == 7) {
          qn0 = *(const f16x8*)(nnb + L::Q16 + koff[0]);
          qn1 = *(const f16x8*)(nnb + L::Q16 + koff[1]);
        }
        fence();
      }
      cb = next_buf(cb);
      adv(ibi, ig);
    };
    for (int j = 0; j < nitem; j += 2) {
      step(j, Sa, Sb);
      end_step_a();
      if (j + 1 >= nitem) break;
      step(j + 1, Sb, Sa);
      end_step_a();
    }
    lds_copies_wait();
    acc_fence4(acc);
    if (slot < 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * half + (r & 3);
        if (kr >= wkeys) continue;
        const float v[4] = {acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
        store_v(P, kvh, kw + kr, col, v);
      }
    } else if (wkeys > 0) {
      float* dst = P.part + ((size_t)slot * P.Hkv + kvh) * PART_WAVE + PART_WAVE / 2 + lane * 4;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(float4*)(dst + (dt * 4 + r4) * 256) =
              float4{acc[dt][4 * r4], acc[dt][4 * r4 + 1], acc[dt][4 * r4 + 2], acc[dt][4 * r4 + 3]};
    }
  } else {
    // ---- role B: dP, dS, dK ------------------------------------------------
    auto seed = [&](const char* b, f32x16& dP) {
      const float* dd = (const float*)(b + L::DD);
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 d4 = *(const float4*)(dd + 8 * r4 + 4 * half);
        dP[4 * r4 + 0] = d4.x;
        dP[4 * r4 + 1] = d4.y;
        dP[4 * r4 + 2] = d4.z;
        dP[4 * r4 + 3] = d4.w;
      }
    };
    const int ds_lane0 = ds_elem(col, half * 16), ds_lane1 = ds_elem(col, half * 16 + 8);  // this lane's two units
    int cb = 0, ibi = nblk - 1, ig = 0;         // item j - 1 of step j: buffer, block, head
    f32x16 dPa, dPb;
    {  // step 0: dP of item 0 only
      const char* b0 = buf(0);
      seed(b0, dPa);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        dPa = mfma32(*(const bf16x8*)(b0 + L::DO + koff[s]), __builtin_bit_cast(bf16x8, fr[s]), dPa);
      stage_next();
      asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // items up to 3 landed
      __syncthreads();
    }
    // the first two dO operands of the next step's dP MFMAs; step j + 1's dP
    // seed is written into the spent dP(j - 1)
    bf16x8 on0, on1;
    {
      const char* b1 = buf(1);
      seed(b1, dPb);
      on0 = *(const bf16x8*)(b1 + L::DO + koff[0]);
      on1 = *(const bf16x8*)(b1 + L::DO + koff[1]);
    }
    // Step j, in two runs of eight MFMAs: the dP MFMAs of item j (unless
    // `last`; a dependent chain) with dS(j - 1) = P dP formed between them
    // (the P role A handed over in step j - 1, dP from the previous step),
    // then dK += dS(j - 1)^T Q(j - 1) (d-tiles innermost) with the two dS
    // stores among them.  The copies of item j + 5 go out in the first run.
    // LDS operands are read two MFMAs ahead; the seed and first two operands
    // of the next step's dP MFMAs (item j + 1) are read at the end of the
    // second run.
    auto step = [&](int j, f32x16& dPg, f32x16& dPn, bool last) {
      const char* gb = buf(cb);               // item j - 1: transpose-read Q
      const char* nb = buf(next_buf(cb));     // item j: dO rows and -D
      const char* nnb = buf(next_buf(next_buf(cb)));  // item j + 1
      const int qb = qlo + SUB * ibi;
      bf16x8 oa[8];
      f16x8 oq[8];  // transpose reads of Q(j - 1): MFMA m = 2 dt + qs
      auto read_oq = [&](int m) {
        const char* q = gb + L::Q16 + (m & 1) * 16 * D * 2;
        oq[m] = cat(lds_read_tr((const f16*)(q + toff[m >> 1][0])), lds_read_tr((const f16*)(q + toff[m >> 1][1])));
      };
      const char* xp = xch + ((j - 1) & 1) * (4 * KV_XCH);
      const f16x8 ph0 = *(const f16x8*)xp;
      const f16x8 ph1 = *(const f16x8*)(xp + 1024);
      if (!last) {
        oa[0] = on0;
        oa[1] = on1;
      }
      fence();
      // dP MFMAs of item j with dS(j - 1) = P dP formed between them
      float ds[16];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (!last) {
          if (s < 6) oa[s + 2] = *(const bf16x8*)(nb + L::DO + koff[s + 2]);
        }
        if (s >= 6) read_oq(2 * (s - 6));
        if (!last) dPn = mfma32(oa[s], __builtin_bit_cast(bf16x8, fr[s]), dPn);
        {
          const f16x8 ph = s < 4 ? ph0 : ph1;
          ds[2 * s] = (float)ph[(2 * s) & 7] * dPg[2 * s];
          ds[2 * s + 1] = (float)ph[(2 * s + 1) & 7] * dPg[2 * s + 1];
        }
        if (s == 1 && !last) stage_next();
        fence();
      }
      f16x8 sa[2];
      sa[0] = pack_f16_rtz(ds);
      sa[1] = pack_f16_rtz(ds + 8);
      f16* blk = P.ds_spare;
      if (DS) {
        const bool own = wkeys > 0 && qb < rhi && qb + SUB > rlo;
        if (own) blk = P.ds + (((size_t)kvr * P.n_dsblk + dsoff + ((qb - P.q0) >> 5)) * G + ig) * (SUB * SUB);
      }
      fence();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int s = 2 * (u & 3) + (u >> 2);  // d-tiles innermost: consecutive MFMAs are independent
        if (u < 6) read_oq(2 * ((u + 2) & 3) + ((u + 2) >> 2));
        acc[s >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(sa[s & 1], oq[s], acc[s >> 1], 0, 0, 0);
        if (DS && u == 2) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sa[0]), (u32x4*)(blk + ds_lane0));
        if (DS && u == 3) __builtin_nontemporal_store(__builtin_bit_cast(u32x4, sa[1]), (u32x4*)(blk + ds_lane1));
        if (!last && u == 6) seed(nnb, dPg);  // item j + 1
        if (!last && u == 7) {
          on0 = *(const bf16x8*)(nnb + L::DO + koff[0]);
          on1 = *(const bf16x8*)(nnb + L::DO + koff[1]);
        }
        fence();
      }
      cb = next_buf(cb);
      adv(ibi, ig);
    };
    int j = 1;
    for (; j + 1 < nitem; j += 2) {
      step(j, dPa, dPb, false);
      end_step();
      step(j + 1, dPb, dPa, false);
      end_step();
    }
    if (j < nitem) {  // one more full step (item j), then the last from dPb
      step(j, dPa, dPb, false);
      end_step();
      step(nitem, dPb, dPa, true);
    } else {
      step(nitem, dPa, dPb, true);
    }
    lds_copies_wait();
    acc_fence4(acc);
    if (slot < 0) {
      const double inv[2] = {P.rope_base > 0.f ? rope_inv(col, D, P.rope_base) : 0.0,
                             P.rope_base > 0.f ? rope_inv(32 + col, D, P.rope_base) : 0.0};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * half + (r & 3);
        if (kr >= wkeys) continue;
        float g[4] = {acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
        store_k(P, kvh, kw + kr, col, inv, g);
      }
    } else if (wkeys > 0) {
      float* dst = P.part + ((size_t)slot * P.Hkv + kvh) * PART_WAVE + lane * 4;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(float4*)(dst + (dt * 4 + r4) * 256) =
              float4{acc[dt][4 * r4], acc[dt][4 * r4 + 1], acc[dt][4 * r4 + 2], acc[dt][4 * r4 + 3]};
    }
  }
}

// Sums the partial slots of each cut sub-tile in slot order (deterministic)
// and stores its dK / dV as the whole-piece epilogue does.  One wavefront per
// cut sub-tile, four per workgroup, and one workgroup per (four sub-tiles, KV
// head, register group g); group g holds accumulator registers 4g..4g+3 of
// every tile (keys 8g + 4*half + 0..3).
__global__ __launch_bounds__(256) void dkv_sum_kernel(KVParams P) {
  const int g = blockIdx.x & 3, rest = blockIdx.x >> 2;
  const int kvh = P.kv0 + rest % P.nkv;
  const int i = (rest / P.nkv) * 4 + (threadIdx.x >> 6);
  if (i >= P.n_sum) return;
  const int32_t* tl = P.kr + (size_t)i * 4;
  const int kw = tl[0], wkeys = tl[1], slot0 = tl[2], np = tl[3];
  const int lane = threadIdx.x & 63;
  float sk[4][4], sv[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) sk[dt][j] = sv[dt][j] = 0.f;
  for (int s = 0; s < np; ++s) {
    const float* src = P.part + ((size_t)(slot0 + s) * P.Hkv + kvh) * PART_WAVE + g * 256 + lane * 4;
    float4 a[4], b[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      a[dt] = *(const float4*)(src + dt * 1024);
      b[dt] = *(const float4*)(src + PART_WAVE / 2 + dt * 1024);
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      sk[dt][0] += a[dt].x;
      sk[dt][1] += a[dt].y;
      sk[dt][2] += a[dt].z;
      sk[dt][3] += a[dt].w;
      sv[dt][0] += b[dt].x;
      sv[dt][1] += b[dt].y;
      sv[dt][2] += b[dt].z;
      sv[dt][3] += b[dt].w;
    }
  }
  // register 4g + j of tile dt <-> key kw + 8g + 4*half + j
  const double inv[2] = {P.rope_base > 0.f ? rope_inv(lane & 31, D, P.rope_base) : 0.0,
                         P.rope_base > 0.f ? rope_inv(32 + (lane & 31), D, P.rope_base) : 0.0};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = 8 * g + 4 * (lane >> 5) + j;
    if (kr >= wkeys) continue;
    float gk[4] = {sk[0][j], sk[1][j], sk[2][j], sk[3][j]};
    const float gv[4] = {sv[0][j], sv[1][j], sv[2][j], sv[3][j]};
    store_k(P, kvh, kw + kr, lane & 31, inv, gk);
    store_v(P, kvh, kw + kr, lane & 31, gv);
  }
}

// ---------------------------------------------------------------------------
// fp32 path.
// ---------------------------------------------------------------------------
// The dS path.  The dK/dV kernel stores the fp16 dS of every (query tile,
// 32-key sub-tile) block it computes, and dQ = scale * dS K becomes one
// product instead of recomputing S and dP (three).  Before dK/dV, prep_kernel
// writes what the recomputing dQ kernel otherwise produces for it: the fp16
// copy of Q (rotated by position when RoPE is on), -D = -(dO . O) and
// -LSE * log2(e), for query rows >= q_start.  Eight lanes per (row, head):
// lane j takes dimensions 8j..8j+7 and their rotate-half partners 64 + 8j..,
// and D is summed over the eight.
struct PrepParams {
  const bf16* q;
  const bf16* o;
  const bf16* dO;
  const float* lse;
  f16* qs;
  float* nld;  // [Hq][nqb][64]: per 32-row query block, -LSE * log2(e), then -D
  int32_t* sat;  // saturation flag (fp16 conversion of Q clamped)
  const int32_t* pos;
  int N, Hq, q0, nqb;
  float rope_base;
};

__global__ __launch_bounds__(256) void prep_kernel(PrepParams P) {
  __shared__ double sInv[D / 2];
  rope_inv_table(sInv, D / 2, D, P.rope_base);
  __syncthreads();
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t pr = gid >> 3;
  const int j = (int)(gid & 7);
  if (pr >= (size_t)P.nqb * 32 * P.Hq) return;  // whole groups of eight lanes
  const int row = P.q0 + (int)(pr / P.Hq), h = (int)(pr % P.Hq);
  const int rb = row - P.q0;
  float* rec = P.nld + ((size_t)h * P.nqb + (rb >> 5)) * 64 + (rb & 31);
  if (row >= P.N) {  // padding rows of the last block: zeros (the dK/dV kernel masks them)
    if (j == 0) rec[0] = rec[32] = 0.f;
    return;
  }
  const size_t off = ((size_t)row * P.Hq + h) * D + 8 * j;
  const bf16x8 q1 = *(const bf16x8*)(P.q + off), q2 = *(const bf16x8*)(P.q + off + D / 2);
  const bf16x8 o1 = *(const bf16x8*)(P.o + off), o2 = *(const bf16x8*)(P.o + off + D / 2);
  const bf16x8 d1 = *(const bf16x8*)(P.dO + off), d2 = *(const bf16x8*)(P.dO + off + D / 2);
  const bool rot = P.rope_base > 0.f;
  const int p = P.pos[row];
  float dsum = 0.f;
  bool sat = false;
  f16x8 h1, h2;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    dsum += (float)d1[e] * (float)o1[e] + (float)d2[e] * (float)o2[e];
    float x1 = (float)q1[e], x2 = (float)q2[e];
    if (rot) {
      float sn, cs;
      rope_sincos_at(p, sInv[8 * j + e], &sn, &cs);
      const float y1 = x1 * cs - x2 * sn;
      x2 = x2 * cs + x1 * sn;
      x1 = y1;
    }
    h1[e] = to_f16_sat(x1, sat);
    h2[e] = to_f16_sat(x2, sat);
  }
  report_sat(P.sat, sat);
  *(f16x8*)(P.qs + off) = h1;
  *(f16x8*)(P.qs + off + D / 2) = h2;
  dsum += __shfl_xor(dsum, 1);
  dsum += __shfl_xor(dsum, 2);
  dsum += __shfl_xor(dsum, 4);
  if (j == 0) {
    rec[0] = -P.lse[(size_t)h * P.N + row] * TA_LOG2E;
    rec[32] = -dsum;
  }
}

struct DSParams {
  const f16* k;   // fp16 K * scale * log2(e) (rotated when RoPE is on)
  const f16* ds;  // [nkv][n_dsblk][G] blocks of 32 keys x 32 positions (ds_elem): this round's KV heads
  bf16* dq;
  const int32_t* pos;
  const int32_t* dq_ptr;
  const int32_t* dq_ent;
  const int32_t* dq_order;
  int N, Hq, Hkv, G, q0, n_dsblk;
  int kv0, nkv;  // this launch's KV heads
  float rope_base;
};

// dQ from the stored dS: one workgroup per (query tile, KV head) and up to
// four heads of its group, one wavefront per head.  For each 32-key sub-tile
// some row of the tile reads (the plan's list, by first key) the sub-tile's
// fp16 K rows and the heads' dS blocks are copied straight into a three-buffer
// LDS ring two entries ahead (48 KB, three workgroups per CU: the dS blocks
// come from HBM and the latency wants many in flight); dQ^T += K^T dS^T
// on 32x32x16 fp16 MFMA, both operands from transpose reads.  The K copy
// carries scale * log2(e), so dQ = ln(2) * the accumulators; rotated back in
// the epilogue.  A fixed order over the list: bitwise repeatable.
constexpr int DS_COPIES = 4;  // copies per wavefront per entry: two of K rows, two of dS

__global__ __launch_bounds__(256, 3) void dq_ds_kernel(DSParams P) {
  __shared__ __attribute__((aligned(1024))) f16 sK[3][SUB * D];
  __shared__ __attribute__((aligned(1024))) f16 sS[3][4][SUB * SUB];
  __shared__ double sInv[D / 2];  // read after the loop's barriers

  const int kvr = blockIdx.x % P.nkv, kvh = P.kv0 + kvr;
  const int tile = as_const(P.dq_order)[blockIdx.x / P.nkv];
  rope_inv_table(sInv, D / 2, D, P.rope_base);
  const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hsub = blockIdx.y * 4 + w;
  const bool active = hsub < P.G;
  const int g = active ? hsub : 0;  // wavefronts without a head copy head 0's blocks and never store
  const int e0 = as_const(P.dq_ptr)[tile], e1 = as_const(P.dq_ptr)[tile + 1];  // e1 > e0: a row reads its own key
  const int last = e1 - 1;

  // copy instruction i of the K rows fills rows 4i..4i+3 (wavefront w: i = w, w + 4);
  // the dS block of this wavefront's head is two 1 KiB copies
  auto stage = [&](int e, int b) {
    const cint_ptr en = as_const(P.dq_ent) + (size_t)e * 4;
    const int kw = en[0], wk = en[1], blk = en[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int i = w + 4 * c;
      const int row = 4 * i + (lane >> 4);
      const size_t off = ((size_t)(kw + min(row, wk - 1)) * P.Hkv + kvh) * D + (((lane & 15) ^ swz(row & 15)) << 3);
      copy16_to_lds(P.k + off, sK[b] + 4 * i * D);
    }
    const f16* src = P.ds + (((size_t)kvr * P.n_dsblk + blk) * P.G + g) * (SUB * SUB) + lane * 8;
    copy16_to_lds_nt(src, sS[b][w]);
    copy16_to_lds_nt(src + 512, sS[b][w] + 512);
  };

  // transpose-read offsets: K^T of d-tile dt (256-byte swizzled rows), dS^T
  // (the ds_elem layout: positions tcol..tcol+3 of one key are 8 contiguous
  // bytes); rows (keys) trow + 8x of each 16-key group kk, soff[kk][x]
  const int trow = half * 4 + ((lane & 15) >> 2);
  const int tcol = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int toff[4][2], soff[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int r = trow + 8 * x;
    soff[0][x] = ds_elem(r, tcol);
    soff[1][x] = ds_elem(16 + r, tcol);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) toff[dt][x] = r * D + (((4 * dt + (tcol >> 3)) ^ swz(r)) << 3) + (tcol & 7);
  }

  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x16{};

  stage(e0, 0);
  stage(min(e0 + 1, last), 1);
  asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // entry e0 landed
  __syncthreads();
  for (int e = e0; e < e1; ++e) {
    const int b = (e - e0) % 3;
    // the buffer refilled here was last read in the previous iteration, before its barrier
    stage(min(e + 2, last), (e - e0 + 2) % 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const f16* sb = sS[b][w];
      const f16x8 bs = cat(lds_read_tr(sb + soff[kk][0]), lds_read_tr(sb + soff[kk][1]));
      const f16* kb = sK[b] + kk * 16 * D;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma32h(cat(lds_read_tr(kb + toff[dt][0]), lds_read_tr(kb + toff[dt][1])), bs, acc[dt]);
    }
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");  // entry e + 1 landed
    __syncthreads();
  }
  lds_copies_wait();

  // dQ^T register r of tile dt <-> d = dt*32 + 8*(r/4) + 4*half + r%4; lane
  // column `col` is dS position col, i.e. row 8*((col%16)/4) + 4*(col/16) +
  // col%4 of the tile; the rotate-half partner d + 64 sits in tile dt + 2.
  const int qi = P.q0 + tile * SUB + 8 * ((col & 15) >> 2) + 4 * (col >> 4) + (col & 3);
  if (active && qi < P.N) {
    constexpr float LN2 = 0.69314718055994530942f;
    float gq[4][16];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) gq[dt][r] = acc[dt][r] * LN2;
    if (P.rope_base > 0.f) {
      const int p = P.pos[qi];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float sn, cs;
          rope_sincos_at(p, sInv[dt * 32 + 8 * (r >> 2) + 4 * half + (r & 3)], &sn, &cs);
          const float y1 = gq[dt][r], y2 = gq[dt + 2][r];
          gq[dt][r] = y1 * cs + y2 * sn;
          gq[dt + 2][r] = y2 * cs - y1 * sn;
        }
    }
    bf16* out = P.dq + ((size_t)qi * P.Hq + kvh * P.G + hsub) * D;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 v;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = (bf16)gq[dt][r4 * 4 + u];
        *(bf16x4*)(out + dt * 32 + r4 * 8 + half * 4) = v;
      }
  }
}

template <int D_>
__global__ __launch_bounds__(TA_BLOCK_M) void dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                             const float* __restrict__ v, const float* __restrict__ o,
                                                             const float* __restrict__ dO, const float* __restrict__ lse,
                                                             float* __restrict__ dq, float* __restrict__ Dd,
                                                             const int32_t* __restrict__ fq_ptr,
                                                             const int32_t* __restrict__ fq_chunk, int N, int Hq,
                                                             int Hkv, float scale, int q0) {
  const int tile = blockIdx.x, h = blockIdx.y, G = Hq / Hkv, kvh = h / G;
  const int i = q0 + tile * TA_BLOCK_M + threadIdx.x;
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
                                                               float scale, int q0) {
  const int32_t* tl = bk + (size_t)blockIdx.x * 4;
  const int kvh = blockIdx.y, G = Hq / Hkv;
  if ((int)threadIdx.x >= tl[1]) return;
  const int j = tl[0] + threadIdx.x, qe = tl[2];
  const size_t ko = ((size_t)j * Hkv + kvh) * D_;
  float gk[D_], gv[D_];
  for (int x = 0; x < D_; ++x) gk[x] = gv[x] = 0.f;
  for (int hs = 0; hs < G; ++hs) {
    const int h = kvh * G + hs;
    for (int i = max(j, q0); i < qe; ++i) {
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

constexpr size_t SUB_SQ = TA_KV_SUB * TA_KV_SUB;

// dS blocks of one KV head (its Hq / Hkv query heads): 32 x 32 fp16 per
// (query tile, sub-tile) block and query head.
static size_t ds_head_bytes(const ta_plan* p, int32_t Hq, int32_t Hkv) {
  return (size_t)p->n_dsblk * (Hq / Hkv) * SUB_SQ * sizeof(f16);
}

// Backward workspace.  ds_heads > 0 (bf16): the dS path with room for the dS
// blocks of ds_heads KV heads at a time (the KV heads then run in rounds of
// that many), plus a spare block.
size_t ta_bwd_ws_heads(const ta_plan* p, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d, float rope_base,
                       int ds_heads) {
  const size_t N = p->n_tokens;
  size_t b = 0;
  if (dt == TA_BF16) {
    b += TA_WS_FLAG_BYTES;                                                           // saturation flag
    b += align256((size_t)Hq * p->n_qtiles * 64 * sizeof(float));                    // -LSE log2(e), -D blocks
    b += align256(N * Hq * d * sizeof(f16)) + align256(N * Hkv * d * sizeof(f16));  // fp16 Q, K
    if (rope_base > 0.f) b += align256(N * Hkv * d * sizeof(bf16));                 // rotated bf16 K
    b += align256((size_t)p->n_kslots * Hkv * bwd::PART_WAVE * sizeof(float));       // dK/dV partials
    if (ds_heads > 0) b += align256((size_t)ds_heads * ds_head_bytes(p, Hq, Hkv)) +  // dS blocks
                           align256(SUB_SQ * sizeof(f16));                           // + a spare one
  } else {
    b += align256(N * Hq * sizeof(float));  // D
    if (rope_base > 0.f) b += align256(N * Hq * d * sizeof(float)) + align256(N * Hkv * d * sizeof(float));
  }
  return b;
}

size_t ta_bwd_ws(const ta_plan* p, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d, float rope_base, bool with_ds) {
  return ta_bwd_ws_heads(p, dt, Hq, Hkv, d, rope_base, with_ds && dt == TA_BF16 ? Hkv : 0);
}

// KV heads whose dS blocks fit a workspace of ws_bytes (0: the recompute path).
static int ds_heads_for(const ta_plan* p, int32_t Hq, int32_t Hkv, int32_t d, float rope_base, size_t ws_bytes) {
  for (int h = Hkv; h >= 1; --h)
    if (ta_bwd_ws_heads(p, TA_BF16, Hq, Hkv, d, rope_base, h) <= ws_bytes) return h;
  return 0;
}

extern "C" ta_status tree_attn_bwd_ws_budget(const ta_plan* p, ta_dtype dt, int32_t Hq, int32_t Hkv, int32_t d,
                                             float rope_base, size_t budget, size_t* bytes,
                                             int32_t* kv_heads_per_round) {
  if (!p || !bytes || !kv_heads_per_round || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return TA_EINVAL;
  if (budget == 0) budget = TA_BWD_WS_BUDGET_DEFAULT;
  const size_t smallest = ta_bwd_ws_heads(p, dt, Hq, Hkv, d, rope_base, 0);
  const int h = dt == TA_BF16 ? ds_heads_for(p, Hq, Hkv, d, rope_base, budget) : 0;
  *kv_heads_per_round = h;
  *bytes = h > 0 ? ta_bwd_ws_heads(p, dt, Hq, Hkv, d, rope_base, h) : smallest;
  return *bytes <= budget ? TA_OK : TA_ENOMEM;
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
  if (p->n_tokens == 0) return TA_OK;  // nothing to read or write (empty tensors may be null)
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return TA_EINVAL;
  // bf16: the dS path when the workspace holds the dS blocks of at least one
  // KV head (the KV heads then run in rounds of as many as fit), else dQ
  // recomputes S and dP
  const size_t need = ta_bwd_ws(p, dt, Hq, Hkv, d, rope_base, false);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  const int ds_heads = dt == TA_BF16 ? ds_heads_for(p, Hq, Hkv, d, rope_base, ws_bytes) : 0;
  const bool ds_path = ds_heads > 0;
  const int N = p->n_tokens;
  if (scale <= 0.f) scale = 1.f / sqrtf((float)d);
  const char* base = (const char*)dplan;
  const int32_t* pos = (const int32_t*)(base + p->off_pos);
  const int32_t* fq_ptr = (const int32_t*)(base + p->off_fq_ptr);
  const int32_t* fq_chunk = (const int32_t*)(base + p->off_fq_chunk);
  const int32_t* fq_order = (const int32_t*)(base + p->off_fq_order);
  const int32_t* bk = (const int32_t*)(base + p->off_bk);
  const int32_t* kp = (const int32_t*)(base + p->off_kp);
  const int32_t* kr = (const int32_t*)(base + p->off_kr);
  const bool rope = rope_base > 0.f;
  char* w = (char*)ws;

  if (dt == TA_BF16) {
    int32_t* sat = (int32_t*)w;
    w += TA_WS_FLAG_BYTES;
    float* nld = (float*)w;
    w += align256((size_t)Hq * p->n_qtiles * 64 * sizeof(float));
    f16* qs = (f16*)w;
    w += align256((size_t)N * Hq * d * sizeof(f16));
    f16* ks = (f16*)w;
    w += align256((size_t)N * Hkv * d * sizeof(f16));
    bf16* krot = rope ? (bf16*)w : nullptr;
    if (rope) w += align256((size_t)N * Hkv * d * sizeof(bf16));
    float* part = (float*)w;
    w += align256((size_t)p->n_kslots * Hkv * bwd::PART_WAVE * sizeof(float));
    f16* dsb = ds_path ? (f16*)w : nullptr;
    f16* ds_spare = ds_path ? (f16*)(w + align256((size_t)ds_heads * ds_head_bytes(p, Hq, Hkv))) : nullptr;
    const int32_t* dq_ptr = (const int32_t*)(base + p->off_dq_ptr);
    const int32_t* dq_ent = (const int32_t*)(base + p->off_dq_ent);
    const int32_t* dq_order = (const int32_t*)(base + p->off_dq_order);
    mark(ev, nev, 0, stream);
    // one pass: fp16 K * scale * log2(e) for dK/dV's scores and, with RoPE,
    // the rotated bf16 K for dQ
    const bf16* kb = rope ? krot : (const bf16*)k;
    if (launch_rope<bf16, f16>((const bf16*)k, ks, pos, N, Hkv, d, rope_base, 0, stream, scale * TA_LOG2E,
                               ds_path ? nullptr : krot, sat) != hipSuccess)
      return TA_EHIP;
    if (ds_path) {
      bwd::PrepParams R;
      R.q = (const bf16*)q;
      R.o = (const bf16*)o;
      R.dO = (const bf16*)dO;
      R.lse = lse;
      R.qs = qs;
      R.nld = nld;
      R.sat = sat;
      R.pos = pos;
      R.N = N;
      R.Hq = Hq;
      R.q0 = p->q_start;
      R.nqb = p->n_qtiles;
      R.rope_base = rope_base;
      const size_t lanes = (size_t)p->n_qtiles * 32 * Hq * 8;
      if (lanes > 0) {
        hipLaunchKernelGGL(bwd::prep_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, stream, R);
        TA_LAUNCH_CHECK();
      }
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
    A.nld = nld;
    A.qs = qs;
    A.sat = sat;
    A.pos = pos;
    A.fq_ptr = fq_ptr;
    A.fq_chunk = fq_chunk;
    A.fq_order = fq_order;
    A.N = N;
    A.Hq = Hq;
    A.Hkv = Hkv;
    A.G = Hq / Hkv;
    A.nqb = p->n_qtiles;
    A.q0 = p->q_start;
    A.scale = scale;
    A.scale_log2 = scale * TA_LOG2E;
    A.rope_base = rope_base;
    if (!ds_path) {
      hipLaunchKernelGGL(bwd::dq_bf16_kernel, dim3(p->n_qtiles * Hkv, (A.G + 3) / 4), dim3(256), 0, stream, A);
      TA_LAUNCH_CHECK();
      mark(ev, nev, 2, stream);
    }

    bwd::KVParams B;
    B.q = qs;
    B.k = ks;
    B.v = (const bf16*)v;
    B.dO = (const bf16*)dO;
    B.nld = nld;
    B.dk = (bf16*)dk;
    B.dv = (bf16*)dv;
    B.pos = pos;
    B.kp = kp;
    B.kr = kr;
    B.part = part;
    B.ds = dsb;
    B.ds_spare = ds_spare;
    B.n_dsblk = (int)p->n_dsblk;
    B.n_sum = p->n_ksplit;
    B.nqb = p->n_qtiles;
    B.N = N;
    B.Hq = Hq;
    B.Hkv = Hkv;
    B.G = Hq / Hkv;
    B.q0 = p->q_start;
    B.scale = scale;
    B.scale_log2 = scale * TA_LOG2E;
    B.rope_base = rope_base;
    bwd::DSParams Q;
    if (ds_path) {
      Q.k = ks;
      Q.ds = dsb;
      Q.dq = (bf16*)dq;
      Q.pos = pos;
      Q.dq_ptr = dq_ptr;
      Q.dq_ent = dq_ent;
      Q.dq_order = dq_order;
      Q.N = N;
      Q.Hq = Hq;
      Q.Hkv = Hkv;
      Q.G = Hq / Hkv;
      Q.q0 = p->q_start;
      Q.n_dsblk = (int)p->n_dsblk;
      Q.rope_base = rope_base;
    }
    // dK/dV (storing dS) and then dQ from the stored dS, for the KV heads
    // whose dS blocks fit the workspace at once: a query head's dQ depends on
    // its own KV head's keys only, so rounds over KV heads give the same
    // results bit for bit.  Without the dS workspace, one round of dK/dV.
    const int per_round = ds_path ? ds_heads : Hkv;
    for (int kv0 = 0; kv0 < Hkv; kv0 += per_round) {
      const int nkv = std::min(per_round, Hkv - kv0);
      B.kv0 = kv0;
      B.nkv = nkv;
      if (ds_path)
        hipLaunchKernelGGL(bwd::dkv_bf16_kernel<true>, dim3(p->n_kpieces * nkv), dim3(512), 0, stream, B);
      else
        hipLaunchKernelGGL(bwd::dkv_bf16_kernel<false>, dim3(p->n_kpieces * nkv), dim3(512), 0, stream, B);
      TA_LAUNCH_CHECK();
      if (p->n_ksplit > 0) {
        hipLaunchKernelGGL(bwd::dkv_sum_kernel, dim3((p->n_ksplit + 3) / 4 * nkv * 4), dim3(256), 0, stream, B);
        TA_LAUNCH_CHECK();
      }
      if (ds_path) {
        if (kv0 == 0) mark(ev, nev, 2, stream);
        Q.kv0 = kv0;
        Q.nkv = nkv;
        if (p->n_qtiles > 0) {
          hipLaunchKernelGGL(bwd::dq_ds_kernel, dim3(p->n_qtiles * nkv, (Q.G + 3) / 4), dim3(256), 0, stream, Q);
          TA_LAUNCH_CHECK();
        }
      }
    }
    mark(ev, nev, 3, stream);
    return TA_OK;
  }

  float* Dd = (float*)w;
  w += align256((size_t)N * Hq * sizeof(float));
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
                       (const float*)o, (const float*)dO, lse, (float*)dq, Dd, fq_ptr, fq_chunk, N, Hq, Hkv, scale,
                       p->q_start);
    hipLaunchKernelGGL(bwd::dkv_f32_kernel<64>, g2, dim3(TA_BLOCK_KV), 0, stream, qq, kk, (const float*)v,
                       (const float*)dO, lse, Dd, (float*)dk, (float*)dv, bk, N, Hq, Hkv, scale,
                       p->q_start);
  } else {
    hipLaunchKernelGGL(bwd::dq_f32_kernel<128>, g1, dim3(TA_BLOCK_M), 0, stream, qq, kk, (const float*)v,
                       (const float*)o, (const float*)dO, lse, (float*)dq, Dd, fq_ptr, fq_chunk, N, Hq, Hkv, scale,
                       p->q_start);
    hipLaunchKernelGGL(bwd::dkv_f32_kernel<128>, g2, dim3(TA_BLOCK_KV), 0, stream, qq, kk, (const float*)v,
                       (const float*)dO, lse, Dd, (float*)dk, (float*)dv, bk, N, Hq, Hkv, scale,
                       p->q_start);
  }
  TA_LAUNCH_CHECK();
  if (rope) {
    const int q0 = p->q_start;  // prefix rows of dQ are not outputs: leave them untouched
    if (launch_rope<float, float>((const float*)dq + (size_t)q0 * Hq * d, (float*)dq + (size_t)q0 * Hq * d,
                                  pos + q0, N - q0, Hq, d, rope_base, 1, stream) != hipSuccess)
      return TA_EHIP;
    if (launch_rope<float, float>((const float*)dk, (float*)dk, pos, N, Hkv, d, rope_base, 1, stream) != hipSuccess)
      return TA_EHIP;
  }
  return TA_OK;
}
