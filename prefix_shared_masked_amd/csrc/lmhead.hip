// Output layer fused with the g_t/K weighted NLL (agent-rl chapter 14,
// section 14.3: the N x V logits are never held whole -- the forward reduces
// them tile by tile, the backward recomputes them chunk by chunk; Tree
// Training post, sections 6.2 and 6.3: loss = sum_t w_t [y_t valid]
// (logsumexp_v(h_t . W_v) - h_t . W_y)).
//
//  - lse_kernel: S^T = W h^T on 32x32x16 bf16 MFMA over tiles of 256 vocab
//    rows x 256 tokens, k in stages of 32 copied HBM -> LDS by direct copies
//    into a four-deep ring; the vocabulary is on the MFMA rows and the tokens
//    on the lanes, so each token's running (max, sum) stays in registers.  A
//    workgroup walks a slice of the vocabulary and writes per-token partials.
//  - merge_kernel: one wavefront per token merges the partials into LSE,
//    forms the label logit h_t . W_y and the weighted token loss; a single
//    workgroup sums the token losses in a fixed order (bitwise reproducible).
//  - ds_kernel (backward, per vocabulary chunk): the same tiles recomputed,
//    epilogue dS = w [valid] (exp(S - LSE) - onehot(y)) in bf16, laid out
//    [tokens rounded up to 32, chunk rows] with zeros past the last token and
//    the last vocabulary row; then gemm_kernel twice on the same tiling:
//    dh += dS W_chunk (fp32 accumulator) and dW_chunk = dS^T h.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"

namespace ta {
namespace lmh {

constexpr int BT = 256;                    // tokens per tile
constexpr int BV = 256;                    // vocabulary rows per tile
constexpr int KS = 32;                     // k per ring stage
constexpr int NBUF = 4;                    // ring depth
constexpr int TILE_BYTES = 256 * KS * 2;   // one operand tile of a stage (16 KB)
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr float L2E = 1.4426950408889634f;

// Accumulating MFMA into AGPRs with all 16 tiles fenced together (see
// mfma32_acc / agpr_fence8 in common.h for the wait-state reasoning).
__device__ __forceinline__ void agpr_fence16(f32x16 (&x)[4][4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0][0]), "+a"(x[0][1]), "+a"(x[0][2]), "+a"(x[0][3]), "+a"(x[1][0]), "+a"(x[1][1]),
                 "+a"(x[1][2]), "+a"(x[1][3]), "+a"(x[2][0]), "+a"(x[2][1]), "+a"(x[2][2]), "+a"(x[2][3]),
                 "+a"(x[3][0]), "+a"(x[3][1]), "+a"(x[3][2]), "+a"(x[3][3]));
}

__device__ __forceinline__ int swz4(int row) { return (row >> 2) & 3; }

// Rows [r0, r0 + 256) x k [k0, k0 + KS) of X ([nrows, Dm] bf16; rows past
// the end repeat the last row) into an LDS tile of 256 rows x 64 bytes whose
// 16-byte pieces sit at position piece ^ swz4(row): the 16 rows read by a
// quarter-wavefront land on 16 distinct bank groups.  Copy q (0..15) fills
// rows 16q..16q+15 (lane l: row 16q + l/4, position l%4); wave w issues
// q = w + 4i.
__device__ __forceinline__ void stage_tile(const bf16* X, int r0, int nrows, int Dm, int k0, char* tile) {
  const int l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = w + 4 * i;
    const int row = 16 * q + (l >> 2);
    const int piece = (l & 3) ^ swz4(row);
    const int gr = min(r0 + row, nrows - 1);
    copy16_to_lds(X + (size_t)gr * Dm + k0 + piece * 8, tile + q * 1024);
  }
}

struct Params {
  const bf16* h;        // [N, Dm]
  const bf16* W;        // [V, Dm]
  const int32_t* labels;
  const float* w;
  const float* lse;     // [N] natural log (ds_kernel)
  float2* part;         // [n_parts][N] (m in log2 units, l) (lse_kernel)
  bf16* ds;             // [N][ld_ds] (ds_kernel): the chunk's dS, token-major
  int ld_ds;            // row stride of ds (the chunk's row capacity)
  int N, V, Dm;
  int n_pad;            // rows of ds: N rounded up to KS (the rows past N are written as zeros)
  int vt_per_wg;        // vocabulary tiles per workgroup
  int vt_first;         // first vocabulary tile of the launch
  int vt_last;          // one past the last vocabulary tile of the launch
  int ignore_index;
};

// The tile loop shared by both kernels: workgroup (blockIdx.x = token tile,
// blockIdx.y = slice of vocabulary tiles) runs every (vocabulary tile,
// k-stage) of its slice through the ring and calls epi(vt, acc) once per
// vocabulary tile with S^T of the 256 x 256 tile in the accumulators:
// acc[i][j] register r <-> vocab row 128*wv + 32*i + 8*(r/4) + 4*half + r%4,
// token 128*wt + 32*j + l%32 of the tile.
template <typename Epi>
__device__ __forceinline__ void tile_loop(const Params& P, char* ring, Epi&& epi) {
  const int t0 = blockIdx.x * BT;
  const int vt0 = P.vt_first + blockIdx.y * P.vt_per_wg;
  const int vt1 = min(P.vt_last, vt0 + P.vt_per_wg);
  if (vt0 >= vt1) return;  // uniform over the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane & 31, half = lane >> 5;
  const int wv = wave & 1, wt = wave >> 1;
  const int nk = P.Dm / KS;
  const int total = (vt1 - vt0) * nk;

  // Copy i of a stage fills rows 16 q .. 16 q + 15 (q = wave + 4 i) of each
  // tile (stage_tile's lane map): with a scalar base at the stage's first row
  // and k column, each lane's byte offset is fixed, the token rows clamped to
  // the last token once; a vocabulary tile that runs past the last row takes
  // the clamped stage_tile.  The stages are issued in order, so a cursor (vt,
  // kk) replaces the division of the stage index.
  const int l = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  uint32_t offw[4], offh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * (wu + 4 * i) + (l >> 2);
    const int piece = (l & 3) ^ swz4(row);
    offw[i] = (uint32_t)(row * P.Dm + piece * 8) * 2u;
    offh[i] = (uint32_t)(min(row, P.N - 1 - t0) * P.Dm + piece * 8) * 2u;
  }
  const uint32_t lds0 = lds_addr(ring);
  int iv = vt0, ik = 0, ip = 0;  // the next stage to issue: vocabulary tile, k stage, index
  auto issue = [&]() {
    const uint32_t lb = lds0 + (ip % NBUF) * STAGE_BYTES;
    const int k0 = ik * KS;
    if ((iv + 1) * BV <= P.V) {
      const bf16* wb = P.W + ((size_t)iv * BV * P.Dm + k0);
#pragma unroll
      for (int i = 0; i < 4; ++i) copy16_to_lds_s(wb, offw[i], lb + (wu + 4 * i) * 1024);
    } else {
      stage_tile(P.W, iv * BV, P.V, P.Dm, k0, ring + (ip % NBUF) * STAGE_BYTES);
    }
    const bf16* hb = P.h + ((size_t)t0 * P.Dm + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) copy16_to_lds_s(hb, offh[i], lb + TILE_BYTES + (wu + 4 * i) * 1024);
    ++ip;
    if (++ik == nk) {
      ik = 0;
      ++iv;
    }
  };

  // per-lane LDS offsets: vocab tile i at abase + 2048 i, token tile j at
  // bbase + 2048 j, k-substep s at po[s]
  const int sw = swz4(rr);
  const int po[2] = {((0 + half) ^ sw) << 4, ((2 + half) ^ sw) << 4};
  const int abase = (128 * wv + rr) * 64;
  const int bbase = TILE_BYTES + (128 * wt + rr) * 64;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  agpr_fence16(acc);

  for (int p = 0; p < min(NBUF - 1, total); ++p) issue();
  for (int it = 0; it < total; ++it) {
    // this wave's copies of stage `it` have landed once at most the copies of
    // the stages issued after it (8 per stage) are outstanding
    const int after = min(NBUF - 2, total - 1 - it);
    if (after >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies landed; every wave is done with stage it - 1
    if (it + NBUF - 1 < total) issue();  // stage it + NBUF - 1 refills the buffer of stage it - 1
    const char* buf = ring + (it % NBUF) * STAGE_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const bf16x8*)(buf + abase + 2048 * i + po[s]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const bf16x8*)(buf + bbase + 2048 * j + po[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma32_acc(acc[i][j], a[i], b[j]);
    }
    if (it % nk == nk - 1) {
      agpr_fence16(acc);
      epi(vt0 + it / nk, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
      agpr_fence16(acc);
    }
  }
  lds_copies_wait();
}

__global__ __launch_bounds__(256, 1) void lse_kernel(Params P) {
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * STAGE_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane & 31, half = lane >> 5;
  const int wv = wave & 1, wt = wave >> 1;
  float m[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
  }
  tile_loop(P, ring, [&](int vt, f32x16 (&acc)[4][4]) {
    const int vb = vt * BV + 128 * wv;  // this wave's first vocabulary row
    // rows at offset 32 i + 8 (r/4) + r%4 >= lim (past the vocabulary) are
    // left out; only the last tile has any
    const int lim = P.V - vb - 4 * half;
    const bool ragged = vb + 128 > P.V;  // uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool in = !ragged || 32 * i + 8 * (r >> 2) + (r & 3) < lim;
          mx = __builtin_elementwise_maximum(mx, in ? acc[i][j][r] : -INFINITY);
        }
      mx = __builtin_elementwise_maximum(mx, __shfl_xor(mx, 32)) * L2E;
      const float mn = __builtin_elementwise_maximum(m[j], mx);
      const float mu = mn == -INFINITY ? 0.f : mn;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool in = !ragged || 32 * i + 8 * (r >> 2) + (r & 3) < lim;
          const float e = exp2f_fast(fmaf(acc[i][j][r], L2E, -mu));
          s += in ? e : 0.f;
        }
      l[j] = l[j] * exp2f_fast(m[j] - mu) + s;
      m[j] = mn;
    }
  });
  // this wave's partial over its half of every vocabulary tile of the slice
  const int slot = blockIdx.y * 2 + wv;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lt = l[j] + __shfl_xor(l[j], 32);
    const int t = blockIdx.x * BT + 128 * wt + 32 * j + rr;
    if (half == 0 && t < P.N) P.part[(size_t)slot * P.N + t] = make_float2(m[j], lt);
  }
}

__global__ __launch_bounds__(256, 1) void ds_kernel(Params P) {
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * STAGE_BYTES];
  // per wavefront, one 32-token x 128-row slice of dS in bf16 on its way to
  // memory: row = token, 16-byte piece c of a row at c ^ (token % 16)
  __shared__ __attribute__((aligned(1024))) char tbuf[4][32 * 256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane & 31, half = lane >> 5;
  const int wv = wave & 1, wt = wave >> 1;
  // the lane's four tokens: log2-scaled LSE, weight (0 when not supervised), label
  float lse2[4], wt_[4];
  int y[4];
  bool tv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = blockIdx.x * BT + 128 * wt + 32 * j + rr;
    tv[j] = t < P.N;
    const int tc = tv[j] ? t : 0;
    y[j] = P.labels[tc];
    const bool valid = tv[j] && y[j] != P.ignore_index && y[j] >= 0 && y[j] < P.V;
    wt_[j] = valid ? P.w[tc] : 0.f;
    lse2[j] = P.lse[tc] * L2E;
  }
  const int vrow0 = P.vt_first * BV;  // first vocabulary row of this chunk
  char* const tb = tbuf[wave];
  tile_loop(P, ring, [&](int vt, f32x16 (&acc)[4][4]) {
    const int vb = vt * BV + 128 * wv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // the lane's token rr: its 128 rows into the slice, 8 bytes at a time
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          // registers 4 r4 .. 4 r4 + 3: four consecutive vocabulary rows
          const int v0 = vb + 32 * i + 8 * r4 + 4 * half;
          bf16x4 o;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float p = exp2f_fast(acc[i][j][4 * r4 + u] * L2E - lse2[j]);
            const float g = wt_[j] * (p - (v0 + u == y[j] ? 1.f : 0.f));
            o[u] = (bf16)(tv[j] && v0 + u < P.V ? g : 0.f);
          }
          *(bf16x4*)(tb + rr * 256 + (((4 * i + r4) ^ (rr & 15)) << 4) + 8 * half) = o;
        }
      // then each store writes four tokens' 256-byte runs: every row up to
      // n_pad and every column of the tile, which the products read as zero
      // padding of their contraction
      const int tj = blockIdx.x * BT + 128 * wt + 32 * j;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int row = 4 * q + (lane >> 4), c = lane & 15;
        const u32x4 v = *(const u32x4*)(tb + row * 256 + ((c ^ (row & 15)) << 4));
        if (tj + row < P.n_pad) *(u32x4*)(P.ds + (size_t)(tj + row) * P.ld_ds + (vb - vrow0) + 8 * c) = v;
      }
    }
    // stores count on vmcnt too and may complete out of order with the ring
    // copies: let them drain so the ring's counted waits stay exact
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  });
}

// One wavefront per token: LSE from the partials, the label logit, the
// weighted token loss.
__global__ __launch_bounds__(256) void merge_kernel(const float2* __restrict__ part, int n_parts, const bf16* __restrict__ h,
                                                    const bf16* __restrict__ W, const int32_t* __restrict__ labels,
                                                    const float* __restrict__ w, int N, int V, int Dm,
                                                    int ignore_index, float* __restrict__ lse_out,
                                                    float* __restrict__ tok_loss, int32_t* __restrict__ err_flag) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= N) return;  // whole wavefronts only
  float m = -INFINITY, l = 0.f;
  for (int p = lane; p < n_parts; p += 64) {
    const float2 q = part[(size_t)p * N + t];
    const float M = __builtin_elementwise_maximum(m, q.x);
    const float Mu = M == -INFINITY ? 0.f : M;
    l = l * exp2f_fast(m - Mu) + q.y * exp2f_fast(q.x - Mu);
    m = M;
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(l, off);
    const float M = __builtin_elementwise_maximum(m, m2);
    const float Mu = M == -INFINITY ? 0.f : M;
    l = l * exp2f_fast(m - Mu) + l2 * exp2f_fast(m2 - Mu);
    m = M;
  }
  const float lse = (m + log2f(l)) * TA_LN2;
  const int y = labels[t];
  const bool bad = y != ignore_index && (y < 0 || y >= V);
  const bool valid = y != ignore_index && !bad;
  float xy = 0.f;
  if (valid) {
    const bf16* hr = h + (size_t)t * Dm;
    const bf16* wr = W + (size_t)y * Dm;
    for (int k = lane * 8; k < Dm; k += 512) {
      const bf16x8 a = *(const bf16x8*)(hr + k), b = *(const bf16x8*)(wr + k);
#pragma unroll
      for (int e = 0; e < 8; ++e) xy = fmaf((float)a[e], (float)b[e], xy);
    }
    for (int off = 32; off > 0; off >>= 1) xy += __shfl_xor(xy, off);
  }
  if (lane == 0) {
    lse_out[t] = lse;
    tok_loss[t] = valid ? w[t] * (lse - xy) : 0.f;
    if (bad && err_flag) *err_flag = 1;
  }
}

__global__ __launch_bounds__(256) void cast_kernel(const float* __restrict__ x, bf16* __restrict__ y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) y[i] = (bf16)x[i];
}

// ---------------------------------------------------------------------------
// The backward's two products, hand-written on the same 256 x 256 tiles,
// written transposed so the MFMA rows run along the model dimension d and
// each lane stores four consecutive d of one output row:
//   dh^T       = W_chunk^T dS^T   (d x tokens;          k = the chunk's vocabulary rows)
//   dW_chunk^T = h^T dS           (d x vocabulary rows; k = tokens)
// A (W_chunk or h, stored [k][d]) is a "k-row" tile of 32 k rows x 256 d
// (512-byte rows) read with the LDS transpose read; B is dS: for dh its rows
// (vocabulary contiguous) form a k-contiguous tile read with 16-byte row
// reads like the logits tiles, for dW it is a k-row tile of 32 tokens x 256
// vocabulary rows.  In a k-row tile the 32-byte unit u of row r sits at
// u ^ (2 (r % 4)): the two adjacent units of the four rows that 32 lanes of
// a transpose read touch then fill a whole 256-byte window of banks (with
// u ^ (r % 4) they shared 128 bytes, a two-way conflict).
struct GemmParams {
  const bf16* A;  // [k][d] rows of A (W_chunk or h)
  int lda, a_rmax, a_cmax;  // row stride; last valid row; columns (d) available
  const bf16* B;  // dS
  int ldb, b_rmax, b_cmax;  // row stride; last valid row; columns available (k-row form)
  int K;          // contraction length, a multiple of KS (operand rows past the data are zero)
  int n_cols;     // output columns (tokens for dh, vocabulary rows for dW)
  int Dm;
  float* out32;   // dh accumulator [tokens][Dm] (fp32), or
  bf16* out16;    // dW_chunk [rows][Dm] (bf16)
  int accumulate; // out32 += (else =)
};

// Rows k0 .. k0 + 31 (clamped to rmax) x columns c0 .. c0 + 255 (clamped to
// cmax - 8) of X [rows][ld] into a k-row tile.  Copy q (0..15) fills rows
// 2q, 2q + 1 (lane i: row 2q + i/32, 16-byte slot i % 32 holding global
// piece ((slot/2) ^ (2 (row % 4))) * 2 + slot % 2); wave w issues q = w + 4i.
__device__ __forceinline__ void stage_krows(const bf16* X, int ld, int rmax, int cmax, int k0, int c0, char* tile) {
  const int l = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = w + 4 * i;
    const int row = 2 * q + (l >> 5);
    const int slot = l & 31;
    const int piece = (((slot >> 1) ^ (2 * (row & 3))) << 1) | (slot & 1);
    const int gc = min(c0 + 8 * piece, cmax - 8);
    const int gr = min(k0 + row, rmax);
    copy16_to_lds(X + (size_t)gr * ld + gc, tile + q * 1024);
  }
}

// B_KC: B is dS rows (dh); else B is a k-row tile of dS (dW).
template <bool B_KC>
__global__ __launch_bounds__(256, 1) void gemm_kernel(GemmParams G) {
  __shared__ __attribute__((aligned(1024))) char ring[NBUF * STAGE_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rr = lane & 31, half = lane >> 5;
  const int wm = wave & 1, wn = wave >> 1;   // this wave's 128 d x 128 columns
  const int c0 = blockIdx.x * 256, d0 = blockIdx.y * 256;
  const int total = G.K / KS;

  // The copies' per-lane byte offsets do not change from stage to stage (the
  // lane-to-row and lane-to-piece maps of stage_krows / stage_tile, with the
  // column clamps), so a stage whose k rows all exist issues each copy from a
  // scalar base (the stage's first k row) plus that fixed offset; only the
  // stage that runs past the last row takes the clamped path.
  const int l = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  uint32_t offa[4], offb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = wu + 4 * i;
    const int row = 2 * q + (l >> 5), slot = l & 31;
    const int piece = (((slot >> 1) ^ (2 * (row & 3))) << 1) | (slot & 1);
    offa[i] = (uint32_t)(row * G.lda + min(d0 + 8 * piece, G.a_cmax - 8)) * 2u;
    if (B_KC) {
      const int brow = 16 * q + (l >> 2);
      const int bpiece = (l & 3) ^ swz4(brow);
      offb[i] = (uint32_t)((size_t)min(c0 + brow, G.b_rmax) * G.ldb + bpiece * 8) * 2u;
    } else {
      offb[i] = (uint32_t)(row * G.ldb + min(c0 + 8 * piece, G.b_cmax - 8)) * 2u;
    }
  }
  const uint32_t lds0 = lds_addr(ring);
  // (dS rows addressed by 32-bit offsets from the stage's column while the
  // whole operand spans less than 4 GiB)
  const bool b_off32 = (size_t)(G.b_rmax + 1) * G.ldb * 2 < ((size_t)1 << 32);
  auto issue = [&](int p) {
    char* buf = ring + (p % NBUF) * STAGE_BYTES;
    const uint32_t lb = lds0 + (p % NBUF) * STAGE_BYTES;
    const int k0 = p * KS;
    if (k0 + KS - 1 <= G.a_rmax) {
#pragma unroll
      for (int i = 0; i < 4; ++i) copy16_to_lds_s(G.A + (size_t)k0 * G.lda, offa[i], lb + (wu + 4 * i) * 1024);
    } else {
      stage_krows(G.A, G.lda, G.a_rmax, G.a_cmax, k0, d0, buf);
    }
    if (B_KC && b_off32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) copy16_to_lds_s(G.B + k0, offb[i], lb + TILE_BYTES + (wu + 4 * i) * 1024);
    } else if (B_KC) {
      stage_tile(G.B, c0, G.b_rmax + 1, G.ldb, k0, buf + TILE_BYTES);
    } else if (k0 + KS - 1 <= G.b_rmax) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        copy16_to_lds_s(G.B + (size_t)k0 * G.ldb, offb[i], lb + TILE_BYTES + (wu + 4 * i) * 1024);
    } else {
      stage_krows(G.B, G.ldb, G.b_rmax, G.b_cmax, k0, c0, buf + TILE_BYTES);
    }
  };

  // Transpose-read offsets (bytes) in a k-row tile for MFMA tile t (32
  // columns at 128 * w + 32 t): the lane reads row 8*half + 4x + x16/4 of
  // k-group s (+ 16 s rows, + 4x rows: immediates) and columns
  // 16 g + 4 (x16 % 4) of the tile, g = (lane / 16) % 2, and receives
  // column lane % 32 with k-slots 16 s + 8 half + 0..7 (consecutive).
  const int x16 = lane & 15, g = (lane >> 4) & 1, q4 = x16 >> 2;
  auto kroff = [&](int w, int t) {
    return (8 * half + q4) * 512 + (((8 * w + 2 * t + g) ^ (2 * q4)) << 5) + 8 * (x16 & 3);
  };
  int aoff[4], boff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    aoff[t] = kroff(wm, t);
    boff[t] = TILE_BYTES + kroff(wn, t);
  }
  // k-contiguous B (as in the logits tiles): row 128 wn + 32 t + rr, piece 2s + half
  const int sw = swz4(rr);
  const int po[2] = {((0 + half) ^ sw) << 4, ((2 + half) ^ sw) << 4};
  const int bbase = TILE_BYTES + (128 * wn + rr) * 64;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  agpr_fence16(acc);

  for (int p = 0; p < min(NBUF - 1, total); ++p) issue(p);
  for (int it = 0; it < total; ++it) {
    const int after = min(NBUF - 2, total - 1 - it);
    if (after >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies of stage it landed; every wave is done with stage it - 1
    if (it + NBUF - 1 < total) issue(it + NBUF - 1);
    const char* buf = ring + (it % NBUF) * STAGE_BYTES;
    // both k-groups' operands are read before the first MFMA
    bf16x8 a[2][4], b[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16* pa = (const bf16*)(buf + aoff[t] + 16 * s * 512);
        a[s][t] = cat(lds_read_tr(pa), lds_read_tr(pa + 4 * 256));
        if (B_KC) {
          b[s][t] = *(const bf16x8*)(buf + bbase + 2048 * t + po[s]);
        } else {
          const bf16* pb = (const bf16*)(buf + boff[t] + 16 * s * 512);
          b[s][t] = cat(lds_read_tr(pb), lds_read_tr(pb + 4 * 256));
        }
      }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mfma32_acc(acc[i][j], a[s][i], b[s][j]);
  }
  lds_copies_wait();
  agpr_fence16(acc);

  // acc[i][j] register r <-> d = d0 + 128 wm + 32 i + 8 (r/4) + 4 half + r%4,
  // column c0 + 128 wn + 32 j + rr
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = c0 + 128 * wn + 32 * j + rr;
    if (c >= G.n_cols) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = d0 + 128 * wm + 32 * i + 8 * r4 + 4 * half;
        if (d >= G.Dm) continue;
        const float4 v = make_float4(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
        if (G.out32) {
          float4* o = (float4*)(G.out32 + (size_t)c * G.Dm + d);
          float4 x = v;
          if (G.accumulate) {
            const float4 y = *o;
            x = make_float4(v.x + y.x, v.y + y.y, v.z + y.z, v.w + y.w);
          }
          *o = x;
        } else {
          const bf16x4 o = {(bf16)v.x, (bf16)v.y, (bf16)v.z, (bf16)v.w};
          *(bf16x4*)(G.out16 + (size_t)c * G.Dm + d) = o;
        }
      }
  }
}

struct Sizes {
  int n_tt, n_vt, vsplit, vt_per_wg, n_parts, chunk_vt, n_chunks;
  int n_pad;
  size_t off_part, off_tok, off_lse, off_ds, off_dh, total;
};

Sizes sizes(int N, int V, int Dm, bool grad, int vocab_chunk) {
  Sizes s{};
  s.n_tt = (N + BT - 1) / BT;
  s.n_vt = (V + BV - 1) / BV;
  // about four workgroups per CU of 256 CUs in the forward
  s.vsplit = std::max(1, std::min(s.n_vt, (1024 + s.n_tt - 1) / s.n_tt));
  s.vt_per_wg = (s.n_vt + s.vsplit - 1) / s.vsplit;
  s.vsplit = (s.n_vt + s.vt_per_wg - 1) / s.vt_per_wg;
  s.n_parts = 2 * s.vsplit;
  // backward chunk: at most ~512 MB of bf16 dS, whole tiles (16K vocabulary rows at 16K tokens:
  // 3% faster than half that, the launches and GEMMs being larger; twice that was slower again)
  if (vocab_chunk > 0) {
    s.chunk_vt = std::max(1, vocab_chunk / BV);
  } else {
    const size_t rows = (size_t(1) << 28) / std::max(N, 1);
    s.chunk_vt = (int)std::max<size_t>(1, rows / BV);
  }
  s.chunk_vt = std::min(s.chunk_vt, s.n_vt);
  s.n_chunks = (s.n_vt + s.chunk_vt - 1) / s.chunk_vt;
  s.n_pad = (N + KS - 1) / KS * KS;
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t x = off;
    off += align256(b);
    return x;
  };
  s.off_part = take((size_t)s.n_parts * N * sizeof(float2));
  s.off_tok = take((size_t)N * sizeof(float));
  s.off_lse = take((size_t)N * sizeof(float));
  if (grad) {
    s.off_ds = take((size_t)s.chunk_vt * BV * s.n_pad * sizeof(bf16));
    s.off_dh = take((size_t)N * Dm * sizeof(float));
  }
  s.total = off;
  return s;
}

}  // namespace lmh

hipError_t launch_sum(const float* v, int n, float* out, hipStream_t st);  // nll.hip

}  // namespace ta

using namespace ta;

extern "C" ta_status tree_lmhead_nll_ws_bytes(int32_t N, int32_t V, int32_t Dm, int32_t need_grad,
                                              int32_t vocab_chunk, size_t* bytes) {
  if (!bytes || N <= 0 || V <= 0 || Dm <= 0 || vocab_chunk < 0) return TA_EINVAL;
  *bytes = lmh::sizes(N, V, Dm, need_grad != 0, vocab_chunk).total;
  return TA_OK;
}

extern "C" ta_status tree_lmhead_nll(ta_dtype dt, const void* h, const void* W, const int32_t* labels,
                                     const float* w, int32_t N, int32_t V, int32_t Dm, int32_t ignore_index,
                                     int32_t vocab_chunk, float* loss, float* lse, void* dh, void* dW,
                                     int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != TA_BF16) return TA_EUNSUPPORTED;
  if (!h || !W || !labels || !w || !loss || N <= 0 || V <= 0 || Dm <= 0 || vocab_chunk < 0) return TA_EINVAL;
  if (Dm % lmh::KS != 0) return TA_EUNSUPPORTED;
  if ((dh == nullptr) != (dW == nullptr)) return TA_EINVAL;
  if ((int64_t)N * Dm > INT32_MAX || (int64_t)V * Dm > ((int64_t)1 << 40)) return TA_ERANGE;
  const bool grad = dh != nullptr;
  const lmh::Sizes S = lmh::sizes(N, V, Dm, grad, vocab_chunk);
  if (!ws || ws_bytes < S.total) return TA_ENOMEM;
  char* wsb = (char*)ws;
  float2* part = (float2*)(wsb + S.off_part);
  float* tok = (float*)(wsb + S.off_tok);
  float* lse_b = lse ? lse : (float*)(wsb + S.off_lse);

  lmh::Params P{};
  P.h = (const bf16*)h;
  P.W = (const bf16*)W;
  P.labels = labels;
  P.w = w;
  P.lse = lse_b;
  P.part = part;
  P.N = N;
  P.V = V;
  P.Dm = Dm;
  P.ignore_index = ignore_index;
  P.vt_per_wg = S.vt_per_wg;
  P.vt_first = 0;
  P.vt_last = S.n_vt;
  hipLaunchKernelGGL(lmh::lse_kernel, dim3(S.n_tt, S.vsplit), dim3(256), 0, stream, P);
  TA_LAUNCH_CHECK();
  hipLaunchKernelGGL(lmh::merge_kernel, dim3((N + 3) / 4), dim3(256), 0, stream, (const float2*)part, S.n_parts,
                     (const bf16*)h, (const bf16*)W, labels, w, N, V, Dm, ignore_index, lse_b, tok, err_flag);
  TA_LAUNCH_CHECK();
  if (launch_sum(tok, N, loss, stream) != hipSuccess) return TA_EHIP;
  if (!grad) return TA_OK;

  bf16* ds = (bf16*)(wsb + S.off_ds);
  float* dh_acc = (float*)(wsb + S.off_dh);
  P.ds = ds;
  P.n_pad = S.n_pad;
  P.ld_ds = S.chunk_vt * lmh::BV;
  for (int c = 0; c < S.n_chunks; ++c) {
    const int vt_a = c * S.chunk_vt, vt_b = std::min(S.n_vt, vt_a + S.chunk_vt);
    const int v0 = vt_a * lmh::BV, cv = std::min(V, vt_b * lmh::BV) - v0;  // rows of this chunk
    P.vt_first = vt_a;
    P.vt_last = vt_b;
    // about four workgroups per CU, each walking a few vocabulary tiles
    const int ntile = vt_b - vt_a;
    P.vt_per_wg = std::max(1, std::min(ntile, ntile * S.n_tt / 1024));
    hipLaunchKernelGGL(lmh::ds_kernel, dim3(S.n_tt, (ntile + P.vt_per_wg - 1) / P.vt_per_wg), dim3(256), 0, stream,
                       P);
    TA_LAUNCH_CHECK();
    // dh^T += W_chunk^T dS^T over the chunk's rows (rounded up to KS: dS is zero past V), then
    // dW_chunk^T = h^T dS over the tokens (rounded up: dS is zero past N)
    lmh::GemmParams G{};
    G.Dm = Dm;
    G.A = (const bf16*)W + (size_t)v0 * Dm;
    G.lda = Dm;
    G.a_rmax = V - 1 - v0;
    G.a_cmax = Dm;
    G.B = ds;
    G.ldb = P.ld_ds;
    G.b_rmax = N - 1;
    G.b_cmax = P.ld_ds;
    G.K = (cv + lmh::KS - 1) / lmh::KS * lmh::KS;
    G.n_cols = N;
    G.out32 = dh_acc;
    G.accumulate = c > 0;
    hipLaunchKernelGGL(lmh::gemm_kernel<true>, dim3(S.n_tt, (Dm + 255) / 256), dim3(256), 0, stream, G);
    TA_LAUNCH_CHECK();
    G.A = (const bf16*)h;
    G.a_rmax = N - 1;
    G.b_rmax = S.n_pad - 1;
    G.K = S.n_pad;
    G.n_cols = cv;
    G.out32 = nullptr;
    G.out16 = (bf16*)dW + (size_t)v0 * Dm;
    G.accumulate = 0;
    hipLaunchKernelGGL(lmh::gemm_kernel<false>, dim3((cv + 255) / 256, (Dm + 255) / 256), dim3(256), 0, stream, G);
    TA_LAUNCH_CHECK();
  }
  const size_t nel = (size_t)N * Dm;
  hipLaunchKernelGGL(lmh::cast_kernel, dim3((unsigned)std::min<size_t>((nel + 255) / 256, 16384)), dim3(256), 0,
                     stream, dh_acc, (bf16*)dh, nel);
  TA_LAUNCH_CHECK();
  return TA_OK;
}
