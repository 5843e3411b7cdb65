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
//    [N, chunk rows]; then two plain GEMMs on the library's matrix kernels:
//    dh += dS W_chunk (fp32 accumulator) and dW_chunk = dS^T h.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <map>
#include <mutex>

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

  auto issue = [&](int p) {
    const int vt = vt0 + p / nk, kk = p % nk;
    char* buf = ring + (p % NBUF) * STAGE_BYTES;
    stage_tile(P.W, vt * BV, P.V, P.Dm, kk * KS, buf);
    stage_tile(P.h, t0, P.N, P.Dm, kk * KS, buf + TILE_BYTES);
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

  for (int p = 0; p < min(NBUF - 1, total); ++p) issue(p);
  for (int it = 0; it < total; ++it) {
    // this wave's copies of stage `it` have landed once at most the copies of
    // the stages issued after it (8 per stage) are outstanding
    const int after = min(NBUF - 2, total - 1 - it);
    if (after >= 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // every wave's copies landed; every wave is done with stage it - 1
    if (it + NBUF - 1 < total) issue(it + NBUF - 1);  // refills the buffer of stage it - 1
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
  tile_loop(P, ring, [&](int vt, f32x16 (&acc)[4][4]) {
    const int vb = vt * BV + 128 * wv;
    const bool ragged = vb + 128 > P.V;  // uniform
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = blockIdx.x * BT + 128 * wt + 32 * j + rr;
      bf16* row = P.ds + (size_t)(tv[j] ? t : 0) * P.ld_ds + (vb - vrow0) + 4 * half;
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
            o[u] = (bf16)(v0 + u < P.V ? g : 0.f);
          }
          if (tv[j] && (!ragged || v0 < P.V)) *(bf16x4*)(row + 32 * i + 8 * r4) = o;
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
// Plain GEMMs of the backward on the library matrix kernels.  One handle per
// device, created on first use and kept for the life of the process.
std::mutex g_mu;
std::map<int, hipblasLtHandle_t> g_handles;

hipblasLtHandle_t lt_handle() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_handles.find(dev);
  if (it != g_handles.end()) return it->second;
  hipblasLtHandle_t hd = nullptr;
  if (hipblasLtCreate(&hd) != HIPBLAS_STATUS_SUCCESS) return nullptr;
  g_handles[dev] = hd;
  return hd;
}

// D = op(A) op(B) + beta D in column-major terms; A, B bf16, D of type dtD,
// fp32 compute.  m x n result, k the contraction.
ta_status lt_gemm(bool ta_, bool tb, int m, int n, int k, const void* A, int lda, const void* B, int ldb, void* D,
                  hipDataType dtD, int ldd, float beta, void* ws, size_t wsb, hipStream_t st) {
  hipblasLtHandle_t hd = lt_handle();
  if (!hd) return TA_EHIP;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  ta_status rc = TA_OK;
  const hipblasOperation_t opa = ta_ ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  const uint64_t wsz = wsb;
  hipblasLtMatmulHeuristicResult_t res{};
  int got = 0;
  const float alpha = 1.f;
  if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, ta_ ? k : m, ta_ ? m : k, lda) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, tb ? n : k, tb ? k : n, ldb) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ld, dtD, m, n, ldd) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz, sizeof(wsz)) !=
          HIPBLAS_STATUS_SUCCESS) {
    rc = TA_EHIP;
  } else if (hipblasLtMatmulAlgoGetHeuristic(hd, desc, la, lb, ld, ld, pref, 1, &res, &got) != HIPBLAS_STATUS_SUCCESS ||
             got < 1) {
    rc = TA_EUNSUPPORTED;
  } else if (hipblasLtMatmul(hd, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &res.algo, ws, wsb, st) !=
             HIPBLAS_STATUS_SUCCESS) {
    rc = TA_EHIP;
  }
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return rc;
}

constexpr size_t LT_WS = size_t(64) << 20;  // library GEMM workspace

struct Sizes {
  int n_tt, n_vt, vsplit, vt_per_wg, n_parts, chunk_vt, n_chunks;
  size_t off_part, off_tok, off_lse, off_ds, off_dh, off_lt, total;
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
    s.off_ds = take((size_t)s.chunk_vt * BV * N * sizeof(bf16));
    s.off_dh = take((size_t)N * Dm * sizeof(float));
    s.off_lt = take(LT_WS);
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
  void* ltws = wsb + S.off_lt;
  P.ds = ds;
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
    // column-major views: dS is (cv x N) with ld = ld_ds; W_chunk (Dm x cv), h (Dm x N), dh (Dm x N),
    // dW_chunk (Dm x cv)
    ta_status st = lmh::lt_gemm(false, false, Dm, N, cv, (const bf16*)W + (size_t)v0 * Dm, Dm, ds, P.ld_ds, dh_acc,
                                HIP_R_32F, Dm, c == 0 ? 0.f : 1.f, ltws, lmh::LT_WS, stream);
    if (st != TA_OK) return st;
    st = lmh::lt_gemm(false, true, Dm, cv, N, h, Dm, ds, P.ld_ds, (bf16*)dW + (size_t)v0 * Dm, HIP_R_16BF, Dm, 0.f,
                      ltws, lmh::LT_WS, stream);
    if (st != TA_OK) return st;
  }
  const size_t nel = (size_t)N * Dm;
  hipLaunchKernelGGL(lmh::cast_kernel, dim3((unsigned)std::min<size_t>((nel + 255) / 256, 16384)), dim3(256), 0,
                     stream, dh_acc, (bf16*)dh, nel);
  TA_LAUNCH_CHECK();
  return TA_OK;
}
