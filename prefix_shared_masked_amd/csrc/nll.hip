// g_t/K weighted negative log-likelihood (Tree Training post, sections 6.2,
// 6.3 and 12): loss = sum_t w_t [y_t valid] (logsumexp(x_t) - x_t[y_t]) and
// dlogits_t = w_t [y_t valid] (softmax(x_t) - onehot(y_t)).
//
// One workgroup per row streams the row twice (max/sum, then the gradient;
// 16-byte pieces when the rows allow);
// per-row losses go to the workspace and a single workgroup sums them in a
// fixed order, so the loss is bitwise reproducible.  The work is HBM-bound:
// the row is read twice and the gradient written once.
#include "common.h"

namespace ta {
namespace nll {

constexpr int THREADS = 256;

__device__ __forceinline__ void merge_ms(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

__global__ __launch_bounds__(THREADS) void row_kernel(const float* __restrict__ logits, const int32_t* __restrict__ labels,
                                                      const float* __restrict__ w, int V, int ignore_index,
                                                      float* __restrict__ row_loss, float* __restrict__ dlogits,
                                                      int32_t* __restrict__ err_flag) {
  __shared__ float sm[THREADS / 64], ss[THREADS / 64];
  const int row = blockIdx.x;
  const float* x = logits + (size_t)row * V;
  float m = -INFINITY, s = 0.f;
  // A masked logit (-inf) adds nothing: its term is skipped rather than
  // evaluated as exp(-inf - -inf).
  for (int j = threadIdx.x; j < V; j += THREADS) {
    const float v = x[j];
    if (v > m) {
      s = s * expf(m - v) + 1.f;
      m = v;
    } else if (v != -INFINITY) {
      s += expf(v - m);
    }
  }
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    merge_ms(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
  for (int i = 1; i < THREADS / 64; ++i) merge_ms(m, s, sm[i], ss[i]);
  const float lse = m + logf(s);

  const int y = labels[row];
  const bool bad = y != ignore_index && (y < 0 || y >= V);
  const bool valid = y != ignore_index && !bad;
  const float wr = valid ? w[row] : 0.f;
  if (threadIdx.x == 0) {
    row_loss[row] = valid ? wr * (lse - x[y]) : 0.f;
    if (bad && err_flag) *err_flag = 1;
  }
  if (dlogits) {
    float* g = dlogits + (size_t)row * V;
    for (int j = threadIdx.x; j < V; j += THREADS) {
      const float p = expf(x[j] - lse) - (j == y ? 1.f : 0.f);
      g[j] = wr * p;
    }
  }
}

// The same for rows of a multiple of four floats on 16-byte boundaries: each
// lane streams 16-byte pieces, four in flight, folds a piece into its running
// (max, sum) with one rescale (branch-free: M = max(m, piece max), s = s *
// 2^((m - M) log2 e) + sum 2^((v - M) log2 e)), and writes the gradient as
// 16-byte pieces.  exp2 is the hardware's; the reductions keep a fixed order.
constexpr int UNROLL = 4;

// Masked logits (-inf) contribute exp2(-inf) = 0; while every value seen so
// far is -inf, the reference is taken as 0 so no -inf - -inf is evaluated.
__device__ __forceinline__ void fold4(float& m, float& s, const float4& v) {
  const float pm = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
  const float M = fmaxf(m, pm);
  const float Mu = M == -INFINITY ? 0.f : M;
  const float e = exp2f_fast((v.x - Mu) * TA_LOG2E) + exp2f_fast((v.y - Mu) * TA_LOG2E) +
                  exp2f_fast((v.z - Mu) * TA_LOG2E) + exp2f_fast((v.w - Mu) * TA_LOG2E);
  s = (m == -INFINITY ? 0.f : s * exp2f_fast((m - M) * TA_LOG2E)) + e;
  m = M;
}

__global__ __launch_bounds__(THREADS) void row4_kernel(const float* __restrict__ logits, const int32_t* __restrict__ labels,
                                                       const float* __restrict__ w, int V, int ignore_index,
                                                       float* __restrict__ row_loss, float* __restrict__ dlogits,
                                                       int32_t* __restrict__ err_flag) {
  __shared__ float sm[THREADS / 64], ss[THREADS / 64];
  const int row = blockIdx.x;
  const float* x = logits + (size_t)row * V;
  const float4* x4 = (const float4*)x;
  const int V4 = V / 4;
  float m = -INFINITY, s = 0.f;
  int j = threadIdx.x;
  for (; j + (UNROLL - 1) * THREADS < V4; j += UNROLL * THREADS) {
    float4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = x4[j + u * THREADS];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) fold4(m, s, v[u]);
  }
  for (; j < V4; j += THREADS) fold4(m, s, x4[j]);
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    merge_ms(m, s, m2, s2);
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  m = sm[0];
  s = ss[0];
  for (int i = 1; i < THREADS / 64; ++i) merge_ms(m, s, sm[i], ss[i]);
  const float lse = m + logf(s);

  const int y = labels[row];
  const bool bad = y != ignore_index && (y < 0 || y >= V);
  const bool valid = y != ignore_index && !bad;
  const float wr = valid ? w[row] : 0.f;
  if (threadIdx.x == 0) {
    row_loss[row] = valid ? wr * (lse - x[y]) : 0.f;
    if (bad && err_flag) *err_flag = 1;
  }
  if (dlogits) {
    float4* g4 = (float4*)(dlogits + (size_t)row * V);
    auto grad = [&](int jj, const float4& v) {
      float4 g;
      g.x = wr * (exp2f_fast((v.x - lse) * TA_LOG2E) - (4 * jj == y ? 1.f : 0.f));
      g.y = wr * (exp2f_fast((v.y - lse) * TA_LOG2E) - (4 * jj + 1 == y ? 1.f : 0.f));
      g.z = wr * (exp2f_fast((v.z - lse) * TA_LOG2E) - (4 * jj + 2 == y ? 1.f : 0.f));
      g.w = wr * (exp2f_fast((v.w - lse) * TA_LOG2E) - (4 * jj + 3 == y ? 1.f : 0.f));
      g4[jj] = g;
    };
    int jj = threadIdx.x;
    for (; jj + (UNROLL - 1) * THREADS < V4; jj += UNROLL * THREADS) {
      float4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) v[u] = x4[jj + u * THREADS];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) grad(jj + u * THREADS, v[u]);
    }
    for (; jj < V4; jj += THREADS) grad(jj, x4[jj]);
  }
}

__global__ __launch_bounds__(1024) void sum_kernel(const float* __restrict__ v, int n, float* __restrict__ out) {
  __shared__ float sh[1024];
  float a = 0.f;
  for (int i = threadIdx.x; i < n; i += 1024) a += v[i];
  sh[threadIdx.x] = a;
  __syncthreads();
  for (int st = 512; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) sh[threadIdx.x] += sh[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = sh[0];
}

}  // namespace nll

// Fixed-order sum of n floats into *out by one workgroup (shared with the
// fused output-layer loss).
hipError_t launch_sum(const float* v, int n, float* out, hipStream_t st) {
  hipLaunchKernelGGL(nll::sum_kernel, dim3(1), dim3(1024), 0, st, v, n, out);
  return hipGetLastError();
}

}  // namespace ta

using namespace ta;

extern "C" ta_status tree_nll_ws_bytes(int32_t N, int32_t V, size_t* bytes) {
  if (!bytes || N < 0 || V <= 0) return TA_EINVAL;
  *bytes = align256((size_t)(N > 0 ? N : 1) * sizeof(float));
  return TA_OK;
}

extern "C" ta_status tree_weighted_nll(ta_dtype dt, const void* logits, const int32_t* labels, const float* w,
                                       int32_t N, int32_t V, int32_t ignore_index, float* loss, void* dlogits,
                                       int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dt != TA_F32) return TA_EUNSUPPORTED;
  if (N < 0 || V <= 0 || !loss) return TA_EINVAL;
  if (N > 0 && (!logits || !labels || !w)) return TA_EINVAL;
  size_t need;
  tree_nll_ws_bytes(N, V, &need);
  if (!ws || ws_bytes < need) return TA_ENOMEM;
  float* rl = (float*)ws;
  if (N > 0) {
    const bool vec = V % 4 == 0 && (uintptr_t)logits % 16 == 0 && (uintptr_t)dlogits % 16 == 0;
    if (vec)
      hipLaunchKernelGGL(nll::row4_kernel, dim3(N), dim3(nll::THREADS), 0, stream, (const float*)logits, labels, w,
                         V, ignore_index, rl, (float*)dlogits, err_flag);
    else
      hipLaunchKernelGGL(nll::row_kernel, dim3(N), dim3(nll::THREADS), 0, stream, (const float*)logits, labels, w, V,
                         ignore_index, rl, (float*)dlogits, err_flag);
    TA_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(nll::sum_kernel, dim3(1), dim3(1024), 0, stream, rl, N, loss);
  TA_LAUNCH_CHECK();
  return TA_OK;
}
