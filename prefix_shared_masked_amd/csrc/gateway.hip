// Gateway data movement for partitioned tree attention (Tree Training post,
// section 8.2) and the partition-at-a-time forward/backward drivers.
//
// A partition's local rows are its root's ancestor chain (the gateway K/V it
// reads from the partitions above it) followed by its own rows.  On one
// device the "export" of the gateway is a row gather out of the whole tree's
// tensors, and the relay of the gateway gradient is a row scatter-add into an
// fp32 accumulator: the per-device work of a multi-device run, done in turn.
//
// All kernels here are plain HBM-bound copies: one 16-byte (or 4-byte) unit
// per lane, consecutive lanes on consecutive units of a row, so every row is
// read and written with full coalescing (the row map entry a lane needs is a
// cached 4-byte read shared by the lanes of that row).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "partition_internal.h"
#include "plan_internal.h"

namespace ta {
namespace gw {

constexpr int kThreads = 256;

// dst[o][i][:] = i < n_zero ? 0 : src[o][idx[i]][:] for i in [0, n_rows),
// o in [0, n_outer); a row is `units` elements of type U.
template <typename U>
__global__ void __launch_bounds__(kThreads) gather_kernel(const U* __restrict__ src, const int32_t* __restrict__ idx,
                                                           U* __restrict__ dst, int n_rows, int n_zero, int units,
                                                           int64_t src_outer, int64_t dst_outer, int total) {
  for (int t = blockIdx.x * kThreads + threadIdx.x; t < total; t += gridDim.x * kThreads) {
    const int ru = t / units, u = t - ru * units;
    const int o = ru / n_rows, i = ru - o * n_rows;
    U val{};
    if (i >= n_zero) val = src[o * src_outer + (int64_t)idx[i] * units + u];
    dst[o * dst_outer + (int64_t)i * units + u] = val;
  }
}

// dst[o][idx[i]][:] = src[o][i][:] for i in [0, n_rows).
template <typename U>
__global__ void __launch_bounds__(kThreads) scatter_kernel(const U* __restrict__ src, const int32_t* __restrict__ idx,
                                                            U* __restrict__ dst, int n_rows, int units,
                                                            int64_t src_outer, int64_t dst_outer, int total) {
  for (int t = blockIdx.x * kThreads + threadIdx.x; t < total; t += gridDim.x * kThreads) {
    const int ru = t / units, u = t - ru * units;
    const int o = ru / n_rows, i = ru - o * n_rows;
    dst[o * dst_outer + (int64_t)idx[i] * units + u] = src[o * src_outer + (int64_t)i * units + u];
  }
}

__device__ __forceinline__ void load4(const bf16* p, float* x) {
  const bf16x4 v = *(const bf16x4*)p;
  for (int j = 0; j < 4; ++j) x[j] = (float)v[j];
}
__device__ __forceinline__ void load4(const float* p, float* x) {
  const f32x4 v = *(const f32x4*)p;
  for (int j = 0; j < 4; ++j) x[j] = v[j];
}

// acc[idx[i]][:] += float(src[i][:]) over rows of `quads` x 4 elements.  The
// rows of one call map to distinct global rows, so no two lanes add into the
// same element and plain read-modify-write is exact and deterministic.
template <typename T>
__global__ void __launch_bounds__(kThreads) scatter_add_kernel(const T* __restrict__ src,
                                                                const int32_t* __restrict__ idx,
                                                                float* __restrict__ acc, int quads, int total) {
  for (int t = blockIdx.x * kThreads + threadIdx.x; t < total; t += gridDim.x * kThreads) {
    const int i = t / quads, u = t - i * quads;
    float x[4];
    load4(src + (int64_t)t * 4, x);
    f32x4* a = (f32x4*)(acc + ((int64_t)idx[i] * quads + u) * 4);
    f32x4 s = *a;
    for (int j = 0; j < 4; ++j) s[j] += x[j];
    *a = s;
  }
}

// y = bf16(x) (round to nearest even), 4 elements per lane.
__global__ void __launch_bounds__(kThreads) cast_kernel(const float* __restrict__ x, bf16* __restrict__ y,
                                                         int64_t quads) {
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < quads; t += (int64_t)gridDim.x * kThreads) {
    const f32x4 v = ((const f32x4*)x)[t];
    bf16x4 r;
    for (int j = 0; j < 4; ++j) r[j] = (bf16)v[j];
    ((bf16x4*)y)[t] = r;
  }
}

__global__ void __launch_bounds__(kThreads) zero_kernel(f32x4* __restrict__ x, int64_t quads) {
  for (int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x; t < quads; t += (int64_t)gridDim.x * kThreads)
    x[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Grid: enough workgroups to cover the work up to 64 per CU (grid-stride
// beyond that); every launch here is a streaming copy.
inline int blocks_for(int64_t total) {
  const int64_t b = (total + kThreads - 1) / kThreads;
  return (int)std::max<int64_t>(1, std::min<int64_t>(b, 256 * 64));
}

// Row gather/scatter on rows of row_bytes bytes, in 16-byte units when the
// row size and both bases allow it, else 4-byte units.
hipError_t gather(const void* src, const int32_t* idx, void* dst, int n_rows, int n_zero, size_t row_bytes,
                  int n_outer, size_t src_outer_bytes, size_t dst_outer_bytes, hipStream_t st) {
  if (n_rows <= 0 || n_outer <= 0) return hipSuccess;
  if (row_bytes % 4) return hipErrorInvalidValue;
  const bool v16 = row_bytes % 16 == 0 && src_outer_bytes % 16 == 0 && dst_outer_bytes % 16 == 0 &&
                   (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  const size_t ub = v16 ? 16 : 4;
  const int units = (int)(row_bytes / ub);
  const int64_t total64 = (int64_t)n_outer * n_rows * units;
  if (total64 > INT32_MAX) return hipErrorInvalidValue;
  const int total = (int)total64;
  if (v16)
    gather_kernel<u32x4><<<blocks_for(total), kThreads, 0, st>>>((const u32x4*)src, idx, (u32x4*)dst, n_rows, n_zero,
                                                                  units, src_outer_bytes / 16, dst_outer_bytes / 16,
                                                                  total);
  else
    gather_kernel<uint32_t><<<blocks_for(total), kThreads, 0, st>>>((const uint32_t*)src, idx, (uint32_t*)dst, n_rows,
                                                                     n_zero, units, src_outer_bytes / 4,
                                                                     dst_outer_bytes / 4, total);
  return hipGetLastError();
}

hipError_t scatter(const void* src, const int32_t* idx, void* dst, int n_rows, size_t row_bytes, int n_outer,
                   size_t src_outer_bytes, size_t dst_outer_bytes, hipStream_t st) {
  if (n_rows <= 0 || n_outer <= 0) return hipSuccess;
  if (row_bytes % 4) return hipErrorInvalidValue;
  const bool v16 = row_bytes % 16 == 0 && src_outer_bytes % 16 == 0 && dst_outer_bytes % 16 == 0 &&
                   (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  const size_t ub = v16 ? 16 : 4;
  const int units = (int)(row_bytes / ub);
  const int64_t total64 = (int64_t)n_outer * n_rows * units;
  if (total64 > INT32_MAX) return hipErrorInvalidValue;
  const int total = (int)total64;
  if (v16)
    scatter_kernel<u32x4><<<blocks_for(total), kThreads, 0, st>>>((const u32x4*)src, idx, (u32x4*)dst, n_rows, units,
                                                                   src_outer_bytes / 16, dst_outer_bytes / 16, total);
  else
    scatter_kernel<uint32_t><<<blocks_for(total), kThreads, 0, st>>>((const uint32_t*)src, idx, (uint32_t*)dst,
                                                                      n_rows, units, src_outer_bytes / 4,
                                                                      dst_outer_bytes / 4, total);
  return hipGetLastError();
}

hipError_t scatter_add(ta_dtype dt, const void* src, const int32_t* idx, float* acc, int n_rows, int row_elems,
                       hipStream_t st) {
  if (n_rows <= 0) return hipSuccess;
  const int quads = row_elems / 4;
  const int64_t total64 = (int64_t)n_rows * quads;
  if (total64 > INT32_MAX) return hipErrorInvalidValue;
  const int total = (int)total64;
  if (dt == TA_BF16)
    scatter_add_kernel<bf16><<<blocks_for(total), kThreads, 0, st>>>((const bf16*)src, idx, acc, quads, total);
  else
    scatter_add_kernel<float><<<blocks_for(total), kThreads, 0, st>>>((const float*)src, idx, acc, quads, total);
  return hipGetLastError();
}

hipError_t zero(float* x, int64_t n, hipStream_t st) {
  zero_kernel<<<blocks_for(n / 4), kThreads, 0, st>>>((f32x4*)x, n / 4);
  return hipGetLastError();
}

hipError_t cast(const float* x, bf16* y, int64_t n, hipStream_t st) {
  cast_kernel<<<blocks_for(n / 4), kThreads, 0, st>>>(x, y, n / 4);
  return hipGetLastError();
}

// Workspace layout of the drivers (offsets in bytes, each 256-aligned).
// The local attention workspace comes first, so its saturation flag is the
// first word of the partition workspace, as in tree_attn_fwd / _bwd.
struct WsLayout {
  size_t attn, attn_bytes, q, k, v, o, lse, dO, dq, dk, dv, acc_k, acc_v, total;
};

WsLayout layout(const ta_partition* P, int op, ta_dtype dt, int Hq, int Hkv, int d, float rope_base) {
  const size_t es = dt == TA_BF16 ? 2 : 4;
  const size_t R = (size_t)P->max_local, N = (size_t)P->n_tokens;
  const size_t qb = align256(R * Hq * d * es), kb = align256(R * Hkv * d * es);
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t b) {
    const size_t x = off;
    off += b;
    return x;
  };
  size_t attn = 0;
  for (int p = 0; p < P->n_parts; ++p) {
    const ta_plan* pl = P->plans[p];
    if (!pl) continue;
    size_t b = 0;
    tree_attn_ws_bytes(pl, op, dt, Hq, Hkv, d, rope_base, &b);
    attn = std::max(attn, b);
  }
  L.attn_bytes = align256(attn);
  L.attn = take(L.attn_bytes);
  L.q = take(qb);
  L.k = take(kb);
  L.v = take(kb);
  L.o = take(qb);
  L.lse = take(align256(R * Hq * sizeof(float)));
  if (op == 1) {
    L.dO = take(qb);
    L.dq = take(qb);
    L.dk = take(kb);
    L.dv = take(kb);
    if (dt == TA_BF16) {  // fp32 relay accumulators (fp32 dk/dv serve directly)
      L.acc_k = take(align256(N * Hkv * d * sizeof(float)));
      L.acc_v = take(align256(N * Hkv * d * sizeof(float)));
    }
  }
  L.total = off;
  return L;
}

ta_status check(const ta_partition* P, const void* dpart, ta_dtype dt, int Hq, int Hkv, int d) {
  if (!P || !dpart) return TA_EINVAL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return TA_EINVAL;
  if (dt == TA_BF16) {
    if (d != 128) return TA_EUNSUPPORTED;
  } else if (dt == TA_F32) {
    if (d != 64 && d != 128) return TA_EUNSUPPORTED;
  } else {
    return TA_EUNSUPPORTED;
  }
  return TA_OK;
}

#define GW_HIP(x)                              \
  do {                                         \
    if ((x) != hipSuccess) return TA_EHIP;     \
  } while (0)
#define GW_TA(x)                               \
  do {                                         \
    const ta_status s_ = (x);                  \
    if (s_ != TA_OK) return s_;                \
  } while (0)

}  // namespace gw
}  // namespace ta

using namespace ta;

extern "C" ta_status tree_partition_upload(const ta_partition* P, void* dpart, size_t bytes, hipStream_t stream) {
  if (!P || !dpart) return TA_EINVAL;
  if (bytes < P->device_bytes) return TA_ENOMEM;
  char* base = (char*)dpart;
  for (int p = 0; p < P->n_parts; ++p) {
    const ta_plan* pl = P->plans[p];
    if (!pl) continue;
    const ta_status st = tree_plan_upload(pl, base + P->off_plan[p], pl->device_bytes, stream);
    if (st != TA_OK) return st;
    const size_t rows = size_t(P->tok_ptr[p + 1] - P->tok_ptr[p]);
    if (hipMemcpyAsync(base + P->off_idx[p], P->tok_idx.data() + P->tok_ptr[p], rows * sizeof(int32_t),
                       hipMemcpyHostToDevice, stream) != hipSuccess)
      return TA_EHIP;
  }
  return TA_OK;
}

extern "C" ta_status tree_partition_ws_bytes(const ta_partition* P, int32_t op, ta_dtype dt, int32_t Hq, int32_t Hkv,
                                             int32_t d, float rope_base, size_t* bytes) {
  if (!P || !bytes || (op != 0 && op != 1)) return TA_EINVAL;
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return TA_EINVAL;
  *bytes = gw::layout(P, op, dt, Hq, Hkv, d, rope_base).total;
  return TA_OK;
}

extern "C" ta_status tree_partition_fwd(const ta_partition* P, const void* dpart, ta_dtype dt, const void* q,
                                        const void* k, const void* v, int32_t Hq, int32_t Hkv, int32_t d, float scale,
                                        float rope_base, void* o, float* lse, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  GW_TA(gw::check(P, dpart, dt, Hq, Hkv, d));
  if (!q || !k || !v || !o || !lse) return TA_EINVAL;
  const gw::WsLayout L = gw::layout(P, 0, dt, Hq, Hkv, d, rope_base);
  if (!ws || ws_bytes < L.total) return TA_ENOMEM;
  char* w = (char*)ws;
  const char* dp = (const char*)dpart;
  const size_t es = dt == TA_BF16 ? 2 : 4, qrow = (size_t)Hq * d * es, krow = (size_t)Hkv * d * es;
  const size_t N = (size_t)P->n_tokens;
  for (int p = 0; p < P->n_parts; ++p) {
    const ta_plan* pl = P->plans[p];
    if (!pl) continue;
    const int R = pl->n_tokens, q0 = pl->q_start;
    const int32_t* idx = (const int32_t*)(dp + P->off_idx[p]);
    // gateway: the chain's K/V come from the partitions above; its Q rows are zeros
    GW_HIP(gw::gather(q, idx, w + L.q, R, q0, qrow, 1, 0, 0, stream));
    GW_HIP(gw::gather(k, idx, w + L.k, R, 0, krow, 1, 0, 0, stream));
    GW_HIP(gw::gather(v, idx, w + L.v, R, 0, krow, 1, 0, 0, stream));
    GW_TA(tree_attn_fwd(pl, dp + P->off_plan[p], dt, w + L.q, w + L.k, w + L.v, Hq, Hkv, d, scale, rope_base,
                        w + L.o, (float*)(w + L.lse), w + L.attn, L.attn_bytes, stream));
    // own rows back to the whole tree: O rows, LSE columns ([Hq, N] layout)
    GW_HIP(gw::scatter(w + L.o + q0 * qrow, idx + q0, o, R - q0, qrow, 1, 0, 0, stream));
    GW_HIP(gw::scatter(w + L.lse + q0 * sizeof(float), idx + q0, lse, R - q0, sizeof(float), Hq,
                       (size_t)R * sizeof(float), N * sizeof(float), stream));
  }
  return TA_OK;
}

extern "C" ta_status tree_partition_bwd(const ta_partition* P, const void* dpart, ta_dtype dt, const void* q,
                                        const void* k, const void* v, const void* o, const float* lse, const void* dO,
                                        int32_t Hq, int32_t Hkv, int32_t d, float scale, float rope_base, void* dq,
                                        void* dk, void* dv, void* ws, size_t ws_bytes, hipStream_t stream) {
  GW_TA(gw::check(P, dpart, dt, Hq, Hkv, d));
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return TA_EINVAL;
  if ((uintptr_t)dk % 16 || (uintptr_t)dv % 16) return TA_EINVAL;
  const gw::WsLayout L = gw::layout(P, 1, dt, Hq, Hkv, d, rope_base);
  if (!ws || ws_bytes < L.total) return TA_ENOMEM;
  char* w = (char*)ws;
  const char* dp = (const char*)dpart;
  const size_t es = dt == TA_BF16 ? 2 : 4, qrow = (size_t)Hq * d * es, krow = (size_t)Hkv * d * es;
  const size_t N = (size_t)P->n_tokens;
  const int kel = Hkv * d;
  float* acc_k = dt == TA_BF16 ? (float*)(w + L.acc_k) : (float*)dk;
  float* acc_v = dt == TA_BF16 ? (float*)(w + L.acc_v) : (float*)dv;
  GW_HIP(gw::zero(acc_k, (int64_t)N * kel, stream));
  GW_HIP(gw::zero(acc_v, (int64_t)N * kel, stream));
  for (int p = 0; p < P->n_parts; ++p) {
    const ta_plan* pl = P->plans[p];
    if (!pl) continue;
    const int R = pl->n_tokens, q0 = pl->q_start;
    const int32_t* idx = (const int32_t*)(dp + P->off_idx[p]);
    GW_HIP(gw::gather(q, idx, w + L.q, R, q0, qrow, 1, 0, 0, stream));
    GW_HIP(gw::gather(k, idx, w + L.k, R, 0, krow, 1, 0, 0, stream));
    GW_HIP(gw::gather(v, idx, w + L.v, R, 0, krow, 1, 0, 0, stream));
    GW_HIP(gw::gather(o, idx, w + L.o, R, q0, qrow, 1, 0, 0, stream));
    GW_HIP(gw::gather(dO, idx, w + L.dO, R, q0, qrow, 1, 0, 0, stream));
    GW_HIP(gw::gather(lse, idx, w + L.lse, R, q0, sizeof(float), Hq, N * sizeof(float), (size_t)R * sizeof(float),
                      stream));
    GW_TA(tree_attn_bwd(pl, dp + P->off_plan[p], dt, w + L.q, w + L.k, w + L.v, w + L.o, (const float*)(w + L.lse),
                        w + L.dO, Hq, Hkv, d, scale, rope_base, w + L.dq, w + L.dk, w + L.dv, w + L.attn,
                        L.attn_bytes, stream));
    GW_HIP(gw::scatter(w + L.dq + q0 * qrow, idx + q0, dq, R - q0, qrow, 1, 0, 0, stream));
    // relay: every local key row, the gateway chain included, into fp32
    GW_HIP(gw::scatter_add(dt, w + L.dk, idx, acc_k, R, kel, stream));
    GW_HIP(gw::scatter_add(dt, w + L.dv, idx, acc_v, R, kel, stream));
  }
  if (dt == TA_BF16) {
    GW_HIP(gw::cast(acc_k, (bf16*)dk, (int64_t)N * kel, stream));
    GW_HIP(gw::cast(acc_v, (bf16*)dv, (int64_t)N * kel, stream));
  }
  return TA_OK;
}
