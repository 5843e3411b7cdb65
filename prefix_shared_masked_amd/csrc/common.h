// Device helpers shared by the gfx950 kernels: bf16 vectors, MFMA wrappers,
// the LDS transpose read, and launch error mapping.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "tree_attn.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16-byte load/store unit (a native vector: selects stay in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define TA_LOG2E 1.4426950408889634f
#define TA_LN2 0.6931471805599453f

namespace ta {

// 32x32x16 bf16 MFMA: C[32x32] += A[32x16] B[16x32].  Lane l holds row l%32
// of A and column l%32 of B, each with the 8 k-slots of half l/32; C is held
// as 16 registers per lane, register r <-> row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Accumulating 32x32x16 bf16 MFMA whose accumulator lives in AGPRs, for
// loop-carried accumulators that nothing but these MFMAs touches between
// agpr_fence8() points.  The compiler's hazard recognizer does not look inside
// inline asm, so the asm carries its own wait states: a VALU write of a VGPR
// needs two wait states before an MFMA may read it as A or B (the compiler
// itself spaces builtin MFMAs that way), and s_nop 2 gives three.  Chained
// MFMAs into the same accumulator need none.
__device__ __forceinline__ void mfma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the accumulators' MFMA writes and any other access (an
// XDL 16-pass result needs at most 18; this gives 24), and between VALU
// writes (zero init) and the first MFMA.  The accumulators are operands, so
// their initialisation and epilogue reads cannot move across the fence.
__device__ __forceinline__ void agpr_fence8(f32x16 (&x)[4], f32x16 (&y)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(x[0]), "+a"(x[1]), "+a"(x[2]), "+a"(x[3]), "+a"(y[0]), "+a"(y[1]), "+a"(y[2]), "+a"(y[3]));
}

// Wait states between VALU writes of accumulators (zero init) and the first
// MFMA, and between the last MFMA writes and the epilogue reads; the
// accumulators are asm operands, so neither can move across the fence.
__device__ __forceinline__ void acc_fence4(f32x16 (&x)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

// Same shape with fp16 operands (same rate; 10 stored mantissa bits).
__device__ __forceinline__ f32x16 mfma32h(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// fp32 -> fp16 for the score operands: a value beyond the largest finite
// fp16 (65504) clamps to +-65504, so it never becomes inf inside a score, and
// sets `sat`; NaN passes through unchanged (the NaN-propagating maximum and
// minimum), so a NaN input still shows up as NaN in the outputs it reaches.
__device__ __forceinline__ f16 to_f16_sat(float x, bool& sat) {
  sat |= fabsf(x) > 65504.f;  // false for NaN
  return (f16)__builtin_elementwise_minimum(__builtin_elementwise_maximum(x, -65504.f), 65504.f);
}
// Raise a caller-visible saturation flag (a device int32; may be null) from
// every lane that clamped.  Every writer stores the same 1.
__device__ __forceinline__ void report_sat(int32_t* flag, bool sat) {
  if (flag && sat) *(volatile int32_t*)flag = 1;
}

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane x points at row x/4, columns 4*(x%4)..+3 of a 4x16 bf16 block and
// receives column x of that block (its 4 rows).
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// The transpose read moves 16-bit elements whatever their type.
__device__ __forceinline__ f16x4 lds_read_tr(const f16* p) {
  return __builtin_bit_cast(f16x4, lds_read_tr((const bf16*)p));
}
// Eight floats to fp16, rounding toward zero: out-of-range values clamp to
// +-65504 instead of becoming infinities.
__device__ __forceinline__ f16x8 pack_f16_rtz(const float* x) {
  uint4 w;
  w.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x[0], x[1]));
  w.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x[2], x[3]));
  w.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x[4], x[5]));
  w.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x[6], x[7]));
  return __builtin_bit_cast(f16x8, w);
}

// Eight floats to fp16, rounding to nearest even (for values in [0, 1]).
__device__ __forceinline__ f16x8 pack_f16_rte(const float* x) {
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, f16x8);
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& a, const bf16x4& b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f16x8 cat(const f16x4& a, const f16x4& b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotary angle pos * base^(-2i/d): the product and the reduction by
// quadrants (multiples of pi/2) are done in double precision, so long depths
// lose no accuracy; sin and cos of the remainder r in [-pi/4, pi/4] come from
// their Taylor series (truncation error below 2e-9 at |r| = pi/4).  The
// inverse frequency base^(-2i/d) depends on i alone: kernels that rotate many
// elements compute it once per dimension (rope_inv, into LDS or a register)
// and then call rope_sincos_at; the two paths give bitwise the same values.
__device__ __forceinline__ double rope_inv(int i, int d, float base) {
  return exp2(-(2.0 * i / d) * log2((double)base));
}
__device__ __forceinline__ void rope_sincos_at(int pos, double inv, float* s, float* c) {
  const double ang = (double)pos * inv;
  const double half_pi = 1.5707963267948966;
  const double kq = rint(ang * 0.63661977236758134);  // 2/pi: a multiply, not a division
  const float r = (float)(ang - kq * half_pi);
  const float r2 = r * r;
  const float sr = r * (1.f + r2 * (-1.f / 6 + r2 * (1.f / 120 + r2 * (-1.f / 5040 + r2 * (1.f / 362880)))));
  const float cr = 1.f + r2 * (-0.5f + r2 * (1.f / 24 + r2 * (-1.f / 720 + r2 * (1.f / 40320 + r2 * (-1.f / 3628800)))));
  const int q = (int)((long long)kq & 3);
  *s = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
  *c = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
}
__device__ __forceinline__ void rope_sincos(int pos, int i, int d, float base, float* s, float* c) {
  rope_sincos_at(pos, rope_inv(i, d, base), s, c);
}
// The inverse frequencies of dimensions 0 .. n-1 into LDS by the first n
// threads of the workgroup (the caller puts a barrier before reading them).
__device__ __forceinline__ void rope_inv_table(double* tab, int n, int d, float base) {
  if ((int)threadIdx.x < n) tab[threadIdx.x] = base > 0.f ? rope_inv(threadIdx.x, d, base) : 0.0;
}

// Gathered key chunk of the plan: slot v -> packed key index and the end of
// the DFS interval of the key's node (row i reads the key iff key <= i < kend).
// K/V tiles staged by direct global-to-LDS copies use rows of 128 16-bit
// elements (256 bytes) with no padding; the 16-byte piece p of row r is
// stored at piece p ^ swz(r).  swz moves the row's low two bits to the high
// two bits of the piece index and bits 2-3 to the low two (a bijection on
// 0..15): the 16 rows that one 16-byte row read touches land on 16 distinct
// pieces, and the 4 rows x 4 pieces of each half of a transpose read land
// on 16 distinct pieces (measured on gfx950: transpose reads ~134 B/clk/CU
// with this layout against ~110 for a padded 288-byte pitch).
__device__ __forceinline__ constexpr int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// One 16-byte global-to-LDS copy per lane (global_load_lds_dwordx4): lane i
// writes lds_base + 16 i, where lds_base (taken from M0; one wait state after
// writing it) is the same for the whole wavefront.  The copy bypasses VGPRs
// and counts on the vector-memory counter.  It is issued from inline asm
// because the compiler cannot tell that the copies target the buffer nobody
// is reading and would wait for them before every LDS read; the cost is that
// the copies are invisible to its wait-count bookkeeping, so whoever reads the
// data must first run lds_copies_wait() (then a workgroup barrier).  M0 is
// listed as clobbered for the reader; the compiler reserves M0 and emits no
// other M0 use in these kernels (checked in the generated code), so nothing
// it keeps there is lost.
// The LDS address of a generic pointer into shared memory: a flat address in
// the LDS aperture holds the LDS offset in its low 32 bits (the aperture base
// is the high half), so truncation gives it without the null check an
// address-space cast carries.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
__device__ __forceinline__ void copy16_to_lds(const void* g, const void* lds_base) {
  const uint32_t a = lds_addr(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(a) : "memory", "m0");
}
// Non-temporal variant: the data streams past the caches.
__device__ __forceinline__ void copy16_to_lds_nt(const void* g, const void* lds_base) {
  const uint32_t a = lds_addr(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(a)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_copies_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Scalar-base forms: lane i copies the bytes at sbase + voff_i, where sbase
// is wave-uniform (an SGPR pair) and voff_i a 32-bit per-lane byte offset,
// into lds + 16 i (16-byte form) or lds + 4 i (4-byte form).  A loop whose
// per-lane offsets do not change only recomputes the scalar base, so a copy
// costs no vector instructions.  lds is an LDS byte address (lds_addr).
// The base goes through readfirstlane so it is an SGPR pair even where the
// compiler cannot prove it uniform.  The builtin returns int: each half is
// taken back to uint32_t before widening, or the low half would be
// sign-extended into the high one.
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | (uint64_t)lo;
}
__device__ __forceinline__ void copy16_to_lds_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(sbase)),
               "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(uniform_ptr(sbase)),
               "s"(lds)
               : "memory", "m0");
}

// Plan tables are read-only for a kernel's lifetime.  Reading them through
// the constant address space lets uniform reads become scalar loads, which
// issue early and never make the vector-memory counter wait on them.
typedef const int32_t __attribute__((address_space(4)))* cint_ptr;
__device__ __forceinline__ cint_ptr as_const(const int32_t* p) { return (cint_ptr)p; }

// A chunk record held in registers: [nseg nkeys full -], kstart[4],
// vstart[4], kend[4].  Loaded with four uniform 16-byte reads before any use,
// so slot lookups below are register selects only.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef const i32x4 __attribute__((address_space(4)))* ci32x4_ptr;
struct ChunkRec {
  i32x4 h, ks, ko, ke;
};
__device__ __forceinline__ ChunkRec load_chunk(cint_ptr ch) {
  const ci32x4_ptr p = (ci32x4_ptr)ch;
  return ChunkRec{p[0], p[1], p[2], p[3]};
}
__device__ __forceinline__ void chunk_slot(const ChunkRec& c, int v, int& phys, int& kend) {
  int j = c.ks[0] + (v - c.ko[0]), e = c.ke[0];
#pragma unroll
  for (int x = 1; x < TA_CHUNK_MAX_SEG; ++x) {
    const bool in = c.ko[x] <= v;
    j = in ? c.ks[x] + (v - c.ko[x]) : j;
    e = in ? c.ke[x] : e;
  }
  phys = v < c.h[1] ? j : c.ks[0];  // padding slot: a valid row, never visible
  kend = v < c.h[1] ? e : 0;
}

// Key index and DFS-interval end of slot v of a gathered chunk.  All fields
// are read with uniform indices (scalar loads) and the segment is picked per
// lane with selects; unused segments carry offsets past the last slot.
template <class Ptr>
__device__ __forceinline__ void chunk_slot(Ptr ch, int v, int& phys, int& kend) {
  int j = ch[4] + (v - ch[8]), e = ch[12];
#pragma unroll
  for (int x = 1; x < TA_CHUNK_MAX_SEG; ++x) {
    const int ks = ch[4 + x], ko = ch[8 + x], ke = ch[12 + x];
    j = ko <= v ? ks + (v - ko) : j;
    e = ko <= v ? ke : e;
  }
  phys = v < ch[1] ? j : ch[4];  // padding slot: a valid row, never visible
  kend = v < ch[1] ? e : 0;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// RoPE / conversion pass over a [N, H, d] tensor (attn_fwd.hip); the result
// is multiplied by mul before the conversion to To.  A non-null y2 also
// receives the rotated values (without mul) in bf16.
template <typename Ti, typename To>
hipError_t launch_rope(const Ti* x, To* y, const int32_t* pos, int N, int H, int d, float base, int transpose,
                       hipStream_t st, float mul = 1.f, bf16* y2 = nullptr, int32_t* sat_flag = nullptr);

// Saturation flag of the bf16 attention calls: a device int32 at the start of
// their workspaces (the scratch they use starts TA_WS_FLAG_BYTES later).
constexpr size_t TA_WS_FLAG_BYTES = 256;

}  // namespace ta

namespace ta {
// Record events[i] on the stream when the caller asked for stage timing.
inline void mark(hipEvent_t* ev, int32_t n, int32_t i, hipStream_t st) {
  if (ev && i < n && ev[i]) (void)hipEventRecord(ev[i], st);
}
}  // namespace ta

#define TA_LAUNCH_CHECK()                            \
  do {                                               \
    if (hipGetLastError() != hipSuccess) return TA_EHIP; \
  } while (0)
