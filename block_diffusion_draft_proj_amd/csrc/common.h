// Internal device helpers shared by the gfx950 kernels of the DFlash hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 16;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, round-robin WG dispatch

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// 16-byte global loads / stores.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Byte permute of the 8-byte value {hi:lo}: result byte i = byte sel[i] (v_perm_b32).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// Low halves of a and b -> {b.lo : a.lo};  high halves -> {b.hi : a.hi}.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm(b, a, 0x07060302u); }

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 (nearest even) of the exact sum a + b of two fp64 values, rounded once.
// The fp64 sum s and its rounding error e (two-sum) hold the exact value.  It is
// narrowed to fp32 by round-to-odd -- truncate toward zero, then set the last bit
// if anything was dropped -- which keeps enough of the discarded part that the
// fp32 -> bf16 nearest-even step (16 bits narrower) equals a direct rounding of
// the exact value.  s is a double (not float) so no step rounds on its own.
__device__ __forceinline__ uint16_t bf16_of_exact_sum(double a, double b) {
#pragma clang fp contract(off)
  const double s = a + b;
  const double bb = s - a;
  const double e = (a - (s - bb)) + (b - bb);
  const float f = (float)s;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != s) {
    if (fabs(back) > fabs(s)) u -= 1u;   // f was rounded away from zero: step back
    u |= 1u;
  } else if (e != 0.0) {                 // s is an fp32 value; the exact sum is just off it
    if ((e < 0.0) != (f < 0.0)) u -= 1u; // ... on the side of zero
    u |= 1u;
  }
  return f32_to_bf16(__uint_as_float(u));
}

// bf16 (nearest even) of the exact value a*c + b*d of fp32 inputs, rounded once.
// Fast path: y = fma(a, c, fl(b*d)) is within 2^-24 (|b d| + |y|) of the exact value
// (one product rounding, one fma rounding); whenever y lies farther than twice that
// from the midpoint of its bf16 interval, the exact value rounds to the same bf16 as
// y (it cannot cross that midpoint, nor reach the midpoints of the neighbouring
// intervals, half a step away).  Otherwise (rare: within ~2^-15 of a step around the
// midpoint) the exact value is rounded through fp64 (bf16_of_exact_sum; products of
// two fp32 values are exact in fp64).
__device__ __forceinline__ uint16_t bf16_of_exact_dot2(float a, float c, float b, float d) {
  const float bd = b * d;
  const float y = __builtin_fmaf(a, c, bd);
  const uint32_t u = __float_as_uint(y);
  const float mid = __uint_as_float((u & 0xffff0000u) | 0x8000u);  // same sign and binade as y
  const float dist = fabsf(y - mid);                               // exact (same binade)
  const float err = (fabsf(bd) + fabsf(y)) * 0x1p-23f + 0x1p-140f;
  if (dist > err && (u & 0x7f800000u) != 0x7f800000u) return f32_to_bf16(y);
  return bf16_of_exact_sum((double)a * (double)c, (double)b * (double)d);
}

// One rotate-half RoPE pair (lo = x_j, hi = x_{j+d/2}) with fp32 cos / sin: each
// output is the exact rotation rounded once to bf16.
__device__ __forceinline__ void rope_pair_bf16(float lo, float hi, float c, float s, uint16_t& ylo,
                                               uint16_t& yhi) {
  ylo = bf16_of_exact_dot2(lo, c, hi, -s);
  yhi = bf16_of_exact_dot2(hi, c, lo, s);
}

#define LDS_AS __attribute__((address_space(3)))

// 16 bytes per lane from `src` into LDS at `lds_base` + 16 * lane (global_load_lds,
// LDS side lane-contiguous; `lds_base` must be wave-uniform).
// Issued as inline assembly on purpose: the compiler cannot tell which LDS bytes
// the DMA writes, so with the builtin it waits for every outstanding load before
// any LDS read it cannot prove disjoint (e.g. a transpose read), which empties a
// stage ring.  Completion is tracked by hand (wait_vmcnt + barrier); loads the
// compiler does not see can only make its own vmcnt waits stricter, never looser.
// M0 is saved and restored around the load since the compiler reserves it.
// The _nt form marks data read exactly once (non-temporal): measured on this
// part, that lifts a plain streaming read from ~6.2 to ~7.1 TB/s.
__device__ __forceinline__ void lds_dma16_nt(const void* src, char* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)lds_base);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(m0) : "memory");
}
__device__ __forceinline__ void lds_dma16(const void* src, char* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)lds_base);
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(m0) : "memory");
}

// Same load addressed as a wave-uniform base (SGPR pair) plus a 32-bit per-lane
// byte offset, into LDS byte address `m0` (wave-uniform): no 64-bit address math
// per lane.
// The base goes through readfirstlane so that it is provably wave-uniform: where the
// compiler's uniformity analysis loses track of it, an "s" operand would otherwise be
// handed a VGPR pair.
__device__ __forceinline__ void lds_dma16_nt_sv(const void* sbase, uint32_t voff, uint32_t m0) {
  const uint64_t a = (uint64_t)(uintptr_t)sbase;
  // readfirstlane returns int: each half goes back to uint32 before widening, or the
  // low half would be sign-extended into the high one.
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t u = ((uint64_t)hi << 32) | lo;
  const void* base = (const void*)(uintptr_t)u;
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(base), "s"(m0) : "memory");
}

// Non-temporal global_load_lds into LDS byte address `m0` (wave-uniform).
__device__ __forceinline__ void lds_dma16_nt_m0(const void* src, uint32_t m0) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(m0) : "memory");
}

// global_load_lds (cached) into LDS byte address `m0` (wave-uniform).
__device__ __forceinline__ void lds_dma16_m0(const void* src, uint32_t m0) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(src), "s"(m0) : "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS only.  __syncthreads() also orders global
// memory, which makes every wave wait for all of its outstanding global loads
// (vmcnt(0)) and so drains any register prefetch at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Accelerator die (XCD) the wave runs on: HW_REG_XCC_ID (hardware register 20),
// bits 3:0, on gfx950.
__device__ __forceinline__ uint32_t xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);
}

// Device-side error bits (workspace word 0), as declared in the public header.
constexpr uint32_t kDevErrCtxLen = 1u, kDevErrPageId = 2u, kDevErrRow = 4u, kDevErrMerge = 8u,
                   kDevErrXcd = 16u, kDevErrAccept = 32u;

__device__ __forceinline__ void set_dev_error(uint32_t* err_word, uint32_t bit) {
  __hip_atomic_fetch_or(err_word, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dflash
