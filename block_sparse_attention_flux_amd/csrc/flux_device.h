// Device-side helpers shared by the gfx950 kernels of libflux.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Reinterpret 32 bits as fp32.  Takes the value, not a vector element: a
// __builtin_bit_cast applied directly to an ext_vector element lvalue reads
// element 0 with this compiler, whatever the index.
__device__ __forceinline__ float u32_as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Wait until every vector memory operation this wave issued has completed
// (loads returned, stores acknowledged): s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16-byte global load / store of raw bits.
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// 16-byte streaming load (non-temporal: data read once, not kept in the caches)
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// v_exp_f32: 2^x, exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Both 32-lane halves of v after v_permlane32_swap: lo[l] = v[l % 32],
// hi[l] = v[l % 32 + 32] (one VALU op, no LDS).
__device__ __forceinline__ void halves(float v, float& lo, float& hi) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  lo = u32_as_f32(r[0]);
  hi = u32_as_f32(r[1]);
}
// max / sum of lanes l and l ^ 32, the same value (and bits) in both lanes
__device__ __forceinline__ float max_halves(float v) {
  float lo, hi;
  halves(v, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_halves(float v) {
  float lo, hi;
  halves(v, lo, hi);
  return lo + hi;
}

// The values of lanes l & ~16 and l | 16 (the two 16-lane rows of a 32-lane
// half) after v_permlane16_swap, in both lanes (one VALU op, no LDS).
__device__ __forceinline__ void quarters(float v, float& lo, float& hi) {
  const uint32_t x = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  lo = u32_as_f32(r[0]);
  hi = u32_as_f32(r[1]);
}
// max / sum of lanes l and l ^ 16, the same value (and bits) in both lanes
__device__ __forceinline__ float max_quarters(float v) {
  float lo, hi;
  quarters(v, lo, hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float sum_quarters(float v) {
  float lo, hi;
  quarters(v, lo, hi);
  return lo + hi;
}

// a.x + a.y + c for a packed bf16 pair a (v_dot2c_f32_bf16 against (1, 1))
__device__ __forceinline__ float add_bf16_pair(uint32_t a, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), c, false);
}

}  // namespace flux
