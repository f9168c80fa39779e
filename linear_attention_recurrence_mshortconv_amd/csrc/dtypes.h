// bf16 / fp32 helpers for the device code (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace chm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float(uint32_t(u) << 16); }

// Two fp32 -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  bf16x2 b = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// Load / store 8 consecutive elements as fp32, from bf16 or fp32 storage.
__device__ __forceinline__ void load8(const uint16_t* p, float* out) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  out[0] = bf_lo(u.x); out[1] = bf_hi(u.x); out[2] = bf_lo(u.y); out[3] = bf_hi(u.y);
  out[4] = bf_lo(u.z); out[5] = bf_hi(u.z); out[6] = bf_lo(u.w); out[7] = bf_hi(u.w);
}
__device__ __forceinline__ void load8(const float* p, float* out) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]); u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]); u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ float to_f32(uint16_t u) { return bf2f(u); }
__device__ __forceinline__ float to_f32(float f) { return f; }
__device__ __forceinline__ void from_f32(uint16_t* p, float f) { *p = f2bf(f); }
__device__ __forceinline__ void from_f32(float* p, float f) { *p = f; }

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads() it
// does not wait for outstanding global loads and stores, so prefetches and
// write-backs stay in flight across it (the compiler still waits for a load
// before its result is used).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Work is spread over the 8 XCDs round-robin by block id; this maps the
// hardware block id to a logical id so that each XCD gets one contiguous range
// of logical ids (neighbouring tiles then share that XCD's L2). `nblk` must be
// the launched grid size, a multiple of 8.
__device__ __forceinline__ uint32_t xcd_contiguous_id(uint32_t hw_id, uint32_t nblk) {
  const uint32_t per_xcd = nblk / 8u;
  return (hw_id % 8u) * per_xcd + hw_id / 8u;
}

}  // namespace chm
