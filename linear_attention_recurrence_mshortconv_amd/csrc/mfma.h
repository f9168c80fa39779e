// MFMA fragments, bf16 packing, lane exchanges and buffer loads shared by the
// chunked KDA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

#include "dtypes.h"

namespace chm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;


// alpha is raised to at least e^{-7.5} (bf16 0x3A11) as the chunked kernels load it:
// their decay factors are products of up to 8 alphas and their reciprocals, which then
// stay within e^{+-60}, so both factors of every bf16 product keep full precision and
// the reciprocals stay finite. A token with a smaller alpha (alpha = 0 included) keeps
// 5.5e-4 of each decayed channel instead of less, below the bf16 resolution of a result.
constexpr uint32_t kAlphaMin2 = 0x3A113A11u;
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t clamp_alpha2(uint32_t u) {   // both bf16 halves (positive)
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, u),
                                                                 __builtin_bit_cast(u16x2_t, kAlphaMin2)));
}

__device__ __forceinline__ f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ uint2 pack4(const f32x4& v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ uint2 pack4(const float4& v) {
  return make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}
__device__ __forceinline__ uint4 pack8(const f32x4& lo, const f32x4& hi) {
  return make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                    pack_bf16x2(hi[2], hi[3]));
}
__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }
__device__ __forceinline__ float4 unpack4(uint2 u) {
  return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
}
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ __forceinline__ float4 rcp4(float4 a) {
  return make_float4(__builtin_amdgcn_rcpf(a.x), __builtin_amdgcn_rcpf(a.y), __builtin_amdgcn_rcpf(a.z),
                     __builtin_amdgcn_rcpf(a.w));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// sum of squares of the bf16 pair(s) in u (v_dot2_f32_bf16)
__device__ __forceinline__ float sq2(uint32_t u, float c) {
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, u);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, c, false);
}
__device__ __forceinline__ float dot4(uint2 u) { return sq2(u.y, sq2(u.x, 0.f)); }

// Position of channel (or token) c inside its row: within each group of 32 the
// order is 0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31.
__device__ __forceinline__ constexpr int cpos(int c) {
  return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Register-level lane exchanges.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_f<0xB1>(v); }              // quad_perm 1,0,3,2
__device__ __forceinline__ float lane_xor2(float v) { return dpp_f<0x4E>(v); }              // quad_perm 2,3,0,1
__device__ __forceinline__ float lane_xor4(float v) { return dpp_f<0x1B>(dpp_f<0x141>(v)); } // half mirror, quad reverse
__device__ __forceinline__ float lane_xor8(float v) { return dpp_f<0x128>(v); }             // row_ror 8
// lanes < 32 get lo + (lane + 32)'s lo, lanes >= 32 get (lane - 32)'s hi + hi
__device__ __forceinline__ float halve32(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(lo), __float_as_int(hi), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
// the same across 16-lane rows: lanes with bit 4 clear get lo + lo', set get hi' + hi
__device__ __forceinline__ float halve16(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(lo), __float_as_int(hi), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Sum 16 per-lane values over the 32 lanes of each half-wave by recursive
// halving; every lane returns the half-wave total of value (lane >> 1) & 15.
__device__ __forceinline__ float half_sum16(const float (&a)[16], int lane) {
  float b8[8], b4[4], b2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = halve16(a[j], a[j + 8]);
  const bool u3 = (lane >> 3) & 1, u2 = (lane >> 2) & 1, u1 = (lane >> 1) & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) b4[j] = (u3 ? b8[j + 4] : b8[j]) + lane_xor8(u3 ? b8[j] : b8[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b2[j] = (u2 ? b4[j + 2] : b4[j]) + lane_xor4(u2 ? b4[j] : b4[j + 2]);
  float b1 = (u1 ? b2[1] : b2[0]) + lane_xor2(u1 ? b2[0] : b2[1]);
  b1 += lane_xor1(b1);
  return b1;
}

// Sum 16 per-lane values over the 16 lanes of each DPP row by recursive halving; lane
// l16 of the row returns the row total of value l16.
__device__ __forceinline__ float row_sum16(const float (&a)[16], int l16) {
  float b8[8], b4[4], b2[2];
  const bool u3 = (l16 >> 3) & 1, u2 = (l16 >> 2) & 1, u1 = (l16 >> 1) & 1, u0 = l16 & 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = (u3 ? a[j + 8] : a[j]) + lane_xor8(u3 ? a[j] : a[j + 8]);
#pragma unroll
  for (int j = 0; j < 4; ++j) b4[j] = (u2 ? b8[j + 4] : b8[j]) + lane_xor4(u2 ? b8[j] : b8[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b2[j] = (u1 ? b4[j + 2] : b4[j]) + lane_xor2(u1 ? b4[j] : b4[j + 2]);
  return (u0 ? b2[1] : b2[0]) + lane_xor1(u0 ? b2[0] : b2[1]);
}

// third descriptor word of a raw buffer resource on gfx9
constexpr int kRsrcW3 = 0x00020000;
// A buffer offset past every bound (2^31 as the unsigned offset the hardware sees): channels beyond
// a head's dk / dv read zero and are not stored. Bounds stay at or below 2^31 bytes (64 token rows
// of at most 2^25 bytes), and offset plus any token row offset stays below 2^32.
constexpr int kOffOut = INT32_MIN;
__device__ __forceinline__ uint2 ld_buf64(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v[0], v[1]);
}

__device__ __forceinline__ uint4 ld128(const uint16_t* base, int idx) {
  return *reinterpret_cast<const uint4*>(base + idx);
}
// Transposing LDS read: within each 16-lane group, lane i receives element i%4
// of the 8-byte reads of lanes 4j + i/4 (j = 0..3) as its element j.
__device__ __forceinline__ uint2 ld_tr(const uint16_t* p) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace
}  // namespace chm
