// Cross-lane sums inside a wave64 for the token-by-token kernels, where a column of the
// state is spread over the 16 lanes of one DPP row (row-threads) and a wave holds four
// such columns, one per DPP row.
#pragma once
#include <hip/hip_runtime.h>

namespace chm {

// x moved from the lane given by the DPP control CTRL (all rows and banks)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the 16 lanes of a DPP row, in every lane: xor 1, xor 2 (quad permutes), then
// the half-row and row mirrors
__device__ __forceinline__ float sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four columns of one wave), in every lane
__device__ __forceinline__ float sum_cols4(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
  x = __int_as_float(r[0]) + __int_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Sums over the four columns of one wave (lanes l, l ^ 16, l ^ 32, l ^ 48) of NV values at
// once (NV a multiple of 4): a permlane16 swap of two values leaves the first's pair sums in
// wave rows 0 and 2 and the second's in rows 1 and 3, and a permlane32 swap of two such
// results completes four values, one per wave row: out[n] in wave row w is the total of
// v[4 n + w].
template <int NV>
__device__ __forceinline__ void sum_cols4_many(const float (&v)[NV], float (&out)[NV / 4]) {
  float s1[NV / 2];
#pragma unroll
  for (int m = 0; m < NV / 2; ++m) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(v[2 * m]), __float_as_int(v[2 * m + 1]), false,
                                                    false);
    s1[m] = __int_as_float(r[0]) + __int_as_float(r[1]);
  }
#pragma unroll
  for (int n = 0; n < NV / 4; ++n) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(s1[2 * n]), __float_as_int(s1[2 * n + 1]), false,
                                                    false);
    out[n] = __int_as_float(r[0]) + __int_as_float(r[1]);
  }
}

}  // namespace chm
