// Device helpers shared by the kernel files: bf16 conversions with the rounding the
// oracle uses, wave64 reductions on DPP, the arg-max key, int8 unpacking.  Internal.
#pragma once
#include "qd_common.h"
#include <math.h>

namespace qd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
// round to nearest even: the hardware conversion (v_cvt_pk_bf16_f32 on gfx950), the same
// bits as adding 0x7FFF plus the lowest kept bit and truncating, for every finite input
// (f32 denormals are kept, the default for this code)
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

// wave64 reductions on DPP: quad swaps, half-row and row mirrors give every lane its
// 16-lane row total; two row broadcasts fold the four rows into lane 63, which is read
// back as a wave-uniform value
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(0.0f, v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(0.0f, v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(0.0f, v);       // row_half_mirror
  v += dpp_f<0x140>(0.0f, v);       // row_mirror
  v += dpp_f<0x142, 0xa>(0.0f, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xc>(0.0f, v);  // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
// the total of each 16-lane row, in every lane of the row (the first four steps above)
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(0.0f, v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(0.0f, v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(0.0f, v);  // row_half_mirror
  v += dpp_f<0x140>(0.0f, v);  // row_mirror
  return v;
}
// v combined with the value of lane l ^ 16 (row swap) or l ^ 32 (half swap) through the
// gfx950 lane-swap instructions instead of an LDS permute: swapping a register with itself
// leaves each lane its own value in one result and its partner's in the other
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v, v));
  v = fmaxf(v, dpp_f<0x4E>(v, v));
  v = fmaxf(v, dpp_f<0x141>(v, v));
  v = fmaxf(v, dpp_f<0x140>(v, v));
  v = fmaxf(v, dpp_f<0x142, 0xa>(v, v));
  v = fmaxf(v, dpp_f<0x143, 0xc>(v, v));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// 256-thread block reductions through LDS
__device__ __forceinline__ float block_sum256(float v, float* red4) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red4[wid] = v;
  __syncthreads();
  return red4[0] + red4[1] + red4[2] + red4[3];
}
__device__ __forceinline__ float block_max256(float v, float* red4) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red4[wid] = v;
  __syncthreads();
  return fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
}

// arg-max key: larger value wins, equal values go to the lower index; -0.0 == +0.0
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  if (v == 0.0f) v = 0.0f;
  uint32_t u = __float_as_uint(v);
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

// unpack 16 signed int8 codes to float
__device__ __forceinline__ void i8x16_to_f32(const int4 v, float* f) {
  const int w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) f[j * 4 + e] = (float)((int)((uint32_t)w4[j] << (24 - 8 * e)) >> 24);
}

}  // namespace qd
