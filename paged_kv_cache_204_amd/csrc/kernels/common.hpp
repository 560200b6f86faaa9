// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 halves of a packed 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// ---- cross-lane reductions without LDS traffic ------------------------------
// DPP within 16-lane rows, v_permlane16/32_swap across rows (gfx950).
constexpr int kDppXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppMirror8 = 0x141;  // row_half_mirror: lane i <-> 7 - i within 8
constexpr int kDppMirror16 = 0x140; // row_mirror: lane i <-> 15 - i within 16
constexpr int kDppXor8 = 0x128;     // row_ror 8: lane i <-> i ^ 8 within 16

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of W lanes (W = 2, 4, 8 or 16); every lane of
// the group gets the total.  Mirror steps pair lanes so that, with the two
// quad swaps after them, each lane has added all W values once.
template <int W>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (W >= 16) x += dpp_f32<kDppMirror16>(x);
  if constexpr (W >= 8) x += dpp_f32<kDppMirror8>(x);
  if constexpr (W >= 2) x += dpp_f32<kDppXor1>(x);
  if constexpr (W >= 4) x += dpp_f32<kDppXor2>(x);
  return x;
}
template <int W>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (W >= 16) x = fmaxf(x, dpp_f32<kDppMirror16>(x));
  if constexpr (W >= 8) x = fmaxf(x, dpp_f32<kDppMirror8>(x));
  if constexpr (W >= 2) x = fmaxf(x, dpp_f32<kDppXor1>(x));
  if constexpr (W >= 4) x = fmaxf(x, dpp_f32<kDppXor2>(x));
  return x;
}

// The value of lane l ^ 16 (resp. l ^ 32) combined with lane l's own: the
// swap returns the pair {own, partner} in the two results.
__device__ __forceinline__ float xor16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_max(float v) {
  return xor32_max(xor16_max(group_max<16>(v)));
}
__device__ __forceinline__ float wave_sum(float v) {
  return xor32_sum(xor16_sum(group_sum<16>(v)));
}

// Workgroup barrier that orders LDS traffic only.  __syncthreads() also
// fences global memory, which makes every wave drain its in-flight global
// loads (prefetches included) at each barrier; here only LDS operations are
// waited for, so loads issued ahead stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 2^x with the hardware instruction (results below 2^-126 flush to zero).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

}  // namespace pkv
