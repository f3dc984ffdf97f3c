// Device helpers shared by the HIP kernels of the verification library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace sv {

// bf16 is carried as its 16-bit pattern; arithmetic is always fp32 or fp64.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
  using storage = float;
  __device__ __forceinline__ static float load(const void* p, size_t i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ __forceinline__ static void store(void* p, size_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
};
template <> struct io<bf16_t> {
  using storage = uint16_t;
  __device__ __forceinline__ static float load(const void* p, size_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  __device__ __forceinline__ static void store(void* p, size_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  }
};

__device__ __forceinline__ void flag_error(int32_t* err, int32_t bit) {
  if (err) atomicOr(err, bit);
}

// Sum over aligned groups of W lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Data-parallel-primitive lane moves within rows of 16 lanes (VALU operand
// modifiers, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over each row of 16 lanes, result in every lane of the row:
// rotate by 8, rotate by 4, then swap lane pairs 2 apart and 1 apart.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0x128>(v);  // row_ror:8
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0xb1>(v);   // quad_perm [1,0,3,2]
  return v;
}

}  // namespace sv
