// Shared device helpers of the HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

constexpr float kLog2e = 1.4426950408889634f;  // log2(e): exp(x) = 2^(x * log2 e)
constexpr float kLn2 = 0.69314718055994531f;    // ln(2)
constexpr float kNegInf = -__builtin_inff();

// 2^x on the transcendental unit (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap with both operands x: result [0] holds lanes 0..31 of x in
// both halves of the wave, result [1] holds lanes 32..63 of x in both halves, so
// every lane sees its own value and that of lane ^ 32.

// max of a value and its lane ^ 32 partner (both halves end with the same value).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// sum of a value and its lane ^ 32 partner, added in lane order (low + high) in
// both halves so the two halves hold bit-identical results.
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                            __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

}  // namespace osm
