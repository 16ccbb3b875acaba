// ss_common.h -- device helpers shared by the libss kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element loads: fp32 as is, bf16 is the top half of an fp32 (exact widening).
__device__ __forceinline__ float load_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^x on the transcendental unit (v_exp_f32). Inputs below -126 flush to 0,
// which is the correct limit for a decay factor.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32), x > 0 and normal.
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(x) = log(1 + e^x), accurate to a few ulp in fp32 over the whole range.
// For x > 15, e^-x < 3.1e-7 and softplus(x) = x + e^-x to within fp32 rounding of x.
// Otherwise with e = e^x, log1p(e) is computed as log(1+e) * e / ((1+e) - 1), which
// cancels the rounding of 1+e (the classic log1p identity); for tiny e the quotient
// degenerates and log1p(e) = e is exact to fp32.
__device__ __forceinline__ float softplus(float x) {
  if (x > 15.0f) return x + fast_exp2(-x * kLog2e);
  const float e = fast_exp2(x * kLog2e);
  const float w = 1.0f + e;
  const float m = w - 1.0f;
  if (m == 0.0f) return e;
  return fast_log2(w) * kLn2 * (e / m);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z); for z < -88 the denominator is inf and
// the result is -0, the correct limit.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + fast_exp2(-z * kLog2e)); }

}  // namespace ss
