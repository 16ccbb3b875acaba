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

// softplus(x) = max(x, 0) + log1p(t), t = e^-|x| in (0, 1].
// log1p(t) is log(w) for w = fl(1 + t) plus the rounding error of w: with m = w - 1 (exact
// for w in [1, 2]) and d = t - m (exact), log(1 + t) = log(w) + log(1 + d/w) ~ log(w) + d/w,
// and 1/w ~ 1 - m to the accuracy this tiny correction needs. When t < 2^-24, w = 1, m = 0
// and the result is t itself. max(x, 0) is one v_max_f32: the builtin fmax first quiets a
// possible signalling NaN with a second instruction wherever x comes from another basic block
// (the step is computed only with the softplus flag set, a runtime branch in every kernel); a
// quiet NaN gives the same result either way. Cost: 2 transcendentals and 7 simple VALU ops.
__device__ __forceinline__ float softplus(float x) {
  const float t = fast_exp2(-__builtin_fabsf(x) * kLog2e);
  const float w = 1.0f + t;
  const float m = w - 1.0f;
  const float d = t - m;
  const float corr = __builtin_fmaf(-d, m, d);
  const float lp = __builtin_fmaf(fast_log2(w), kLn2, corr);
  float mx;
  asm("v_max_f32 %0, 0, %1" : "=v"(mx) : "v"(x));
  return mx + lp;
}

// Input coefficient of the exact zero-order hold, (e^x - 1)/A for x = dt*A, given
// ab = e^x (as computed for the decay) and inv_a = 1/A. For |x| < 1/16 it is
// dt*(1 + x/2 + x^2/6 + x^3/24 + x^4/120), whose truncation is below 1.3e-9 relative (and
// which is dt at A = 0); otherwise (ab - 1)/A, where |ab - 1| > 0.06 keeps the rounding of
// ab below 2e-6 relative. The subtraction ab - 1 alone would lose all accuracy as x -> 0.
// Both sides are evaluated and one selected: the series is made opaque before the select,
// which the compiler otherwise turned into an exec-mask branch per state (both sides taken
// wherever the lanes of a wave disagree, plus the mask bookkeeping).
__device__ __forceinline__ float zoh_coef(float dt, float x, float ab, float inv_a) {
  const float p = __builtin_fmaf(
      x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f),
      1.0f);
  float small = dt * p;
  asm("" : "+v"(small));
  return __builtin_fabsf(x) < 0.0625f ? small : (ab - 1.0f) * inv_a;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z), with the reciprocal on the transcendental unit.
// For z < -88, e^-z = inf and the result is z * 0 = -0, the correct limit.
__device__ __forceinline__ float silu(float z) { return z * fast_rcp(1.0f + fast_exp2(-z * kLog2e)); }

// Wave issue priority from progress through the sequence: 3 in the first quarter down to 0
// in the last. A CU holds several workgroups of the same scan; among waves of equal
// priority the SIMD issues from the oldest, so without this the first resident workgroup
// runs as if alone and finishes in about half the time of the last, and the CU spends
// the tail of the launch at a third of its occupancy. Dropping the priority of a wave that
// has moved ahead lets the others catch up at every quarter (measured on the 130M-layer
// forward: the slowest of three co-resident workgroups 343K -> 300K cycles, kernel -7%).
// (Comparisons only: the arguments are wave-uniform, so this is a few scalar instructions.)
__device__ __forceinline__ void progress_priority(int64_t done, int64_t total) {
  if (4 * done < total)
    __builtin_amdgcn_s_setprio(3);
  else if (2 * done < total)
    __builtin_amdgcn_s_setprio(2);
  else if (4 * done < 3 * total)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Causal depthwise convolution + SiLU of the conv prologue for token t of one channel:
// silu(cb + w4[0] x_{t-3} + w4[1] x_{t-2} + w4[2] x_{t-1} + w4[3] x_t), the taps of a
// shorter filter right-aligned in w4 (zeros in front).
__device__ __forceinline__ float conv4_silu(const float (&w4)[4], float cb, float xm3, float xm2, float xm1,
                                            float x0) {
  float p = __builtin_fmaf(w4[0], xm3, cb);
  p = __builtin_fmaf(w4[1], xm2, p);
  p = __builtin_fmaf(w4[2], xm1, p);
  p = __builtin_fmaf(w4[3], x0, p);
  return silu(p);
}

// The four right-aligned taps of channel d's filter (kconv <= 4 taps) and its bias.
__device__ __forceinline__ void conv_taps(const float* conv_w, const float* conv_b, int kconv, int64_t d,
                                          float (&w4)[4], float& cb) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int tap = m - (4 - kconv);
    w4[m] = tap >= 0 ? conv_w[d * kconv + tap] : 0.0f;
  }
  cb = conv_b ? conv_b[d] : 0.0f;
}

// Input x at token tau of channel (b, d) for the conv window: the sequence for tau >= 0,
// the conv state (the kconv - 1 inputs before the sequence, oldest first) or 0 before it.
template <typename T>
__device__ __forceinline__ float conv_input(const T* x, const float* conv_state, int kconv, int64_t b,
                                            int64_t d, int64_t tau, int64_t seqlen, int64_t dim) {
  if (tau >= 0) return load_elem(x, (b * seqlen + tau) * dim + d);
  const int64_t j = (kconv - 1) + tau;
  return (conv_state && j >= 0) ? conv_state[(b * dim + d) * (kconv - 1) + j] : 0.0f;
}

}  // namespace ss
