// ss_step.hip -- one decode step of the selective scan, state carried in place.
// (Input term dt*B, or the exact zero-order hold (abar - 1)/A * B when StepArgs::zoh is set.)
//
// Recurrent inference with a fixed-size state and constant work per token
// ("Mamba：选择性状态空间模型入门教程", table "Mamba vs Transformer vs RNN", and the step
// function (input, state) -> (output, new state) of "Mamba架构深度解析", section
// "Mamba的创新：选择性状态空间模型"). The update itself is the ss_fwd update for one t.
//
// One lane per (b, d). The 16-float state row of a lane is contiguous (64 bytes), so a
// wave reads and writes 4 KiB of consecutive state with 16-byte vector accesses. When a
// wave never straddles two batch rows (dim a multiple of 64) B_t and C_t are wave-uniform
// and come in through scalar loads. The step is bound by the state traffic (128 B per
// channel per token) and the fp32 state never leaves HBM between steps.
#include "ss_common.h"
#include "ss_kernels.h"

namespace ss {

template <int NS, typename T, bool GATE, bool UNIFORM_ROW, bool VEC, bool ZOH>
__global__ __launch_bounds__(256) void step_kernel(StepArgs a) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t total = a.batch * a.dim;
  if (j >= total) return;
  const int ns = NS > 0 ? NS : a.dstate;
  int64_t b = j / a.dim;
  if (UNIFORM_ROW) b = __builtin_amdgcn_readfirstlane(static_cast<int>(b));
  const int64_t d = j - b * a.dim;
  const T* __restrict__ Bm = static_cast<const T*>(a.B) + b * ns;
  const T* __restrict__ Cm = static_cast<const T*>(a.C) + b * ns;
  float* __restrict__ st = a.state + j * ns;

  float h[16];
  if (VEC) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(st)[q];
      h[4 * q] = v.x; h[4 * q + 1] = v.y; h[4 * q + 2] = v.z; h[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int n = 0; n < 16; ++n) h[n] = (n < ns) ? st[n] : 0.0f;
  }

  const float x = load_elem(static_cast<const T*>(a.delta), j) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
  const float dt = a.softplus ? softplus(x) : x;
  const float uv = load_elem(static_cast<const T*>(a.u), j);
  const float du = dt * uv;
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    if (n < ns) {
      const float an = a.A[d * ns + n];
      const float x2 = dt * (an * kLog2e);
      const float ab = fast_exp2(x2);
      const float bu = ZOH ? zoh_coef(dt, x2 * kLn2, ab, 1.0f / an) * uv : du;
      h[n] = __builtin_fmaf(ab, h[n], bu * load_elem(Bm, n));
      acc = __builtin_fmaf(load_elem(Cm, n), h[n], acc);
    }
  }
  float yv = __builtin_fmaf(a.D ? a.D[d] : 0.0f, uv, acc);
  if (GATE) yv *= silu(load_elem(static_cast<const T*>(a.z), j));
  a.y[j] = yv;

  if (VEC) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<float4*>(st)[q] = make_float4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3]);
  } else {
#pragma unroll
    for (int n = 0; n < 16; ++n)
      if (n < ns) st[n] = h[n];
  }
}

template <int NS, typename T, bool GATE, bool UNI, bool VEC>
static hipError_t launch_step(const StepArgs& a, hipStream_t s) {
  const int64_t total = a.batch * a.dim;
  const unsigned grid = static_cast<unsigned>((total + 255) / 256);
  if (a.zoh)
    hipLaunchKernelGGL((step_kernel<NS, T, GATE, UNI, VEC, true>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel<NS, T, GATE, UNI, VEC, false>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, bool GATE>
static hipError_t launch_step_g(const StepArgs& a, hipStream_t s) {
  const bool uni = (a.dim % 64) == 0;
  const bool vec = a.dstate == 16 && (reinterpret_cast<uintptr_t>(a.state) % 16) == 0;
  if (vec) return uni ? launch_step<16, T, GATE, true, true>(a, s) : launch_step<16, T, GATE, false, true>(a, s);
  return uni ? launch_step<0, T, GATE, true, false>(a, s) : launch_step<0, T, GATE, false, false>(a, s);
}

hipError_t step(const StepArgs& a, hipStream_t s) {
  const bool g = a.z != nullptr;
  if (a.dtype == kBF16) return g ? launch_step_g<uint16_t, true>(a, s) : launch_step_g<uint16_t, false>(a, s);
  return g ? launch_step_g<float, true>(a, s) : launch_step_g<float, false>(a, s);
}

}  // namespace ss
