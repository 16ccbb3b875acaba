// ss_fwd_seq.hip -- reference-layout selective-scan forward: one lane per (b, d) channel,
// sequential in t, the N states in registers.
//
// The recurrence of "Mamba：选择性状态空间模型入门教程" (section "Mamba 的关键创新：
// 选择性机制") per channel, discretised as in "架构变体：Mamba/SSM" (section "离散化"):
//   dt = softplus(delta + bias); abar = exp(dt A[d,n]); h = abar h + (bbar B_t[n]) u;
//   y = (C_t . h + D u) silu(z),
// with bbar = dt, or the exact zero-order hold (abar - 1)/A[d,n] when ZOH is set.
// A wave covers 64 consecutive channels of one batch row, so every lane of the wave reads
// the same B_t and C_t (scalar loads) and u, delta, z, y are read/written as 64
// consecutive elements. The expanded (L x N) state lives only in registers.
// This kernel is the simple, always-applicable path (any dim, any dstate <= 16, ragged
// channel tails); the tiled kernel covers the common shapes faster. The state starts at
// h0 when one is given, else at zero. With the conv prologue (CONV) u_t is
// silu(conv_b + conv_w * x) over a sliding window of the last 4 inputs kept in registers.
#include "ss_common.h"
#include "ss_kernels.h"

namespace ss {

template <int NS, typename T, bool GATE, bool ZOH, bool CONV>
__global__ __launch_bounds__(64) void fwd_seq_kernel(FwdArgs a) {
  const int64_t nblk_d = (a.dim + 63) / 64;
  const int64_t b = blockIdx.x / nblk_d;
  const int64_t d = (blockIdx.x % nblk_d) * 64 + threadIdx.x;
  const bool active = d < a.dim;
  const int64_t dd = active ? d : a.dim - 1;  // inactive lanes mirror the last channel
  const int ns = NS > 0 ? NS : a.dstate;
  const T* __restrict__ u = static_cast<const T*>(a.u);
  const T* __restrict__ dl = static_cast<const T*>(a.delta);
  const T* __restrict__ zz = static_cast<const T*>(a.z);
  const T* __restrict__ Bm = static_cast<const T*>(a.B);
  const T* __restrict__ Cm = static_cast<const T*>(a.C);

  float A2[16], h[16], iA[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    A2[n] = (n < ns) ? a.A[dd * ns + n] * kLog2e : 0.0f;
    if (ZOH) iA[n] = (n < ns) ? 1.0f / a.A[dd * ns + n] : 0.0f;
    h[n] = (n < ns && a.h0) ? a.h0[(b * a.dim + dd) * ns + n] : 0.0f;
  }
  const float bias = a.delta_bias ? a.delta_bias[dd] : 0.0f;
  const float Dd = a.D ? a.D[dd] : 0.0f;
  float w4[4], cb = 0.0f, xw0 = 0.0f, xw1 = 0.0f, xw2 = 0.0f;  // conv taps and window
  if (CONV) {
    conv_taps(a.conv_w, a.conv_b, a.kconv, dd, w4, cb);
    xw0 = conv_input(u, a.conv_state, a.kconv, b, dd, -3, a.seqlen, a.dim);
    xw1 = conv_input(u, a.conv_state, a.kconv, b, dd, -2, a.seqlen, a.dim);
    xw2 = conv_input(u, a.conv_state, a.kconv, b, dd, -1, a.seqlen, a.dim);
  }

  for (int64_t t = 0; t < a.seqlen; ++t) {
    const int64_t e = (b * a.seqlen + t) * a.dim + dd;
    const int64_t r = (b * a.seqlen + t) * ns;
    const float x = load_elem(dl, e) + bias;
    const float dt = a.softplus ? softplus(x) : x;
    float uv = load_elem(u, e);
    if (CONV) {
      const float xt = uv;
      uv = conv4_silu(w4, cb, xw0, xw1, xw2, xt);
      xw0 = xw1;
      xw1 = xw2;
      xw2 = xt;
      if (a.u_out && active) a.u_out[e] = uv;
    }
    const float du = dt * uv;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      if (n < ns) {
        const float x2 = dt * A2[n];
        const float ab = fast_exp2(x2);
        const float bu = ZOH ? zoh_coef(dt, x2 * kLn2, ab, iA[n]) * uv : du;
        h[n] = __builtin_fmaf(ab, h[n], bu * load_elem(Bm, r + n));
        acc = __builtin_fmaf(load_elem(Cm, r + n), h[n], acc);
      }
    }
    float yv = __builtin_fmaf(Dd, uv, acc);
    if (GATE) yv *= silu(load_elem(zz, e));
    if (active) a.y[e] = yv;
  }
  if (a.last_state && active) {
#pragma unroll
    for (int n = 0; n < 16; ++n)
      if (n < ns) a.last_state[(b * a.dim + d) * ns + n] = h[n];
  }
}

template <int NS, typename T, bool GATE, bool ZOH>
static void launch_seq_c(const FwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch * ((a.dim + 63) / 64)));
  if (a.kconv > 0)
    hipLaunchKernelGGL((fwd_seq_kernel<NS, T, GATE, ZOH, true>), grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_seq_kernel<NS, T, GATE, ZOH, false>), grid, dim3(64), 0, s, a);
}

template <int NS, typename T, bool GATE>
static hipError_t launch_seq(const FwdArgs& a, hipStream_t s) {
  if (a.zoh)
    launch_seq_c<NS, T, GATE, true>(a, s);
  else
    launch_seq_c<NS, T, GATE, false>(a, s);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_seq_t(const FwdArgs& a, hipStream_t s) {
  const bool g = a.z != nullptr;
  switch (a.dstate) {
    case 16: return g ? launch_seq<16, T, true>(a, s) : launch_seq<16, T, false>(a, s);
    case 8: return g ? launch_seq<8, T, true>(a, s) : launch_seq<8, T, false>(a, s);
    case 4: return g ? launch_seq<4, T, true>(a, s) : launch_seq<4, T, false>(a, s);
    default: return g ? launch_seq<0, T, true>(a, s) : launch_seq<0, T, false>(a, s);
  }
}

hipError_t fwd_seq(const FwdArgs& a, hipStream_t s) {
  return a.dtype == kBF16 ? launch_seq_t<uint16_t>(a, s) : launch_seq_t<float>(a, s);
}

}  // namespace ss
