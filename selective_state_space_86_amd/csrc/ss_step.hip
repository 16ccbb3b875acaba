// ss_step.hip -- one decode step of the selective scan, state carried in place.
// (Input term dt*B, or the exact zero-order hold (abar - 1)/A * B when StepArgs::zoh is set.)
//
// Recurrent inference with a fixed-size state and constant work per token
// ("Mamba：选择性状态空间模型入门教程", table "Mamba vs Transformer vs RNN", and the step
// function (input, state) -> (output, new state) of "Mamba架构深度解析", section
// "Mamba的创新：选择性状态空间模型"). The update itself is the ss_fwd update for one t.
//
// dstate == 16 (the common case) runs step_quad_kernel, four lanes per channel (below).
// Otherwise one lane per (b, d): the state row of a lane is contiguous, read and written
// with 16-byte vector accesses when aligned; when a wave never straddles two batch rows
// (dim a multiple of 64) B_t and C_t are wave-uniform and come in through scalar loads.
// The step is bound by the state traffic (128 B per channel per token); the fp32 state
// never leaves HBM between steps.
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

// dstate == 16: four lanes per channel, lane q of a quad holding states 4q..4q+3. Every
// state, A and B/C access is then one 16-byte vector per lane with consecutive lanes on
// consecutive 16-byte pieces, so a wave moves 1 KiB of state per instruction (in-place
// read+write of the 84 MB state measured 5.6 TB/s this way against 4.8 TB/s with 64 bytes
// per lane). y is the quad's sum, formed by two DPP quad permutes.
template <typename T>
struct Vec4In;
template <>
struct Vec4In<float> {
  static __device__ __forceinline__ float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
};
template <>
struct Vec4In<uint16_t> {
  static __device__ __forceinline__ float4 load(const uint16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  }
};

// The state is read once and written once per step and not touched again until the next
// step: its loads and stores carry the non-temporal hint. At 256 x 5120 x 16 (84 MB) the
// step took 35.0 us with it against 39.9 us without (hinting only the stores changed
// nothing).
typedef float nt4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt(const float4* p) {
  const nt4_t v = __builtin_nontemporal_load(reinterpret_cast<const nt4_t*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(float4* p, float4 v) {
  nt4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nt4_t*>(p));
}

template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <typename T, bool GATE, bool ZOH>
__device__ __forceinline__ void step_quad_channel(const StepArgs& a, int64_t j, int64_t b, int64_t d, int q,
                                                  const float4 hv, const float4 av, const float4 bv,
                                                  const float4 cv, float x, float uv, float zv, float4* st) {
  const float dt = a.softplus ? softplus(x) : x;
  const float du = dt * uv;
  float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float an[4] = {av.x, av.y, av.z, av.w}, bn[4] = {bv.x, bv.y, bv.z, bv.w},
              cn[4] = {cv.x, cv.y, cv.z, cv.w};
  float acc = 0.0f;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float x2 = dt * (an[n] * kLog2e);
    const float ab = fast_exp2(x2);
    const float bu = ZOH ? zoh_coef(dt, x2 * kLn2, ab, 1.0f / an[n]) * uv : du;
    h[n] = __builtin_fmaf(ab, h[n], bu * bn[n]);
    acc = __builtin_fmaf(cn[n], h[n], acc);
  }
  acc += quad_perm<0xB1>(acc);  // quad_perm [1,0,3,2]
  acc += quad_perm<0x4E>(acc);  // quad_perm [2,3,0,1]
  st_nt(st, make_float4(h[0], h[1], h[2], h[3]));
  if (q == 0) {
    float yv = __builtin_fmaf(a.D ? a.D[d] : 0.0f, uv, acc);
    if (GATE) yv *= silu(zv);
    a.y[j] = yv;
  }
}

// A workgroup covers 64 consecutive channels d of RB batch rows (ROWS) or, in general,
// 64 * RB consecutive (b, d) pairs. Lane (quad p, quarter q) handles quarter q of RB
// channels, all of whose loads are issued before any arithmetic. In the ROWS layout the RB
// channels are the same d in RB batch rows, so the lane reads its 16 bytes of A once for
// all of them (A is shared by the batch; read per (b, d) it would move as many bytes as
// the state).
template <typename T, bool GATE, bool ZOH, bool ROWS, int RB>
__global__ __launch_bounds__(256) void step_quad_kernel(StepArgs a) {
  const int q = threadIdx.x & 3;
  const int p = threadIdx.x >> 2;
  const int64_t total = a.batch * a.dim;
  float4 hv[RB], av[RB], bv[RB], cv[RB];
  float xv[RB], uv[RB], zv[RB];
  int64_t jj[RB], bb[RB], dd[RB];
  if (ROWS) {
    const int64_t ngd = a.dim / 64;
    const int64_t d = (blockIdx.x % ngd) * 64 + p;
    const int64_t b0 = (blockIdx.x / ngd) * RB;
    const float4 a4 = reinterpret_cast<const float4*>(a.A)[d * 4 + q];
    const float bias = a.delta_bias ? a.delta_bias[d] : 0.0f;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t b = b0 + r, j = b * a.dim + d;
      jj[r] = j;
      bb[r] = b;
      dd[r] = d;
      hv[r] = ld_nt(reinterpret_cast<const float4*>(a.state) + j * 4 + q);
      av[r] = a4;
      bv[r] = Vec4In<T>::load(static_cast<const T*>(a.B) + b * 16 + 4 * q);
      cv[r] = Vec4In<T>::load(static_cast<const T*>(a.C) + b * 16 + 4 * q);
      xv[r] = load_elem(static_cast<const T*>(a.delta), j) + bias;
      uv[r] = load_elem(static_cast<const T*>(a.u), j);
      zv[r] = GATE ? load_elem(static_cast<const T*>(a.z), j) : 0.0f;
    }
  } else {
    const int64_t c0 = static_cast<int64_t>(blockIdx.x) * (64 * RB);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int64_t j = c0 + p + 64 * r;
      const int64_t jc = j < total ? j : total - 1;  // whole quads agree
      const int64_t b = jc / a.dim;
      const int64_t d = jc - b * a.dim;
      jj[r] = j;
      bb[r] = b;
      dd[r] = d;
      hv[r] = ld_nt(reinterpret_cast<const float4*>(a.state) + jc * 4 + q);
      av[r] = reinterpret_cast<const float4*>(a.A)[d * 4 + q];
      bv[r] = Vec4In<T>::load(static_cast<const T*>(a.B) + b * 16 + 4 * q);
      cv[r] = Vec4In<T>::load(static_cast<const T*>(a.C) + b * 16 + 4 * q);
      xv[r] = load_elem(static_cast<const T*>(a.delta), jc) + (a.delta_bias ? a.delta_bias[d] : 0.0f);
      uv[r] = load_elem(static_cast<const T*>(a.u), jc);
      zv[r] = GATE ? load_elem(static_cast<const T*>(a.z), jc) : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    if (jj[r] < total)
      step_quad_channel<T, GATE, ZOH>(a, jj[r], bb[r], dd[r], q, hv[r], av[r], bv[r], cv[r], xv[r], uv[r],
                                      zv[r], reinterpret_cast<float4*>(a.state) + jj[r] * 4 + q);
  }
}

template <typename T, bool GATE, bool ZOH>
static void launch_step_quad_z(const StepArgs& a, hipStream_t s) {
  constexpr int RB = 2;  // 256 x 5120 x 16: 34.2 us per step; 1 row 37.1, 4 rows 35.0, 8 rows 38.9
  const unsigned grid = static_cast<unsigned>((a.batch * a.dim + 64 * RB - 1) / (64 * RB));
  if (a.dim % 64 == 0 && a.batch % RB == 0)
    hipLaunchKernelGGL((step_quad_kernel<T, GATE, ZOH, true, RB>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((step_quad_kernel<T, GATE, ZOH, false, RB>), dim3(grid), dim3(256), 0, s, a);
}

template <typename T, bool GATE>
static hipError_t launch_step_quad(const StepArgs& a, hipStream_t s) {
  if (a.zoh)
    launch_step_quad_z<T, GATE, true>(a, s);
  else
    launch_step_quad_z<T, GATE, false>(a, s);
  return hipGetLastError();
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
  auto al = [](const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; };
  if (a.dstate == 16 && al(a.state, 16) && al(a.A, 16) && al(a.B, 4 * sizeof(T)) && al(a.C, 4 * sizeof(T)) &&
      a.batch * a.dim <= (int64_t(1) << 29))
    return launch_step_quad<T, GATE>(a, s);
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
