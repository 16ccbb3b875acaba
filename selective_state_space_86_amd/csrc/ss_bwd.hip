// ss_bwd.hip -- backward of the selective scan (gfx950): gradients of a loss L with respect
// to u, delta, A, B, C, D, z, delta_bias and h0, given dL/dy and optionally dL/dlast_state.
//
// For one channel, with lam_t[n] = dL/dh_t[n] and mu_t[n] = abar_t[n] lam_t[n] (what token t
// passes back to h_{t-1}), the chain rule of the forward recurrence gives
//   ds_t = dy_t silu(z_t),  dz_t = dy_t s_t silu'(z_t),  s_t = C_t . h_t + D u_t
//   lam_t[n] = ds_t C_t[n] + mu_{t+1}[n],  mu_L = dL/dlast_state,  dh0 = mu_0
//   dB_t[n] += lam_t[n] dt_t u_t,  dC_t[n] += ds_t h_t[n]       (summed over channels)
//   du_t = ds_t D + dt_t sum_n lam_t[n] B_t[n]
//   ddt_t = u_t sum_n lam_t[n] B_t[n] + sum_n A[n] lam_t[n] abar_t[n] h_{t-1}[n]
//   dA[n] += dt_t lam_t[n] abar_t[n] h_{t-1}[n]                  (summed over batch and t)
//   ddelta_t = ddt_t sigmoid(delta_t + bias) with softplus, dbias += ddelta_t, dD += ds_t u_t
// and abar_t h_{t-1} = h_t - dt_t B_t u_t, so only the states h_t themselves are needed.
// The reverse recurrence mu_t = abar_t (ds_t C_t + mu_{t+1}) is linear with the same
// decays as the forward one, so it is chunked the same way (an associative fold of chunk
// aggregates, run from the end of the sequence).
//
// Following "Mamba：选择性状态空间的线性时间序列建模" (section "第二个创新：硬件感知算法":
// the backward recomputes the expanded states instead of reading them from HBM), nothing
// of size (batch, L, dim, N) is stored:
//   1. bwd_ckpt_kernel runs the forward scan keeping only the state at the start of every
//      tile of 16*TC tokens (workspace, 4*16/(16*TC) bytes per (b, t, d)).
//   2. bwd_chunked_kernel walks the tiles from last to first. Per tile it recomputes the
//      states from the checkpoint (local pass, chunk fold, true recurrence kept in
//      registers), then runs the adjoint: local reverse pass, reverse fold, and the true
//      reverse recurrence that forms every gradient term. dB_t and dC_t (shared by the
//      16 channels of the workgroup) are summed over the 16 lanes of a row through LDS and
//      written as per-group partials; dA, dD, dbias are summed over the rows at the end.
//   3. bwd_reduce_kernel adds the partials over channel groups (dB, dC) and batch rows
//      (dA, dD, dbias). Every sum has a fixed order: results are deterministic.
// Lane layout as in the forward: lane i of a row of 16 is channel c0+i, the 16 rows are 16
// consecutive chunks of TC tokens, and lane n of a row holds B_t[n], C_t[n], broadcast to
// the row by DPP row_newbcast:n. dstate < 16 is padded: lanes n >= dstate read B = C = 0
// and A = 0, which keeps those states at zero and their adjoint at zero.
#include <utility>

#include "ss_common.h"
#include "ss_kernels.h"

namespace ss {
namespace {

constexpr int kS = 16 * 16 + 16;  // LDS [chunk or row][n][lane] stride, padded against bank conflicts

template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + N, 0xf, 0xf, false));
}

template <typename F, int... Ns>
__device__ __forceinline__ void unroll16_impl(F&& f, std::integer_sequence<int, Ns...>) {
  (f(std::integral_constant<int, Ns>{}), ...);
}
// f(std::integral_constant<int, n>) for n = 0..15 (compile-time n for the DPP broadcasts)
template <typename F>
__device__ __forceinline__ void unroll16(F&& f) {
  unroll16_impl(f, std::make_integer_sequence<int, 16>{});
}

__device__ __forceinline__ float sigmoid(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }

// exp(x) - 1 for the decay of a whole chunk, x = A * (sum of its steps) (x2 = x * log2 e):
// a short series for |x| < 1/16 (truncation < 1.3e-9 relative), the hardware exp above.
// Folding chunks as carry + em1 * carry never rounds the factor exp(x) itself: v_exp_f32
// returns values just below 1 about 0.13 ulp low on average, which over thousands of
// slowly decaying steps would bias the carried state and adjoint by ~1e-5 relative and
// more, while the series' error is random and far smaller.
__device__ __forceinline__ float chunk_em1(float x2) {
  const float x = x2 * kLn2;
  const float p = __builtin_fmaf(
      x, __builtin_fmaf(x, __builtin_fmaf(x, __builtin_fmaf(x, 1.0f / 120.0f, 1.0f / 24.0f), 1.0f / 6.0f), 0.5f),
      1.0f);
  return __builtin_fabsf(x) < 0.0625f ? x * p : fast_exp2(x2) - 1.0f;
}

template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i) {
  return load_elem(static_cast<const T*>(p), i);
}

struct Lane {
  int64_t b, c0, c, cc;
  int k, i;
  bool cvalid;
};

__device__ __forceinline__ Lane lane_of(const BwdArgs& a) {
  Lane l;
  const int64_t g = blockIdx.x;
  l.b = g / a.ngroups;
  l.c0 = (g % a.ngroups) * 16;
  l.i = threadIdx.x & 15;
  l.k = threadIdx.x >> 4;
  l.c = l.c0 + l.i;
  l.cvalid = l.c < a.dim;
  l.cc = l.cvalid ? l.c : a.dim - 1;
  return l;
}

// Forward scan from h0 (or zero), storing the state at the start of every tile:
// ckpt[((b * ntiles + tile) * dimp + c) * 16 + n].
template <typename T, int TC>
__global__ __launch_bounds__(256) void bwd_ckpt_kernel(BwdArgs a) {
  __shared__ float lds_p[16 * kS];
  __shared__ float lds_h[16 * kS];
  const Lane l = lane_of(a);
  const int64_t L = a.seqlen, N = a.dstate, dimp = a.ngroups * 16;
  constexpr int TT = 16 * TC;
  float A2[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) A2[n] = n < N ? a.A[l.cc * N + n] * kLog2e : 0.0f;
  const float bias = a.delta_bias ? a.delta_bias[l.cc] : 0.0f;
  float carry = (a.h0 && l.k < N) ? a.h0[(l.b * a.dim + l.cc) * N + l.k] : 0.0f;
  for (int64_t tile = 0; tile < a.ntiles; ++tile) {
    const int64_t t0 = tile * TT;
    a.ckpt[((l.b * a.ntiles + tile) * dimp + l.c) * 16 + l.k] = carry;
    if (tile == a.ntiles - 1) break;  // the state after the last tile is not needed
    float h[16], dsum = 0.0f;
#pragma unroll
    for (int n = 0; n < 16; ++n) h[n] = 0.0f;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const int64_t t = t0 + l.k * TC + j;  // full tile: every t < L
      const int64_t e = (l.b * L + t) * a.dim + l.cc;
      const float x = ld<T>(a.delta, e) + bias;
      const float dt = a.softplus ? softplus(x) : x;
      const float dtu = dt * ld<T>(a.u, e);
      const float vb = l.i < N ? ld<T>(a.B, (l.b * L + t) * N + l.i) : 0.0f;
      dsum += dt;
      unroll16([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        const float ab = fast_exp2(dt * A2[n]);
        h[n] = __builtin_fmaf(ab, h[n], dtu * row_bcast<n>(vb));
      });
    }
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      lds_p[l.k * kS + n * 16 + l.i] = chunk_em1(A2[n] * dsum);
      lds_h[l.k * kS + n * 16 + l.i] = h[n];
    }
    __syncthreads();
    // lane (k, i) owns state n = k of channel i: fold the 16 chunks in order
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int o = jj * kS + l.k * 16 + l.i;
      carry = __builtin_fmaf(lds_p[o], carry, carry + lds_h[o]);
    }
    __syncthreads();
  }
}

template <typename T, bool GATE, int TC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_chunked_kernel(BwdArgs a) {
  __shared__ float lds_p[16 * kS];       // chunk prod-abar, then chunk carries
  __shared__ float lds_v[16 * kS];       // chunk end values (state, then adjoint)
  __shared__ float lds_r[4][2][4 * kS];  // per wave: dB and dC terms [row][n][lane]
  const Lane l = lane_of(a);
  const int64_t L = a.seqlen, N = a.dstate, dimp = a.ngroups * 16;
  constexpr int TT = 16 * TC;
  const int w = threadIdx.x >> 6, rw = l.k & 3;

  float A2[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) A2[n] = n < N ? a.A[l.cc * N + n] * kLog2e : 0.0f;
  const float bias = a.delta_bias ? a.delta_bias[l.cc] : 0.0f;
  const float Dd = a.D ? a.D[l.cc] : 0.0f;
  // adjoint carried from later tiles: lane (k, i) owns state n = k of channel i
  float rcarry = (a.dlast && l.cvalid && l.k < N) ? a.dlast[(l.b * a.dim + l.c) * N + l.k] : 0.0f;
  float dAacc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) dAacc[n] = 0.0f;
  float dDacc = 0.0f, dbacc = 0.0f;

  for (int64_t tile = a.ntiles - 1; tile >= 0; --tile) {
    const int64_t t0 = tile * TT;
    // per-token inputs of this lane's chunk (tokens past the end: zero step, zero dy)
    float dt[TC], dtu[TC], uu[TC], ds[TC], sg[TC], vb[TC], vc[TC], dyv[TC], dsl[TC];
    bool ok[TC];
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const int64_t t = t0 + l.k * TC + j;
      const bool tv = t < L;
      ok[j] = tv && l.cvalid;
      const int64_t tt = tv ? t : L - 1;
      const int64_t e = (l.b * L + tt) * a.dim + l.cc;
      const float x = ld<T>(a.delta, e) + bias;
      dt[j] = tv ? (a.softplus ? softplus(x) : x) : 0.0f;
      sg[j] = a.softplus ? sigmoid(x) : 1.0f;
      uu[j] = ld<T>(a.u, e);
      dtu[j] = dt[j] * uu[j];
      dyv[j] = ok[j] ? a.dy[e] : 0.0f;
      float g = 1.0f;
      dsl[j] = 0.0f;
      if (GATE) {
        const float zv = ld<T>(a.z, e);
        const float s = fast_rcp(1.0f + fast_exp2(-zv * kLog2e));
        g = zv * s;
        dsl[j] = s * __builtin_fmaf(zv, 1.0f - s, 1.0f);
      }
      ds[j] = dyv[j] * g;
      vb[j] = l.i < N ? ld<T>(a.B, (l.b * L + tt) * N + l.i) : 0.0f;
      vc[j] = l.i < N ? ld<T>(a.C, (l.b * L + tt) * N + l.i) : 0.0f;
    }

    // forward local pass from a zero state: decays and chunk aggregates
    float ex[TC][16], h[16], dsum = 0.0f;
#pragma unroll
    for (int n = 0; n < 16; ++n) h[n] = 0.0f;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      dsum += dt[j];
      unroll16([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        ex[j][n] = fast_exp2(dt[j] * A2[n]);
        h[n] = __builtin_fmaf(ex[j][n], h[n], dtu[j] * row_bcast<n>(vb[j]));
      });
    }
    __syncthreads();  // the previous tile's readers of lds_p / lds_v are done
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      lds_p[l.k * kS + n * 16 + l.i] = chunk_em1(A2[n] * dsum);  // chunk decay - 1
      lds_v[l.k * kS + n * 16 + l.i] = h[n];
    }
    __syncthreads();
    {  // forward fold from the checkpoint; each lane overwrites exactly what it read
      float carry = a.ckpt[((l.b * a.ntiles + tile) * dimp + l.c) * 16 + l.k];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const int o = jj * kS + l.k * 16 + l.i;
        const float pm = lds_p[o], hv = lds_v[o];
        lds_p[o] = carry;
        lds_v[o] = pm;  // keep the chunk decay for the reverse fold
        carry = __builtin_fmaf(pm, carry, carry + hv);
      }
    }
    __syncthreads();
    float q[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) q[n] = lds_p[l.k * kS + n * 16 + l.i];

    // true states of the chunk, the pre-gate output s and dz
    float H[TC][16];
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      float s = Dd * uu[j];
      unroll16([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        q[n] = __builtin_fmaf(ex[j][n], q[n], dtu[j] * row_bcast<n>(vb[j]));
        H[j][n] = q[n];
        s = __builtin_fmaf(row_bcast<n>(vc[j]), q[n], s);
      });
      if (GATE && ok[j]) {
        const int64_t e = (l.b * L + t0 + l.k * TC + j) * a.dim + l.c;
        a.dz[e] = dyv[j] * s * dsl[j];
      }
    }

    // reverse local pass from a zero adjoint: the chunk aggregate mu_loc
    float mu[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) mu[n] = 0.0f;
#pragma unroll
    for (int j = TC - 1; j >= 0; --j) {
      unroll16([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        mu[n] = ex[j][n] * __builtin_fmaf(ds[j], row_bcast<n>(vc[j]), mu[n]);
      });
    }
    __syncthreads();  // every lane has read its forward carry-in
#pragma unroll
    for (int n = 0; n < 16; ++n) lds_p[l.k * kS + n * 16 + l.i] = mu[n];
    __syncthreads();
    {  // reverse fold, from the last chunk to the first (lds_v still holds the chunk decays)
#pragma unroll
      for (int jj = 15; jj >= 0; --jj) {
        const int o = jj * kS + l.k * 16 + l.i;
        const float pm = lds_v[o], mv = lds_p[o];
        lds_p[o] = rcarry;  // adjoint entering chunk jj from its end
        rcarry = __builtin_fmaf(pm, rcarry, rcarry + mv);
      }
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 16; ++n) mu[n] = lds_p[l.k * kS + n * 16 + l.i];

    // true reverse recurrence and the gradient terms, token by token from the chunk end
    float* rB = &lds_r[w][0][rw * kS];
    float* rC = &lds_r[w][1][rw * kS];
#pragma unroll
    for (int j = TC - 1; j >= 0; --j) {
      float sb = 0.0f, ga = 0.0f;
      unroll16([&](auto nc) {
        constexpr int n = decltype(nc)::value;
        const float cn = row_bcast<n>(vc[j]);
        const float bn = row_bcast<n>(vb[j]);
        const float lam = __builtin_fmaf(ds[j], cn, mu[n]);
        const float g = lam * (H[j][n] - dtu[j] * bn);  // lam * abar_t h_{t-1}
        dAacc[n] = __builtin_fmaf(dt[j], g, dAacc[n]);
        ga = __builtin_fmaf(A2[n], g, ga);
        sb = __builtin_fmaf(lam, bn, sb);
        rB[n * 16 + l.i] = lam * dtu[j];
        rC[n * 16 + l.i] = ds[j] * H[j][n];
        mu[n] = ex[j][n] * lam;
      });
      const int64_t t = t0 + l.k * TC + j;
      if (ok[j]) {
        const int64_t e = (l.b * L + t) * a.dim + l.c;
        const float ddt = __builtin_fmaf(uu[j], sb, ga * kLn2);
        const float dd = ddt * sg[j];
        a.du[e] = __builtin_fmaf(ds[j], Dd, dt[j] * sb);
        a.ddelta[e] = dd;
        dbacc += dd;
        dDacc = __builtin_fmaf(ds[j], uu[j], dDacc);
      }
      // sum the 16 channels of this row: lane i takes state n = i
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      float sB = 0.0f, sC = 0.0f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        sB += rB[l.i * 16 + m];
        sC += rC[l.i * 16 + m];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (t < L && l.i < N) {
        const int64_t o = ((l.b * a.ngroups + (l.c0 >> 4)) * L + t) * N + l.i;
        a.part_bc[o] = sB;
        a.part_bc[a.batch * a.ngroups * L * N + o] = sC;
      }
    }
  }
  if (a.dh0 && l.cvalid && l.k < N) a.dh0[(l.b * a.dim + l.c) * N + l.k] = rcarry;

  // dA, dD and dbias of this workgroup: sum the 16 rows
  __syncthreads();
#pragma unroll
  for (int n = 0; n < 16; ++n) lds_p[l.k * kS + n * 16 + l.i] = dAacc[n];
  lds_v[l.k * 16 + l.i] = dDacc;
  lds_v[256 + l.k * 16 + l.i] = dbacc;
  __syncthreads();
  {
    float s = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) s += lds_p[kk * kS + l.k * 16 + l.i];
    float* pc = a.part_ch + (l.b * dimp + l.c) * 18;
    if (l.k < N) pc[l.k] = s;
    if (l.k == 0 || l.k == 1) {
      float t = 0.0f;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) t += lds_v[l.k * 256 + kk * 16 + l.i];
      pc[16 + l.k] = t;
    }
  }
}

// dB, dC: sum over channel groups; dA, dD, dbias: sum over batch rows.
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs a) {
  const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nbc = a.batch * a.seqlen * a.dstate;
  const int64_t dimp = a.ngroups * 16;
  if (j < nbc) {
    const int64_t b = j / (a.seqlen * a.dstate), r = j % (a.seqlen * a.dstate);
    const int64_t plane = a.batch * a.ngroups * a.seqlen * a.dstate;
    float sb = 0.0f, sc = 0.0f;
    for (int64_t g = 0; g < a.ngroups; ++g) {
      const int64_t o = (b * a.ngroups + g) * a.seqlen * a.dstate + r;
      sb += a.part_bc[o];
      sc += a.part_bc[plane + o];
    }
    a.dB[j] = sb;
    a.dC[j] = sc;
  }
  const int64_t jc = j - nbc;
  if (jc >= 0 && jc < a.dim * (a.dstate + 2)) {
    const int64_t d = jc / (a.dstate + 2), q = jc % (a.dstate + 2);
    const int slot = q < a.dstate ? static_cast<int>(q) : static_cast<int>(16 + (q - a.dstate));
    float s = 0.0f;
    for (int64_t b = 0; b < a.batch; ++b) s += a.part_ch[(b * dimp + d) * 18 + slot];
    if (q < a.dstate) a.dA[d * a.dstate + q] = s;
    else if (q == a.dstate) { if (a.dD) a.dD[d] = s; }
    else if (a.dbias) a.dbias[d] = s;
  }
}

template <typename T, int TC>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch * a.ngroups));
  hipLaunchKernelGGL((bwd_ckpt_kernel<T, TC>), grid, dim3(256), 0, s, a);
  if (a.z)
    hipLaunchKernelGGL((bwd_chunked_kernel<T, true, TC>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_chunked_kernel<T, false, TC>), grid, dim3(256), 0, s, a);
  const int64_t total = a.batch * a.seqlen * a.dstate + a.dim * (a.dstate + 2);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_tile_tokens() { return 16 * kBwdChunk; }

size_t bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  const int64_t ngroups = (dim + 15) / 16, dimp = ngroups * 16;
  const int64_t ntiles = seqlen > 0 ? (seqlen + bwd_tile_tokens() - 1) / bwd_tile_tokens() : 0;
  const int64_t floats = batch * ntiles * dimp * 16              // tile-start states
                         + 2 * batch * ngroups * seqlen * dstate  // dB, dC per channel group
                         + batch * dimp * 18;                     // dA, dD, dbias per batch row
  return static_cast<size_t>(floats) * sizeof(float);
}

hipError_t bwd(const BwdArgs& a, hipStream_t s) {
  return a.dtype == kBF16 ? launch_bwd_t<uint16_t, kBwdChunk>(a, s) : launch_bwd_t<float, kBwdChunk>(a, s);
}

}  // namespace ss
