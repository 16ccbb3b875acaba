// ss_fwd_state.hip -- state-parallel selective-scan forward (gfx950), any dstate <= 16.
// The default for dstate != 16 (at dstate 16 the time-chunked kernel is faster: this one
// spends a workgroup barrier, an LDS transpose of B/C and one of the outputs per 16 tokens,
// which costs more than the chunked kernel's fix-up; measured 208 us vs 174 us at the
// 130M shape).
//
// The same recurrence as the other forward kernels ("Mamba：选择性状态空间模型入门教程",
// section "Mamba 的关键创新：选择性机制"; "架构变体：Mamba/SSM", section "离散化"), with
// the parallelism taken from the states instead of from time:
//
//  * A workgroup (4 waves) owns 16 consecutive channels of one batch row. Row r of 16 lanes
//    is channel c0+r and lane n of the row is state n: every lane runs one (channel, state)
//    recurrence h_t = abar_t h_{t-1} + dt_t B_t[n] u_t sequentially over the whole sequence,
//    so there is no chunk carry, no combine and no fix-up.
//  * Time advances in blocks of 16 tokens. The per-token work of a block (softplus of the
//    step, dt*u, the gate, D*u) is spread over the row: lane n computes it for token n of
//    the block. The update of token j then reads dt_j and dt_j*u_j from lane j through DPP
//    row_newbcast:j folded into the multiplies that consume them, so each state update is
//    v_mul_dpp (dt*A), v_exp, v_mul_dpp (dt*u*B), v_fma (state), v_mul (C*h): 4 VALU ops
//    and one transcendental.
//  * y_t = sum_n C_t[n] h_t[n] is a sum across the 16 lanes of a row. Each lane writes its
//    16 products of the block to LDS and lane j sums the 16 products of token j (a
//    transpose through LDS, inside one wave: no workgroup barrier).
//  * B and C of a block (16 tokens x 16 states, shared by the 16 channels) are loaded once
//    per workgroup, one element per thread, and staged transposed in LDS so lane n reads
//    its 16 values B_t[n], C_t[n] with four 16-byte reads each; the next block's inputs
//    are requested before the current block is computed (double-buffered LDS, one
//    workgroup barrier per block).
// dstate < 16 leaves lanes n >= dstate with A = B = C = 0, a state that stays zero.
#include "ss_chunk_ops.h"

namespace ss {
namespace {

using chunk::ldf;
using chunk::rsrc;

constexpr int kRowStride = 16 * 16 + 16;  // LDS [row][token][lane], padded

#define SS_DPP_ROW_S(j) " row_newbcast:" #j " row_mask:0xf bank_mask:0xf\n"

// One token of the block for this lane's state: x = dt_j A2; abar = 2^x; h = abar h +
// (du_j) B_j; p_j = C_j h. dt_j and du_j come from lane j (row_newbcast:j). Pipelined two
// tokens deep so each exp result is consumed >= 2 instructions after it is produced; every
// register a DPP instruction reads is written before the block (the s_nop covers the last
// writes before it), which meets the DPP read-after-write wait states.
#define SS_ST(j, j2, E)                                                         \
  "v_mul_f32_dpp %[bu], %[vdu], %[b" #j "]" SS_DPP_ROW_S(j)                     \
  "v_fma_f32 %[h], %[e" #E "], %[h], %[bu]\n"                                   \
  "v_mul_f32_dpp %[x], %[vdt], %[a2]" SS_DPP_ROW_S(j2)                          \
  "v_exp_f32 %[e" #E "], %[x]\n"                                                \
  "v_mul_f32 %[p" #j "], %[c" #j "], %[h]\n"
#define SS_ST_LAST(j, E)                                                        \
  "v_mul_f32_dpp %[bu], %[vdu], %[b" #j "]" SS_DPP_ROW_S(j)                     \
  "v_fma_f32 %[h], %[e" #E "], %[h], %[bu]\n"                                   \
  "v_mul_f32 %[p" #j "], %[c" #j "], %[h]\n"

// Token j's decay lives in e0 (j even) or e1 (j odd); the exp of token j+2 overwrites it
// right after token j's state update has read it.
__device__ __forceinline__ void state_block(float& h, float a2, float vdt, float vdu, const float (&b)[16],
                                            const float (&c)[16], float (&p)[16]) {
  float x, bu, ea, eb;
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32_dpp %[x], %[vdt], %[a2]" SS_DPP_ROW_S(0)
      "v_exp_f32 %[e0], %[x]\n"
      "v_mul_f32_dpp %[x], %[vdt], %[a2]" SS_DPP_ROW_S(1)
      "v_exp_f32 %[e1], %[x]\n"
      SS_ST(0, 2, 0) SS_ST(1, 3, 1) SS_ST(2, 4, 0) SS_ST(3, 5, 1) SS_ST(4, 6, 0) SS_ST(5, 7, 1)
      SS_ST(6, 8, 0) SS_ST(7, 9, 1) SS_ST(8, 10, 0) SS_ST(9, 11, 1) SS_ST(10, 12, 0) SS_ST(11, 13, 1)
      SS_ST(12, 14, 0) SS_ST(13, 15, 1) SS_ST_LAST(14, 0) SS_ST_LAST(15, 1)
      : [h] "+v"(h), [x] "=&v"(x), [bu] "=&v"(bu), [e0] "=&v"(ea), [e1] "=&v"(eb), SS_OPS16(p, "=&v")
      : [a2] "v"(a2), [vdt] "v"(vdt), [vdu] "v"(vdu), SS_OPS16(b, "v"), SS_OPS16(c, "v"));
}
#undef SS_ST
#undef SS_ST_LAST

// Per-lane inputs of one 16-token block: token n's raw step, u and z (for this lane's
// channel), and this thread's share of the block's B and C (one element of each).
struct StateIn {
  float raw, uu, zz, bsh, csh;
};

constexpr int kBcStride = 16 + 4;  // LDS [n][token] rows of B and C, padded

template <typename T, bool GATE>
__global__ __launch_bounds__(256) void fwd_state_kernel(FwdArgs a) {
  __shared__ float lds_p[16 * kRowStride];            // [row][token][lane]: y reduction
  __shared__ float lds_bc[2][2][16 * kBcStride];      // [buffer][B or C][n][token]

  const int64_t ngd = (a.dim + 15) / 16;
  const int64_t g = chunk::group_of(blockIdx.x, a.batch * ngd);
  const int64_t b = g / ngd;
  const int64_t c0 = (g % ngd) * 16;
  const int tid = threadIdx.x;
  const int n = tid & 15;   // state of this lane; token n of a block for per-token work
  const int r = tid >> 4;   // channel row
  const int64_t c = c0 + r;
  const bool cvalid = c < a.dim;
  const int64_t cc = cvalid ? c : a.dim - 1;
  const int64_t L = a.seqlen, N = a.dstate;
  const bool sv = n < N;

  const float a2 = sv ? a.A[cc * N + n] * kLog2e : 0.0f;
  const float bias = a.delta_bias ? a.delta_bias[cc] : 0.0f;
  const float Dd = a.D ? a.D[cc] : 0.0f;
  float h = (a.h0 && sv) ? a.h0[(b * a.dim + cc) * N + n] : 0.0f;

  const uint32_t tok_row = static_cast<uint32_t>(a.dim * sizeof(T));
  const T* U = static_cast<const T*>(a.u);
  const T* DL = static_cast<const T*>(a.delta);
  const T* Z = static_cast<const T*>(a.z);
  const T* Bm = static_cast<const T*>(a.B);
  const T* Cm = static_cast<const T*>(a.C);
  T* tag = nullptr;
  // thread tid loads element (token tid / 16, state tid % 16) of a block's B and C
  const int bt = tid >> 4, bn = tid & 15;
  const uint32_t bc_off = bn < N ? static_cast<uint32_t>((bt * N + bn) * sizeof(T)) : 0x7fffffffu;

  auto load = [&](StateIn& x, int64_t t0) {
    const int64_t last = L - 1 - t0;  // tokens past the end re-read the last token
    const int64_t tn = min(static_cast<int64_t>(n), last);
    const int64_t e0 = (b * L + t0) * a.dim;
    const int64_t left = (a.batch * L * a.dim - e0) * static_cast<int64_t>(sizeof(T));
    // (rows past the last channel read the last channel: computed, never stored)
    const uint32_t off = static_cast<uint32_t>(tn) * tok_row + static_cast<uint32_t>(cc * sizeof(T));
    x.raw = ldf(tag, rsrc(DL + e0, left), off, 0);
    x.uu = ldf(tag, rsrc(U + e0, left), off, 0);
    x.zz = GATE ? ldf(tag, rsrc(Z + e0, left), off, 0) : 0.0f;
    // B and C rows of the block: tokens past the end read 0 (their step is 0 anyway)
    const int64_t bc0 = (b * L + t0) * N;
    const int64_t valid_bytes = min(static_cast<int64_t>(16), L - t0) * N * static_cast<int64_t>(sizeof(T));
    x.bsh = ldf(tag, rsrc(Bm + bc0, valid_bytes), bc_off, 0);
    x.csh = ldf(tag, rsrc(Cm + bc0, valid_bytes), bc_off, 0);
  };
  auto stage = [&](const StateIn& x, int buf) {  // transpose the block's B, C into LDS
    lds_bc[buf][0][bn * kBcStride + bt] = x.bsh;
    lds_bc[buf][1][bn * kBcStride + bt] = x.csh;
  };

  float* lp = lds_p + r * kRowStride;
  StateIn cur, nxt;
  load(cur, 0);
  stage(cur, 0);
  __syncthreads();
  int buf = 0;
  for (int64_t t0 = 0; t0 < L; t0 += 16, buf ^= 1) {
    progress_priority(t0, L);
    const bool more = t0 + 16 < L;
    if (more) load(nxt, t0 + 16);
    // per-token work for token t0 + n (a zero step past the end is the identity)
    const bool tv = t0 + n < L;
    const float xr = cur.raw + bias;
    float dt = a.softplus ? softplus(xr) : xr;
    dt = tv ? dt : 0.0f;
    const float du = dt * cur.uu;
    const float gate = GATE ? silu(cur.zz) : 1.0f;
    const float du_skip = Dd * cur.uu;
    // B_t[n], C_t[n] of the block's 16 tokens for this lane's state n
    float bv[16], cv[16];
    {
      const float4* qb = reinterpret_cast<const float4*>(&lds_bc[buf][0][n * kBcStride]);
      const float4* qc = reinterpret_cast<const float4*>(&lds_bc[buf][1][n * kBcStride]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 vb = qb[m], vc = qc[m];
        bv[4 * m] = vb.x; bv[4 * m + 1] = vb.y; bv[4 * m + 2] = vb.z; bv[4 * m + 3] = vb.w;
        cv[4 * m] = vc.x; cv[4 * m + 1] = vc.y; cv[4 * m + 2] = vc.z; cv[4 * m + 3] = vc.w;
      }
    }

    float p[16];
    state_block(h, a2, dt, du, bv, cv, p);

    // y of token t0 + j is the sum over the row's lanes of p[j]: lane j sums it
#pragma unroll
    for (int j = 0; j < 16; ++j) lp[j * 16 + n] = p[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    float s0 = 0.0f, s1 = 0.0f;
    const float4* q = reinterpret_cast<const float4*>(lp + n * 16);
#pragma unroll
    for (int m = 0; m < 4; m += 2) {
      const float4 v0 = q[m], v1 = q[m + 1];
      s0 += (v0.x + v0.y) + (v0.z + v0.w);
      s1 += (v1.x + v1.y) + (v1.z + v1.w);
    }
    if (tv && cvalid) a.y[(b * L + t0 + n) * a.dim + c] = ((s0 + s1) + du_skip) * gate;
    if (more) stage(nxt, buf ^ 1);
    // one barrier per block: the next block's B, C are staged, and every wave is done
    // with this block's buffer (rewritten two blocks later) and its y-reduction rows
    __syncthreads();
    cur = nxt;
  }
  if (a.last_state && cvalid && sv) a.last_state[(b * a.dim + c) * N + n] = h;
}

template <typename T>
hipError_t launch_state_t(const FwdArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch * ((a.dim + 15) / 16)));
  if (a.z)
    hipLaunchKernelGGL((fwd_state_kernel<T, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_state_kernel<T, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool fwd_state_supported(const FwdArgs& a) { return a.dstate <= 16 && !a.zoh && a.kconv == 0 && a.seqlen > 0; }

hipError_t fwd_state(const FwdArgs& a, hipStream_t s) {
  return a.dtype == kBF16 ? launch_state_t<uint16_t>(a, s) : launch_state_t<float>(a, s);
}

}  // namespace ss
