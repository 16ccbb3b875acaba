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
// and lam_t[n] abar_t[n] h_{t-1}[n] = mu_t[n] h_{t-1}[n]: the adjoint passed back times the
// state entering the token, which the reverse pass holds (the previous token's true state or
// the chunk's carry-in), so only the states h_t themselves are needed.
// The reverse recurrence mu_t = abar_t (ds_t C_t + mu_{t+1}) is linear with the same
// decays as the forward one, so it is chunked the same way (an associative fold of chunk
// aggregates, run from the end of the sequence).
//
// Following "Mamba：选择性状态空间的线性时间序列建模" (section "第二个创新：硬件感知算法":
// the backward recomputes the expanded states instead of reading them from HBM), nothing
// of size (batch, L, dim, N) is stored:
//   1. bwd_ckpt_kernel runs the forward scan keeping only the state at the start of every
//      32 tokens (workspace, 2 bytes per (b, t, d)).
//   2. bwd_chunked_kernel walks the tiles from last to first. Per tile it recomputes the
//      states from the checkpoint (local pass, chunk fold, true recurrence kept in
//      registers), then runs the adjoint: local reverse pass, reverse fold, and the true
//      reverse recurrence that forms every gradient term. dB_t and dC_t (shared by the
//      16 channels of the workgroup) are summed over the 16 lanes of a row through LDS and
//      written as per-group partials; dA, dD, dbias are summed over the rows at the end.
//   3. bwd_reduce_kernel adds the partials over channel groups (dB, dC) and batch rows
//      (dA, dD, dbias). Every sum has a fixed order: results are deterministic.
// Lane layout as in the forward: lane i of a row of 16 is channel c0+i, the 16 or 32 rows are
// consecutive chunks of TC tokens, and lane n of a row holds B_t[n], C_t[n], broadcast to
// the row by DPP row_newbcast:n. dstate < 16 is padded: lanes n >= dstate read B = C = 0
// and A = 0, which keeps those states at zero and their adjoint at zero.
#include <utility>

#include "ss_chunk_ops.h"
#include "ss_split.h"

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
// the series x + x^2/2 + x^3/6, evaluated in x2, for |x| < 1/64, the hardware exp above.
// Folding chunks as carry + em1 * carry never rounds the factor exp(x) itself: v_exp_f32
// returns values just below 1 about 0.13 ulp low on average, which over thousands of
// slowly decaying steps would bias the carried state and adjoint by ~1e-5 relative and
// more. Where the exp is used (|x| >= 1/64) a carried value decays by e^-1 within 64
// chunks, so its bias stays below ~5e-7 relative; the series' truncation, below
// x^3/24 < 1.6e-7 relative to em1, adds up to less than that over the slow decays.
// Cost: 6 VALU and an exp, without a branch: the exp is made opaque before the select, which
// the compiler otherwise turned into a branch around it (an exec-mask branch per state and
// chunk, both sides taken wherever the lanes disagree).
__device__ __forceinline__ float chunk_em1(float x2) {
  constexpr float c1 = kLn2, c2 = kLn2 * kLn2 / 2.0f, c3 = kLn2 * kLn2 * kLn2 / 6.0f;
  const float p = x2 * __builtin_fmaf(x2, __builtin_fmaf(x2, c3, c2), c1);
  float e = fast_exp2(x2);
  asm("" : "+v"(e));
  return __builtin_fabsf(x2) < kLog2e / 64.0f ? p : e - 1.0f;
}

// ---- hand-scheduled per-token blocks of the backward (16 states of one token) ----------
// Conventions as the forward's local_step: B_t[n] and C_t[n] are read from lane n of the
// row by DPP row_newbcast:n folded into the consuming instruction; every VGPR a DPP
// instruction reads is written >= 2 instructions earlier (or before the block, which
// starts with s_nop 1); every exp result is consumed >= 2 instructions later.

// Forward local pass of one token: e[n] = 2^(dt a2[n]); h[n] = e[n] h[n] + dtu B[n].
#define BW_L(n, n2)                                                           \
  "v_mul_f32_dpp %[t], %[vb], %[dtu]" SS_DPP_ROW(n)                           \
  "v_fma_f32 %[h" #n "], %[e" #n "], %[h" #n "], %[t]\n"                      \
  "v_mul_f32 %[x], %[dt], %[a" #n2 "]\n"                                      \
  "v_exp_f32 %[e" #n2 "], %[x]\n"
#define BW_L_END(n)                                                           \
  "v_mul_f32_dpp %[t], %[vb], %[dtu]" SS_DPP_ROW(n)                           \
  "v_fma_f32 %[h" #n "], %[e" #n "], %[h" #n "], %[t]\n"

__device__ __forceinline__ void bwd_local(float (&h)[16], float (&e)[16], const float (&a)[16], float dt,
                                          float dtu, float vb) {
  float x, t;
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32 %[x], %[dt], %[a0]\n"
      "v_exp_f32 %[e0], %[x]\n"
      "v_mul_f32 %[x], %[dt], %[a1]\n"
      "v_exp_f32 %[e1], %[x]\n"
      BW_L(0, 2) BW_L(1, 3) BW_L(2, 4) BW_L(3, 5) BW_L(4, 6) BW_L(5, 7) BW_L(6, 8) BW_L(7, 9)
      BW_L(8, 10) BW_L(9, 11) BW_L(10, 12) BW_L(11, 13) BW_L(12, 14) BW_L(13, 15)
      BW_L_END(14) BW_L_END(15)
      : SS_OPS16(h, "+v"), SS_OPS16(e, "=&v"), [x] "=&v"(x), [t] "=&v"(t)
      : SS_OPS16(a, "v"), [dt] "v"(dt), [dtu] "v"(dtu), [vb] "v"(vb));
}
#undef BW_L
#undef BW_L_END

// The reverse kernel's local pass over a chunk of two tokens, keeping each token's input
// terms bu[n] = dtu B[n] for the true-state pass (which then needs no multiply of its own).
// First token (state from zero): bu0 and e0, the state after it being bu0.
__device__ __forceinline__ void bwd_local_first_bu(float (&bu)[16], float (&e)[16], const float (&a)[16],
                                                   float dt, float dtu, float vb) {
  float x0, x1;
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32 %[x0], %[dt], %[a0]\n"
      "v_exp_f32 %[e0], %[x0]\n"
      "v_mul_f32_dpp %[bu0], %[vb], %[dtu]" SS_DPP_ROW(0)
      "v_mul_f32 %[x1], %[dt], %[a1]\n"
      "v_exp_f32 %[e1], %[x1]\n"
      "v_mul_f32_dpp %[bu1], %[vb], %[dtu]" SS_DPP_ROW(1)
      "v_mul_f32 %[x0], %[dt], %[a2]\n"
      "v_exp_f32 %[e2], %[x0]\n"
      "v_mul_f32_dpp %[bu2], %[vb], %[dtu]" SS_DPP_ROW(2)
      "v_mul_f32 %[x1], %[dt], %[a3]\n"
      "v_exp_f32 %[e3], %[x1]\n"
      "v_mul_f32_dpp %[bu3], %[vb], %[dtu]" SS_DPP_ROW(3)
      "v_mul_f32 %[x0], %[dt], %[a4]\n"
      "v_exp_f32 %[e4], %[x0]\n"
      "v_mul_f32_dpp %[bu4], %[vb], %[dtu]" SS_DPP_ROW(4)
      "v_mul_f32 %[x1], %[dt], %[a5]\n"
      "v_exp_f32 %[e5], %[x1]\n"
      "v_mul_f32_dpp %[bu5], %[vb], %[dtu]" SS_DPP_ROW(5)
      "v_mul_f32 %[x0], %[dt], %[a6]\n"
      "v_exp_f32 %[e6], %[x0]\n"
      "v_mul_f32_dpp %[bu6], %[vb], %[dtu]" SS_DPP_ROW(6)
      "v_mul_f32 %[x1], %[dt], %[a7]\n"
      "v_exp_f32 %[e7], %[x1]\n"
      "v_mul_f32_dpp %[bu7], %[vb], %[dtu]" SS_DPP_ROW(7)
      "v_mul_f32 %[x0], %[dt], %[a8]\n"
      "v_exp_f32 %[e8], %[x0]\n"
      "v_mul_f32_dpp %[bu8], %[vb], %[dtu]" SS_DPP_ROW(8)
      "v_mul_f32 %[x1], %[dt], %[a9]\n"
      "v_exp_f32 %[e9], %[x1]\n"
      "v_mul_f32_dpp %[bu9], %[vb], %[dtu]" SS_DPP_ROW(9)
      "v_mul_f32 %[x0], %[dt], %[a10]\n"
      "v_exp_f32 %[e10], %[x0]\n"
      "v_mul_f32_dpp %[bu10], %[vb], %[dtu]" SS_DPP_ROW(10)
      "v_mul_f32 %[x1], %[dt], %[a11]\n"
      "v_exp_f32 %[e11], %[x1]\n"
      "v_mul_f32_dpp %[bu11], %[vb], %[dtu]" SS_DPP_ROW(11)
      "v_mul_f32 %[x0], %[dt], %[a12]\n"
      "v_exp_f32 %[e12], %[x0]\n"
      "v_mul_f32_dpp %[bu12], %[vb], %[dtu]" SS_DPP_ROW(12)
      "v_mul_f32 %[x1], %[dt], %[a13]\n"
      "v_exp_f32 %[e13], %[x1]\n"
      "v_mul_f32_dpp %[bu13], %[vb], %[dtu]" SS_DPP_ROW(13)
      "v_mul_f32 %[x0], %[dt], %[a14]\n"
      "v_exp_f32 %[e14], %[x0]\n"
      "v_mul_f32_dpp %[bu14], %[vb], %[dtu]" SS_DPP_ROW(14)
      "v_mul_f32 %[x1], %[dt], %[a15]\n"
      "v_exp_f32 %[e15], %[x1]\n"
      "v_mul_f32_dpp %[bu15], %[vb], %[dtu]" SS_DPP_ROW(15)
      : SS_OPS16(bu, "=&v"), SS_OPS16(e, "=&v"), [x0] "=&v"(x0), [x1] "=&v"(x1)
      : SS_OPS16(a, "v"), [dt] "v"(dt), [dtu] "v"(dtu), [vb] "v"(vb));
}
// Second token from the state p after the first: bu, e and h[n] = e[n] p[n] + bu[n].
__device__ __forceinline__ void bwd_local_next_bu(float (&h)[16], float (&bu)[16], float (&e)[16],
                                                  const float (&p)[16], const float (&a)[16], float dt,
                                                  float dtu, float vb) {
  float x0, x1;
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32 %[x0], %[dt], %[a0]\n"
      "v_exp_f32 %[e0], %[x0]\n"
      "v_mul_f32 %[x1], %[dt], %[a1]\n"
      "v_exp_f32 %[e1], %[x1]\n"
      "v_mul_f32_dpp %[bu0], %[vb], %[dtu]" SS_DPP_ROW(0)
      "v_fma_f32 %[h0], %[e0], %[p0], %[bu0]\n"
      "v_mul_f32 %[x0], %[dt], %[a2]\n"
      "v_exp_f32 %[e2], %[x0]\n"
      "v_mul_f32_dpp %[bu1], %[vb], %[dtu]" SS_DPP_ROW(1)
      "v_fma_f32 %[h1], %[e1], %[p1], %[bu1]\n"
      "v_mul_f32 %[x1], %[dt], %[a3]\n"
      "v_exp_f32 %[e3], %[x1]\n"
      "v_mul_f32_dpp %[bu2], %[vb], %[dtu]" SS_DPP_ROW(2)
      "v_fma_f32 %[h2], %[e2], %[p2], %[bu2]\n"
      "v_mul_f32 %[x0], %[dt], %[a4]\n"
      "v_exp_f32 %[e4], %[x0]\n"
      "v_mul_f32_dpp %[bu3], %[vb], %[dtu]" SS_DPP_ROW(3)
      "v_fma_f32 %[h3], %[e3], %[p3], %[bu3]\n"
      "v_mul_f32 %[x1], %[dt], %[a5]\n"
      "v_exp_f32 %[e5], %[x1]\n"
      "v_mul_f32_dpp %[bu4], %[vb], %[dtu]" SS_DPP_ROW(4)
      "v_fma_f32 %[h4], %[e4], %[p4], %[bu4]\n"
      "v_mul_f32 %[x0], %[dt], %[a6]\n"
      "v_exp_f32 %[e6], %[x0]\n"
      "v_mul_f32_dpp %[bu5], %[vb], %[dtu]" SS_DPP_ROW(5)
      "v_fma_f32 %[h5], %[e5], %[p5], %[bu5]\n"
      "v_mul_f32 %[x1], %[dt], %[a7]\n"
      "v_exp_f32 %[e7], %[x1]\n"
      "v_mul_f32_dpp %[bu6], %[vb], %[dtu]" SS_DPP_ROW(6)
      "v_fma_f32 %[h6], %[e6], %[p6], %[bu6]\n"
      "v_mul_f32 %[x0], %[dt], %[a8]\n"
      "v_exp_f32 %[e8], %[x0]\n"
      "v_mul_f32_dpp %[bu7], %[vb], %[dtu]" SS_DPP_ROW(7)
      "v_fma_f32 %[h7], %[e7], %[p7], %[bu7]\n"
      "v_mul_f32 %[x1], %[dt], %[a9]\n"
      "v_exp_f32 %[e9], %[x1]\n"
      "v_mul_f32_dpp %[bu8], %[vb], %[dtu]" SS_DPP_ROW(8)
      "v_fma_f32 %[h8], %[e8], %[p8], %[bu8]\n"
      "v_mul_f32 %[x0], %[dt], %[a10]\n"
      "v_exp_f32 %[e10], %[x0]\n"
      "v_mul_f32_dpp %[bu9], %[vb], %[dtu]" SS_DPP_ROW(9)
      "v_fma_f32 %[h9], %[e9], %[p9], %[bu9]\n"
      "v_mul_f32 %[x1], %[dt], %[a11]\n"
      "v_exp_f32 %[e11], %[x1]\n"
      "v_mul_f32_dpp %[bu10], %[vb], %[dtu]" SS_DPP_ROW(10)
      "v_fma_f32 %[h10], %[e10], %[p10], %[bu10]\n"
      "v_mul_f32 %[x0], %[dt], %[a12]\n"
      "v_exp_f32 %[e12], %[x0]\n"
      "v_mul_f32_dpp %[bu11], %[vb], %[dtu]" SS_DPP_ROW(11)
      "v_fma_f32 %[h11], %[e11], %[p11], %[bu11]\n"
      "v_mul_f32 %[x1], %[dt], %[a13]\n"
      "v_exp_f32 %[e13], %[x1]\n"
      "v_mul_f32_dpp %[bu12], %[vb], %[dtu]" SS_DPP_ROW(12)
      "v_fma_f32 %[h12], %[e12], %[p12], %[bu12]\n"
      "v_mul_f32 %[x0], %[dt], %[a14]\n"
      "v_exp_f32 %[e14], %[x0]\n"
      "v_mul_f32_dpp %[bu13], %[vb], %[dtu]" SS_DPP_ROW(13)
      "v_fma_f32 %[h13], %[e13], %[p13], %[bu13]\n"
      "v_mul_f32 %[x1], %[dt], %[a15]\n"
      "v_exp_f32 %[e15], %[x1]\n"
      "v_mul_f32_dpp %[bu14], %[vb], %[dtu]" SS_DPP_ROW(14)
      "v_fma_f32 %[h14], %[e14], %[p14], %[bu14]\n"
      "v_mul_f32_dpp %[bu15], %[vb], %[dtu]" SS_DPP_ROW(15)
      "v_fma_f32 %[h15], %[e15], %[p15], %[bu15]\n"
      : SS_OPS16(h, "=&v"), SS_OPS16(bu, "=&v"), SS_OPS16(e, "=&v"), [x0] "=&v"(x0), [x1] "=&v"(x1)
      : SS_OPS16(p, "v"), SS_OPS16(a, "v"), [dt] "v"(dt), [dtu] "v"(dtu), [vb] "v"(vb));
}

// The state after a chunk's first token from zero when its decay is not needed: h[n] = dtu B[n].
__device__ __forceinline__ void bwd_input_term(float (&h)[16], float dtu, float vb) {
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32_dpp %[h0], %[vb], %[dtu]" SS_DPP_ROW(0)
      "v_mul_f32_dpp %[h1], %[vb], %[dtu]" SS_DPP_ROW(1)
      "v_mul_f32_dpp %[h2], %[vb], %[dtu]" SS_DPP_ROW(2)
      "v_mul_f32_dpp %[h3], %[vb], %[dtu]" SS_DPP_ROW(3)
      "v_mul_f32_dpp %[h4], %[vb], %[dtu]" SS_DPP_ROW(4)
      "v_mul_f32_dpp %[h5], %[vb], %[dtu]" SS_DPP_ROW(5)
      "v_mul_f32_dpp %[h6], %[vb], %[dtu]" SS_DPP_ROW(6)
      "v_mul_f32_dpp %[h7], %[vb], %[dtu]" SS_DPP_ROW(7)
      "v_mul_f32_dpp %[h8], %[vb], %[dtu]" SS_DPP_ROW(8)
      "v_mul_f32_dpp %[h9], %[vb], %[dtu]" SS_DPP_ROW(9)
      "v_mul_f32_dpp %[h10], %[vb], %[dtu]" SS_DPP_ROW(10)
      "v_mul_f32_dpp %[h11], %[vb], %[dtu]" SS_DPP_ROW(11)
      "v_mul_f32_dpp %[h12], %[vb], %[dtu]" SS_DPP_ROW(12)
      "v_mul_f32_dpp %[h13], %[vb], %[dtu]" SS_DPP_ROW(13)
      "v_mul_f32_dpp %[h14], %[vb], %[dtu]" SS_DPP_ROW(14)
      "v_mul_f32_dpp %[h15], %[vb], %[dtu]" SS_DPP_ROW(15)
      : SS_OPS16(h, "=&v")
      : [dtu] "v"(dtu), [vb] "v"(vb));
}

// True forward step from the previous states P with the kept input terms:
// H[n] = e[n] P[n] + bu[n]; s += C[n] H[n] (the DPP fmac of state n two fmas later).
__device__ __forceinline__ void bwd_true_bu(const float (&P)[16], float (&H)[16], const float (&e)[16],
                                            const float (&b)[16], float vc, float& s) {
  asm volatile(
      "s_nop 1\n"
      "v_fma_f32 %[H0], %[e0], %[P0], %[b0]\n"
      "v_fma_f32 %[H1], %[e1], %[P1], %[b1]\n"
      "v_fma_f32 %[H2], %[e2], %[P2], %[b2]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H0]" SS_DPP_ROW(0)
      "v_fma_f32 %[H3], %[e3], %[P3], %[b3]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H1]" SS_DPP_ROW(1)
      "v_fma_f32 %[H4], %[e4], %[P4], %[b4]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H2]" SS_DPP_ROW(2)
      "v_fma_f32 %[H5], %[e5], %[P5], %[b5]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H3]" SS_DPP_ROW(3)
      "v_fma_f32 %[H6], %[e6], %[P6], %[b6]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H4]" SS_DPP_ROW(4)
      "v_fma_f32 %[H7], %[e7], %[P7], %[b7]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H5]" SS_DPP_ROW(5)
      "v_fma_f32 %[H8], %[e8], %[P8], %[b8]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H6]" SS_DPP_ROW(6)
      "v_fma_f32 %[H9], %[e9], %[P9], %[b9]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H7]" SS_DPP_ROW(7)
      "v_fma_f32 %[H10], %[e10], %[P10], %[b10]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H8]" SS_DPP_ROW(8)
      "v_fma_f32 %[H11], %[e11], %[P11], %[b11]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H9]" SS_DPP_ROW(9)
      "v_fma_f32 %[H12], %[e12], %[P12], %[b12]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H10]" SS_DPP_ROW(10)
      "v_fma_f32 %[H13], %[e13], %[P13], %[b13]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H11]" SS_DPP_ROW(11)
      "v_fma_f32 %[H14], %[e14], %[P14], %[b14]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H12]" SS_DPP_ROW(12)
      "v_fma_f32 %[H15], %[e15], %[P15], %[b15]\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H13]" SS_DPP_ROW(13)
      "s_nop 1\n"
      "v_fmac_f32_dpp %[s], %[vc], %[H14]" SS_DPP_ROW(14)
      "v_fmac_f32_dpp %[s], %[vc], %[H15]" SS_DPP_ROW(15)
      : SS_OPS16(H, "=&v"), [s] "+v"(s)
      : SS_OPS16(P, "v"), SS_OPS16(e, "v"), SS_OPS16(b, "v"), [vc] "v"(vc));
}
// Without s (no gate): H[n] = e[n] P[n] + bu[n].
__device__ __forceinline__ void bwd_true_states_bu(const float (&P)[16], float (&H)[16], const float (&e)[16],
                                                   const float (&b)[16]) {
  asm volatile(
      "v_fma_f32 %[H0], %[e0], %[P0], %[b0]\n"
      "v_fma_f32 %[H1], %[e1], %[P1], %[b1]\n"
      "v_fma_f32 %[H2], %[e2], %[P2], %[b2]\n"
      "v_fma_f32 %[H3], %[e3], %[P3], %[b3]\n"
      "v_fma_f32 %[H4], %[e4], %[P4], %[b4]\n"
      "v_fma_f32 %[H5], %[e5], %[P5], %[b5]\n"
      "v_fma_f32 %[H6], %[e6], %[P6], %[b6]\n"
      "v_fma_f32 %[H7], %[e7], %[P7], %[b7]\n"
      "v_fma_f32 %[H8], %[e8], %[P8], %[b8]\n"
      "v_fma_f32 %[H9], %[e9], %[P9], %[b9]\n"
      "v_fma_f32 %[H10], %[e10], %[P10], %[b10]\n"
      "v_fma_f32 %[H11], %[e11], %[P11], %[b11]\n"
      "v_fma_f32 %[H12], %[e12], %[P12], %[b12]\n"
      "v_fma_f32 %[H13], %[e13], %[P13], %[b13]\n"
      "v_fma_f32 %[H14], %[e14], %[P14], %[b14]\n"
      "v_fma_f32 %[H15], %[e15], %[P15], %[b15]\n"
      : SS_OPS16(H, "=&v")
      : SS_OPS16(P, "v"), SS_OPS16(e, "v"), SS_OPS16(b, "v"));
}

// Reverse local step of one token: m[n] = e[n] (m[n] + ds C[n]).
#define BW_R(n)                                                               \
  "v_fmac_f32_dpp %[m" #n "], %[vc], %[ds]" SS_DPP_ROW(n)                     \
  "v_mul_f32 %[m" #n "], %[e" #n "], %[m" #n "]\n"

__device__ __forceinline__ void bwd_rlocal(float (&m)[16], const float (&e)[16], float ds, float vc) {
  asm volatile(
      "s_nop 1\n"
      BW_R(0) BW_R(1) BW_R(2) BW_R(3) BW_R(4) BW_R(5) BW_R(6) BW_R(7)
      BW_R(8) BW_R(9) BW_R(10) BW_R(11) BW_R(12) BW_R(13) BW_R(14) BW_R(15)
      : SS_OPS16(m, "+v")
      : SS_OPS16(e, "v"), [ds] "v"(ds), [vc] "v"(vc));
}
#undef BW_R

// bwd_rlocal for the last token of a chunk, whose adjoint starts at zero: m[n] = e[n] ds C[n].
__device__ __forceinline__ void bwd_rlocal_first(float (&m)[16], const float (&e)[16], float ds, float vc) {
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32_dpp %[m0], %[vc], %[ds]" SS_DPP_ROW(0)
      "v_mul_f32_dpp %[m1], %[vc], %[ds]" SS_DPP_ROW(1)
      "v_mul_f32_dpp %[m2], %[vc], %[ds]" SS_DPP_ROW(2)
      "v_mul_f32_dpp %[m3], %[vc], %[ds]" SS_DPP_ROW(3)
      "v_mul_f32_dpp %[m4], %[vc], %[ds]" SS_DPP_ROW(4)
      "v_mul_f32_dpp %[m5], %[vc], %[ds]" SS_DPP_ROW(5)
      "v_mul_f32_dpp %[m6], %[vc], %[ds]" SS_DPP_ROW(6)
      "v_mul_f32_dpp %[m7], %[vc], %[ds]" SS_DPP_ROW(7)
      "v_mul_f32_dpp %[m8], %[vc], %[ds]" SS_DPP_ROW(8)
      "v_mul_f32_dpp %[m9], %[vc], %[ds]" SS_DPP_ROW(9)
      "v_mul_f32_dpp %[m10], %[vc], %[ds]" SS_DPP_ROW(10)
      "v_mul_f32_dpp %[m11], %[vc], %[ds]" SS_DPP_ROW(11)
      "v_mul_f32_dpp %[m12], %[vc], %[ds]" SS_DPP_ROW(12)
      "v_mul_f32_dpp %[m13], %[vc], %[ds]" SS_DPP_ROW(13)
      "v_mul_f32_dpp %[m14], %[vc], %[ds]" SS_DPP_ROW(14)
      "v_mul_f32_dpp %[m15], %[vc], %[ds]" SS_DPP_ROW(15)
      "v_mul_f32 %[m0], %[e0], %[m0]\n"
      "v_mul_f32 %[m1], %[e1], %[m1]\n"
      "v_mul_f32 %[m2], %[e2], %[m2]\n"
      "v_mul_f32 %[m3], %[e3], %[m3]\n"
      "v_mul_f32 %[m4], %[e4], %[m4]\n"
      "v_mul_f32 %[m5], %[e5], %[m5]\n"
      "v_mul_f32 %[m6], %[e6], %[m6]\n"
      "v_mul_f32 %[m7], %[e7], %[m7]\n"
      "v_mul_f32 %[m8], %[e8], %[m8]\n"
      "v_mul_f32 %[m9], %[e9], %[m9]\n"
      "v_mul_f32 %[m10], %[e10], %[m10]\n"
      "v_mul_f32 %[m11], %[e11], %[m11]\n"
      "v_mul_f32 %[m12], %[e12], %[m12]\n"
      "v_mul_f32 %[m13], %[e13], %[m13]\n"
      "v_mul_f32 %[m14], %[e14], %[m14]\n"
      "v_mul_f32 %[m15], %[e15], %[m15]\n"
      : SS_OPS16(m, "=&v")
      : SS_OPS16(e, "v"), [ds] "v"(ds), [vc] "v"(vc));
}

// True reverse step of one token and its gradient terms, the adjoint in m on entry:
//   lam = m[n] + ds C[n] (kept in m[n]);  sb += B[n] lam;  o[n] = e[n] lam (the adjoint
//   passed to the previous token);  g = o[n] P[n] (= lam abar h_prev, P the states entering
//   the token);  dA[n] += dt g;  ga += A2[n] g;
//   LDS: lam at row n of the dB block, H[n] at row n of the dC block (column: this lane's
//   channel c, in the 16-byte quarter (c >> 2) ^ (n >> 2) of the row; ad[q] addresses the
//   lane's word for the rows n with n >> 2 = q). The channel sums weight them by dtu and ds
//   (bwd_rowsum). Written straight from lam and H, which nothing overwrites while the writes
//   are in flight: the new adjoint goes to o, and the caller alternates m and o by token.
#define BW_G(n, G, AD, OB, OC)                                                \
  "v_fmac_f32_dpp %[m" #n "], %[vc], %[ds]" SS_DPP_ROW(n)                     \
  "v_mul_f32 %[o" #n "], %[e" #n "], %[m" #n "]\n"                            \
  "v_mul_f32 %[" G "], %[o" #n "], %[P" #n "]\n"                              \
  "v_fmac_f32_dpp %[sb], %[vb], %[m" #n "]" SS_DPP_ROW(n)                     \
  "ds_write_b32 %[" AD "], %[m" #n "] offset:" OB "\n"                        \
  "ds_write_b32 %[" AD "], %[H" #n "] offset:" OC "\n"                        \
  "v_fmac_f32 %[dA" #n "], %[dt], %[" G "]\n"                                 \
  "v_fmac_f32 %[ga], %[a" #n "], %[" G "]\n"

__device__ __forceinline__ void bwd_grad(float (&m)[16], float (&o)[16], float (&dA)[16], const float (&H)[16],
                                         const float (&P)[16], const float (&e)[16], const float (&a)[16],
                                         float dt, float ds, float vb, float vc, float& ga, float& sb,
                                         const uint32_t (&ad)[4]) {
  float g0, g1;
  asm volatile(
      "s_nop 1\n"
      BW_G(0, "g0", "ad0", "0", "4352")
      BW_G(1, "g1", "ad0", "64", "4416")
      BW_G(2, "g0", "ad0", "128", "4480")
      BW_G(3, "g1", "ad0", "192", "4544")
      BW_G(4, "g0", "ad1", "256", "4608")
      BW_G(5, "g1", "ad1", "320", "4672")
      BW_G(6, "g0", "ad1", "384", "4736")
      BW_G(7, "g1", "ad1", "448", "4800")
      BW_G(8, "g0", "ad2", "512", "4864")
      BW_G(9, "g1", "ad2", "576", "4928")
      BW_G(10, "g0", "ad2", "640", "4992")
      BW_G(11, "g1", "ad2", "704", "5056")
      BW_G(12, "g0", "ad3", "768", "5120")
      BW_G(13, "g1", "ad3", "832", "5184")
      BW_G(14, "g0", "ad3", "896", "5248")
      BW_G(15, "g1", "ad3", "960", "5312")
      : SS_OPS16(m, "+v"), SS_OPS16(o, "=&v"), SS_OPS16(dA, "+v"), [ga] "+v"(ga), [sb] "+v"(sb),
        [g0] "=&v"(g0), [g1] "=&v"(g1)
      : SS_OPS16(H, "v"), SS_OPS16(P, "v"), SS_OPS16(e, "v"), SS_OPS16(a, "v"), [dt] "v"(dt), [ds] "v"(ds),
        [vb] "v"(vb), [vc] "v"(vc), [ad0] "v"(ad[0]), [ad1] "v"(ad[1]), [ad2] "v"(ad[2]), [ad3] "v"(ad[3])
      : "memory");
}
#undef BW_G

// Channel sums of one token's dB and dC terms for state n (the reading lane's index in its
// row): b0..b3 and c0..c3 are the logical channel quarters of row n of the dB and dC blocks;
// channel c's terms are weighted by dtu and ds of channel c, broadcast from lane c of the row:
//   sb = sum_c dtu_c lam_c[n],  sc = sum_c ds_c H_c[n].
__device__ __forceinline__ void bwd_rowsum(float4 b0, float4 b1, float4 b2, float4 b3, float4 c0, float4 c1,
                                           float4 c2, float4 c3, float dtu, float ds, float& sb, float& sc) {
  sb = 0.0f;
  sc = 0.0f;
  asm volatile(
      "s_nop 1\n"
      "v_fmac_f32_dpp %[sb], %[dtu], %[b0x]" SS_DPP_ROW(0)
      "v_fmac_f32_dpp %[sc], %[ds], %[c0x]" SS_DPP_ROW(0)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b0y]" SS_DPP_ROW(1)
      "v_fmac_f32_dpp %[sc], %[ds], %[c0y]" SS_DPP_ROW(1)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b0z]" SS_DPP_ROW(2)
      "v_fmac_f32_dpp %[sc], %[ds], %[c0z]" SS_DPP_ROW(2)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b0w]" SS_DPP_ROW(3)
      "v_fmac_f32_dpp %[sc], %[ds], %[c0w]" SS_DPP_ROW(3)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b1x]" SS_DPP_ROW(4)
      "v_fmac_f32_dpp %[sc], %[ds], %[c1x]" SS_DPP_ROW(4)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b1y]" SS_DPP_ROW(5)
      "v_fmac_f32_dpp %[sc], %[ds], %[c1y]" SS_DPP_ROW(5)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b1z]" SS_DPP_ROW(6)
      "v_fmac_f32_dpp %[sc], %[ds], %[c1z]" SS_DPP_ROW(6)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b1w]" SS_DPP_ROW(7)
      "v_fmac_f32_dpp %[sc], %[ds], %[c1w]" SS_DPP_ROW(7)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b2x]" SS_DPP_ROW(8)
      "v_fmac_f32_dpp %[sc], %[ds], %[c2x]" SS_DPP_ROW(8)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b2y]" SS_DPP_ROW(9)
      "v_fmac_f32_dpp %[sc], %[ds], %[c2y]" SS_DPP_ROW(9)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b2z]" SS_DPP_ROW(10)
      "v_fmac_f32_dpp %[sc], %[ds], %[c2z]" SS_DPP_ROW(10)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b2w]" SS_DPP_ROW(11)
      "v_fmac_f32_dpp %[sc], %[ds], %[c2w]" SS_DPP_ROW(11)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b3x]" SS_DPP_ROW(12)
      "v_fmac_f32_dpp %[sc], %[ds], %[c3x]" SS_DPP_ROW(12)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b3y]" SS_DPP_ROW(13)
      "v_fmac_f32_dpp %[sc], %[ds], %[c3y]" SS_DPP_ROW(13)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b3z]" SS_DPP_ROW(14)
      "v_fmac_f32_dpp %[sc], %[ds], %[c3z]" SS_DPP_ROW(14)
      "v_fmac_f32_dpp %[sb], %[dtu], %[b3w]" SS_DPP_ROW(15)
      "v_fmac_f32_dpp %[sc], %[ds], %[c3w]" SS_DPP_ROW(15)
      : [sb] "+v"(sb), [sc] "+v"(sc)
      : [dtu] "v"(dtu), [ds] "v"(ds), [b0x] "v"(b0.x), [b0y] "v"(b0.y), [b0z] "v"(b0.z), [b0w] "v"(b0.w), [b1x] "v"(b1.x), [b1y] "v"(b1.y), [b1z] "v"(b1.z), [b1w] "v"(b1.w), [b2x] "v"(b2.x), [b2y] "v"(b2.y), [b2z] "v"(b2.z), [b2w] "v"(b2.w), [b3x] "v"(b3.x), [b3y] "v"(b3.y), [b3z] "v"(b3.z), [b3w] "v"(b3.w),
        [c0x] "v"(c0.x), [c0y] "v"(c0.y), [c0z] "v"(c0.z), [c0w] "v"(c0.w), [c1x] "v"(c1.x), [c1y] "v"(c1.y), [c1z] "v"(c1.z), [c1w] "v"(c1.w), [c2x] "v"(c2.x), [c2y] "v"(c2.y), [c2z] "v"(c2.z), [c2w] "v"(c2.w), [c3x] "v"(c3.x), [c3y] "v"(c3.y), [c3z] "v"(c3.z), [c3w] "v"(c3.w));
}

// bwd_grad for the 32-row tiles, writing the weighted terms themselves (lam = m + ds C[n] in
// m[n]):
//   LDS[ad + 64 n] = lam dtu (dB term);  LDS[ad + RC + 64 n] = ds H[n] (dC term);
//   sb += B[n] lam;  m[n] = e[n] lam (the adjoint passed to the previous token);
//   g = m[n] P[n] (= lam abar h_prev, P the states entering the token);
//   dA[n] += dt g;  ga += A2[n] g.
// The LDS data registers rotate over three temporaries, g over two.
#define BW_GP(n, T, U, G, OB, OC)                                              \
  "v_fmac_f32_dpp %[m" #n "], %[vc], %[ds]" SS_DPP_ROW(n)                     \
  "v_mul_f32 %[" U "], %[ds], %[H" #n "]\n"                                   \
  "v_mul_f32 %[" T "], %[m" #n "], %[dtu]\n"                                  \
  "v_fmac_f32_dpp %[sb], %[vb], %[m" #n "]" SS_DPP_ROW(n)                     \
  "ds_write_b32 %[ad], %[" T "] offset:" OB "\n"                              \
  "ds_write_b32 %[ad], %[" U "] offset:" OC "\n"                              \
  "v_mul_f32 %[m" #n "], %[e" #n "], %[m" #n "]\n"                            \
  "v_mul_f32 %[" G "], %[m" #n "], %[P" #n "]\n"                              \
  "v_fmac_f32 %[dA" #n "], %[dt], %[" G "]\n"                                 \
  "v_fmac_f32 %[ga], %[a" #n "], %[" G "]\n"

__device__ __forceinline__ void bwd_grad_products(float (&m)[16], float (&dA)[16], const float (&H)[16],
                                         const float (&P)[16], const float (&e)[16], const float (&a)[16],
                                         float dt, float dtu, float ds, float vb, float vc, float& ga,
                                         float& sb, uint32_t ad) {
  float t0, t1, t2, u0, u1, u2, g0, g1;
  asm volatile(
      "s_nop 1\n"
      BW_GP(0, "t0", "u0", "g0", "0", "4352")
      BW_GP(1, "t1", "u1", "g1", "64", "4416")
      BW_GP(2, "t2", "u2", "g0", "128", "4480")
      BW_GP(3, "t0", "u0", "g1", "192", "4544")
      BW_GP(4, "t1", "u1", "g0", "256", "4608")
      BW_GP(5, "t2", "u2", "g1", "320", "4672")
      BW_GP(6, "t0", "u0", "g0", "384", "4736")
      BW_GP(7, "t1", "u1", "g1", "448", "4800")
      BW_GP(8, "t2", "u2", "g0", "512", "4864")
      BW_GP(9, "t0", "u0", "g1", "576", "4928")
      BW_GP(10, "t1", "u1", "g0", "640", "4992")
      BW_GP(11, "t2", "u2", "g1", "704", "5056")
      BW_GP(12, "t0", "u0", "g0", "768", "5120")
      BW_GP(13, "t1", "u1", "g1", "832", "5184")
      BW_GP(14, "t2", "u2", "g0", "896", "5248")
      BW_GP(15, "t0", "u0", "g1", "960", "5312")
      : SS_OPS16(m, "+v"), SS_OPS16(dA, "+v"), [ga] "+v"(ga), [sb] "+v"(sb), [t0] "=&v"(t0), [t1] "=&v"(t1),
        [t2] "=&v"(t2), [u0] "=&v"(u0), [u1] "=&v"(u1), [u2] "=&v"(u2), [g0] "=&v"(g0), [g1] "=&v"(g1)
      : SS_OPS16(H, "v"), SS_OPS16(P, "v"), SS_OPS16(e, "v"), SS_OPS16(a, "v"), [dt] "v"(dt), [dtu] "v"(dtu),
        [ds] "v"(ds), [vb] "v"(vb), [vc] "v"(vc), [ad] "v"(ad)
      : "memory");
}
#undef BW_GP

// LDS byte address of a __shared__ float (for the ds_write instructions of bwd_grad).
__device__ __forceinline__ uint32_t lds_addr(float* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) float*)(p)));
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

__device__ __forceinline__ Lane lane_at(const BwdArgs& a, int64_t g) {
  Lane l;
  l.b = g / a.ngroups;
  l.c0 = (g % a.ngroups) * 16;
  l.i = threadIdx.x & 15;
  l.k = threadIdx.x >> 4;
  l.c = l.c0 + l.i;
  l.cvalid = l.c < a.dim;
  l.cc = l.cvalid ? l.c : a.dim - 1;
  return l;
}

// The workgroup's group index gi and sequence part: with SPLIT a work item from the queue
// (ss_split.h), the chain running from the last part to the first when `reverse`; without,
// the forward's mapping, which keeps neighbouring groups (sharing 128-byte lines of the
// (.., dim) arrays) on one XCD: with the workgroup id as the group, two (fp32) or four (bf16)
// XCDs each fetched every line (130M checkpoint kernel: 0.41 GB read per call for 0.20 GB
// of inputs).
template <bool SPLIT>
__device__ __forceinline__ void work_item(const BwdArgs& a, bool reverse, uint32_t& item_s, int64_t& gi,
                                          int64_t& part) {
  gi = SPLIT ? static_cast<int64_t>(blockIdx.x) : chunk::group_of(blockIdx.x, a.batch * a.ngroups);
  part = 0;
  if (SPLIT) {
    const int64_t groups = a.batch * a.ngroups;
    if (threadIdx.x == 0) item_s = split::take(a.split_ws, groups);
    __syncthreads();
    const uint32_t item = __builtin_amdgcn_readfirstlane(item_s);  // rank * groups + gi
    const int64_t rank = item / groups;
    gi = item % groups;
    part = reverse ? a.parts - 1 - rank : rank;
  }
}

// Forward scan from h0 (or zero), storing the state at the start of every tile of the
// reverse kernel (bwd_tile_tokens() = 32 tokens): ckpt[((b * ntiles + tile) * dimp + c) * 16
// + n]. It runs its own, longer chunks (CTC tokens, tiles of 16 * CTC tokens) with the
// hand-scheduled local step; the folding lane writes a checkpoint whenever the state it
// carries reaches a multiple of 32 tokens. The inputs of the next tile are requested before
// the current one is computed.
// R rows (time chunks): 16 (4 waves) or 32 (8 waves, for shapes with fewer channel groups
// than twice the CUs, where 4-wave workgroups would leave SIMDs with one wave); with 32 the
// rows 16..31 own no state in the fold.
// With SPLIT, a workgroup scans one part of its group's sequence, from the state the previous
// part publishes, and publishes its own end state.
template <typename T, int CTC, int R, bool SPLIT>
__global__ __launch_bounds__(R * 16) __attribute__((amdgpu_waves_per_eu(R == 16 ? 4 : 2)))
void bwd_ckpt_kernel(BwdArgs a) {
  static_assert(CTC * 4 == 32 || CTC * 8 == 32 || CTC * 16 == 32, "checkpoints every 32 tokens");
  static_assert(R == 16 || R == 32, "16 or 32 chunks per tile");
  constexpr int kPer = 32 / CTC;  // chunks per checkpoint interval
  // With 32 rows, rows 16..31 own no state in the fold: the aggregate arrays alternate by
  // tile, so those rows go on to the next tile's local pass while rows 0..15 fold (a tile's
  // arrays are written again two tiles later, after every row has passed the first barrier
  // of the tile between, which the folding rows reach only after their fold).
  constexpr int NB = R == 32 ? 2 : 1;
  __shared__ float lds_p2[NB][R * kS];
  __shared__ float lds_h2[NB][R * kS];
  __shared__ uint32_t item_s, seen_s;
  int buf = 0;
  int64_t gi, part;
  work_item<SPLIT>(a, false, item_s, gi, part);
  const Lane l = lane_at(a, gi);
  const int64_t L = a.seqlen, N = a.dstate, dimp = a.ngroups * 16, groups = a.batch * a.ngroups;
  constexpr int TT = R * CTC;
  const int64_t t_begin = SPLIT ? part * a.part_len : 0;
  const int64_t t_end = SPLIT ? min(L, t_begin + a.part_len) : L;
  float A2[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) A2[n] = n < N ? a.A[l.cc * N + n] * kLog2e : 0.0f;
  const float bias = a.delta_bias ? a.delta_bias[l.cc] : 0.0f;
  float carry = (a.h0 && part == 0 && l.k < N) ? a.h0[(l.b * a.dim + l.cc) * N + l.k] : 0.0f;
  if (SPLIT && part > 0) {  // start from the state the previous part ends with
    const int64_t slot = (part - 1) * groups + gi;
    if (threadIdx.x == 0) seen_s = split::poll(a.split_ws, slot, a.split_wait_limit) ? 1u : 0u;
    __syncthreads();  // (the state loads are issued after thread 0 has seen the flag)
    // a wait that gave up leaves the state unknown: continue from NaN (counted in the header)
    if (l.k < 16)
      carry = __builtin_amdgcn_readfirstlane(seen_s) ? split::load_state(a.split_ws, a.split_cap, slot, l.k, l.i)
                                                     : __builtin_nanf("");
  }

  // lane (k, i): tokens t0 + k*CTC + j of channel cc and B_t[i]; fixed 32-bit byte offsets
  const uint32_t tok_row = static_cast<uint32_t>(a.dim * sizeof(T));
  const uint32_t bc_row = static_cast<uint32_t>(N * sizeof(T));
  const uint32_t col = static_cast<uint32_t>((l.cc - l.c0) * sizeof(T));
  const uint32_t bcol = l.i < N ? static_cast<uint32_t>(l.i * sizeof(T)) : 0x7fffffffu;
  T* tag = nullptr;
  struct In {  // raw element bits, widened where used (a widening next to the load would wait for it)
    chunk::Bits<T> x[CTC], u[CTC], b[CTC];
  };
  // The tile at t0: buffer resources and its last token (tokens past the end re-read it).
  struct Src {
    __amdgpu_buffer_rsrc_t rd, ru, rb;
    int last;
  };
  auto src_of = [&](int64_t t0) {
    Src r;
    const int64_t e0 = (l.b * L + t0) * a.dim + l.c0;
    const int64_t bc0 = (l.b * L + t0) * N;
    const int64_t left = (a.batch * L * a.dim - e0) * static_cast<int64_t>(sizeof(T));
    const int64_t bleft = (a.batch * L * N - bc0) * static_cast<int64_t>(sizeof(T));
    r.rd = chunk::rsrc(static_cast<const T*>(a.delta) + e0, left);
    r.ru = chunk::rsrc(static_cast<const T*>(a.u) + e0, left);
    r.rb = chunk::rsrc(static_cast<const T*>(a.B) + bc0, bleft);
    r.last = static_cast<int>(min(L - 1 - t0, static_cast<int64_t>(TT - 1)));
    return r;
  };
  auto fetch_token = [&](In& r, const Src& sr, int j) {
    const uint32_t tt = static_cast<uint32_t>(min(l.k * CTC + j, sr.last));  // past the end: last token
    r.x[j] = chunk::ldr<T>(sr.rd, tt * tok_row + col, 0);
    r.u[j] = chunk::ldr<T>(sr.ru, tt * tok_row + col, 0);
    r.b[j] = chunk::ldr<T>(sr.rb, bcol == 0x7fffffffu ? bcol : tt * bc_row + bcol, 0);
  };
  auto fetch = [&](In& r, int64_t t0) {
    const Src sr = src_of(t0);
#pragma unroll
    for (int j = 0; j < CTC; ++j) fetch_token(r, sr, j);
  };
  In cur, nxt;
  if (a.ntiles > 0) {
    fetch(cur, t_begin);
    // (the first tile's registers get a definition that is not a load: with a load on one
    // path into the loop and copies on the other, the compiler waits at the start of every
    // tile for the loads just issued)
#pragma unroll
    for (int j = 0; j < CTC; ++j) asm volatile("" : "+v"(cur.x[j]), "+v"(cur.u[j]), "+v"(cur.b[j]));
  }
  asm volatile("" : "+v"(carry));  // (likewise the loaded initial state)
  for (int64_t t0 = t_begin; t0 < t_end; t0 += TT) {
    if (!SPLIT) progress_priority(t0, L);
    // The next tile's inputs, token by token: token j's loads are issued right after this
    // tile's token j is consumed, so a tile's requests reach the memory pipeline spread over
    // its local pass rather than all at its start (the last tile re-requests itself, unused:
    // loads under a branch make the compiler wait for all of them where the paths join).
    const Src nsrc = src_of(t0 + TT < t_end ? t0 + TT : t0);
    float h[16], e[16], dsum = 0.0f;
    // tokens of this lane's chunk inside the sequence (32-bit, once per tile)
    const int nval = static_cast<int>(min(L - t0, static_cast<int64_t>(TT))) - l.k * CTC;
#pragma unroll
    for (int j = 0; j < CTC; ++j) {
      const float x = chunk::as_f32<T>(cur.x[j]) + bias;
      float dt = a.softplus ? softplus(x) : x;
      dt = j < nval ? dt : 0.0f;  // a zero step is the identity
      dsum += dt;
      if (j == 0)  // (the state starts at zero: the first token's decay does not enter it)
        bwd_input_term(h, dt * chunk::as_f32<T>(cur.u[j]), chunk::as_f32<T>(cur.b[j]));
      else
        bwd_local(h, e, A2, dt, dt * chunk::as_f32<T>(cur.u[j]), chunk::as_f32<T>(cur.b[j]));
      fetch_token(nxt, nsrc, j);
    }
    float* lds_p = lds_p2[buf];
    float* lds_h = lds_h2[buf];
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      lds_p[l.k * kS + n * 16 + l.i] = chunk_em1(A2[n] * dsum);
      lds_h[l.k * kS + n * 16 + l.i] = h[n];
    }
    __syncthreads();
    // lane (k, i), k < 16, owns state n = k of channel i: fold the R chunks in order, keeping
    // the state at every multiple of 32 tokens (the checkpoint interval)
    constexpr int kCk = R / kPer;  // checkpoints per tile
    float ckv[kCk];
    if (R == 16 || l.k < 16) {
#pragma unroll
      for (int jj = 0; jj < R; ++jj) {
        if (jj % kPer == 0) ckv[jj / kPer] = carry;
        const int o = jj * kS + l.k * 16 + l.i;
        carry = __builtin_fmaf(lds_p[o], carry, carry + lds_h[o]);
      }
    }
    {  // the checkpoints, stored unconditionally through a resource based at this tile's first
       // one and ending with this batch row's last: a lane that owns no state stores to an
       // offset past every range, checkpoints past the sequence fall past this one (dropped).
       // A store under a branch would make the compiler wait for every memory operation in
       // flight where the paths join, the next tile's loads included.
      const int64_t tile0 = t0 / 32;
      const int64_t ck0 = (l.b * a.ntiles + tile0) * dimp * 16;
      const auto rck = chunk::rsrc(a.ckpt + ck0, (a.ntiles - tile0) * dimp * 16 * 4);
      const uint32_t voff = (R == 16 || l.k < 16) ? static_cast<uint32_t>((l.c * 16 + l.k) * 4) : chunk::kDropOffset;
      uint32_t ck_row = static_cast<uint32_t>(dimp * 16 * 4);  // bytes per checkpoint interval
      asm volatile("" : "+s"(ck_row));
#pragma unroll
      for (int m = 0; m < kCk; ++m)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ckv[m]), rck, voff, m * ck_row, 0);
    }
    if (NB == 1) __syncthreads();  // (one set of arrays: the next tile writes it)
    buf = NB == 2 ? buf ^ 1 : 0;
    cur = nxt;
  }
  if (SPLIT && part < a.parts - 1) {  // publish the end state for the next part
    const int64_t slot = part * groups + gi;
    if (l.k < 16) split::store_state(a.split_ws, a.split_cap, slot, l.k, l.i, carry);
    split::finish_stores();
    __syncthreads();
    if (threadIdx.x == 0) split::publish(a.split_ws, slot);
  }
}

// R rows (time chunks) as the checkpoint kernel: 16 (4 waves, two workgroups per CU) or 32
// (8 waves, one workgroup per CU); a tile is R * TC tokens (32 or 64), a multiple of the
// checkpoint interval. With SPLIT, a workgroup runs one part of its group's sequence, the
// chain going from the last part to the first: it starts from the adjoint the later part
// publishes, publishes the adjoint entering its own first tile, and leaves its dA/dD/dbias
// sums in its part's block of part_ch.
template <typename T, bool GATE, int TC, int R, bool SPLIT>
__global__ __launch_bounds__(R * 16) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_chunked_kernel(BwdArgs a) {
  static_assert(R == 16 || R == 32, "16 or 32 chunks per tile");
  // [0]: chunk decays - 1, [1]: chunk end states then forward carries; after the carries
  // are read, the same 2 R kS floats hold the per-wave dB/dC reduction blocks
  // [wave][dB or dC][row][n][lane] (R/4 x 2 x 4 x kS floats)
  __shared__ __attribute__((aligned(16))) float lds_eh[2][R * kS];
  __shared__ float lds_m[R * kS];  // chunk adjoint aggregates, then reverse carries
  __shared__ uint32_t item_s, seen_s;
  int64_t gi, part;
  work_item<SPLIT>(a, true, item_s, gi, part);
  const Lane l = lane_at(a, gi);
  const int64_t L = a.seqlen, N = a.dstate, dimp = a.ngroups * 16, groups = a.batch * a.ngroups;
  constexpr int TT = R * TC;
  constexpr int CK = TT / 32;  // checkpoint intervals per tile
  static_assert(CK * 32 == TT, "a tile is a whole number of checkpoint intervals");
  const int64_t nt = (L + TT - 1) / TT;  // this kernel's tiles
  const int64_t tile_lo = SPLIT ? part * (a.part_len / TT) : 0;                      // first tile
  const int64_t tile_hi = SPLIT ? min(nt, tile_lo + a.part_len / TT) : nt;  // past the last
  const int w = threadIdx.x >> 6, rw = l.k & 3;

  float A2[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) A2[n] = n < N ? a.A[l.cc * N + n] * kLog2e : 0.0f;
  float bias = a.delta_bias ? a.delta_bias[l.cc] : 0.0f;
  float Dd = a.D ? a.D[l.cc] : 0.0f;
  // Fold ownership: lane (k, i) owns state n = k & 15 of channel i. With 16 rows every lane
  // runs both folds; with 32, rows 0..15 run the forward fold and rows 16..31 the reverse
  // one, at the same time (the folds read the same chunk decays and write different arrays).
  const int own_n = l.k & 15;
  const bool fwd_owner = R == 16 || l.k < 16;
  const bool rev_owner = R == 16 || l.k >= 16;
  // adjoint carried from later tiles (the reverse fold's lanes)
  float rcarry = (a.dlast && (!SPLIT || part == a.parts - 1) && l.cvalid && rev_owner && own_n < N)
                     ? a.dlast[(l.b * a.dim + l.c) * N + own_n] : 0.0f;
  if (SPLIT && part < a.parts - 1) {  // start from the adjoint the later part publishes
    const int64_t slot = part * groups + gi;
    if (threadIdx.x == 0) seen_s = split::poll(a.split_ws, slot, a.split_wait_limit) ? 1u : 0u;
    __syncthreads();  // (the state loads are issued after thread 0 has seen the flag)
    if (rev_owner)
      rcarry = __builtin_amdgcn_readfirstlane(seen_s) ? split::load_state(a.split_ws, a.split_cap, slot, own_n, l.i)
                                                      : __builtin_nanf("");
  }
  float dAacc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) dAacc[n] = 0.0f;
  float dDacc = 0.0f, dbacc = 0.0f;

  // raw inputs of a tile's chunk for this lane, as stored bits (widened where used: a
  // widening next to the load would wait for it); the tile processed next (the earlier one)
  // is requested before this one is computed
  struct Raw {
    chunk::Bits<T> x[TC], u[TC], z[TC], b[TC], c[TC];
    uint32_t dy[TC];
  };
  // Buffer loads from fixed per-lane offsets, the token step in the SGPR offset (full tiles);
  // the sequence's last tile, which may be partial, re-reads its last token instead of
  // reading past the end. Lanes past dstate read state dstate - 1 and discard it. Every load
  // of a call is issued unconditionally (loads under a branch make the compiler wait for all
  // of them where the paths join, which would turn the prefetch into a stall).
  const int64_t nb = l.i < N ? l.i : N - 1;
  const uint32_t tok_row = static_cast<uint32_t>(a.dim * sizeof(T));
  const uint32_t dy_row = static_cast<uint32_t>(a.dim * 4);
  const uint32_t bc_row = static_cast<uint32_t>(N * sizeof(T));
  const uint32_t col = static_cast<uint32_t>((l.cc - l.c0) * sizeof(T));
  const uint32_t dcol = static_cast<uint32_t>((l.cc - l.c0) * 4);
  const uint32_t bcol = static_cast<uint32_t>(nb * sizeof(T));
  T* tag = nullptr;
  float* ftag = nullptr;
  auto tile_rsrc = [&](int64_t t0, __amdgpu_buffer_rsrc_t (&r)[6]) {
    const int64_t e0 = (l.b * L + t0) * a.dim + l.c0;
    const int64_t bc0 = (l.b * L + t0) * N;
    r[0] = chunk::rsrc_tile(static_cast<const T*>(a.delta) + e0);
    r[1] = chunk::rsrc_tile(static_cast<const T*>(a.u) + e0);
    r[2] = chunk::rsrc_tile(GATE ? static_cast<const T*>(a.z) + e0 : static_cast<const T*>(a.u) + e0);
    r[3] = chunk::rsrc_tile(a.dy + e0);
    r[4] = chunk::rsrc_tile(static_cast<const T*>(a.B) + bc0);
    r[5] = chunk::rsrc_tile(static_cast<const T*>(a.C) + bc0);
  };
  // (live = false: every load of the call is dropped by the range check and returns 0)
  auto fetch_full = [&](Raw& r, int64_t t0, bool live) {
    __amdgpu_buffer_rsrc_t rs[6];
    tile_rsrc(t0, rs);
    uint32_t tr = tok_row, dr = dy_row;  // (token steps formed here: SGPRs only while issuing)
    asm volatile("" : "+s"(tr), "+s"(dr));
    const uint32_t vt = live ? static_cast<uint32_t>(l.k * TC) * tok_row + col : chunk::kDropOffset;
    const uint32_t vd = live ? static_cast<uint32_t>(l.k * TC) * dy_row + dcol : chunk::kDropOffset;
    const uint32_t vbc = live ? static_cast<uint32_t>(l.k * TC) * bc_row + bcol : chunk::kDropOffset;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      r.x[j] = chunk::ldr<T>(rs[0], vt, j * tr);
      r.u[j] = chunk::ldr<T>(rs[1], vt, j * tr);
      r.z[j] = GATE ? chunk::ldr<T>(rs[2], vt, j * tr) : chunk::Bits<T>(0);
      r.dy[j] = chunk::ldb(ftag, rs[3], vd, j * dr);
      r.b[j] = chunk::ldr<T>(rs[4], vbc, j * bc_row);
      r.c[j] = chunk::ldr<T>(rs[5], vbc, j * bc_row);
    }
  };
  auto fetch_tail = [&](Raw& r, int64_t t0) {
    __amdgpu_buffer_rsrc_t rs[6];
    tile_rsrc(t0, rs);
    const int last = static_cast<int>(min(L - 1 - t0, static_cast<int64_t>(TT - 1)));
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const uint32_t tt = static_cast<uint32_t>(min(l.k * TC + j, last));  // past the end: last token
      r.x[j] = chunk::ldr<T>(rs[0], tt * tok_row + col, 0);
      r.u[j] = chunk::ldr<T>(rs[1], tt * tok_row + col, 0);
      r.z[j] = GATE ? chunk::ldr<T>(rs[2], tt * tok_row + col, 0) : chunk::Bits<T>(0);
      r.dy[j] = chunk::ldb(ftag, rs[3], tt * dy_row + dcol, 0);
      r.b[j] = chunk::ldr<T>(rs[4], tt * bc_row + bcol, 0);
      r.c[j] = chunk::ldr<T>(rs[5], tt * bc_row + bcol, 0);
    }
  };
  Raw cur, nxt;
  // the checkpointed state entering each tile (lane (k, i): state n = k of channel i), also
  // requested a tile ahead: read where it is used, its latency would stall every tile
  // (rows 16..31 of a 32-row tile own no state: they read state k - 16, unused)
  const uint32_t ck_off = static_cast<uint32_t>((l.c * 16 + (l.k & 15)) * 4);
  // store offsets of token 0 of this lane's chunk: (batch, L, dim) gradients and the dB/dC
  // partials; a lane past the last channel (or past dstate) stores past every range
  const uint32_t e_off = l.cvalid ? static_cast<uint32_t>((l.k * TC * a.dim + l.c) * 4) : chunk::kDropOffset;
  const uint32_t bc_off = l.i < N ? static_cast<uint32_t>((l.k * TC * N + l.i) * 4) : chunk::kDropOffset;
  auto ckpt_of = [&](int64_t tile) {
    const auto r = chunk::rsrc_tile(a.ckpt + (l.b * a.ntiles + tile * CK) * dimp * 16);
    return __builtin_amdgcn_raw_buffer_load_b32(r, ck_off, 0, 0);
  };
  uint32_t ck_cur = 0u, ck_nxt = 0u;
  if (tile_hi > tile_lo) {
    const int64_t tl = tile_hi - 1;
    if ((tl + 1) * TT <= L)
      fetch_full(cur, tl * TT, true);
    else
      fetch_tail(cur, tl * TT);
    ck_cur = ckpt_of(tl);
    // (a definition that is not a load for the first tile's registers: with a load on one path
    // into the loop and copies on the other, the compiler waits at the start of every tile for
    // the loads just issued)
#pragma unroll
    for (int j = 0; j < TC; ++j)
      asm volatile("" : "+v"(cur.x[j]), "+v"(cur.u[j]), "+v"(cur.z[j]), "+v"(cur.b[j]), "+v"(cur.c[j]), "+v"(cur.dy[j]));
    asm volatile("" : "+v"(ck_cur));
  }
  // (also the per-channel constants, loaded on every path into the loop: one left in flight
  // on a path that skips the loop makes the compiler wait at the top of every tile for all
  // memory operations before it, the previous tile's stores included)
  asm volatile("" : "+v"(rcarry), "+v"(bias), "+v"(Dd));
#pragma unroll
  for (int n = 0; n < 16; ++n) asm volatile("" : "+v"(A2[n]));
  for (int64_t tile = tile_hi - 1; tile >= tile_lo; --tile) {
    // wave priorities: the local passes and folds at 0 and the gradient phase after them at
    // 1, so a wave that fell behind catches up before the next tile's barriers (3B long
    // context, split: 18.20-18.26 against 18.36-18.40 ms with none, and 18.42-18.47 with the
    // local phase raised instead; 1.4B, unsplit: 1.448 against 1.555 ms with the progress
    // priority the forward's unsplit plans use)
    __builtin_amdgcn_s_setprio(0);
    const int64_t t0 = tile * TT;
    // the earlier tile, always a full one (the tile before the first re-reads tile 0, unused;
    // a sequence of one, partial, tile has no full tile to read: its loads are all dropped).
    // No branch around the loads: a loaded value that merges with another path's is widened
    // where the paths join, and that waits for the load.
    fetch_full(nxt, tile > 0 ? t0 - TT : 0, nt > 1);
    ck_nxt = ckpt_of(tile > 0 ? tile - 1 : 0);
    // tokens of this lane's chunk inside the sequence (TC except in the last tile)
    const int nval = static_cast<int>(min(static_cast<int64_t>(TC), max(static_cast<int64_t>(0), L - t0 - l.k * TC)));
    // per-token inputs of this lane's chunk (tokens past the end: zero step, zero dy)
    float dt[TC], dtu[TC], uu[TC], ds[TC], sg[TC], vb[TC], vc[TC], dyv[TC], dsl[TC];
    bool ok[TC], tvs[TC];
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const bool tv = j < nval;
      tvs[j] = tv;
      ok[j] = tv && l.cvalid;
      const float x = chunk::as_f32<T>(cur.x[j]) + bias;
      dt[j] = tv ? (a.softplus ? softplus(x) : x) : 0.0f;
      sg[j] = a.softplus ? sigmoid(x) : 1.0f;
      uu[j] = chunk::as_f32<T>(cur.u[j]);
      dtu[j] = dt[j] * uu[j];
      dyv[j] = ok[j] ? __uint_as_float(cur.dy[j]) : 0.0f;
      float g = 1.0f;
      dsl[j] = 0.0f;
      if (GATE) {
        const float zv = chunk::as_f32<T>(cur.z[j]);
        const float s = fast_rcp(1.0f + fast_exp2(-zv * kLog2e));
        g = zv * s;
        dsl[j] = s * __builtin_fmaf(zv, 1.0f - s, 1.0f);
      }
      ds[j] = dyv[j] * g;
      vb[j] = l.i < N ? chunk::as_f32<T>(cur.b[j]) : 0.0f;
      vc[j] = l.i < N ? chunk::as_f32<T>(cur.c[j]) : 0.0f;
    }

    // forward local pass from a zero state: decays and chunk aggregates
    static_assert(TC == 2, "the local pass keeps two tokens' input terms");
    float ex[TC][16], bu[TC][16], h[16];
    const float dsum = dt[0] + dt[1];
    bwd_local_first_bu(bu[0], ex[0], A2, dt[0], dtu[0], vb[0]);
    bwd_local_next_bu(h, bu[1], ex[1], bu[0], A2, dt[1], dtu[1], vb[1]);
    // reverse local pass from a zero adjoint (it needs only the decays): the chunk
    // aggregate mu_loc, so both folds share one pair of barriers
    float mu[16];
#pragma unroll
    for (int j = TC - 1; j >= 0; --j) {
      if (j == TC - 1)
        bwd_rlocal_first(mu, ex[j], ds[j], vc[j]);
      else
        bwd_rlocal(mu, ex[j], ds[j], vc[j]);
    }

    __syncthreads();  // the previous tile is done with every LDS array
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      lds_eh[0][l.k * kS + n * 16 + l.i] = chunk_em1(A2[n] * dsum);  // chunk decay - 1
      lds_eh[1][l.k * kS + n * 16 + l.i] = h[n];
      lds_m[l.k * kS + n * 16 + l.i] = mu[n];
    }
    __syncthreads();
    {  // the forward fold from the checkpoint and the reverse fold from the adjoint of the
       // later tile, over state own_n of channel i; each lane overwrites exactly the words it
       // read, and the two folds write different arrays
      if (fwd_owner) {
        float carry = __uint_as_float(ck_cur);
#pragma unroll
        for (int jj = 0; jj < R; ++jj) {
          const int o = jj * kS + own_n * 16 + l.i;
          const float pm = lds_eh[0][o], hv = lds_eh[1][o];
          lds_eh[1][o] = carry;  // state entering chunk jj
          carry = __builtin_fmaf(pm, carry, carry + hv);
        }
      }
      if (rev_owner) {
#pragma unroll
        for (int jj = R - 1; jj >= 0; --jj) {
          const int o = jj * kS + own_n * 16 + l.i;
          const float pm = lds_eh[0][o], mv = lds_m[o];
          lds_m[o] = rcarry;  // adjoint entering chunk jj from its end
          rcarry = __builtin_fmaf(pm, rcarry, rcarry + mv);
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    float q[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      q[n] = lds_eh[1][l.k * kS + n * 16 + l.i];
      mu[n] = lds_m[l.k * kS + n * 16 + l.i];
    }
    __syncthreads();  // every lane has its carries: lds_eh is free for the reductions

    // Stores go through buffer resources based at this tile, a masked lane's to an offset
    // past the range (dropped), so no store sits under a branch: the compiler would wait there
    // for every memory operation in flight, the next tile's prefetch included.
    // (resources based at this tile with offsets fixed per lane and the token step in the SGPR
    // offset; every store of a token inside the sequence is in bounds, the others go to the
    // drop offset)
    const int64_t eb = (l.b * L + t0) * a.dim;
    const auto rdu = chunk::rsrc_tile(a.du + eb);
    const auto rdd = chunk::rsrc_tile(a.ddelta + eb);
    const auto rdz = chunk::rsrc_tile(GATE ? a.dz + eb : a.du + eb);
    const int64_t plane = a.batch * a.ngroups * L * N;
    const int64_t pb = ((l.b * a.ngroups + (l.c0 >> 4)) * L + t0) * N;
    const auto rpb = chunk::rsrc_tile(a.part_bc + pb);
    const auto rpc = chunk::rsrc_tile(a.part_bc + plane + pb);
    uint32_t er = dy_row, pr = static_cast<uint32_t>(N * 4);
    asm volatile("" : "+s"(er), "+s"(pr));

    // true states of the chunk, the pre-gate output s and dz
    float H[TC][16];
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      if constexpr (GATE) {
        float s = Dd * uu[j];
        bwd_true_bu(j == 0 ? q : H[j > 0 ? j - 1 : 0], H[j], ex[j], bu[j], vc[j], s);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dyv[j] * s * dsl[j]), rdz,
                                              tvs[j] ? e_off : chunk::kDropOffset, j * er, 0);
      } else {
        bwd_true_states_bu(j == 0 ? q : H[j > 0 ? j - 1 : 0], H[j], ex[j], bu[j]);
      }
    }

    // true reverse recurrence and the gradient terms, token by token from the chunk end
    float* rB = &lds_eh[0][0] + w * (2 * 4 * kS) + rw * kS;  // this row's dB block; dC 4*kS on
    const float* rC = rB + 4 * kS;
    // Two ways to sum the dB and dC terms over the 16 channels of a row. With 16-row tiles
    // (two workgroups per CU) the terms are written unweighted and the sums weight them by a
    // DPP broadcast of each channel's dtu and ds, 2 VALU per update fewer (130M backward 0.673
    // -> 0.630 ms, 1.4B 1.735 -> 1.648 ms). With 32-row tiles the eight waves of the CU's one
    // workgroup reach their LDS bursts in step, and that layout made them wait 51% longer to
    // issue LDS instructions (3B long context: 14.43 -> 15.14 ms), so they write the weighted
    // terms and sum them with plain adds as each quarter arrives.
    if constexpr (R == 32) {
      const uint32_t rad = lds_addr(rB + l.i);
#pragma unroll
      for (int j = TC - 1; j >= 0; --j) {
        float sb = 0.0f, ga = 0.0f;
        bwd_grad_products(mu, dAacc, H[j], j == 0 ? q : H[j > 0 ? j - 1 : 0], ex[j], A2, dt[j], dtu[j], ds[j],
                          vb[j], vc[j], ga, sb, rad);
        {
          const uint32_t off = tvs[j] ? e_off : chunk::kDropOffset;
          const float ddt = __builtin_fmaf(uu[j], sb, ga * kLn2);
          const float dd = ddt * sg[j];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__builtin_fmaf(ds[j], Dd, dt[j] * sb)), rdu, off, j * er, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dd), rdd, off, j * er, 0);
          dbacc += ok[j] ? dd : 0.0f;
          dDacc = ok[j] ? __builtin_fmaf(ds[j], uu[j], dDacc) : dDacc;
        }
        // sum the 16 channels of this row: lane i takes state n = i (the block is this row's
        // own and LDS runs a wave's operations in order: the fences only keep the compiler
        // from moving the accesses across the other lanes' writes)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float sB = 0.0f, sC = 0.0f;
        {
          // (lane i reads the quarters of its 64-byte row in the order starting at i / 4: rows
          // of lanes i and i + 4 sit 256 bytes apart, on the same banks, so in one 16-byte read
          // the 16 lanes of a row touch 16 different bank groups only when their quarters differ)
          const float4* qb = reinterpret_cast<const float4*>(rB + l.i * 16);
          const float4* qc = reinterpret_cast<const float4*>(rC + l.i * 16);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int mm = (m + (l.i >> 2)) & 3;
            const float4 vb4 = qb[mm], vc4 = qc[mm];
            sB += (vb4.x + vb4.y) + (vb4.z + vb4.w);
            sC += (vc4.x + vc4.y) + (vc4.z + vc4.w);
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
          const uint32_t off = tvs[j] ? bc_off : chunk::kDropOffset;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sB), rpb, off, j * pr, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sC), rpc, off, j * pr, 0);
        }
      }
    } else {
      // write addresses of bwd_grad: this lane's channel c at quarter (c >> 2) ^ q of the rows n
      // with n >> 2 = q (rows of lanes i and i + 4 lie 256 bytes apart, on the same banks: with the
      // quarters swizzled by n >> 2, the 16 lanes of a row reading one logical quarter touch 16
      // different bank groups, and every lane finds channel c at the same logical position, so
      // the channel sums can take c's weights by a DPP broadcast from lane c)
      uint32_t rad[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        rad[q4] = lds_addr(rB) + static_cast<uint32_t>(16 * ((l.i >> 2) ^ q4) + 4 * (l.i & 3));
      const int sw = l.i >> 2;
      float mo[16];  // the adjoint's second register set (bwd_grad alternates them by token)
      static_assert(TC % 2 == 0, "the adjoint ends each tile in mu");
      const float4* qb = reinterpret_cast<const float4*>(rB + l.i * 16);
      const float4* qc = reinterpret_cast<const float4*>(rC + l.i * 16);
      // Channel sums of the row (lane i takes state n = i), software-pipelined: a token's LDS
      // reads are issued after its terms are written and summed only after the next token's
      // gradient block, whose writes go to the same block but queue behind the reads (LDS runs
      // a wave's operations in order; the block is this row's own). The fences only keep the
      // compiler from moving the accesses across the other lanes' writes.
      float4 qbv[4], qcv[4];  // the pending token's quarters
      auto rowsum_store = [&](int jt) {
        float sB, sC;
        bwd_rowsum(qbv[0], qbv[1], qbv[2], qbv[3], qcv[0], qcv[1], qcv[2], qcv[3], dtu[jt], ds[jt], sB, sC);
        const uint32_t off = tvs[jt] ? bc_off : chunk::kDropOffset;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sB), rpb, off, jt * pr, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sC), rpc, off, jt * pr, 0);
      };
#pragma unroll
      for (int j = TC - 1; j >= 0; --j) {
        float sb = 0.0f, ga = 0.0f;
        if (((TC - 1 - j) & 1) == 0)
          bwd_grad(mu, mo, dAacc, H[j], j == 0 ? q : H[j > 0 ? j - 1 : 0], ex[j], A2, dt[j], ds[j], vb[j], vc[j],
                   ga, sb, rad);
        else
          bwd_grad(mo, mu, dAacc, H[j], j == 0 ? q : H[j > 0 ? j - 1 : 0], ex[j], A2, dt[j], ds[j], vb[j], vc[j],
                   ga, sb, rad);
        if (j < TC - 1) rowsum_store(j + 1);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          qbv[m4] = qb[m4 ^ sw];
          qcv[m4] = qc[m4 ^ sw];
        }
        {
          const uint32_t off = tvs[j] ? e_off : chunk::kDropOffset;
          const float ddt = __builtin_fmaf(uu[j], sb, ga * kLn2);
          const float dd = ddt * sg[j];
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__builtin_fmaf(ds[j], Dd, dt[j] * sb)), rdu, off, j * er, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dd), rdd, off, j * er, 0);
          dbacc += ok[j] ? dd : 0.0f;
          dDacc = ok[j] ? __builtin_fmaf(ds[j], uu[j], dDacc) : dDacc;
        }
      }
      rowsum_store(0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    cur = nxt;
    ck_cur = ck_nxt;
  }
  if (SPLIT && part > 0) {  // publish the adjoint entering this part for the earlier one
    const int64_t slot = (part - 1) * groups + gi;
    if (rev_owner) split::store_state(a.split_ws, a.split_cap, slot, own_n, l.i, rcarry);
    split::finish_stores();
    __syncthreads();
    if (threadIdx.x == 0) split::publish(a.split_ws, slot);
  } else if (a.dh0 && l.cvalid && rev_owner && own_n < N) {
    a.dh0[(l.b * a.dim + l.c) * N + own_n] = rcarry;
  }

  // dA, dD and dbias of this workgroup: sum the R rows
  __syncthreads();
#pragma unroll
  for (int n = 0; n < 16; ++n) lds_eh[0][l.k * kS + n * 16 + l.i] = dAacc[n];
  lds_m[l.k * 16 + l.i] = dDacc;
  lds_m[R * 16 + l.k * 16 + l.i] = dbacc;
  __syncthreads();
  if (R == 16 || l.k < 16) {
    float s = 0.0f;
#pragma unroll
    for (int kk = 0; kk < R; ++kk) s += lds_eh[0][kk * kS + l.k * 16 + l.i];
    float* pc = a.part_ch + ((part * a.batch + l.b) * dimp + l.c) * 18;
    if (l.k < N) pc[l.k] = s;
    if (l.k == 0 || l.k == 1) {
      float t = 0.0f;
#pragma unroll
      for (int kk = 0; kk < R; ++kk) t += lds_m[l.k * R * 16 + kk * 16 + l.i];
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
    const int64_t gstride = a.seqlen * a.dstate;
    const float* pb = a.part_bc + b * a.ngroups * gstride + r;
    float sb = 0.0f, sc = 0.0f;
    // eight groups' loads are issued before they are added (in group order, as one by one):
    // with few outputs per CU (130M: 4 workgroups) a load-add chain left the reads latency
    // bound at ~3.7 TB/s
    int64_t g = 0;
    for (; g + 8 <= a.ngroups; g += 8) {
      float vb[8], vc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        vb[k] = pb[(g + k) * gstride];
        vc[k] = pb[plane + (g + k) * gstride];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        sb += vb[k];
        sc += vc[k];
      }
    }
    for (; g < a.ngroups; ++g) {
      sb += pb[g * gstride];
      sc += pb[plane + g * gstride];
    }
    a.dB[j] = sb;
    a.dC[j] = sc;
  }
  const int64_t jc = j - nbc;
  if (jc >= 0 && jc < a.dim * (a.dstate + 2)) {
    const int64_t d = jc / (a.dstate + 2), q = jc % (a.dstate + 2);
    const int slot = q < a.dstate ? static_cast<int>(q) : static_cast<int>(16 + (q - a.dstate));
    float s = 0.0f;
    const int64_t nparts = a.parts > 1 ? a.parts : 1;
    for (int64_t p = 0; p < nparts; ++p)
      for (int64_t b = 0; b < a.batch; ++b) s += a.part_ch[((p * a.batch + b) * dimp + d) * 18 + slot];
    if (q < a.dstate) a.dA[d * a.dstate + q] = s;
    else if (q == a.dstate) { if (a.dD) a.dD[d] = s; }
    else if (a.dbias) a.dbias[d] = s;
  }
}

template <typename T, int TC, int R>
void launch_bwd_scans(const BwdArgs& a, hipStream_t s) {
  const unsigned groups = static_cast<unsigned>(a.batch * a.ngroups);
  BwdArgs c = a;  // the checkpoint kernel runs its own parts
  c.parts = a.ckpt_parts;
  c.part_len = a.ckpt_part_len;
  // each split kernel starts from a cleared region header and flags (ss_split.h)
  if (c.parts > 1) {
    (void)split::clear(a.split_ws, a.split_cap, s);
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, 8, R, true>), dim3(groups * c.parts), dim3(R * 16), 0, s, c);
  } else {
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, 8, R, false>), dim3(groups), dim3(R * 16), 0, s, c);
  }
  const dim3 grid(groups * static_cast<unsigned>(a.parts > 1 ? a.parts : 1));
  if (a.parts > 1) {
    (void)split::clear(a.split_ws, a.split_cap, s);
    if (a.z)
      hipLaunchKernelGGL((bwd_chunked_kernel<T, true, TC, R, true>), grid, dim3(R * 16), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_chunked_kernel<T, false, TC, R, true>), grid, dim3(R * 16), 0, s, a);
  } else {
    if (a.z)
      hipLaunchKernelGGL((bwd_chunked_kernel<T, true, TC, R, false>), grid, dim3(R * 16), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_chunked_kernel<T, false, TC, R, false>), grid, dim3(R * 16), 0, s, a);
  }
}

template <typename T, int TC>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  if (a.rows == 32)
    launch_bwd_scans<T, TC, 32>(a, s);
  else
    launch_bwd_scans<T, TC, 16>(a, s);
  const int64_t total = a.batch * a.seqlen * a.dstate + a.dim * (a.dstate + 2);
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t bwd_tile_tokens() { return 16 * kBwdChunk; }

// 32 rows (8 waves, one workgroup per CU at two waves per SIMD) or 16 (4 waves, two per CU).
// A CU finishes one 8-wave workgroup's group in ~0.6 of the time it takes for two 4-wave
// workgroups sharing it (L = 32K, bf16: 256 groups 4.45 ms with 32 rows, 512 groups 7.4 ms
// with 16), so 32 rows pay while their rounds (with the split) stay under 1/0.6 of the one
// round that 16-row pairs need for at most two groups per CU.
int bwd_rows(int64_t groups, int64_t seqlen, int cus) {
  if (groups >= 2 * static_cast<int64_t>(cus)) return 16;
  const int p = bwd_split_parts(groups, 32, false, seqlen, cus);
  const double rounds = static_cast<double>((groups * p + cus - 1) / cus) / p;
  return 0.6 * (rounds > 1.0 ? rounds : 1.0) < 1.0 ? 32 : 16;
}

size_t bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  const int64_t ngroups = (dim + 15) / 16, dimp = ngroups * 16;
  const int64_t ntiles = seqlen > 0 ? (seqlen + bwd_tile_tokens() - 1) / bwd_tile_tokens() : 0;
  const int64_t floats = batch * ntiles * dimp * 16              // tile-start states
                         + 2 * batch * ngroups * seqlen * dstate  // dB, dC per channel group
                         + kBwdMaxParts * batch * dimp * 18;      // dA, dD, dbias per part and row
  return static_cast<size_t>(floats) * sizeof(float);
}

// Parts of whole tiles of both kernels (the checkpoint kernel's tile, R * 8 tokens, is the
// longer).
int64_t bwd_split_part_len(int64_t seqlen, int rows, int parts) {
  const int64_t tile = static_cast<int64_t>(rows) * 8;
  const int64_t per = (seqlen + parts - 1) / parts;
  return (per + tile - 1) / tile * tile;
}

// When the groups leave part of the last round of resident slots empty, split as the forward
// does: the fewest parts within 5% of the best of max(1, ceil(groups * parts / slots) /
// parts). The reverse kernel (~205-215 VGPRs) holds one 32-row or two 16-row workgroups per CU,
// the checkpoint kernel (at most 128 VGPRs with 16 rows, 35 KB of LDS) one 32-row or four
// 16-row ones. At the 130M shape (768 groups
// of 16-row tiles) the reverse kernel's two parts took it from 569 to 526 us, and the
// checkpoint kernel, whose slots hold all 768 groups at once, ran 9 us slower split; at 1024 groups
// (two whole rounds of the reverse kernel) two parts measured 2% slower.
int bwd_split_parts(int64_t groups, int rows, bool ckpt, int64_t seqlen, int cus) {
  const int64_t slots = static_cast<int64_t>(rows == 32 ? 1 : (ckpt ? 4 : 2)) * cus;
  if (groups <= slots || seqlen <= 0) return 1;
  auto time = [&](int p) {
    const double rounds = static_cast<double>((groups * p + slots - 1) / slots);
    return rounds / p > 1.0 ? rounds / p : 1.0;
  };
  int best = 1;
  double tbest = time(1);
  for (int p = 2; p <= kBwdMaxParts; ++p) {
    const int64_t len = bwd_split_part_len(seqlen, rows, p);
    if ((seqlen + len - 1) / len != p) continue;  // too short for p parts of whole tiles
    if (time(p) < 0.95 * tbest) {
      best = p;
      tbest = time(p);
    }
  }
  return best;
}

hipError_t bwd(const BwdArgs& a, hipStream_t s) {
  return a.dtype == kBF16 ? launch_bwd_t<uint16_t, kBwdChunk>(a, s) : launch_bwd_t<float, kBwdChunk>(a, s);
}

}  // namespace ss
