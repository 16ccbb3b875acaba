// ss_proj.hip -- the input projections of the selective scan on the matrix cores (gfx950).
//
// B_t, C_t and the step are linear maps of the token's input vector ("Mamba：选择性状态空间
// 模型入门教程", section "Mamba 的关键创新：选择性机制"; "Mamba：选择性状态空间的线性时间
// 序列建模", table "算法对比（核心直觉）": s_B(x_t), s_C(x_t) of shape (B, L, N)), the step
// map taken low-rank: for every token t,
//   xp_t = W_x u_t (rank + 2N outputs), delta_raw_t = W_dt xp_t[0:rank],
//   B_t = xp_t[rank : rank+N], C_t = xp_t[rank+N : rank+2N].
// Optionally u_t is formed on the fly from the block input x as silu(conv_b + sum of the causal
// depthwise conv taps over x_{t-K+1..t}) (the short convolution and SiLU in front of the SSM,
// "Mamba：选择性状态空间的线性时间序列建模", section "架构：极简设计"), so u never goes
// through HBM. Both products are dense contractions and run on MFMA:
// v_mfma_f32_16x16x4_f32 for fp32 operands, v_mfma_f32_16x16x32_bf16 for bf16, fp32
// accumulation either way.
//
// A workgroup is 4 waves and owns TOK = 16 S consecutive tokens (S strips of 16).
//  * Phase 1 (xp^T = W_x X^T) is split over K: wave w takes a quarter of the channel lines
//    and computes all T1 = RT + 2 output tiles (RT for the step part, rows >= rank zero; one
//    for B, one for C) for all S strips, so each fragment it loads feeds T1 or S MFMAs and
//    nothing is shared in the main loop. Both operands come straight from global memory as
//    whole 128-byte lines (two K blocks per stage), turned into MFMA fragments with one DPP
//    row rotate per register; each tile's registers are reloaded for the next stage right
//    after they are turned into fragments, so one stage of products covers every load.
//    With the convolution, the window x_{t-1..t-3} of lane i is taken from lanes i-1..i-3 of
//    the same 16-lane row (DPP row rotates; the previous strip, or a halo load for the first
//    one, supplies the rows' first lanes), and a token whose window crosses the start of its
//    sequence takes the conv state (or zeros) there. A bf16 convolution output enters the
//    MFMA as a hi and a lo bf16 part, so it keeps ~2^-17 relative precision.
//  * The four partial sums of every (strip, tile) are added in a fixed order through LDS,
//    two (strip, tile) units per wave per round; B and C leave from there, the step part goes
//    to an LDS copy of xp (fp32, or bf16 hi and lo parts).
//  * Phase 2 computes delta_raw^T = W_dt xp^T: wave w takes every fourth group of 16 TG
//    channels, with the W_dt fragments (the A operand) from global memory as line pairs of K
//    steps, reloaded for the next group as they are used, and the xp fragments (the B
//    operand) from the LDS copy. The A rows of a group are permuted so that each lane ends up
//    with consecutive channels of one token: every store is 16 bytes of a row.
// The loads are bound by the L1's request rate (64-byte requests, a few dozen in flight per
// CU), so the weights, which every workgroup reads in full, set the time at small token
// counts.
// Shapes the host side guarantees: dim % 8 == 0, rank % 8 == 0, rank <= 16 RT, dstate <= 16,
// 16-byte aligned u, W_x, W_dt and delta_raw, element-aligned B and C, 1 <= kconv <= 4.
#include "ss_chunk_ops.h"

namespace ss {
namespace {

using chunk::kDropOffset;
using chunk::rsrc;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// MFMA step e of a 16-byte K block: fp32 takes 4 steps of K = 4 (element e of each operand),
// bf16 one step of K = 32.
__device__ __forceinline__ f32x4 mfma_step(float*, const u32x4& a, const u32x4& b, int e, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_step(uint16_t*, const u32x4& a, const u32x4& b, int, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                 0, 0, 0);
}

// Lane i of each 16-lane row receives lane (i - J) mod 16 of the same row.
template <int J>
__device__ __forceinline__ u32x4 row_ror(const u32x4& v) {
  u32x4 r;
#pragma unroll
  for (int d = 0; d < 4; ++d)
    r[d] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v[d]), 0x120 + J, 0xf, 0xf, false));
  return r;
}

// Full-line loads to MFMA fragments. Load h of a 16-row block gives lane (i, q) row 8h + (i & 7),
// 16-byte piece q + 4 (i >> 3) of a 128-byte line (each load reads 8 whole lines: the L1
// tags and requests go by the line, and half-line loads run at half the rate); the fragment
// of the line's half t wants row i, piece q + 4t in lane (i, q). Rows i < 8 of half 0 and
// rows i >= 8 of half 1 are already in place; the rest are 8 lanes away in the other load.
__device__ __forceinline__ void line_halves(const u32x4& g0, const u32x4& g1, int li, u32x4& t0, u32x4& t1) {
  const u32x4 r0 = row_ror<8>(g0), r1 = row_ror<8>(g1);
  const bool lo = li < 8;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    t0[d] = lo ? g0[d] : r1[d];
    t1[d] = lo ? r0[d] : g1[d];
  }
}

// the CH channel values of a 16-byte piece as floats
__device__ __forceinline__ void unpack(float*, const u32x4& v, float (&f)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(v[e]);
}
__device__ __forceinline__ void unpack(uint16_t*, const u32x4& v, float (&f)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = __uint_as_float(v[d] << 16);
    f[2 * d + 1] = __uint_as_float(v[d] & 0xffff0000u);
  }
}

template <typename T, int RT, int S, bool CONV>
__global__ __launch_bounds__(256) void proj_kernel(ProjArgs a) {
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr bool BF = ES == 2;
  constexpr int T1 = RT + 2;            // phase-1 output tiles
  constexpr int CH = 16 / ES;           // channels per lane and stage
  constexpr int KBW = 4 * CH;           // channels per K block (16 fp32, 32 bf16)
  constexpr int KSTEP = BF ? 1 : 4;     // MFMA steps per 16-byte K block
  constexpr int TOK = 16 * S;
  constexpr int RC = 8 / S;             // tiles per reduction round (8 units, 2 per wave)
  constexpr int NR = (T1 + RC - 1) / RC;
  constexpr int NS = BF ? RT / 2 : RT;  // phase-2 K steps (32 ranks bf16, 16 ranks fp32)
  constexpr int TG = BF ? 4 : 2;        // phase-2 tiles per group
  constexpr int GC = 16 * TG;           // channels per phase-2 group
  constexpr int XS = BF ? 16 * RT + 8 : 16 * RT + 4;  // xp copy row stride (elements; odd 16-byte units)
  T* tag = nullptr;

  __shared__ f32x4 part[2][4][8][64];                   // partial tiles, double-buffered by round
  __shared__ __attribute__((aligned(16))) T xph[TOK * XS];               // xp (fp32) or its hi part
  __shared__ __attribute__((aligned(16))) uint16_t xpl[BF ? TOK * XS : 8];  // bf16 lo part
  __shared__ __attribute__((aligned(16))) float cwl[CONV ? 4 * 2 * 5 * 2 * KBW : 4];  // conv taps per wave

  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int li = l & 15, lq = l >> 4;
  const int64_t M = a.tokens, dim = a.dim, N = a.dstate, rank = a.rank;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TOK;
  const int64_t row_bytes = dim * ES;

  // ---- phase 1 -------------------------------------------------------------------------------
  // A stage is one 128-byte line of every row: two K blocks of KBW channels.
  constexpr int KL = 2 * KBW;
  const int lr = li & 7, lp = lq + 4 * (li >> 3);  // row within 8 and 16-byte piece of a line load
  const int64_t nkb = (dim + KL - 1) / KL;
  const int64_t kb_lo = nkb * w / 4, kb_hi = nkb * (w + 1) / 4;

  // this workgroup's input rows (and, with the convolution, the 16 before them)
  const int hb = (CONV && tok0 >= 16) ? 16 : 0;
  const int64_t rows_here = (M - tok0 + hb) < (TOK + hb) ? (M - tok0 + hb) : (TOK + hb);
  const auto rx = rsrc(static_cast<const T*>(a.u) + (tok0 - hb) * dim, rows_here * row_bytes);
  uint32_t xoff[S][2];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) xoff[s][h] = static_cast<uint32_t>((hb + 16 * s + 8 * h + lr) * row_bytes);
  uint32_t hoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) hoff[h] = hb ? static_cast<uint32_t>((8 * h + lr) * row_bytes) : kDropOffset;

  const auto rwx = rsrc(a.W_x, (rank + 2 * N) * row_bytes);
  uint32_t woff[T1][2];  // byte offset of row 8h + lr of each tile (kDropOffset: a zero row)
#pragma unroll
  for (int c = 0; c < T1; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = 8 * h + lr;
      int64_t r = -1;
      if (c < RT) r = 16 * c + i < rank ? 16 * c + i : -1;
      else if (i < N) r = (c == RT ? rank : rank + N) + i;
      woff[c][h] = r >= 0 ? static_cast<uint32_t>(r * row_bytes) : kDropOffset;
    }

  // convolution: taps right-aligned to 4 (zeros in front for kconv < 4) and the bias
  const int K = a.kconv;
  const auto rcw = rsrc(a.conv_w, CONV ? dim * K * 4 : 0);
  const auto rcb = rsrc(a.conv_b, (CONV && a.conv_b) ? dim * 4 : 0);
  const auto rcs = rsrc(a.conv_state, (CONV && a.conv_state) ? (M / a.seqlen) * dim * (K - 1) * 4 : 0);
  int pc[S];  // min(position in the sequence, 3) of this lane's token in each strip
  if constexpr (CONV) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t p = (tok0 + 16 * s + li) % a.seqlen;
      pc[s] = p < 3 ? static_cast<int>(p) : 3;
    }
  }

  f32x4 acc[S][T1];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int c = 0; c < T1; ++c) acc[s][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Raw line loads of the next stage. Each stage reloads a tile's registers right after
  // turning them into fragments, so one stage of products covers every load and the live
  // registers stay near one stage's worth.
  u32x4 wr[T1][2], xr[S][2], hr[2];
  float cr[5];
  // (issued for every stage, also past the wave's last block, where every offset is dropped:
  // loads under a branch would make the compiler wait for all of them before each stage)
  auto load_w = [&](int c, int64_t kb) {
    const int64_t kk = kb * KL + lp * CH;
    const bool in = kb < kb_hi && kk < dim;
    const uint32_t ko = static_cast<uint32_t>(kk * ES);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      wr[c][h] = __builtin_amdgcn_raw_buffer_load_b128(
          rwx, (in && woff[c][h] != kDropOffset) ? woff[c][h] + ko : kDropOffset, 0, 0);
  };
  auto load_x = [&](int64_t kb) {
    const int64_t kk = kb * KL + lp * CH;
    const bool in = kb < kb_hi && kk < dim;
    const uint32_t ko = static_cast<uint32_t>(kk * ES);
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        xr[s][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xoff[s][h] + ko : kDropOffset, 0, 0);
    if constexpr (CONV) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        hr[h] = __builtin_amdgcn_raw_buffer_load_b128(rx, (in && hb) ? hoff[h] + ko : kDropOffset, 0, 0);
      // lane l < KL: the taps and bias of channel kb*KL + l
      const int64_t ch = kb * KL + l;
      const bool cin = kb < kb_hi && l < KL && ch < dim;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int t = m - (4 - K);
        const uint32_t off = (cin && t >= 0) ? static_cast<uint32_t>((ch * K + t) * 4) : kDropOffset;
        cr[m] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rcw, off, 0, 0));
      }
      cr[4] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rcb, (cin && a.conv_b) ? static_cast<uint32_t>(ch * 4) : kDropOffset, 0, 0));
    }
  };

  // the B operands of one stage: the inputs, or u from the convolution over them (bf16: a hi
  // and a lo part, BP = 2 operands per strip and K block)
  constexpr int BP = (CONV && BF) ? 2 : 1;
  auto make_operands = [&](int64_t kb, u32x4 (&xb)[S][2][BP]) {
    u32x4 xf[S][2];
#pragma unroll
    for (int s = 0; s < S; ++s) line_halves(xr[s][0], xr[s][1], li, xf[s][0], xf[s][1]);
    if constexpr (!CONV) {
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) xb[s][kh][0] = xf[s][kh];
    } else {
      u32x4 hf[2];
      line_halves(hr[0], hr[1], li, hf[0], hf[1]);
      // the stage's taps through a wave-private LDS slot, read back per lane's channels
      float* cs = cwl + (w * 2 + static_cast<int>(kb & 1)) * (5 * KL);
      if (l < KL) {
#pragma unroll
        for (int m = 0; m < 5; ++m) cs[m * KL + l] = cr[m];
      }
      // (LDS executes a wave's operations in order; the fences only keep the compiler from
      // moving the accesses across the other lanes' writes)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float wv[5][CH];
#pragma unroll
        for (int m = 0; m < 5; ++m)
#pragma unroll
          for (int v = 0; v < CH / 4; ++v) {
            const f32x4 t4 = *reinterpret_cast<const f32x4*>(cs + m * KL + kh * KBW + lq * CH + 4 * v);
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[m][4 * v + e] = t4[e];
          }
        const int64_t ch0 = kb * KL + kh * KBW + lq * CH;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const u32x4 cur = xf[s][kh];
          const u32x4 prev = s == 0 ? hf[kh] : xf[s - 1][kh];
          // window position m holds x_{t-3+m}; the value lane i needs from x_{t-J} sits in lane
          // i - J of this strip or, for i < J, in lane 16 + i - J of the previous one: select
          // at the source lane, then rotate
          u32x4 sel1, sel2, sel3;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            sel1[d] = li < 15 ? cur[d] : prev[d];
            sel2[d] = li < 14 ? cur[d] : prev[d];
            sel3[d] = li < 13 ? cur[d] : prev[d];
          }
          float xw[4][CH];
          unpack(tag, cur, xw[3]);
          unpack(tag, row_ror<1>(sel1), xw[2]);
          unpack(tag, row_ror<2>(sel2), xw[1]);
          unpack(tag, row_ror<3>(sel3), xw[0]);
          if (pc[s] < 3) {  // the window reaches before the sequence: conv state or zeros there
            const int p = pc[s];
            const int64_t tok = tok0 + 16 * s + li;
            const int64_t b = tok / a.seqlen;
#pragma unroll
            for (int jj = 1; jj <= 3; ++jj) {
              if (jj > p) {
                const int idx = (K - 1) + p - jj;  // position in the conv state, oldest first
#pragma unroll
                for (int e = 0; e < CH; ++e) {
                  const int64_t ch = ch0 + e;
                  const bool ok = a.conv_state && idx >= 0 && tok < M && ch < dim;
                  const uint32_t off =
                      ok ? static_cast<uint32_t>(((b * dim + ch) * (K - 1) + idx) * 4) : kDropOffset;
                  xw[3 - jj][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rcs, off, 0, 0));
                }
              }
            }
            // wait here (vmcnt(0)) for these loads: waited for after the branch, they would
            // make every stage wait for all the prefetched ones
            __builtin_amdgcn_s_waitcnt(0x0f70);
          }
          float uv[CH];
#pragma unroll
          for (int e = 0; e < CH; ++e) {
            float p = wv[4][e];
            p = __builtin_fmaf(wv[0][e], xw[0][e], p);
            p = __builtin_fmaf(wv[1][e], xw[1][e], p);
            p = __builtin_fmaf(wv[2][e], xw[2][e], p);
            p = __builtin_fmaf(wv[3][e], xw[3][e], p);
            uv[e] = silu(p);
          }
          if constexpr (!BF) {
            xb[s][kh][0] = u32x4{__float_as_uint(uv[0]), __float_as_uint(uv[1]), __float_as_uint(uv[2]),
                                 __float_as_uint(uv[3])};
          } else {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t h0 = bf16_bits(uv[2 * d]), h1 = bf16_bits(uv[2 * d + 1]);
              const uint32_t l0 = bf16_bits(uv[2 * d] - bf16_value(h0)), l1 = bf16_bits(uv[2 * d + 1] - bf16_value(h1));
              xb[s][kh][0][d] = h0 | (h1 << 16);
              xb[s][kh][BP - 1][d] = l0 | (l1 << 16);
            }
          }
        }
      }
    }
  };

  // (the prologue issues its loads in the loop's order, so the waits at the loop head can
  // count on it)
  load_x(kb_lo);
#pragma unroll
  for (int c = 0; c < T1; ++c) {
    __builtin_amdgcn_sched_barrier(0);
    load_w(c, kb_lo);
  }
  for (int64_t kb = kb_lo; kb < kb_hi; ++kb) {
    // (scheduling barriers keep each reload right after the fragments it replaces were made
    // and ahead of the products: left alone, the scheduler moves loads down and products up)
    __builtin_amdgcn_sched_barrier(0);
    u32x4 xb[S][2][BP];
    make_operands(kb, xb);
    __builtin_amdgcn_sched_barrier(0);
    load_x(kb + 1);
#pragma unroll
    for (int c = 0; c < T1; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      u32x4 wf[2];
      line_halves(wr[c][0], wr[c][1], li, wf[0], wf[1]);
      load_w(c, kb + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < KSTEP; ++e)
#pragma unroll
          for (int b = 0; b < BP; ++b)
#pragma unroll
            for (int s = 0; s < S; ++s) acc[s][c] = mfma_step(tag, wf[kh], xb[s][kh][b], e, acc[s][c]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- reduction of the four K quarters ------------------------------------------------------
  {
    const auto rb = rsrc(static_cast<T*>(a.B) + tok0 * N, (M - tok0) * N * ES);
    const auto rc = rsrc(static_cast<T*>(a.C) + tok0 * N, (M - tok0) * N * ES);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int buf = r & 1;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int cc = 0; cc < RC; ++cc)
          if (r * RC + cc < T1) part[buf][w][s * RC + cc][l] = acc[s][r * RC + cc];
      __syncthreads();
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int unit = w + 4 * uu, s = unit / RC, c = r * RC + unit % RC;
        if (c < T1) {
          const f32x4 v = ((part[buf][0][unit][l] + part[buf][1][unit][l]) + part[buf][2][unit][l]) +
                          part[buf][3][unit][l];
          const int tl = 16 * s + li;  // lane (li, lq) holds xp[token tl][16 c + 4 lq + 0..3]
          if (c < RT) {
            if constexpr (BF) {
              uint32_t h[4], lo[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                h[e] = bf16_bits(v[e]);
                lo[e] = bf16_bits(v[e] - bf16_value(h[e]));
              }
              *reinterpret_cast<u32x2*>(xph + tl * XS + 16 * c + 4 * lq) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
              *reinterpret_cast<u32x2*>(xpl + tl * XS + 16 * c + 4 * lq) =
                  u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
            } else {
              *reinterpret_cast<f32x4*>(xph + tl * XS + 16 * c + 4 * lq) = v;
            }
          } else {
            const auto& ro = c == RT ? rb : rc;
            const int n0 = 4 * lq;
            if (N == 16) {
              const uint32_t off = static_cast<uint32_t>((tl * 16 + n0) * ES);
              if constexpr (BF) {
                const u32x2 pk = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
                __builtin_amdgcn_raw_buffer_store_b64(pk, ro, off, 0, 0);
              } else {
                __builtin_amdgcn_raw_buffer_store_b128(
                    u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])},
                    ro, off, 0, 0);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t off = n0 + e < N ? static_cast<uint32_t>((tl * N + n0 + e) * ES) : kDropOffset;
                if constexpr (BF)
                  __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_bits(v[e])), ro, off, 0, 0);
                else
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), ro, off, 0, 0);
              }
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- phase 2: delta_raw^T = W_dt xp^T --------------------------------------------------------
  const auto rdt = rsrc(a.W_dt, dim * rank * ES);
  const auto rd = rsrc(static_cast<T*>(a.delta_raw) + tok0 * dim, (M - tok0) * row_bytes);
  const int64_t ngroups = (dim + GC - 1) / GC;
  const int64_t ngw = ngroups > w ? (ngroups - w + 3) / 4 : 0;
  // W_dt fragments come as line pairs of K steps (128 bytes of a row), like phase 1's loads
  constexpr int NP = (NS + 1) / 2;
  constexpr int SW = BF ? 32 : 16;  // ranks per K step
  u32x4 vr[NP][TG][2];  // raw line loads of the next group, reloaded as they are used
  // Row i of tile t in group g: bf16 pairs (t even, t odd) take channels so that lane
  // (i, q) ends with channels 32 (t/2) + 8q .. + 7; fp32 tile t takes 16 t + i.
  auto dt_chan = [&](int64_t g, int t, int i) -> int64_t {
    if constexpr (BF) return g * GC + 32 * (t >> 1) + 8 * (i >> 2) + 4 * (t & 1) + (i & 3);
    else return g * GC + 16 * t + i;
  };
  auto load_dt = [&](int p, int t, int64_t g, bool live) {  // live = false: all dropped
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t d = live ? dt_chan(g, t, 8 * h + lr) : dim;
      const int64_t kk = 2 * p * SW + lp * CH;
      const uint32_t off = (d < dim && kk < rank) ? static_cast<uint32_t>((d * rank + kk) * ES) : kDropOffset;
      vr[p][t][h] = __builtin_amdgcn_raw_buffer_load_b128(rdt, off, 0, 0);
    }
  };
  auto run_group = [&](int64_t g, bool next_live) {
    f32x4 o[S][TG];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int t = 0; t < TG; ++t) o[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // B operands of steps 2p, 2p+1 from the LDS copy of xp (bf16: hi and lo parts)
      constexpr int NB = BF ? 2 : 1;
      u32x4 bx[2][S][NB];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int st = 2 * p + kh;
        if (st >= NS) break;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          if constexpr (BF) {
            const int at = (16 * s + li) * XS + 32 * st + 8 * lq;
            bx[kh][s][0] = *reinterpret_cast<const u32x4*>(xph + at);
            bx[kh][s][NB - 1] = *reinterpret_cast<const u32x4*>(xpl + at);
          } else {
            bx[kh][s][0] = *reinterpret_cast<const u32x4*>(xph + (16 * s + li) * XS + 16 * st + 4 * lq);
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TG; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        u32x4 af[2];
        line_halves(vr[p][t][0], vr[p][t][1], li, af[0], af[1]);
        load_dt(p, t, g + 4, next_live);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (2 * p + kh >= NS) break;
#pragma unroll
          for (int e = 0; e < KSTEP; ++e)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
              for (int s = 0; s < S; ++s) o[s][t] = mfma_step(tag, af[kh], bx[kh][s][b], e, o[s][t]);
        }
      }
    }
    // lane (i, q), register r of tile t: delta_raw[token 16 s + i][channel of row 4q + r]
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t tl = 16 * s + li;
      if constexpr (BF) {
#pragma unroll
        for (int p = 0; p < TG / 2; ++p) {
          const int64_t d = g * GC + 32 * p + 8 * lq;
          const f32x4 e0 = o[s][2 * p], e1 = o[s][2 * p + 1];
          const u32x4 pk = {bf16_bits(e0[0]) | (bf16_bits(e0[1]) << 16), bf16_bits(e0[2]) | (bf16_bits(e0[3]) << 16),
                            bf16_bits(e1[0]) | (bf16_bits(e1[1]) << 16), bf16_bits(e1[2]) | (bf16_bits(e1[3]) << 16)};
          __builtin_amdgcn_raw_buffer_store_b128(
              pk, rd, d < dim ? static_cast<uint32_t>(tl * row_bytes + d * ES) : kDropOffset, 0, 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          const int64_t d = g * GC + 16 * t + 4 * lq;
          const f32x4 e0 = o[s][t];
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(e0[0]), __float_as_uint(e0[1]), __float_as_uint(e0[2]), __float_as_uint(e0[3])}, rd,
              d < dim ? static_cast<uint32_t>(tl * row_bytes + d * ES) : kDropOffset, 0, 0);
        }
      }
    }
  };

  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int t = 0; t < TG; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      load_dt(p, t, w, ngw > 0);
    }
  for (int64_t j = 0; j < ngw; ++j) run_group(w + 4 * j, j + 1 < ngw);
  __builtin_amdgcn_sched_barrier(0);
}

// Token-split variant for many tokens: each wave owns 64 tokens (four strips) and the whole K
// range, and the weights go through LDS once per workgroup of 256 tokens, so every weight byte
// fetched through L1 serves four times the tokens of the split-K kernel. Phase 1 stages one
// 128-byte line of every W_x row per step (two K blocks, double-buffered, one barrier per
// step); each wave reads its A fragments from there and its own inputs from global memory.
// The accumulators hold complete sums, so B, C and the phase-2 operands come straight from
// them. Phase 2 stages W_dt a group of 64 channels at a time (contiguous rows, read as whole
// lines) and every wave applies each group to its own tokens.
template <typename T, int RT>
__global__ __launch_bounds__(256) void proj_tok_kernel(ProjArgs a) {
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr bool BF = ES == 2;
  constexpr int T1 = RT + 2;
  constexpr int CH = 16 / ES;
  constexpr int KBW = 4 * CH;
  constexpr int KL = 2 * KBW;                       // channels per staged line
  constexpr int KSTEP = BF ? 1 : 4;
  constexpr int S = 4;                              // strips per wave
  constexpr int NS = BF ? RT / 2 : RT;              // phase-2 K steps
  constexpr int TG = 4, GC = 64;                    // phase-2 tiles and channels per group
  constexpr int LROW = 144;                         // staged W_x row: one line + 16 bytes
  constexpr int WST = T1 * 16 * LROW;               // one staged line of every tile
  constexpr int WPT = (T1 * 128 + 255) / 256;       // 16-byte pieces per thread and step
  constexpr int DROW = 16 * RT * ES + 16;           // staged W_dt row (bytes)
  constexpr int DST = GC * DROW;
  constexpr int DPT = (GC * RT * ES + 255) / 256;   // 16-byte pieces per thread and group
  constexpr int JUNK = (WST > DST ? WST : DST) * 2;  // 16 bytes per thread for pieces past the end
  __shared__ __attribute__((aligned(16))) unsigned char lds[JUNK + 256 * 16];
  T* tag = nullptr;

  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int li = l & 15, lq = l >> 4;
  const int lr = li & 7, lp = lq + 4 * (li >> 3);
  const int64_t M = a.tokens, dim = a.dim, N = a.dstate, rank = a.rank;
  const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * (64 * S);
  const int64_t row_bytes = dim * ES;
  const int tw = 64 * w;  // this wave's first token within the workgroup

  // ---- phase 1 ------------------------------------------------------------------------------
  const int64_t nkb = (dim + KL - 1) / KL;
  const int64_t rows_here = (M - tok0) < 64 * S ? (M - tok0) : 64 * S;
  const auto rx = rsrc(static_cast<const T*>(a.u) + tok0 * dim, rows_here * row_bytes);
  uint32_t xoff[S][2];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) xoff[s][h] = static_cast<uint32_t>((tw + 16 * s + 8 * h + lr) * row_bytes);

  // staging map: piece k = tid + 256 j is tile k / 128, row (k / 8) % 16, 16-byte piece k % 8
  const auto rwx = rsrc(a.W_x, (rank + 2 * N) * row_bytes);
  uint32_t goff[WPT], loff[WPT];
  int gpc[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int k = tid + 256 * j;
    const int c = k >> 7, r = (k >> 3) & 15, pc = k & 7;
    int64_t row = -1;
    if (k < T1 * 128) {
      if (c < RT) row = 16 * c + r < rank ? 16 * c + r : -1;
      else if (r < N) row = (c == RT ? rank : rank + N) + r;
    }
    goff[j] = row >= 0 ? static_cast<uint32_t>(row * row_bytes) : kDropOffset;
    // (a piece past the last tile loads nothing and is stored to this thread's junk slot:
    // stores under a branch would make the compiler wait for every load in flight)
    loff[j] = k < T1 * 128 ? static_cast<uint32_t>(c * 16 * LROW + r * LROW + pc * 16)
                           : static_cast<uint32_t>(JUNK + 16 * tid);
    gpc[j] = k < T1 * 128 ? pc : -1;
  }
  u32x4 wst[WPT], xr[S][2];
  auto load_w = [&](int64_t kb) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int64_t kk = kb * KL + gpc[j] * CH;
      const bool in = gpc[j] >= 0 && kb < nkb && kk < dim && goff[j] != kDropOffset;
      wst[j] = __builtin_amdgcn_raw_buffer_load_b128(rwx, in ? goff[j] + static_cast<uint32_t>(kk * ES) : kDropOffset,
                                                     0, 0);
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int j = 0; j < WPT; ++j)
      *reinterpret_cast<u32x4*>(lds + (gpc[j] >= 0 ? buf * WST + loff[j] : loff[j])) = wst[j];
  };
  auto load_x = [&](int64_t kb) {
    const int64_t kk = kb * KL + lp * CH;
    const bool in = kb < nkb && kk < dim;
    const uint32_t ko = static_cast<uint32_t>(kk * ES);
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        xr[s][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xoff[s][h] + ko : kDropOffset, 0, 0);
  };

  f32x4 acc[S][T1];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int c = 0; c < T1; ++c) acc[s][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Step kb: after the barrier the staged line kb is complete in buffer kb & 1 and every wave
  // is done with buffer (kb + 1) & 1, which then takes line kb + 1 (loaded during step kb - 1).
  load_w(0);
  store_w(0);
  load_w(1);
  load_x(0);
  for (int64_t kb = 0; kb < nkb; ++kb) {
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    store_w(static_cast<int>((kb + 1) & 1));
    __builtin_amdgcn_sched_barrier(0);
    load_w(kb + 2);
    u32x4 xf[S][2];
#pragma unroll
    for (int s = 0; s < S; ++s) line_halves(xr[s][0], xr[s][1], li, xf[s][0], xf[s][1]);
    __builtin_amdgcn_sched_barrier(0);
    load_x(kb + 1);
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* lb = lds + static_cast<int>(kb & 1) * WST + li * LROW + lq * 16;
    // tile c + 1's fragments are read while tile c's products run
    u32x4 af[2][2];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) af[0][kh] = *reinterpret_cast<const u32x4*>(lb + kh * 64);
#pragma unroll
    for (int c = 0; c < T1; ++c) {
      if (c + 1 < T1) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
          af[(c + 1) & 1][kh] = *reinterpret_cast<const u32x4*>(lb + (c + 1) * 16 * LROW + kh * 64);
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < KSTEP; ++e)
#pragma unroll
          for (int s = 0; s < S; ++s) acc[s][c] = mfma_step(tag, af[c & 1][kh], xf[s][kh], e, acc[s][c]);
      // (keep the reads of tile c + 1 ahead of tile c's products)
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KSTEP * S, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- B and C: lane (i, q), register r of tile RT / RT+1 holds B / C[token i][4q + r] ---------
  {
    const auto rb = rsrc(static_cast<T*>(a.B) + tok0 * N, (M - tok0) * N * ES);
    const auto rc = rsrc(static_cast<T*>(a.C) + tok0 * N, (M - tok0) * N * ES);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int tl = tw + 16 * s + li;
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const f32x4 v = acc[s][RT + cc];
        const auto& ro = cc == 0 ? rb : rc;
        const int n0 = 4 * lq;
        if (N == 16) {
          const uint32_t off = static_cast<uint32_t>((tl * 16 + n0) * ES);
          if constexpr (BF) {
            const u32x2 pk = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16), bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(pk, ro, off, 0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}, ro,
                off, 0, 0);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t off = n0 + e < N ? static_cast<uint32_t>((tl * N + n0 + e) * ES) : kDropOffset;
            if constexpr (BF)
              __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_bits(v[e])), ro, off, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[e]), ro, off, 0, 0);
          }
        }
      }
    }
  }

  // ---- phase 2: delta_raw^T = W_dt xp^T ------------------------------------------------------
  // B operands from the accumulators: fp32 step (c, e) is register e of tile c (rank
  // 16c + 4q + e); bf16 step st packs tiles 2st and 2st+1 (ranks 32st + 16 (e/4) + 4q + e%4)
  // as a hi and a lo part.
  constexpr int NB = BF ? NS : 1;
  u32x4 xh[S][NB], xl[S][NB];
  if constexpr (BF) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint32_t hv[2], lv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int e = 2 * d + u;
            const float v = acc[s][2 * st + (e >> 2)][e & 3];
            hv[u] = bf16_bits(v);
            lv[u] = bf16_bits(v - bf16_value(hv[u]));
          }
          xh[s][st][d] = hv[0] | (hv[1] << 16);
          xl[s][st][d] = lv[0] | (lv[1] << 16);
        }
  }

  const auto rdt = rsrc(a.W_dt, dim * rank * ES);
  const auto rd = rsrc(static_cast<T*>(a.delta_raw) + tok0 * dim, (M - tok0) * row_bytes);
  const int64_t ngroups = (dim + GC - 1) / GC;
  const int64_t grp_bytes = GC * rank * ES;  // a group's rows are contiguous in W_dt
  uint32_t dl[DPT];
  int drow[DPT];
#pragma unroll
  for (int j = 0; j < DPT; ++j) {
    const int64_t o = 16 * static_cast<int64_t>(tid + 256 * j);
    const int64_t row = o / (rank * ES), col = o % (rank * ES);
    drow[j] = o < grp_bytes ? static_cast<int>(row) : -1;
    dl[j] = o < grp_bytes ? static_cast<uint32_t>(row * DROW + col) : static_cast<uint32_t>(JUNK + 16 * tid);
  }
  u32x4 dst[DPT];
  auto load_dt = [&](int64_t g) {
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
      const bool in = drow[j] >= 0 && g < ngroups && g * GC + drow[j] < dim;
      dst[j] = __builtin_amdgcn_raw_buffer_load_b128(
          rdt, in ? static_cast<uint32_t>(g * grp_bytes + 16 * (tid + 256 * j)) : kDropOffset, 0, 0);
    }
  };
  auto store_dt = [&](int buf) {
#pragma unroll
    for (int j = 0; j < DPT; ++j)
      *reinterpret_cast<u32x4*>(lds + (drow[j] >= 0 ? buf * DST + dl[j] : dl[j])) = dst[j];
  };

  __syncthreads();  // phase 1 is done with the staging area
  load_dt(0);
  store_dt(0);
  load_dt(1);
  for (int64_t g = 0; g < ngroups; ++g) {
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    store_dt(static_cast<int>((g + 1) & 1));
    __builtin_amdgcn_sched_barrier(0);
    load_dt(g + 2);
    __builtin_amdgcn_sched_barrier(0);
    const unsigned char* db = lds + static_cast<int>(g & 1) * DST;
    f32x4 o[S][TG];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int t = 0; t < TG; ++t) o[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // A fragment of (step st, tile t); the next one is read while the current products run
    auto read_a = [&](int st, int t) -> u32x4 {
      if constexpr (BF) {
        // row li of tile t: channel 32 (t/2) + 8 (li/4) + 4 (t%2) + li%4 of the group
        const int dm = 32 * (t >> 1) + 8 * (li >> 2) + 4 * (t & 1) + (li & 3);
        const unsigned char* rp = db + dm * DROW + (32 * st + 4 * lq) * 2;
        const u32x2 lo8 = *reinterpret_cast<const u32x2*>(rp);
        const u32x2 hi8 = *reinterpret_cast<const u32x2*>(rp + 32);
        return u32x4{lo8[0], lo8[1], hi8[0], hi8[1]};
      } else {
        return *reinterpret_cast<const u32x4*>(db + (16 * t + li) * DROW + (16 * st + 4 * lq) * 4);
      }
    };
    u32x4 av[2];
    av[0] = read_a(0, 0);
#pragma unroll
    for (int it = 0; it < NS * TG; ++it) {
      const int st = it / TG, t = it % TG;
      if (it + 1 < NS * TG) av[(it + 1) & 1] = read_a((it + 1) / TG, (it + 1) % TG);
      const u32x4 a0 = av[it & 1];
      if constexpr (BF) {
#pragma unroll
        for (int s = 0; s < S; ++s) o[s][t] = mfma_step(tag, a0, xh[s][st], 0, o[s][t]);
#pragma unroll
        for (int s = 0; s < S; ++s) o[s][t] = mfma_step(tag, a0, xl[s][st], 0, o[s][t]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int s = 0; s < S; ++s)
            o[s][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a0[e]), acc[s][st][e], o[s][t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, BF ? 2 : 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, BF ? 2 * S : 4 * S, 0);
    }
    // lane (i, q), register r of tile t: delta_raw[token i][channel of row 4q + r]
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t tl = tw + 16 * s + li;
      if constexpr (BF) {
#pragma unroll
        for (int pp = 0; pp < TG / 2; ++pp) {
          const int64_t d = g * GC + 32 * pp + 8 * lq;
          const f32x4 e0 = o[s][2 * pp], e1 = o[s][2 * pp + 1];
          const u32x4 pk = {bf16_bits(e0[0]) | (bf16_bits(e0[1]) << 16), bf16_bits(e0[2]) | (bf16_bits(e0[3]) << 16),
                            bf16_bits(e1[0]) | (bf16_bits(e1[1]) << 16), bf16_bits(e1[2]) | (bf16_bits(e1[3]) << 16)};
          __builtin_amdgcn_raw_buffer_store_b128(
              pk, rd, d < dim ? static_cast<uint32_t>(tl * row_bytes + d * ES) : kDropOffset, 0, 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < TG; ++t) {
          const int64_t d = g * GC + 16 * t + 4 * lq;
          const f32x4 e0 = o[s][t];
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(e0[0]), __float_as_uint(e0[1]), __float_as_uint(e0[2]), __float_as_uint(e0[3])}, rd,
              d < dim ? static_cast<uint32_t>(tl * row_bytes + d * ES) : kDropOffset, 0, 0);
        }
      }
    }
  }
}

// Strips per workgroup: the accumulators take 4 T1 S registers per lane, the convolution's
// window and taps about 100 more (the choices keep every variant free of spills).
constexpr int strips(int rt, bool conv, int es) {
  if (conv) return (rt <= 2 || (es == 4 && rt <= 4)) ? 4 : (rt <= 10 ? 2 : 1);
  return rt <= 10 ? 4 : ((rt <= 12 || es == 2) ? 2 : 1);
}

template <typename T, int RT, bool CONV>
hipError_t launch_proj(const ProjArgs& a, hipStream_t s) {
  constexpr int S = strips(RT, CONV, static_cast<int>(sizeof(T)));
  const int64_t per = 16 * S;
  const dim3 grid(static_cast<unsigned>((a.tokens + per - 1) / per));
  hipLaunchKernelGGL((proj_kernel<T, RT, S, CONV>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int RT>
hipError_t launch_proj_tok(const ProjArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.tokens + 255) / 256));
  hipLaunchKernelGGL((proj_tok_kernel<T, RT>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t proj_tok_t(const ProjArgs& a, int rt, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {
    if (rt == 3) return launch_proj_tok<T, 3>(a, s);
  }
  switch (rt) {
    case 2: return launch_proj_tok<T, 2>(a, s);
    case 4: return launch_proj_tok<T, 4>(a, s);
    case 6: return launch_proj_tok<T, 6>(a, s);
    case 8: return launch_proj_tok<T, 8>(a, s);
    default: return launch_proj_tok<T, 10>(a, s);
  }
}

template <typename T, bool CONV>
hipError_t proj_t(const ProjArgs& a, int rt, hipStream_t s) {
  if constexpr (sizeof(T) == 4) {  // fp32 also has 3 step tiles (rank 48: 1536 / 32)
    if (rt == 3) return launch_proj<T, 3, CONV>(a, s);
  }
  switch (rt) {
    case 2: return launch_proj<T, 2, CONV>(a, s);
    case 4: return launch_proj<T, 4, CONV>(a, s);
    case 6: return launch_proj<T, 6, CONV>(a, s);
    case 8: return launch_proj<T, 8, CONV>(a, s);
    case 10: return launch_proj<T, 10, CONV>(a, s);
    case 12: return launch_proj<T, 12, CONV>(a, s);
    default: return launch_proj<T, 16, CONV>(a, s);
  }
}

}  // namespace

// Step tiles: the smallest instantiated count covering rank (rank <= 256 by the host check);
// bf16 needs an even count (one MFMA step covers two tiles), fp32 also has 3.
int proj_step_tiles(int64_t rank, int dtype) {
  const int need = static_cast<int>((rank + 15) / 16);
  if (dtype != kBF16 && need == 3) return 3;
  for (int rt : {2, 4, 6, 8, 10, 12, 16})
    if (rt >= need) return rt;
  return 16;
}

hipError_t proj(const ProjArgs& a, int cus, hipStream_t s) {
  const int rt = proj_step_tiles(a.rank, a.dtype);
  const bool conv = a.kconv > 0;
  // the token-split kernel once there are enough tokens for a workgroup of 256 on every CU
  if (!conv && rt <= 10 && a.tokens >= 256 * static_cast<int64_t>(cus))
    return a.dtype == kBF16 ? proj_tok_t<uint16_t>(a, rt, s) : proj_tok_t<float>(a, rt, s);
  if (a.dtype == kBF16) return conv ? proj_t<uint16_t, true>(a, rt, s) : proj_t<uint16_t, false>(a, rt, s);
  return conv ? proj_t<float, true>(a, rt, s) : proj_t<float, false>(a, rt, s);
}

}  // namespace ss
