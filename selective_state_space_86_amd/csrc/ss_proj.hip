// ss_proj.hip -- the input projections of the selective scan on the matrix cores (gfx950).
//
// B_t, C_t and the step are linear maps of the token's input vector ("Mamba：选择性状态空间
// 模型入门教程", section "Mamba 的关键创新：选择性机制"; "Mamba：选择性状态空间的线性时间
// 序列建模", table "算法对比（核心直觉）": s_B(x_t), s_C(x_t) of shape (B, L, N)), the step
// map taken low-rank: for every token t,
//   xp_t = W_x u_t (rank + 2N outputs), delta_raw_t = W_dt xp_t[0:rank],
//   B_t = xp_t[rank : rank+N], C_t = xp_t[rank+N : rank+2N].
// Both products are dense contractions, so they run on MFMA: v_mfma_f32_16x16x4_f32 for fp32
// operands, v_mfma_f32_16x16x32_bf16 for bf16, fp32 accumulation either way.
//
// A workgroup is 4 waves; a wave owns S strips of 16 consecutive tokens.
//  * Phase 1 computes xp transposed, D = W_x X^T, in T1 = RT + 2 output tiles of 16 rows
//    (RT tiles for the step part, rows >= rank zero; one tile for B, one for C). The A operand
//    (W_x, shared by all waves) goes through LDS in chunks of 4 16-byte units per row; the B
//    operand (a strip's inputs) is loaded straight from HBM, 16 bytes per lane. Lane (i, q)
//    of a 16-byte unit holds channels k0 + (4h + q) * CH .. + CH - 1 (CH = 4 fp32 / 8 bf16),
//    and both operands use that same channel-to-K map, so the contraction covers every
//    channel once whatever order the MFMA steps take.
//  * The phase-1 accumulators are laid out exactly as the A operand of phase 2: lane
//    (token i, q) holds xp[i][16c + 4q + r] in register r of tile c. Phase 2 computes
//    delta_raw = xp[:, :rank] W_dt^T per 32-channel group with W_dt staged in LDS and no
//    transpose of the intermediate (fp32: K index 4q of step (c, r) is rank 16c + 4q + r;
//    bf16: one step covers tiles 2s and 2s+1, and the fp32 intermediate enters as a hi and a
//    lo bf16 part, two MFMAs, so its rounding stays near 2^-17 relative).
//  * B and C leave from tiles RT and RT + 1; delta_raw from the phase-2 accumulators. bf16
//    outputs are rounded to nearest even.
// Shapes the host side guarantees: dim % 8 == 0, rank % 8 == 0, rank <= 16 RT, dstate <= 16,
// 16-byte aligned u, W_x, W_dt and delta_raw.
#include "ss_chunk_ops.h"

namespace ss {
namespace {

using chunk::kDropOffset;
using chunk::rsrc;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kCh = 4;  // elements per 16-byte unit
};
template <>
struct Elem<uint16_t> {
  static constexpr int kCh = 8;
};

constexpr int kUnits = 4;       // 16-byte units per W_x row and phase-1 LDS chunk (one MFMA K block)
constexpr int kGroup = 32;      // channels per phase-2 group: two 16-channel output tiles

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// one K block of phase 1: a = 16 bytes of W_x, b = 16 bytes of the inputs
__device__ __forceinline__ f32x4 mfma_block(float*, const u32x4& a, const u32x4& b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ f32x4 mfma_block(uint16_t*, const u32x4& a, const u32x4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                 0, 0, 0);
}

__device__ __forceinline__ void store_elem(float*, __amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void store_elem(uint16_t*, __amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(static_cast<unsigned short>(bf16_bits(v)), r, off, 0, 0);
}

template <typename T, int RT, int S>
__global__ __launch_bounds__(256) void proj_kernel(ProjArgs a) {
  constexpr int T1 = RT + 2;                  // phase-1 output tiles
  constexpr int ROWS = T1 * 16;               // W_x rows staged per chunk (zeros where absent)
  constexpr int CH = Elem<T>::kCh;
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int RPU = RT * 16 / CH;           // 16-byte units per staged W_dt row (RT*16 ranks)
  constexpr int P1 = ROWS * (kUnits + 1);     // padded rows (one spare unit against bank conflicts)
  constexpr int P2 = kGroup * (RPU + 1);
  constexpr int HALF = P1 > P2 ? P1 : P2;
  __shared__ u32x4 lds[2 * HALF];
  T* tag = nullptr;

  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  const int li = l & 15, lq = l >> 4;
  const int64_t M = a.tokens, dim = a.dim, N = a.dstate, rank = a.rank;
  const int64_t wg_tok0 = static_cast<int64_t>(blockIdx.x) * (64 * S);
  const int64_t row_bytes = dim * ES;

  // inputs of this workgroup's tokens; tokens past M read 0 (range check)
  const auto ru = rsrc(static_cast<const T*>(a.u) + wg_tok0 * dim, (M - wg_tok0) * row_bytes);
  uint32_t xrow[S];
#pragma unroll
  for (int s = 0; s < S; ++s) xrow[s] = static_cast<uint32_t>((w * 16 * S + s * 16 + li) * row_bytes);

  // ---- phase 1: xp^T = W_x X^T ------------------------------------------------------------
  const auto rwx = rsrc(a.W_x, (rank + 2 * N) * row_bytes);
  constexpr int EPL = (ROWS * kUnits + 255) / 256;  // staged units per lane and chunk
  // source row of staged row r (-1: zero row)
  auto wx_row = [&](int r) -> int64_t {
    const int c = r >> 4, i = r & 15;
    if (c < RT) return 16 * c + i < rank ? 16 * c + i : -1;
    if (i >= N) return -1;
    return c == RT ? rank + i : rank + N + i;
  };
  auto load_wx = [&](u32x4 (&v)[EPL], int64_t k0) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const int e = tid + 256 * m;
      const int r = e / kUnits, un = e % kUnits;
      const int64_t kk = k0 + un * CH;
      const int64_t sr = e < ROWS * kUnits ? wx_row(r) : -1;
      const uint32_t off = (sr >= 0 && kk < dim) ? static_cast<uint32_t>((sr * dim + kk) * ES) : kDropOffset;
      v[m] = __builtin_amdgcn_raw_buffer_load_b128(rwx, off, 0, 0);
    }
  };
  auto store_wx = [&](const u32x4 (&v)[EPL], int buf) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const int e = tid + 256 * m;
      if (e < ROWS * kUnits) lds[buf * HALF + (e / kUnits) * (kUnits + 1) + e % kUnits] = v[m];
    }
  };
  auto load_x = [&](u32x4 (&x)[S], int64_t k0) {
    const int64_t kk = k0 + lq * CH;
#pragma unroll
    for (int s = 0; s < S; ++s)
      x[s] = __builtin_amdgcn_raw_buffer_load_b128(ru, kk < dim ? xrow[s] + static_cast<uint32_t>(kk * ES) : kDropOffset,
                                                   0, 0);
  };

  f32x4 acc[S][T1];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int c = 0; c < T1; ++c) acc[s][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int KB = kUnits * CH;  // channels per chunk
  const int64_t nchunks = (dim + KB - 1) / KB;
  {
    u32x4 wv[EPL];
    load_wx(wv, 0);
    store_wx(wv, 0);
  }
  __syncthreads();
  u32x4 xc[S], xn[S];
  load_x(xc, 0);
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int buf = static_cast<int>(ci & 1);
    const bool more = ci + 1 < nchunks;
    u32x4 wv[EPL];
    if (more) {
      load_wx(wv, (ci + 1) * KB);
      load_x(xn, (ci + 1) * KB);
    }
    const u32x4* lb = lds + buf * HALF;
#pragma unroll
    for (int c = 0; c < T1; ++c) {
      const u32x4 av = lb[(c * 16 + li) * (kUnits + 1) + lq];
#pragma unroll
      for (int s = 0; s < S; ++s) acc[s][c] = mfma_block(tag, av, xc[s], acc[s][c]);
    }
    if (more) {
      store_wx(wv, buf ^ 1);
#pragma unroll
      for (int s = 0; s < S; ++s) xc[s] = xn[s];
    }
    __syncthreads();
  }

  // ---- B and C ----------------------------------------------------------------------------
  {
    const int64_t bc0 = wg_tok0 * N;
    const auto rb = rsrc(static_cast<T*>(a.B) + bc0, (M - wg_tok0) * N * ES);
    const auto rc = rsrc(static_cast<T*>(a.C) + bc0, (M - wg_tok0) * N * ES);
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int64_t tok = w * 16 * S + s * 16 + li;  // local token of this lane's column
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = 4 * lq + r;
        const uint32_t off = n < N ? static_cast<uint32_t>((tok * N + n) * ES) : kDropOffset;
        store_elem(tag, rb, off, acc[s][RT][r]);
        store_elem(tag, rc, off, acc[s][RT + 1][r]);
      }
    }
  }

  // ---- phase 2: delta_raw = xp[:, :rank] W_dt^T --------------------------------------------
  // The intermediate as phase-2 A operands: fp32 uses acc directly; bf16 packs tiles 2s, 2s+1
  // into 8 bf16 values, as a hi part and a lo (remainder) part.
  constexpr int NS = (sizeof(T) == 4) ? RT : RT / 2;  // bf16 steps (RT is even for bf16)
  i16x8 ahi[S][NS > 0 ? NS : 1], alo[S][NS > 0 ? NS : 1];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = acc[s][2 * st + (e >> 2)][e & 3];
          const uint32_t h = bf16_bits(v);
          ahi[s][st][e] = static_cast<short>(h);
          alo[s][st][e] = static_cast<short>(bf16_bits(v - bf16_value(h)));
        }
  }

  const auto rdt = rsrc(a.W_dt, dim * rank * ES);
  constexpr int GPL = (kGroup * RPU + 255) / 256;  // staged W_dt units per lane and group
  auto load_dt = [&](u32x4 (&v)[GPL], int64_t d0) {
#pragma unroll
    for (int m = 0; m < GPL; ++m) {
      const int e = tid + 256 * m;
      const int r = e / RPU, un = e % RPU;  // channel row within the group, unit along rank
      const int64_t d = d0 + r, rk = static_cast<int64_t>(un) * CH;
      const uint32_t off = (e < kGroup * RPU && d < dim && rk < rank) ? static_cast<uint32_t>((d * rank + rk) * ES)
                                                                       : kDropOffset;
      v[m] = __builtin_amdgcn_raw_buffer_load_b128(rdt, off, 0, 0);
    }
  };
  auto store_dt = [&](const u32x4 (&v)[GPL], int buf) {
#pragma unroll
    for (int m = 0; m < GPL; ++m) {
      const int e = tid + 256 * m;
      if (e < kGroup * RPU) lds[buf * HALF + (e / RPU) * (RPU + 1) + e % RPU] = v[m];
    }
  };

  const auto rd = rsrc(static_cast<T*>(a.delta_raw) + wg_tok0 * dim, (M - wg_tok0) * row_bytes);
  const int64_t ngroups = (dim + kGroup - 1) / kGroup;
  {
    u32x4 dv[GPL];
    load_dt(dv, 0);
    store_dt(dv, 0);
  }
  __syncthreads();
  for (int64_t g = 0; g < ngroups; ++g) {
    const int buf = static_cast<int>(g & 1);
    const bool more = g + 1 < ngroups;
    u32x4 dv[GPL];
    if (more) load_dt(dv, (g + 1) * kGroup);
    const u32x4* lb = lds + buf * HALF;
    f32x4 o[S][2];
#pragma unroll
    for (int s = 0; s < S; ++s) o[s][0] = o[s][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const u32x4* row = lb + (16 * t + li) * (RPU + 1);
      if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int c = 0; c < RT; ++c) {
          const u32x4 bv = row[4 * c + lq];  // ranks 16c + 4lq .. +3
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int s = 0; s < S; ++s)
              o[s][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(acc[s][c][r], __uint_as_float(bv[r]), o[s][t], 0, 0, 0);
        }
      } else {
        const u32x2* row2 = reinterpret_cast<const u32x2*>(row);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          // ranks 16(2st) + 4lq .. +3 and 16(2st+1) + 4lq .. +3, 4 bf16 each
          const u32x2 lo8 = row2[(32 * st + 4 * lq) / 4];
          const u32x2 hi8 = row2[(32 * st + 16 + 4 * lq) / 4];
          const u32x4 bv = {lo8[0], lo8[1], hi8[0], hi8[1]};
          const bf16x8 b8 = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
          for (int s = 0; s < S; ++s) {
            o[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ahi[s][st]), b8, o[s][t], 0, 0, 0);
            o[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo[s][st]), b8, o[s][t], 0, 0, 0);
          }
        }
      }
    }
    // lane (channel li, q) holds tokens 4q .. 4q+3 of each strip for channel d0 + 16t + li
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int64_t d = g * kGroup + 16 * t + li;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t tok = w * 16 * S + s * 16 + 4 * lq + r;
          const uint32_t off = d < dim ? static_cast<uint32_t>(tok * row_bytes + d * ES) : kDropOffset;
          store_elem(tag, rd, off, o[s][t][r]);
        }
    }
    if (more) store_dt(dv, buf ^ 1);
    __syncthreads();
  }
}

template <typename T, int RT, int S>
hipError_t launch_proj(const ProjArgs& a, hipStream_t s) {
  const int64_t per = 64 * S;
  const dim3 grid(static_cast<unsigned>((a.tokens + per - 1) / per));
  hipLaunchKernelGGL((proj_kernel<T, RT, S>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t proj_t(const ProjArgs& a, int rt, int strips, hipStream_t s) {
  if (strips == 2) {
    switch (rt) {
      case 2: return launch_proj<T, 2, 2>(a, s);
      case 4: return launch_proj<T, 4, 2>(a, s);
      case 6: return launch_proj<T, 6, 2>(a, s);
      case 8: return launch_proj<T, 8, 2>(a, s);
      default: return launch_proj<T, 10, 2>(a, s);
    }
  }
  switch (rt) {
    case 2: return launch_proj<T, 2, 1>(a, s);
    case 4: return launch_proj<T, 4, 1>(a, s);
    case 6: return launch_proj<T, 6, 1>(a, s);
    case 8: return launch_proj<T, 8, 1>(a, s);
    case 10: return launch_proj<T, 10, 1>(a, s);
    case 12: return launch_proj<T, 12, 1>(a, s);
    default: return launch_proj<T, 16, 1>(a, s);
  }
}

}  // namespace

// Step tiles: the instantiated even count covering rank (rank <= 256 by the host check).
int proj_step_tiles(int64_t rank) {
  const int need = static_cast<int>((rank + 15) / 16);
  for (int rt : {2, 4, 6, 8, 10, 12, 16})
    if (rt >= need) return rt;
  return 16;
}

// Two strips per wave (128 tokens per workgroup) halve the W_x and W_dt reads per token and
// are used when that still leaves at least two workgroups per CU and the accumulators fit.
hipError_t proj(const ProjArgs& a, int cus, hipStream_t s) {
  const int rt = proj_step_tiles(a.rank);
  const int max_rt = a.dtype == kBF16 ? 6 : 10;  // the bf16 hi/lo operands need more registers
  const int strips = (rt <= max_rt && (a.tokens + 127) / 128 >= 2 * static_cast<int64_t>(cus)) ? 2 : 1;
  return a.dtype == kBF16 ? proj_t<uint16_t>(a, rt, strips, s) : proj_t<float>(a, rt, strips, s);
}

}  // namespace ss
