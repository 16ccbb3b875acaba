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
//  * B and C leave from tiles RT and RT + 1; delta_raw from the phase-2 accumulators (bf16
//    through a wave-private LDS block, so that every store is 16 bytes of a full row). bf16
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


// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_value(uint32_t b) { return __uint_as_float(b << 16); }

// Phase-1 MFMA step e of a K block (a = 16 bytes of W_x, b = 16 bytes of the inputs): fp32
// takes 4 steps of K = 4 (element e of each), bf16 one step of K = 32.
__device__ __forceinline__ f32x4 mfma_step(float*, const u32x4& a, const u32x4& b, int e, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_step(uint16_t*, const u32x4& a, const u32x4& b, int, f32x4 acc) {
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
  constexpr int KU = ES == 4 ? 1 : 2;         // MFMA K blocks per phase-1 chunk
  constexpr int CU = 4 * KU;                  // 16-byte units per W_x row and chunk
  constexpr int KB = CU * CH;                 // channels per chunk (16 fp32, 64 bf16)
  constexpr int GC = ES == 4 ? 32 : 64;       // channels per phase-2 group
  constexpr int TG = GC / 16;                 // output tiles per group
  constexpr int RPU = RT * 16 / CH;           // 16-byte units per staged W_dt row (RT*16 ranks)
  constexpr int P1 = ROWS * (CU + 1);         // padded rows (one spare unit against bank conflicts)
  constexpr int P2 = GC * (RPU + 1);
  constexpr int HALF = P1 > P2 ? P1 : P2;
  constexpr int KSTEP = ES == 4 ? 4 : 1;      // MFMA steps per K block
  constexpr int PD = ES == 4 ? 3 : 2;         // chunks (phase 1) / groups (phase 2) in flight
  __shared__ u32x4 lds[2 * HALF];
  // bf16 output tiles pass through a wave-private block so each lane stores 16 bytes of a
  // 128-byte row (direct stores would write 32-byte pieces, twice the HBM write traffic)
  constexpr int SROW = GC + 8;                // bf16 per staged row (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint16_t stage[ES == 2 ? 4 * S * 16 * SROW : 1];
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
  // Chunk c of W_x is requested PD + 1 iterations before it is used and staged in LDS one
  // iteration before; the inputs of chunk c are requested PD iterations before. The loop is
  // unrolled by PD so every register slot is static.
  const auto rwx = rsrc(a.W_x, (rank + 2 * N) * row_bytes);
  constexpr int EPL = (ROWS * CU + 255) / 256;  // staged units per lane and chunk
  auto wx_row = [&](int r) -> int64_t {         // source row of staged row r (-1: zero row)
    const int c = r >> 4, i = r & 15;
    if (c < RT) return 16 * c + i < rank ? 16 * c + i : -1;
    if (i >= N) return -1;
    return c == RT ? rank + i : rank + N + i;
  };
  auto load_wx = [&](u32x4 (&v)[EPL], int64_t k0) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const int e = tid + 256 * m;
      const int r = e / CU, un = e % CU;
      const int64_t kk = k0 + un * CH;
      const int64_t sr = e < ROWS * CU ? wx_row(r) : -1;
      const uint32_t off = (sr >= 0 && kk < dim) ? static_cast<uint32_t>((sr * dim + kk) * ES) : kDropOffset;
      v[m] = __builtin_amdgcn_raw_buffer_load_b128(rwx, off, 0, 0);
    }
  };
  auto store_wx = [&](const u32x4 (&v)[EPL], int buf) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const int e = tid + 256 * m;
      if (e < ROWS * CU) lds[buf * HALF + (e / CU) * (CU + 1) + e % CU] = v[m];
    }
  };
  auto load_x = [&](u32x4 (&x)[S][KU], int64_t k0) {
#pragma unroll
    for (int kb = 0; kb < KU; ++kb) {
      const int64_t kk = k0 + (4 * kb + lq) * CH;
#pragma unroll
      for (int s = 0; s < S; ++s)
        x[s][kb] = __builtin_amdgcn_raw_buffer_load_b128(
            ru, kk < dim ? xrow[s] + static_cast<uint32_t>(kk * ES) : kDropOffset, 0, 0);
    }
  };

  f32x4 acc[S][T1];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int c = 0; c < T1; ++c) acc[s][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t nchunks = (dim + KB - 1) / KB;
  u32x4 wq[PD][EPL], xq[PD][S][KU];
  {
    u32x4 w0[EPL];
    load_wx(w0, 0);
    store_wx(w0, 0);
  }
#pragma unroll
  for (int j = 0; j < PD; ++j) {
    if (j + 1 < nchunks) load_wx(wq[(j + 1) % PD], (j + 1) * KB);
    if (j < nchunks) load_x(xq[j], j * KB);
  }
  __syncthreads();
  for (int64_t base = 0; base < nchunks; base += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int64_t ci = base + j;
      if (ci < nchunks) {
        const u32x4* lb = lds + static_cast<int>(ci & 1) * HALF;
#pragma unroll
        for (int kb = 0; kb < KU; ++kb) {
          u32x4 av[T1];
#pragma unroll
          for (int c = 0; c < T1; ++c) av[c] = lb[(c * 16 + li) * (CU + 1) + 4 * kb + lq];
          // consecutive MFMAs go to different tiles, so none waits on the one before
#pragma unroll
          for (int e = 0; e < KSTEP; ++e)
#pragma unroll
            for (int c = 0; c < T1; ++c)
#pragma unroll
              for (int s = 0; s < S; ++s) acc[s][c] = mfma_step(tag, av[c], xq[j][s][kb], e, acc[s][c]);
        }
        if (ci + 1 < nchunks) store_wx(wq[(j + 1) % PD], static_cast<int>((ci + 1) & 1));
        if (ci + 1 + PD < nchunks) load_wx(wq[(j + 1) % PD], (ci + 1 + PD) * KB);
        if (ci + PD < nchunks) load_x(xq[j], (ci + PD) * KB);
        __syncthreads();
      }
    }
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
  constexpr int NS = (ES == 4) ? RT : RT / 2;  // bf16 steps (RT is even for bf16)
  i16x8 ahi[S][NS], alo[S][NS];
  if constexpr (ES == 2) {
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
  constexpr int GPL = (GC * RPU + 255) / 256;  // staged W_dt units per lane and group
  auto load_dt = [&](u32x4 (&v)[GPL], int64_t d0) {
#pragma unroll
    for (int m = 0; m < GPL; ++m) {
      const int e = tid + 256 * m;
      const int r = e / RPU, un = e % RPU;  // channel row within the group, unit along rank
      const int64_t d = d0 + r, rk = static_cast<int64_t>(un) * CH;
      const uint32_t off = (e < GC * RPU && d < dim && rk < rank) ? static_cast<uint32_t>((d * rank + rk) * ES)
                                                                   : kDropOffset;
      v[m] = __builtin_amdgcn_raw_buffer_load_b128(rdt, off, 0, 0);
    }
  };
  auto store_dt = [&](const u32x4 (&v)[GPL], int buf) {
#pragma unroll
    for (int m = 0; m < GPL; ++m) {
      const int e = tid + 256 * m;
      if (e < GC * RPU) lds[buf * HALF + (e / RPU) * (RPU + 1) + e % RPU] = v[m];
    }
  };

  const auto rd = rsrc(static_cast<T*>(a.delta_raw) + wg_tok0 * dim, (M - wg_tok0) * row_bytes);
  const int64_t ngroups = (dim + GC - 1) / GC;
  u32x4 dq[PD][GPL];
  {
    u32x4 d0v[GPL];
    load_dt(d0v, 0);
    store_dt(d0v, 0);
  }
#pragma unroll
  for (int j = 0; j < PD; ++j)
    if (j + 1 < ngroups) load_dt(dq[(j + 1) % PD], (j + 1) * GC);
  __syncthreads();
  for (int64_t base = 0; base < ngroups; base += PD) {
#pragma unroll
    for (int j = 0; j < PD; ++j) {
      const int64_t g = base + j;
      if (g < ngroups) {
        const u32x4* lb = lds + static_cast<int>(g & 1) * HALF;
        f32x4 o[S][TG];
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int t = 0; t < TG; ++t) o[s][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (ES == 4) {
#pragma unroll
          for (int c = 0; c < RT; ++c) {
            u32x4 bv[TG];
#pragma unroll
            for (int t = 0; t < TG; ++t) bv[t] = lb[(16 * t + li) * (RPU + 1) + 4 * c + lq];  // ranks 16c + 4lq ..
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
              for (int t = 0; t < TG; ++t)
#pragma unroll
                for (int s = 0; s < S; ++s)
                  o[s][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(acc[s][c][r], __uint_as_float(bv[t][r]), o[s][t],
                                                                 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            bf16x8 b8[TG];
#pragma unroll
            for (int t = 0; t < TG; ++t) {
              // ranks 16(2st) + 4lq .. +3 and 16(2st+1) + 4lq .. +3, 4 bf16 each
              const u32x2* row2 = reinterpret_cast<const u32x2*>(lb + (16 * t + li) * (RPU + 1));
              const u32x2 lo8 = row2[8 * st + lq];
              const u32x2 hi8 = row2[8 * st + 4 + lq];
              const u32x4 bv = {lo8[0], lo8[1], hi8[0], hi8[1]};
              b8[t] = __builtin_bit_cast(bf16x8, bv);
            }
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
              for (int s = 0; s < S; ++s)
                o[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ahi[s][st]), b8[t], o[s][t],
                                                                  0, 0, 0);
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
              for (int s = 0; s < S; ++s)
                o[s][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, alo[s][st]), b8[t], o[s][t],
                                                                  0, 0, 0);
          }
        }
        // lane (channel li, q) holds tokens 4q .. 4q+3 of each strip for channel g*GC + 16t + li
        if constexpr (ES == 4) {
#pragma unroll
          for (int t = 0; t < TG; ++t) {
            const int64_t d = g * GC + 16 * t + li;
#pragma unroll
            for (int s = 0; s < S; ++s)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int64_t tok = w * 16 * S + s * 16 + 4 * lq + r;
                const uint32_t off = d < dim ? static_cast<uint32_t>(tok * row_bytes + d * ES) : kDropOffset;
                store_elem(tag, rd, off, o[s][t][r]);
              }
          }
        } else {
          uint16_t* st = stage + w * (S * 16 * SROW);
#pragma unroll
          for (int s = 0; s < S; ++s)
#pragma unroll
            for (int t = 0; t < TG; ++t)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                st[(s * 16 + 4 * lq + r) * SROW + 16 * t + li] = static_cast<uint16_t>(bf16_bits(o[s][t][r]));
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
          // 16 tokens x 128 bytes per strip = 128 pieces of 16 bytes: pieces l and l + 64
#pragma unroll
          for (int s = 0; s < S; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int piece = l + 64 * h, tok = piece >> 3, col = (piece & 7) * 8;
              const u32x4 v = *reinterpret_cast<const u32x4*>(st + (s * 16 + tok) * SROW + col);
              const int64_t d = g * GC + col;
              const int64_t tk = w * 16 * S + s * 16 + tok;
              __builtin_amdgcn_raw_buffer_store_b128(
                  v, rd, d < dim ? static_cast<uint32_t>(tk * row_bytes + d * ES) : kDropOffset, 0, 0);
            }
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        }
        if (g + 1 < ngroups) store_dt(dq[(j + 1) % PD], static_cast<int>((g + 1) & 1));
        if (g + 1 + PD < ngroups) load_dt(dq[(j + 1) % PD], (g + 1 + PD) * GC);
        __syncthreads();
      }
    }
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
  if constexpr (sizeof(T) == 4) {  // fp32 also has 3 step tiles (rank 48: 1536 / 32)
    if (rt == 3) return strips == 2 ? launch_proj<T, 3, 2>(a, s) : launch_proj<T, 3, 1>(a, s);
  }
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

// Step tiles: the smallest instantiated count covering rank (rank <= 256 by the host check);
// bf16 needs an even count (one MFMA step covers two tiles), fp32 also has 3.
int proj_step_tiles(int64_t rank, int dtype) {
  const int need = static_cast<int>((rank + 15) / 16);
  if (dtype != kBF16 && need == 3) return 3;
  for (int rt : {2, 4, 6, 8, 10, 12, 16})
    if (rt >= need) return rt;
  return 16;
}

// Two strips per wave (128 tokens per workgroup) halve the W_x and W_dt reads per token and
// are used when that still leaves at least two workgroups per CU and the accumulators fit.
hipError_t proj(const ProjArgs& a, int cus, hipStream_t s) {
  const int rt = proj_step_tiles(a.rank, a.dtype);
  const int max_rt = a.dtype == kBF16 ? 6 : 10;  // the bf16 hi/lo operands need more registers
  const int strips = (rt <= max_rt && (a.tokens + 127) / 128 >= 2 * static_cast<int64_t>(cus)) ? 2 : 1;
  return a.dtype == kBF16 ? proj_t<uint16_t>(a, rt, strips, s) : proj_t<float>(a, rt, strips, s);
}

}  // namespace ss
