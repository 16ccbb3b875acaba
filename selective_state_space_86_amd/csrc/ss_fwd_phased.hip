// ss_fwd_phased.hip -- time-chunked selective-scan forward for dstate == 16 with the
// default input term and no conv prologue, scheduled in phases (gfx950).
//
// What it computes is the recurrence of "Mamba：选择性状态空间模型入门教程" (section
// "Mamba 的关键创新：选择性机制"): dt = softplus(delta + bias), abar = exp(dt A),
// h = abar h + (dt B_t) u, y = (C_t . h + D u) silu(z). How it computes it follows the
// hardware-aware scan of "Mamba：选择性状态空间的线性时间序列建模" (section "第二个创新：硬件
// 感知算法": a parallel associative scan, fused so the expanded state never leaves the chip)
// and the associative combine of "架构变体：Mamba/SSM" (section "硬件感知算法").
//
// Layout: a workgroup of 8 waves (32 rows of 16 lanes) owns 16 consecutive channels of one
// batch row; lane i of a row is channel c0 + i and holds all 16 fp32 states of it; row k is
// time chunk k (4 tokens) of a 128-token tile. A row sits at one token at a time, so B_t and
// C_t are row-uniform: lane n of the row holds B_t[n] and C_t[n], read by the other lanes of
// the row through DPP row_newbcast:n inside the multiply that consumes them.
//
// Per tile, every wave of the workgroup runs the same phases, separated by barriers so the
// two waves sharing a SIMD stay in the same phase. On gfx950 a wave64 fp32 FMA-class VALU op
// issues in about 2.25 cycles per SIMD and v_exp_f32 in about 8, but when transcendental and
// other VALU ops are interleaved on a SIMD, even across different waves, every VALU op costs
// about 4 cycles; so the exponentials are kept in phases of their own where possible:
//  A (exp phase): per token softplus, the gate, D u, dt u, and for the 16 states the decay
//    abar = 2^(dt A log2 e) and the input term bbar = (dt u) B_t[n]; abar and bbar of the
//    chunk's 4 tokens stay in registers (128 values per lane).
//  B (FMA phase): the chunk's local scan from zero, h = abar h + bbar, and its decay product
//    P = prod abar: the chunk aggregate (P, h_end), the pair of the associative operator
//    (a1, b1) o (a2, b2) = (a2 a1, a2 b1 + b2), goes to LDS.
//  fold: after a barrier, lane (k < 16, i) owns state n = k of channel i and folds the 32
//    chunk aggregates in order, starting from the carry of the previous tile: every chunk's
//    carry-in goes back to LDS, and the carry into the next tile stays in the lane.
//  C (FMA phase): after a barrier, each lane replays its chunk's recurrence from its true
//    carry-in with the stored abar and bbar, and forms y = C_t . h + D u (times the gate) for
//    each token: two VALU ops per state update, where a fix-up of a zero-started local pass
//    would take a multiply and an FMA per update on top of the local pass's own output FMA.
// Per state update: 3 VALU + 1 exp in A (dt A, the exp, bbar), 1 FMA in B, 2 in C, plus the
// decay product (3 multiplies per state per chunk). The (L x N) state never reaches memory.
//
// Memory access as in the other chunked kernel (ss_chunk_ops.h TileLoader): fixed 32-bit
// per-lane offsets into a tile, SGPR tile bases; the next tile's inputs are requested at the
// start of a tile into the other of two input buffers (the loop is unrolled by two, so no
// register copies), from a start clamped to the last tile, so the request is unconditional
// and the compiler keeps it in flight through the whole tile.
#include <algorithm>

#include "ss_chunk_ops.h"
#include "ss_split.h"

namespace ss {
namespace {

using namespace chunk;

constexpr int kR = 32;            // time chunks (rows) per tile
constexpr int kTC = 4;            // tokens per chunk
constexpr int kTile = kR * kTC;   // tokens per tile
constexpr int kPS = 16 * 16 + 16; // (P, h) pairs per chunk in LDS: [n][lane], padded
constexpr int kCS = 16 * 16 + 16; // carries per chunk in LDS: [n][lane], padded

#define SS_BB(n) "v_mul_f32_dpp %[bb" #n "], %[vb], %[w]" SS_DPP_ROW(n)

// bb[n] = B_t[n] * w for the 16 states (B_t[n] from lane n of the row). The DPP source vb may
// have been written by a VALU op just before: two wait states first.
__device__ __forceinline__ void input_terms(float (&bb)[16], float vb, float w) {
  asm volatile("s_nop 1\n" SS_BB(0) SS_BB(1) SS_BB(2) SS_BB(3) SS_BB(4) SS_BB(5) SS_BB(6) SS_BB(7)
               SS_BB(8) SS_BB(9) SS_BB(10) SS_BB(11) SS_BB(12) SS_BB(13) SS_BB(14) SS_BB(15)
               : SS_OPS16(bb, "=&v")
               : [vb] "v"(vb), [w] "v"(w));
}

#define SS_YD(n, Y) "v_fmac_f32_dpp %[" #Y "], %[vc], %[h" #n "]" SS_DPP_ROW(n)

// y += sum_n C_t[n] h[n] (C_t[n] from lane n of the row), in two accumulators.
__device__ __forceinline__ void out_dot(float& y, const float (&h)[16], float vc) {
  float y2 = 0.0f;
  asm volatile("s_nop 1\n" SS_YD(0, y) SS_YD(1, y2) SS_YD(2, y) SS_YD(3, y2) SS_YD(4, y) SS_YD(5, y2)
               SS_YD(6, y) SS_YD(7, y2) SS_YD(8, y) SS_YD(9, y2) SS_YD(10, y) SS_YD(11, y2) SS_YD(12, y)
               SS_YD(13, y2) SS_YD(14, y) SS_YD(15, y2)
               : [y] "+v"(y), [y2] "+v"(y2)
               : SS_OPS16(h, "v"), [vc] "v"(vc));
  y += y2;
}

template <typename T, bool GATE, bool SPLIT, bool SYNC_C>
__global__ __launch_bounds__(kR * 16) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_phased_kernel(FwdArgs a) {
  __shared__ float2 lds_ph[kR * kPS];  // chunk aggregates (P, h_end): [chunk][n][lane]
  __shared__ float lds_c[kR * kCS];    // chunk carry-ins: [chunk][n][lane]
  __shared__ uint32_t item_s, seen_s;

  const int64_t ngd = (a.dim + 15) / 16;
  const int64_t groups = a.batch * ngd;
  const int tid = threadIdx.x;
  const int64_t L = a.seqlen;
  int64_t gi = blockIdx.x, part = 0;  // work item: group index gi, sequence part
  if (SPLIT) {
    if (tid == 0) item_s = split::take(a.split_ws, groups);  // part * groups + gi
    __syncthreads();
    const uint32_t item = __builtin_amdgcn_readfirstlane(item_s);
    part = item / groups;
    gi = item % groups;
  }
  const int64_t t_begin = SPLIT ? part * a.part_len : 0;
  const int64_t t_end = SPLIT ? min(L, t_begin + a.part_len) : L;
  const int64_t t_last = t_begin + (t_end - 1 - t_begin) / kTile * kTile;  // start of the last tile
  const int64_t g = SPLIT ? gi : group_of(gi, groups);
  const int64_t b = g / ngd;
  const int64_t c0 = (g % ngd) * 16;
  const int i = tid & 15;  // channel in the group; the state this lane owns in the fold
  const int k = tid >> 4;  // time chunk (row) in the tile
  const int64_t c = c0 + i;
  const bool cvalid = c < a.dim;
  const int64_t cc = cvalid ? c : a.dim - 1;
  TileLoader<T, GATE, kTC, kR> K(a, b, c0, k, i, cc);

  float A2[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) A2[n] = a.A[cc * 16 + n] * kLog2e;
  const float bias = a.delta_bias ? a.delta_bias[cc] : 0.0f;
  const float Dd = a.D ? a.D[cc] : 0.0f;
  // the state n = k (k < 16) of channel c0 + i, carried across tiles
  float carry = (a.h0 && part == 0 && k < 16) ? a.h0[(b * a.dim + cc) * 16 + k] : 0.0f;
  if (SPLIT && part > 0) {  // start from the state the previous part of this group ends with
    const int64_t slot = (part - 1) * groups + gi;
    if (tid == 0) seen_s = split::poll(a.split_ws, slot, a.split_wait_limit) ? 1u : 0u;
    __syncthreads();  // (the state loads are issued after thread 0 has seen the flag)
    const bool seen = __builtin_amdgcn_readfirstlane(seen_s) != 0u;
    // a wait that gave up leaves the carry unknown: continue from NaN (counted in the header)
    if (k < 16) carry = seen ? split::load_state(a.split_ws, a.split_cap, slot, k, i) : __builtin_nanf("");
  }
  const uint32_t y_row = static_cast<uint32_t>(a.dim * 4);
  const uint32_t y_off = static_cast<uint32_t>(k * kTC) * y_row + static_cast<uint32_t>(i * 4);

  // one tile from the inputs `cur`, with the next tile's inputs requested into `nxt`
  auto tile = [&](const TileIn<kTC>& cur, TileIn<kTC>& nxt, int64_t t0) {
    K.load(nxt, min(t0 + kTile, t_last));  // (the last tile re-requests itself: unused)
    const bool full = t0 + kTile <= t_end;

    // A: step sizes, gate, skip term, decays and input terms of the chunk's 4 tokens
    float e[kTC][16], bb[kTC][16], y[kTC], gate[kTC];
#pragma unroll
    for (int j = 0; j < kTC; ++j) {
      const float x = cur.raw[j] + bias;
      float dt = a.softplus ? softplus(x) : x;
      if (!full) dt = (t0 + k * kTC + j < t_end) ? dt : 0.0f;  // a zero step is the identity
      y[j] = Dd * cur.uu[j];
      gate[j] = GATE ? silu(cur.zz[j]) : 1.0f;
#pragma unroll
      for (int n = 0; n < 16; ++n) e[j][n] = fast_exp2(dt * A2[n]);
      input_terms(bb[j], cur.vb[j], dt * cur.uu[j]);
    }

    // B: the chunk's local scan from zero and its decay product -> LDS
    {
      float h[16], p[16];
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        h[n] = bb[0][n];
        p[n] = e[0][n];
      }
#pragma unroll
      for (int j = 1; j < kTC; ++j)
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          h[n] = __builtin_fmaf(e[j][n], h[n], bb[j][n]);
          p[n] *= e[j][n];
        }
      float2* dst = lds_ph + k * kPS + i;
#pragma unroll
      for (int n = 0; n < 16; ++n) dst[n * 16] = make_float2(p[n], h[n]);
    }
    __syncthreads();

    // fold: lane (k < 16, i) owns state n = k of channel i; carry-in of every chunk in order
    if (k < 16) {
      const float2* src = lds_ph + k * 16 + i;
      float* out = lds_c + k * 16 + i;
#pragma unroll
      for (int j0 = 0; j0 < kR; j0 += 8) {
        float2 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[(j0 + j) * kPS];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          out[(j0 + j) * kCS] = carry;
          carry = __builtin_fmaf(v[j].x, carry, v[j].y);
        }
      }
    }
    __syncthreads();

    // C: the chunk's recurrence from its carry-in; y of every token; stores
    {
      float h[16];
      const float* q = lds_c + k * kCS + i;
#pragma unroll
      for (int n = 0; n < 16; ++n) h[n] = q[n * 16];
      const int64_t y0 = (b * L + t0) * a.dim + c0;
      const auto ry = rsrc(a.y + y0, (a.batch * L * a.dim - y0) * 4);
#pragma unroll
      for (int j = 0; j < kTC; ++j) {
#pragma unroll
        for (int n = 0; n < 16; ++n) h[n] = __builtin_fmaf(e[j][n], h[n], bb[j][n]);
        out_dot(y[j], h, cur.vc[j]);
        const bool ok = full ? cvalid : (cvalid && t0 + k * kTC + j < t_end);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[j] * gate[j]), ry, ok ? y_off : kDropOffset,
                                              j * y_row, 0);
      }
    }
    if (SYNC_C) __syncthreads();  // (keeps the waves of a SIMD in step for the next phase A)
  };

  TileIn<kTC> in0, in1;
  K.load(in0, t_begin);
  for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kTile) {
    tile(in0, in1, t0);
    if (t0 + kTile >= t_end) break;
    tile(in1, in0, t0 + kTile);
  }

  if (SPLIT && part < a.parts - 1) {  // publish this part's end state for the next part
    const int64_t slot = part * groups + gi;
    if (k < 16) split::store_state(a.split_ws, a.split_cap, slot, k, i, carry);
    split::finish_stores();
    __syncthreads();
    if (tid == 0) split::publish(a.split_ws, slot);
  } else if (a.last_state && cvalid && k < 16) {
    a.last_state[(b * a.dim + c) * 16 + k] = carry;
  }
}

template <typename T, bool GATE, bool SYNC_C>
void launch_phased_g(const FwdArgs& a, hipStream_t s) {
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  const dim3 block(kR * 16);
  if (a.parts > 1)
    hipLaunchKernelGGL((fwd_phased_kernel<T, GATE, true, SYNC_C>), dim3(static_cast<unsigned>(groups * a.parts)),
                       block, 0, s, a);
  else
    hipLaunchKernelGGL((fwd_phased_kernel<T, GATE, false, SYNC_C>), dim3(static_cast<unsigned>(groups)), block, 0,
                       s, a);
}

template <typename T>
hipError_t launch_phased_t(const FwdArgs& a, hipStream_t s) {
  if (a.z)
    launch_phased_g<T, true, true>(a, s);
  else
    launch_phased_g<T, false, true>(a, s);
  return hipGetLastError();
}

}  // namespace

bool fwd_phased_supported(const FwdArgs& a) {
  return a.dstate == 16 && a.seqlen > 0 && !a.zoh && a.kconv == 0;
}

ChunkPlan fwd_phased_plan() { return ChunkPlan{kTC, kR}; }

hipError_t fwd_phased(const FwdArgs& a, hipStream_t s) {
  return a.dtype == kBF16 ? launch_phased_t<uint16_t>(a, s) : launch_phased_t<float>(a, s);
}

}  // namespace ss
