// ss_fwd_chunked.hip -- time-chunked selective-scan forward for dstate == 16 (gfx950).
//
// What it computes is the recurrence of "Mamba：选择性状态空间模型入门教程" (section
// "Mamba 的关键创新：选择性机制"), discretised as in "架构变体：Mamba/SSM" (section
// "离散化"); how it computes it follows the hardware-aware scan of "Mamba：选择性状态空间
// 的线性时间序列建模" (section "第二个创新：硬件感知算法": a parallel associative scan,
// fused so the expanded state stays on chip) and the block decomposition of "Mamba架构
// 深度解析" (section "Mamba的创新": split the sequence into blocks, parallel inside a
// block), laid out for 64-wide CDNA waves:
//
//  * A workgroup (4 waves, 16 rows of 16 lanes) owns 16 consecutive channels of one batch
//    row. Lane i of a row is channel c0+i; the 16 rows are 16 consecutive time chunks of
//    TC tokens, so a tile covers 16*TC tokens. Every lane keeps all 16 fp32 states of its
//    channel in registers: softplus, the D term and the gate are paid once per 16 updates.
//  * A row sits at one token at a time, so B_t and C_t are row-uniform: lane n of the row
//    holds B_t[n] and C_t[n], and the update reads them through DPP row_newbcast:n folded
//    into the v_mul / v_fmac that consume them (no LDS, no extra instruction).
//  * Local pass: each lane scans its chunk from a zero state, keeping abar = exp(dt A) of
//    every step in registers. The chunk aggregate (prod abar, end state) is the pair of the
//    associative operator (a1, b1) o (a2, b2) = (a2 a1, a2 b1 + b2) ("架构变体" section
//    "硬件感知算法": the update is associative, so it can be combined as a tree).
//  * Combine: aggregates go to LDS; lane (chunk k, channel i) then owns state n = k and
//    folds the 16 chunk aggregates of channel i in order, producing every chunk's carry-in
//    and the carry into the next tile (kept in that lane's register across tiles).
//  * Fix-up: y_t += sum_n C_t[n] (prod_{s<=t} abar_s[n]) carry[n], from the stored abar;
//    then the gate, and one store per token. The (L x N) state never reaches memory.
// Per state update the local pass issues 4 VALU ops and one v_exp_f32, the fix-up 2 VALU.
// With the exact zero-order-hold input term (ZOH) the local pass also evaluates
// (abar - 1)/A per update (zoh_coef); the combine and the fix-up do not change. With the
// conv prologue (CONV) the u operand is x and each lane first forms
// u_t = silu(conv_b + conv_w * x_{t-3..t}) from its chunk's inputs and the 3 before them.
//
// Memory access: every lane has a fixed 32-bit byte offset into a tile (its chunk row and
// channel); the tile origin and the token step within the chunk live in SGPR base pointers,
// so the loads and stores need no per-access vector address arithmetic. The next tile's
// inputs are requested right after the local pass, so the combine and the fix-up of the
// current tile overlap their latency.
#include <algorithm>

#include "ss_chunk_ops.h"
#include "ss_split.h"

namespace ss {
namespace {

using namespace chunk;

constexpr int kLdsChunkStride = 16 * 16 + 16;  // [chunk][n][lane], padded against bank conflicts

// Sequence split (SPLIT): the work queue and state hand-off of ss_split.h. When the channel
// groups do not fill the resident workgroup slots in whole rounds (the 3B long-context shape:
// 320 groups for 256 one-workgroup CUs, so a second round of 64 would run on a quarter of
// the chip), every group's sequence is cut into parts of whole tiles, one workgroup each;
// part q starts from the carry part q - 1 publishes.

// R rows (time chunks) per workgroup: 16 (4 waves), 12 (3 waves; four such workgroups fit
// a CU where three of 16 do, for shapes with between 3 and 4 channel groups per CU) or 32
// (8 waves, two per SIMD from one workgroup, for shapes with at most 2 groups per CU, where
// 4-wave workgroups leave most SIMDs with a single wave, which issues at about half rate).
// Register budget: TC = 4 must fit 3 waves per SIMD, TC = 8 two; the zero-order-hold
// variant holds 16 more values (1/A) and runs at two.
template <typename T, bool GATE, int TC, bool EARLY, bool ZOH, bool CONV, int R, bool SPLIT>
__global__ __launch_bounds__(R * 16) __attribute__((amdgpu_waves_per_eu(TC <= 4 && !ZOH && R <= 16 ? 3 : 2)))
void fwd_chunked_kernel(FwdArgs a) {
  static_assert(R == 16 || R == 12 || R == 32, "12, 16 or 32 chunks per tile");
  constexpr int NOWN = (16 + R - 1) / R;  // states each lane folds: n = k, k + R (when < 16)
  // The prod-abar/carry array alternates between two buffers by tile, so a tile's
  // aggregates never overwrite carries a slower wave may still be reading after the second
  // barrier of the previous tile. The end states are read only between the two barriers of
  // a tile, so one buffer suffices.
  __shared__ float lds_a2[2][R * kLdsChunkStride];  // chunk prod-abar, then the chunk carries
  __shared__ float lds_h[R * kLdsChunkStride];      // chunk end states

  const int64_t ngd = (a.dim + 15) / 16;
  const int64_t groups = a.batch * ngd;
  const int tid = threadIdx.x;
  const int64_t L = a.seqlen;
  int64_t gi = blockIdx.x, part = 0;  // work item: group index gi, sequence part
  __shared__ uint32_t item_s;
  if (SPLIT) {
    if (tid == 0) item_s = split::take(a.split_ws, groups, a.parts);  // part * groups + gi
    __syncthreads();
    const uint32_t item = __builtin_amdgcn_readfirstlane(item_s);  // (uniform: keep it in SGPRs)
    part = item / groups;
    gi = item % groups;
  }
  const int64_t t_begin = SPLIT ? part * a.part_len : 0;
  const int64_t t_end = SPLIT ? min(L, t_begin + a.part_len) : L;
  const int64_t g = SPLIT ? gi : group_of(gi, groups);
  const int64_t b = g / ngd;
  const int64_t c0 = (g % ngd) * 16;
  const int i = tid & 15;  // channel within the group == the state index this lane owns in the combine
  const int k = tid >> 4;  // time chunk within the tile (row of 16 lanes)
  const int64_t c = c0 + i;
  const bool cvalid = c < a.dim;
  const int64_t cc = cvalid ? c : a.dim - 1;
  TileLoader<T, GATE, TC, R> K(a, b, c0, k, i, cc);

  float A2[16], iA[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    A2[n] = a.A[cc * 16 + n] * kLog2e;
    if (ZOH) iA[n] = 1.0f / a.A[cc * 16 + n];
  }
  const float bias = a.delta_bias ? a.delta_bias[cc] : 0.0f;
  const float Dd = a.D ? a.D[cc] : 0.0f;
  float w4[4], cb = 0.0f;
  if (CONV) conv_taps(a.conv_w, a.conv_b, a.kconv, cc, w4, cb);
  // states n = k (+ R) of channel c0+i, carried across tiles; start at h0 when one is given
  float carry[NOWN];
#pragma unroll
  for (int m = 0; m < NOWN; ++m) {
    const int n = k + m * R;
    carry[m] = (a.h0 && part == 0 && n < 16) ? a.h0[(b * a.dim + cc) * 16 + n] : 0.0f;
  }
  if (SPLIT && part > 0) {  // start from the state the previous part of this group ends with
    const int64_t slot = (part - 1) * groups + gi;
    split::wait(a.split_ws, slot);
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = k + m * R;
      if (n < 16) carry[m] = split::load_state(a.split_ws, a.split_cap, slot, n, i);
    }
    __syncthreads();  // every wave has seen the flag: clear it for the next call
    if (tid == 0) split::clear(a.split_ws, slot);
  }
  const uint32_t y_row = static_cast<uint32_t>(a.dim * 4);
  const uint32_t y_off = static_cast<uint32_t>(k * TC) * y_row + static_cast<uint32_t>(i * 4);

  TileIn<TC> cur, nxt;
  K.load(cur, t_begin);
  int buf = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += R * TC, buf ^= 1) {
    // (a split kernel is the one-workgroup-per-CU plan, where priorities change nothing)
    if (!SPLIT) progress_priority(t0, L);
    const bool full = t0 + R * TC <= t_end;  // (a part other than the last ends on a tile boundary)
    float* lds_a = lds_a2[buf];
    // request the next tile first: the whole tile's work hides its latency
    if (EARLY && t0 + R * TC < t_end) K.load(nxt, t0 + R * TC);

    // local pass from a zero state
    float h[16], ex[TC][16], y[TC], gate[TC], vc[TC];
#pragma unroll
    for (int n = 0; n < 16; ++n) h[n] = 0.0f;
    float dsum = 0.0f;
    if (CONV) {  // u = silu(conv(x)) over the window [3 inputs before the chunk, x_0 .. x_{TC-1}]
      // (the 3 earlier inputs are the end of the previous chunk: cache hits, loaded here
      // rather than prefetched to keep registers for the 16 states)
      float win[TC + 3];
#pragma unroll
      for (int m = 0; m < 3; ++m)
        win[m] = conv_input(static_cast<const T*>(a.u), a.conv_state, a.kconv, b, cc,
                            min(t0 + k * TC - 3 + m, L - 1), L, a.dim);
#pragma unroll
      for (int j = 0; j < TC; ++j) win[j + 3] = cur.uu[j];
      // u_out has y's layout; a null u_out gets an empty range, so every store is dropped
      const int64_t u0 = (b * L + t0) * a.dim + c0;
      const auto ru = rsrc(a.u_out ? a.u_out + u0 : a.y, a.u_out ? (a.batch * L * a.dim - u0) * 4 : 0);
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        cur.uu[j] = conv4_silu(w4, cb, win[j], win[j + 1], win[j + 2], win[j + 3]);
        const bool ok = full ? cvalid : (cvalid && t0 + k * TC + j < L);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cur.uu[j]), ru, ok ? y_off : kDropOffset, j * y_row, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const float x = cur.raw[j] + bias;
      float dt = a.softplus ? softplus(x) : x;
      if (!full) dt = (t0 + k * TC + j < L) ? dt : 0.0f;  // a zero step is the identity
      dsum += dt;
      y[j] = Dd * cur.uu[j];
      if (ZOH)
        local_step_zoh(h, ex[j], A2, iA, dt, cur.uu[j], cur.vb[j], cur.vc[j], y[j]);
      else
        local_step(h, ex[j], A2, dt, dt * cur.uu[j], cur.vb[j], cur.vc[j], y[j]);
      gate[j] = GATE ? silu(cur.zz[j]) : 1.0f;
      vc[j] = cur.vc[j];
    }

    // otherwise request it now: the combine and fix-up below hide its latency
    if (!EARLY && t0 + R * TC < t_end) K.load(nxt, t0 + R * TC);

    // chunk aggregates (prod abar = exp(A * sum dt), end state) to LDS
    {
      float* la = lds_a + k * kLdsChunkStride + i;
      float* lh = lds_h + k * kLdsChunkStride + i;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        float p;
        if (TC <= 4) {  // product of the stored factors: TC-1 multiplies
          p = ex[0][n];
#pragma unroll
          for (int j = 1; j < TC; ++j) p *= ex[j][n];
        } else {        // one multiply and one exp
          p = fast_exp2(A2[n] * dsum);
        }
        la[n * 16] = p;
        lh[n * 16] = h[n];
      }
    }
    __syncthreads();

    // combine: this lane owns state n = k (and k + R) of channel i and folds the R chunks in
    // order (with 32 rows, rows 16..31 own none). Each lane reads exactly the LDS words it then
    // overwrites with carries, so the carry array can alias the prod-abar array without another
    // barrier.
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = k + m * R;
      if (n < 16) {
        float* sa = lds_a + n * 16 + i;
        const float* sh = lds_h + n * 16 + i;
        // (in blocks of at most 16 chunks: all reads of a block first, then its fold)
        constexpr int CB = R < 16 ? R : 16;
#pragma unroll
        for (int j0 = 0; j0 < R; j0 += CB) {
          float av[CB], hv[CB];
#pragma unroll
          for (int j = 0; j < CB; ++j) {
            av[j] = sa[(j0 + j) * kLdsChunkStride];
            hv[j] = sh[(j0 + j) * kLdsChunkStride];
          }
#pragma unroll
          for (int j = 0; j < CB; ++j) {
            sa[(j0 + j) * kLdsChunkStride] = carry[m];  // carry into chunk j0 + j
            carry[m] = __builtin_fmaf(av[j], carry[m], hv[j]);
          }
        }
      }
    }
    __syncthreads();
    float q[16];  // this chunk's carry-in
    {
      const float* lc = lds_a + k * kLdsChunkStride + i;
#pragma unroll
      for (int n = 0; n < 16; ++n) q[n] = lc[n * 16];
    }

    // fix-up with the carry-in, gate, store (unconditionally: a masked lane's store goes to an
    // offset past the buffer range and is dropped, so the compiler sees a fixed number of
    // outstanding stores and never waits for them when the prefetched loads are consumed)
    const int64_t y0 = (b * L + t0) * a.dim + c0;
    const auto ry = rsrc(a.y + y0, (a.batch * L * a.dim - y0) * 4);
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      fixup_step(q, ex[j], vc[j], y[j]);
      const bool ok = full ? cvalid : (cvalid && t0 + k * TC + j < L);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[j] * gate[j]), ry, ok ? y_off : kDropOffset, j * y_row, 0);
    }
    cur = nxt;
  }
  if (SPLIT && item_s / groups < a.parts - 1) {  // publish this part's end state for the next
    const int64_t slot = __builtin_amdgcn_readfirstlane(item_s);  // (re-read: nothing kept live)
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = k + m * R;
      if (n < 16) split::store_state(a.split_ws, a.split_cap, slot, n, i, carry[m]);
    }
    split::finish_stores();
    __syncthreads();
    if (tid == 0) split::publish(a.split_ws, slot);
  } else if (a.last_state && cvalid) {
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = k + m * R;
      if (n < 16) a.last_state[(b * a.dim + c) * 16 + n] = carry[m];
    }
  }
}

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[j] = 0u;
}

template <typename T, bool GATE, int TC, bool ZOH, int R>
void launch_chunked_c(const FwdArgs& a, hipStream_t s) {
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  constexpr bool early = TC <= 4;
  const dim3 block(R * 16);
  if (a.parts > 1) {
    const dim3 grid(static_cast<unsigned>(groups * a.parts));
    if (a.kconv > 0)
      hipLaunchKernelGGL((fwd_chunked_kernel<T, GATE, TC, early, ZOH, true, R, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_chunked_kernel<T, GATE, TC, early, ZOH, false, R, true>), grid, block, 0, s, a);
  } else {
    const dim3 grid(static_cast<unsigned>(groups));
    if (a.kconv > 0)
      hipLaunchKernelGGL((fwd_chunked_kernel<T, GATE, TC, early, ZOH, true, R, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_chunked_kernel<T, GATE, TC, early, ZOH, false, R, false>), grid, block, 0, s, a);
  }
}

template <typename T, bool GATE, int TC, int R>
hipError_t launch_chunked(const FwdArgs& a, hipStream_t s) {
  if (a.zoh)
    launch_chunked_c<T, GATE, TC, true, R>(a, s);
  else
    launch_chunked_c<T, GATE, TC, false, R>(a, s);
  return hipGetLastError();
}

template <typename T, int TC, int R>
hipError_t launch_chunked_g(const FwdArgs& a, hipStream_t s) {
  return a.z ? launch_chunked<T, true, TC, R>(a, s) : launch_chunked<T, false, TC, R>(a, s);
}

template <typename T>
hipError_t launch_chunked_t(const FwdArgs& a, ChunkPlan p, hipStream_t s) {
  if (p.rows == 12) return launch_chunked_g<T, 4, 12>(a, s);
  if (p.rows == 32) return p.chunk_len == 4 ? launch_chunked_g<T, 4, 32>(a, s) : launch_chunked_g<T, 8, 32>(a, s);
  return p.chunk_len == 4 ? launch_chunked_g<T, 4, 16>(a, s) : launch_chunked_g<T, 8, 16>(a, s);
}

}  // namespace

bool fwd_chunked_supported(const FwdArgs& a) { return a.dstate == 16 && a.seqlen > 0; }

// Tile shape. Chunk length 8 halves the per-tile combine cost but needs ~2x the registers
// of 4 (2 resident workgroups of 16 rows per CU instead of 3). The plan:
//  - at most 2 groups per CU (the 3B long-context shape: 320 groups): length 8, 32 rows, so
//    every SIMD holding a group has two of its waves (with the sequence split when the groups
//    outnumber the CUs);
//  - otherwise length 4 with 16 rows (3 resident workgroups per CU). 12-row tiles (3 waves,
//    4 per CU) fill the resident slots better at 1024 groups (the 1.4B shape) but measured
//    slower at steady clock (420 against 398 us at 1.4B, 169 against 136 us at 130M): in a
//    12-row tile a quarter of the folding lanes fold two states. They stay available through
//    ss_fwd_options.chunk_rows.
// The zero-order-hold variant runs at two waves per SIMD either way and keeps 16 rows.
ChunkPlan fwd_chunked_pick(const FwdArgs& a, int cus) {
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  if (a.zoh) return {4, 16};  // the zero-order-hold variant spills registers at 8
  // (32 rows of 8 tokens span 256 tokens of the (.., dim) arrays from one 32-bit tile offset)
  if (groups <= 2 * static_cast<int64_t>(cus)) return (256 * a.dim * 4 < (1LL << 31)) ? ChunkPlan{8, 32} : ChunkPlan{8, 16};
  return ChunkPlan{4, 16};
}

// Resident workgroups per CU of a tile plan (VGPR and LDS budgets): 32 rows, 8 waves at two
// per SIMD: 1; 12 rows: 4; 16 rows: 3 with 4-token chunks (2 with the zero-order hold), 2
// with 8-token chunks.
static int plan_slots_per_cu(const FwdArgs& a, ChunkPlan p) {
  if (p.rows == 32) return 1;
  if (p.rows == 12) return a.zoh ? 2 : 4;
  return (p.chunk_len == 4 && !a.zoh) ? 3 : 2;
}

int64_t fwd_split_part_len(int64_t seqlen, ChunkPlan plan, int parts) {
  const int64_t tile = static_cast<int64_t>(plan.rows) * plan.chunk_len;
  const int64_t per = (seqlen + parts - 1) / parts;
  return (per + tile - 1) / tile * tile;
}

// The split pays when the groups leave part of the last round of resident slots empty and
// there are more groups than slots (a group's parts run one after another, so with fewer
// groups than slots the split cannot shorten anything). Model: a sequence part takes 1/parts
// of a whole-sequence time and the work items run in rounds of `slots`; the time is
// max(1, ceil(groups * parts / slots) / parts). Take the fewest parts within 5% of the best.
int fwd_split_parts(const FwdArgs& a, ChunkPlan plan, int cus) {
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  const int64_t slots = static_cast<int64_t>(plan_slots_per_cu(a, plan)) * cus;
  if (groups <= slots || a.seqlen <= 0) return 1;
  auto time = [&](int p) {
    const double rounds = static_cast<double>((groups * p + slots - 1) / slots);
    return std::max(1.0, rounds / p);
  };
  int best = 1;
  double tbest = time(1);
  for (int p = 2; p <= 8; ++p) {
    const int64_t len = fwd_split_part_len(a.seqlen, plan, p);
    if ((a.seqlen + len - 1) / len != p) continue;  // too short for p parts of whole tiles
    const double t = time(p);
    if (t < 0.95 * tbest) {
      best = p;
      tbest = t;
    }
  }
  return best;
}

int64_t fwd_split_items(int64_t groups, int parts) { return groups * (parts - 1); }

size_t fwd_split_ws_bytes(int64_t cap) { return split::ws_bytes(cap); }

hipError_t fwd_split_ws_clear(uint32_t* ws, size_t bytes, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(bytes / 4);
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 1024));
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, ws, n);
  return hipGetLastError();
}

hipError_t fwd_chunked(const FwdArgs& a, ChunkPlan plan, hipStream_t s) {
  return a.dtype == kBF16 ? launch_chunked_t<uint16_t>(a, plan, s) : launch_chunked_t<float>(a, plan, s);
}

}  // namespace ss
