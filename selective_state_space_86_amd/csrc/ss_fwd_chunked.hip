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
#include <atomic>
#include <type_traits>

#include "ss_chunk_ops.h"
#include "ss_split.h"

namespace ss {
namespace {

using namespace chunk;

constexpr int kLdsChunkStride = 16 * 16 + 16;  // [chunk][n][lane], padded against bank conflicts

// Fix-up weights, for the rows of a 32-row tile that own no state in the fold, computed while
// the other rows fold: token j's stored decays become W_j[n] = C_j[n] P_j[n], with P_j[n] the
// product of the chunk's decays up to token j (kept in p), so that once the carry-in q is
// known the fix-up is y_j += sum_n W_j[n] q[n], one fma per update instead of two. With
// `first`, p starts as the token's decays. (C_j[n] comes from lane n of the row by DPP
// row_newbcast:n; every DPP source is written well before the block, which starts with
// s_nop 1.)
#define SS_PRE_M(n) "v_mul_f32 %[p" #n "], %[p" #n "], %[e" #n "]\n"
#define SS_PRE_C(n) "v_mov_b32 %[p" #n "], %[e" #n "]\n"
#define SS_PRE_W(n) "v_mul_f32_dpp %[e" #n "], %[vc], %[p" #n "]" SS_DPP_ROW(n)
#define SS_PRE(M)                                                                              \
  asm volatile("s_nop 1\n" M(0) M(1) SS_PRE_W(0) M(2) SS_PRE_W(1) M(3) SS_PRE_W(2) M(4)         \
               SS_PRE_W(3) M(5) SS_PRE_W(4) M(6) SS_PRE_W(5) M(7) SS_PRE_W(6) M(8) SS_PRE_W(7)     \
               M(9) SS_PRE_W(8) M(10) SS_PRE_W(9) M(11) SS_PRE_W(10) M(12) SS_PRE_W(11) M(13)      \
               SS_PRE_W(12) M(14) SS_PRE_W(13) M(15) SS_PRE_W(14) SS_PRE_W(15)                     \
               : SS_OPS16(p, "+v"), SS_OPS16(e, "+v")                                              \
               : [vc] "v"(vc))
__device__ __forceinline__ void fixup_weights(float (&p)[16], float (&e)[16], float vc, bool first) {
  if (first)
    SS_PRE(SS_PRE_C);
  else
    SS_PRE(SS_PRE_M);
}
#undef SS_PRE
// y += sum_n w[n] q[n] (even and odd states in separate sums, as fixup_step)
__device__ __forceinline__ void fixup_weighted(const float (&w)[16], const float (&q)[16], float& y) {
  float y2 = w[1] * q[1];
  y = __builtin_fmaf(w[0], q[0], y);
#pragma unroll
  for (int n = 2; n < 16; n += 2) {
    y = __builtin_fmaf(w[n], q[n], y);
    y2 = __builtin_fmaf(w[n + 1], q[n + 1], y2);
  }
  y += y2;
}

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
  __shared__ uint32_t item_s, seen_s;
  if (SPLIT) {
    if (tid == 0) item_s = split::take(a.split_ws, groups);  // part * groups + gi
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
  const int wave_tid0 = __builtin_amdgcn_readfirstlane(tid & ~63);  // the wave's first thread (SGPR)
  const int64_t c = c0 + i;
  const bool cvalid = c < a.dim;
  const int64_t cc = cvalid ? c : a.dim - 1;
  // With 4-token chunks the gate input z is loaded at the start of the tile that uses it (its
  // first use is the fix-up, after the local pass and the fold) instead of being prefetched a
  // tile ahead: it is never carried across the loop, which saves a register copy per token at
  // the back edge (1.4B-layer shape: 334 -> 326 us). With 8-token chunks the prefetched form
  // measured faster (3B-layer shape: 3.55 against 3.58 ms), and it stays.
  constexpr bool ZT = GATE && TC <= 4;
  using Loader = TileLoader<T, GATE && !ZT, TC, R>;
  Loader K(a, b, c0, k, i, cc);

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
    if (tid == 0) seen_s = split::poll(a.split_ws, slot, a.split_wait_limit) ? 1u : 0u;
    __syncthreads();  // (the state loads are issued after thread 0 has seen the flag)
    const bool seen = __builtin_amdgcn_readfirstlane(seen_s) != 0u;
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = k + m * R;
      // a wait that gave up leaves the carry unknown: continue from NaN (reported in the header)
      if (n < 16) carry[m] = seen ? split::load_state(a.split_ws, a.split_cap, slot, n, i) : __builtin_nanf("");
    }
  }
  // Wave priorities. Several workgroups per CU (unsplit plans of at most 16 rows): progress
  // priority (ss_common.h). Otherwise: the fix-up at a raised priority. The waves of a SIMD
  // drift apart because the SIMD issues from the oldest wave first: a younger wave's fix-up
  // runs beside an older wave's next local pass, takes about three times as long, and the
  // older wave then waits for it at the first barrier of every tile (8-wave 3B-layer tiles:
  // 4.85 -> 4.25 ms with the raised fix-up). The local pass steps down from 2 to 0 over its
  // tokens and the fix-up runs at 1: at the 1.4B shape (split, 16 rows) 336 against 343-346
  // us with the fix-up at 2 (341 at 3), the 3B shape unchanged.
#ifndef SS_FIXUP_PRIO
#define SS_FIXUP_PRIO 1
#endif
#ifndef SS_LOCAL_RAMP
#define SS_LOCAL_RAMP 1
#endif
  constexpr bool kProgressPrio = !SPLIT && R <= 16;
  constexpr int kFixupPrio = SS_FIXUP_PRIO;
  const uint32_t y_row = static_cast<uint32_t>(a.dim * 4);
  const uint32_t y_off = static_cast<uint32_t>(k * TC) * y_row + static_cast<uint32_t>(i * 4);
  // a lane past the last channel stores to an offset beyond every buffer range (dropped)
  const uint32_t y_voff = cvalid ? y_off : kDropOffset;

  // One tile: local pass, chunk aggregates, combine, fix-up and stores. TAIL is the
  // sequence's last, partial tile: steps of tokens past the end are forced to 0 (the
  // identity) and their outputs are not stored; a full tile needs no per-token test.
  // With load_next the inputs of the following (full) tile are requested into nxt.
  int buf = 0;
  auto tile = [&](auto tail_c, TileIn<TC>& cur, TileIn<TC>& nxt, int64_t t0, bool load_next) {
    constexpr bool TAIL = decltype(tail_c)::value;
    if (kProgressPrio) progress_priority(t0, L);
    else __builtin_amdgcn_s_setprio(0);
    float* lds_a = lds_a2[buf];
#ifndef SS_TOKEN_LOADS
#define SS_TOKEN_LOADS 1
#endif
    // The next tile's inputs: token j's loads are issued right after this tile's token j is
    // consumed, into the registers it leaves (one tile of latency cover; the requests of a
    // tile are spread over its local pass instead of arriving at the memory pipeline all at
    // once). Without SS_TOKEN_LOADS: at the top of the tile (EARLY) or after the local pass.
    typename Loader::Rsrcs nr;
    if (SS_TOKEN_LOADS && load_next) nr = K.rsrcs(t0 + R * TC);
    if (!SS_TOKEN_LOADS && EARLY && load_next) K.load_full(nxt, t0 + R * TC);
    // tokens of this lane's chunk inside the sequence (TC except in the tail tile)
    const int nval = TAIL ? max(0, min(TC, static_cast<int>(L - t0) - k * TC)) : TC;
    // ZT: this tile's gate inputs (the tail tile's tokens past the end re-read the last token)
    Bits<T> zb[TC];
    if (ZT) {
      const auto rz = rsrc_tile(static_cast<const T*>(a.z) + (b * L + t0) * a.dim + c0);
      if (!TAIL) {
        uint32_t tr = K.tok_row;
        asm volatile("" : "+s"(tr));
#pragma unroll
        for (int j = 0; j < TC; ++j) zb[j] = ldr<T>(rz, K.tok_off, j * tr);
      } else {
        const int last = static_cast<int>(L - 1 - t0);
        const uint32_t col = K.tok_off - static_cast<uint32_t>(k * TC) * K.tok_row;
#pragma unroll
        for (int j = 0; j < TC; ++j)
          zb[j] = ldr<T>(rz, static_cast<uint32_t>(min(k * TC + j, last)) * K.tok_row + col, 0);
      }
    }

    // local pass from a zero state
    float h[16], ex[TC][16], y[TC], gate[TC], vc[TC], uu[TC];
#pragma unroll
    for (int j = 0; j < TC; ++j) uu[j] = as_f32<T>(cur.uu[j]);
    if (ZOH) {
#pragma unroll
      for (int n = 0; n < 16; ++n) h[n] = 0.0f;
    }
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
      for (int j = 0; j < TC; ++j) win[j + 3] = as_f32<T>(cur.uu[j]);
      // u_out has y's layout; a null u_out gets an empty range, so every store is dropped
      const int64_t u0 = (b * L + t0) * a.dim + c0;
      const auto ru = rsrc(a.u_out ? a.u_out + u0 : a.y, a.u_out ? (a.batch * L * a.dim - u0) * 4 : 0);
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        uu[j] = conv4_silu(w4, cb, win[j], win[j + 1], win[j + 2], win[j + 3]);
        const uint32_t vo = TAIL ? ((cvalid && j < nval) ? y_off : kDropOffset) : y_voff;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(uu[j]), ru, vo, j * y_row, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      if (!kProgressPrio && SS_LOCAL_RAMP) {
        switch ((3 * j) / TC) {  // (folds to one instruction per unrolled token)
          case 0: __builtin_amdgcn_s_setprio(2); break;
          case 1: __builtin_amdgcn_s_setprio(1); break;
          default: __builtin_amdgcn_s_setprio(0); break;
        }
      }
      const float x = as_f32<T>(cur.raw[j]) + bias;
      const float vb = as_f32<T>(cur.vb[j]);
      vc[j] = as_f32<T>(cur.vc[j]);
      float dt = a.softplus ? softplus(x) : x;
      if (TAIL) dt = j < nval ? dt : 0.0f;  // a zero step is the identity
      dsum += dt;
      y[j] = Dd * uu[j];
      if (ZOH)
        local_step_zoh(h, ex[j], A2, iA, dt, uu[j], vb, vc[j], y[j]);
      else if (j == 0)
        local_step_first(h, ex[0], A2, dt, dt * uu[0], vb, vc[0], y[0]);
      else
        local_step(h, ex[j], A2, dt, dt * uu[j], vb, vc[j], y[j]);
      gate[j] = (GATE && !ZT) ? silu(as_f32<T>(cur.zz[j])) : 1.0f;
      if (SS_TOKEN_LOADS && load_next) K.load_token(nxt, nr, j);
    }

    if (!SS_TOKEN_LOADS && !EARLY && load_next) K.load_full(nxt, t0 + R * TC);

    // chunk aggregates (prod abar = exp(A * sum dt), end state) to LDS
    // (lane-dependent LDS addresses from the thread id formed here: see lane_in_wave)
    const int tid_t = wave_tid0 + lane_in_wave();
    const int k_t = tid_t >> 4, i_t = tid_t & 15;
    {
      float* la = lds_a + k_t * kLdsChunkStride + i_t;
      float* lh = lds_h + k_t * kLdsChunkStride + i_t;
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
    // barrier. (A two-level fold of 32 chunks, rows 16..31 folding the second half from zero
    // and correcting it after one more barrier, measured 8% slower at the 3B shape.)
#pragma unroll
    for (int m = 0; m < NOWN; ++m) {
      const int n = k + m * R;
      if (n < 16) {
        float* sa = lds_a + (k_t + m * R) * 16 + i_t;
        const float* sh = lds_h + (k_t + m * R) * 16 + i_t;
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
    // (32-row tiles: rows 16..31 are waves 4..7, so the test is uniform per wave)
    const bool weighted = R == 32 && wave_tid0 >= 256;
    float q[16];  // this chunk's carry-in (before it, the running decay product of the weights)
    if (weighted) {
#pragma unroll
      for (int j = 0; j < TC; ++j) fixup_weights(q, ex[j], vc[j], j == 0);
    }
    __syncthreads();
    {
      const float* lc = lds_a + k_t * kLdsChunkStride + i_t;
#pragma unroll
      for (int n = 0; n < 16; ++n) q[n] = lc[n * 16];
    }

    // (32-row tiles: the rows that folded have the longer fix-up, two VALU per update against
    // one for the rows with weights, and run it at priority 3: 3B 3.500/3.504/3.511 ->
    // 3.481/3.487/3.482 ms on one box)
    if (!kProgressPrio) {
      if (R == 32 && wave_tid0 < 256)
        __builtin_amdgcn_s_setprio(3);
      else
        __builtin_amdgcn_s_setprio(kFixupPrio);
    }
    // fix-up with the carry-in, gate, store (unconditionally: a masked lane's store goes to an
    // offset past the buffer range and is dropped, so the compiler sees a fixed number of
    // outstanding stores and never waits for them when the prefetched loads are consumed)
    const int64_t y0 = (b * L + t0) * a.dim + c0;
    const auto ry = rsrc_tile(a.y + y0);
    uint32_t yr = y_row;  // (token steps formed per tile, as in the loads)
    asm volatile("" : "+s"(yr));
    auto store = [&](int j) {
      const uint32_t vo = TAIL ? ((cvalid && j < nval) ? y_off : kDropOffset) : y_voff;
      const float g = ZT ? silu(as_f32<T>(zb[j])) : gate[j];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[j] * g), ry, vo, j * yr, 0);
    };
    if (weighted) {  // (one branch around the whole fix-up: q stays one set of registers)
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        fixup_weighted(ex[j], q, y[j]);
        store(j);
      }
    } else {
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        fixup_step(q, ex[j], vc[j], y[j]);
        store(j);
      }
    }
    buf ^= 1;
  };

  // full tiles (a part other than the last holds only full tiles), then the partial tail
  const int64_t nfull = (t_end - t_begin) / (R * TC);
  TileIn<TC> cur, nxt;
  int64_t t0 = t_begin;
  if (nfull > 0) {
    K.load_full(cur, t0);
    if (GATE && !ZT) {
      cur.settle();
    } else {
#pragma unroll
      for (int j = 0; j < TC; ++j)  // (TileIn::settle without the gate inputs, not carried here)
        asm volatile("" : "+v"(cur.raw[j]), "+v"(cur.uu[j]), "+v"(cur.vb[j]), "+v"(cur.vc[j]));
    }
  }
  for (int64_t it = 0; it < nfull; ++it, t0 += R * TC) {
    tile(std::false_type{}, cur, nxt, t0, it + 1 < nfull);
    cur = nxt;
  }
  if (t0 < t_end) {
    K.load_tail(cur, t0);
    tile(std::true_type{}, cur, nxt, t0, false);
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
// The zero-order-hold variant keeps chunk length 4 (it spills registers at 8) and takes 32
// rows where the plain one does (3B long-context shape: 6.31 against 10.35 ms with 16 rows,
// whose 320 groups of 4 waves left most SIMDs one wave).
ChunkPlan fwd_chunked_pick(const FwdArgs& a, int cus) {
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  if (a.zoh)
    return (groups <= 2 * static_cast<int64_t>(cus) && 128 * a.dim * 4 < (1LL << 31)) ? ChunkPlan{4, 32}
                                                                                       : ChunkPlan{4, 16};
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
// max(1, ceil(groups * parts / slots) / parts). Among the part counts whose modelled time is
// within 5% of the best, take the largest whose parts still span at least 32 tiles: shorter
// work items even out the workgroups' finishing times (at the 3B long-context shape 4, 8 and
// 12 parts model the same; 8 measured 1.1% faster than 4, and its neighbouring groups, which
// share cache lines, drift apart less: 1.076 against 1.094 times the algorithmic bytes), while
// each part adds a hand-off and a tile's start-up (at the 1.4B shape 3 and 6 parts model the
// same, and 6 parts of 11 tiles measured 0.8% slower than 3 of 22).
int fwd_split_parts(const FwdArgs& a, ChunkPlan plan, int cus) {
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  const int64_t slots = static_cast<int64_t>(plan_slots_per_cu(a, plan)) * cus;
  if (groups <= slots || a.seqlen <= 0) return 1;
  auto time = [&](int p) {
    const double rounds = static_cast<double>((groups * p + slots - 1) / slots);
    return std::max(1.0, rounds / p);
  };
  const int64_t tile = static_cast<int64_t>(plan.rows) * plan.chunk_len;
  auto fits = [&](int p) {  // p parts of whole tiles
    const int64_t len = fwd_split_part_len(a.seqlen, plan, p);
    return (a.seqlen + len - 1) / len == p;
  };
  // Among the part counts whose modelled time is within 5% of the best, the largest whose
  // parts still span 40 tiles: shorter parts even out the workgroups' finishing times, and
  // each part pays a start (its first tile's loads, the hand-off); at most 12 parts, whose
  // hand-off slots the fixed scratch of ss_fwd_noalloc holds at the 3B layer's 320 groups.
  double tbest = time(1);
  for (int p = 2; p <= 12; ++p)
    if (fits(p)) tbest = std::min(tbest, time(p));
  int best = 1;
  for (int p = 2; p <= 12; ++p) {
    if (!fits(p) || time(p) > tbest / 0.95) continue;
    if (best == 1 || fwd_split_part_len(a.seqlen, plan, p) >= 40 * tile) best = p;
  }
  return best;
}

int64_t fwd_split_items(int64_t groups, int parts) { return groups * (parts - 1); }

namespace {
__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t j = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; j < n;
       j += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[j] = 0u;
}
}  // namespace

hipError_t split::clear(uint32_t* ws, int64_t cap, hipStream_t s) {
  const int64_t n = split::clear_words(cap);
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n + 255) / 256, 64));
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, ws, n);
  return hipGetLastError();
}

// The fixed scratch of ss_fwd_noalloc: one array per device (every GPU the library runs on
// holds its own copy until the process ends). Host code never passes `noalloc_scratch`
// itself to a kernel (in host code it names a host-side stand-in): it uses the device
// address hipGetSymbolAddress gives, looked up once per device and kept.
static __device__ __align__(256) uint32_t noalloc_scratch[kNoallocScratchBytes / 4];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<uint32_t*> g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch_ptr(uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  uint32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(noalloc_scratch));  // (the current device's copy)
    if (e != hipSuccess) return e;
    p = static_cast<uint32_t*>(q);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t fwd_chunked(const FwdArgs& a, ChunkPlan plan, hipStream_t s) {
  return a.dtype == kBF16 ? launch_chunked_t<uint16_t>(a, plan, s) : launch_chunked_t<float>(a, plan, s);
}

}  // namespace ss
