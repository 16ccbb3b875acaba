// ss_chunk_ops.h -- building blocks of the time-chunked selective-scan kernel (gfx950):
// the hand-scheduled per-token update and fix-up for 16 states, buffer-resource loads,
// and the per-lane tile loader.
//
// Lane layout: a row of 16 lanes holds 16 consecutive channels at
// one token, so B_t and C_t are row-uniform and lane n of the row holds B_t[n], C_t[n];
// the update reads them through DPP row_newbcast:n folded into the consuming v_mul/v_fmac.
#pragma once

#include <type_traits>

#include "ss_common.h"
#include "ss_kernels.h"

namespace ss {
namespace chunk {

#define SS_DPP_ROW(n) " row_newbcast:" #n " row_mask:0xf bank_mask:0xf\n"

// One token of the local pass for all 16 states, software-pipelined so that
//  - each exp result is consumed >= 2 instructions after it is produced, and
//  - each VGPR read by a DPP instruction was written >= 2 instructions earlier
// (the gfx950 transcendental-forwarding and DPP read-after-write wait states).
#define SS_UPD(n, n2)                                                        \
  "v_mul_f32_dpp %[bu], %[vb], %[du]" SS_DPP_ROW(n)                          \
  "v_fma_f32 %[h" #n "], %[e" #n "], %[h" #n "], %[bu]\n"                    \
  "v_mul_f32 %[x], %[dt], %[a" #n2 "]\n"                                     \
  "v_exp_f32 %[e" #n2 "], %[x]\n"                                            \
  "v_fmac_f32_dpp %[y], %[vc], %[h" #n "]" SS_DPP_ROW(n)

#define SS_OPS16(P, r) \
  [P##0] r(P[0]), [P##1] r(P[1]), [P##2] r(P[2]), [P##3] r(P[3]), [P##4] r(P[4]), [P##5] r(P[5]), \
  [P##6] r(P[6]), [P##7] r(P[7]), [P##8] r(P[8]), [P##9] r(P[9]), [P##10] r(P[10]), [P##11] r(P[11]), \
  [P##12] r(P[12]), [P##13] r(P[13]), [P##14] r(P[14]), [P##15] r(P[15])

__device__ __forceinline__ void local_step(float (&h)[16], float (&e)[16], const float (&a)[16], float dt,
                                           float du, float vb, float vc, float& y) {
  float x, bu;
  asm volatile(
      "s_nop 0\n"
      "v_mul_f32 %[x], %[dt], %[a0]\n"
      "v_exp_f32 %[e0], %[x]\n"
      "v_mul_f32 %[x], %[dt], %[a1]\n"
      "v_exp_f32 %[e1], %[x]\n"
      SS_UPD(0, 2) SS_UPD(1, 3) SS_UPD(2, 4) SS_UPD(3, 5) SS_UPD(4, 6) SS_UPD(5, 7)
      SS_UPD(6, 8) SS_UPD(7, 9) SS_UPD(8, 10) SS_UPD(9, 11) SS_UPD(10, 12) SS_UPD(11, 13)
      SS_UPD(12, 14) SS_UPD(13, 15)
      "v_mul_f32_dpp %[bu], %[vb], %[du]" SS_DPP_ROW(14)
      "v_fma_f32 %[h14], %[e14], %[h14], %[bu]\n"
      "v_mul_f32_dpp %[bu], %[vb], %[du]" SS_DPP_ROW(15)
      "v_fma_f32 %[h15], %[e15], %[h15], %[bu]\n"
      "v_fmac_f32_dpp %[y], %[vc], %[h14]" SS_DPP_ROW(14)
      "s_nop 0\n"
      "v_fmac_f32_dpp %[y], %[vc], %[h15]" SS_DPP_ROW(15)
      : SS_OPS16(h, "+v"), SS_OPS16(e, "=&v"), [y] "+v"(y), [x] "=&v"(x), [bu] "=&v"(bu)
      : SS_OPS16(a, "v"), [dt] "v"(dt), [du] "v"(du), [vb] "v"(vb), [vc] "v"(vc));
}

// The first token of a chunk, whose state before it is zero: h[n] = (dt u) B_t[n] with no
// multiply-add, y += C_t[n] h[n], and the decays abar[n] = 2^(dt A'[n]) stored for the chunk
// aggregate and the fix-up (3 VALU + 1 transcendental per state; none of the exps is read
// here). Each h is read by its DPP fmac 2 instructions after the multiply that wrote it
// (as a plain operand: only vb and vc are read through DPP).
#define SS_UPD0(n)                                                           \
  "v_mul_f32_dpp %[h" #n "], %[vb], %[du]" SS_DPP_ROW(n)                     \
  "v_mul_f32 %[x], %[dt], %[a" #n "]\n"                                       \
  "v_exp_f32 %[e" #n "], %[x]\n"                                              \
  "v_fmac_f32_dpp %[y], %[vc], %[h" #n "]" SS_DPP_ROW(n)

__device__ __forceinline__ void local_step_first(float (&h)[16], float (&e)[16], const float (&a)[16], float dt,
                                                 float du, float vb, float vc, float& y) {
  float x;
  asm volatile(
      "s_nop 1\n"  // (the first instruction reads vb through DPP: 2 wait states after its write)
      SS_UPD0(0) SS_UPD0(1) SS_UPD0(2) SS_UPD0(3) SS_UPD0(4) SS_UPD0(5) SS_UPD0(6) SS_UPD0(7)
      SS_UPD0(8) SS_UPD0(9) SS_UPD0(10) SS_UPD0(11) SS_UPD0(12) SS_UPD0(13) SS_UPD0(14) SS_UPD0(15)
      : SS_OPS16(h, "=&v"), SS_OPS16(e, "=&v"), [y] "+v"(y), [x] "=&v"(x)
      : SS_OPS16(a, "v"), [dt] "v"(dt), [du] "v"(du), [vb] "v"(vb), [vc] "v"(vc));
}

// State update of one token from precomputed input terms bbu[n] = bbar[n] * u:
// h[n] = abar[n] h[n] + bbu[n] B_t[n]; y += C_t[n] h[n] (B_t, C_t by row_newbcast:n).
// Pipelined like local_step: each h is read by its DPP fmac >= 2 instructions after the
// fma that wrote it.
#define SS_UPDB(n, n1)                                                        \
  "v_mul_f32_dpp %[t], %[vb], %[bb" #n1 "]" SS_DPP_ROW(n1)                    \
  "v_fma_f32 %[h" #n1 "], %[e" #n1 "], %[h" #n1 "], %[t]\n"                  \
  "v_fmac_f32_dpp %[y], %[vc], %[h" #n "]" SS_DPP_ROW(n)

__device__ __forceinline__ void update_from_terms(float (&h)[16], const float (&e)[16],
                                                  const float (&bb)[16], float vb, float vc, float& y) {
  float t;
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32_dpp %[t], %[vb], %[bb0]" SS_DPP_ROW(0)
      "v_fma_f32 %[h0], %[e0], %[h0], %[t]\n"
      SS_UPDB(0, 1) SS_UPDB(1, 2) SS_UPDB(2, 3) SS_UPDB(3, 4) SS_UPDB(4, 5) SS_UPDB(5, 6)
      SS_UPDB(6, 7) SS_UPDB(7, 8) SS_UPDB(8, 9) SS_UPDB(9, 10) SS_UPDB(10, 11) SS_UPDB(11, 12)
      SS_UPDB(12, 13) SS_UPDB(13, 14) SS_UPDB(14, 15)
      "s_nop 1\n"
      "v_fmac_f32_dpp %[y], %[vc], %[h15]" SS_DPP_ROW(15)
      : SS_OPS16(h, "+v"), [y] "+v"(y), [t] "=&v"(t)
      : SS_OPS16(e, "v"), SS_OPS16(bb, "v"), [vb] "v"(vb), [vc] "v"(vc));
}

// One token of the local pass with the exact zero-order-hold input term bbar = (abar - 1)/A
// (zoh_coef): the decays and input terms of the 16 states first (compiler-scheduled), then
// the pipelined update. Computing them in two phases keeps the live temporaries to one
// array of 16; interleaving everything per state made the compiler spill.
__device__ __forceinline__ void local_step_zoh(float (&h)[16], float (&e)[16], const float (&a)[16],
                                               const float (&ia)[16], float dt, float uu, float vb,
                                               float vc, float& y) {
  float bb[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const float x2 = dt * a[n];
    e[n] = fast_exp2(x2);
    bb[n] = zoh_coef(dt, x2 * kLn2, e[n], ia[n]) * uu;
  }
  update_from_terms(h, e, bb, vb, vc, y);
}

#define SS_FIX_M(n) "v_mul_f32 %[q" #n "], %[q" #n "], %[e" #n "]\n"
#define SS_FIX_F(n, Y) "v_fmac_f32_dpp %[" #Y "], %[vc], %[q" #n "]" SS_DPP_ROW(n)

// Fix-up of one token: q[n] *= abar_t[n]; y += C_t[n] q[n] (C_t[n] via row_newbcast:n).
// Each q is read by the DPP fmac >= 2 instructions after its multiply; even and odd states
// accumulate into separate registers so consecutive fmacs do not wait on each other (the odd
// sum starts with a multiply instead of a cleared register).
__device__ __forceinline__ void fixup_step(float (&q)[16], const float (&e)[16], float vc, float& y) {
  float y2;
  asm volatile(
      SS_FIX_M(0) SS_FIX_M(1) SS_FIX_M(2) SS_FIX_F(0, y) SS_FIX_M(3)
      "v_mul_f32_dpp %[y2], %[vc], %[q1]" SS_DPP_ROW(1)
      SS_FIX_M(4)
      SS_FIX_F(2, y) SS_FIX_M(5) SS_FIX_F(3, y2) SS_FIX_M(6) SS_FIX_F(4, y) SS_FIX_M(7) SS_FIX_F(5, y2)
      SS_FIX_M(8) SS_FIX_F(6, y) SS_FIX_M(9) SS_FIX_F(7, y2) SS_FIX_M(10) SS_FIX_F(8, y) SS_FIX_M(11)
      SS_FIX_F(9, y2) SS_FIX_M(12) SS_FIX_F(10, y) SS_FIX_M(13) SS_FIX_F(11, y2) SS_FIX_M(14)
      SS_FIX_F(12, y) SS_FIX_M(15) SS_FIX_F(13, y2) SS_FIX_F(14, y) SS_FIX_F(15, y2)
      : SS_OPS16(q, "+v"), [y] "+v"(y), [y2] "=&v"(y2)
      : SS_OPS16(e, "v"), [vc] "v"(vc));
  y += y2;
}

// Buffer resource (gfx9 V#) over [base, base + bytes): loads take an SGPR descriptor, a
// per-lane 32-bit offset and an SGPR offset, so addressing costs no vector instructions.
// Accesses past `bytes` read 0 / are dropped by the hardware range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes > 0x7fffffffLL ? 0x7fffffff : static_cast<int32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}
// A resource over [base, base + 2^31 - 1) for accesses known to be in bounds (a tile's
// loads and stores; only kDropOffset lies outside): no per-tile range arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_tile(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), 0x7fffffff, 0x00020000);
}
// A per-lane byte offset beyond every range rsrc() creates (those are clamped to 2^31 - 1):
// a buffer store at it is dropped by the range check, a load returns 0.
constexpr uint32_t kDropOffset = 0x80000000u;
// Raw element bits (the b32/b16 builtins move raw bits as unsigned integers), widened to
// fp32 where they are used (as_f32): a prefetched tile stays in the registers the loads
// wrote, so nothing reads them, and nothing waits for them, before the tile is consumed.
__device__ __forceinline__ uint32_t ldb(float*, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t ldb(uint16_t*, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0));
}
template <typename T>
__device__ __forceinline__ float as_f32(uint32_t w) {
  return __uint_as_float(sizeof(T) == 2 ? w << 16 : w);  // bf16 is the top half of an fp32
}
// Raw bits in the element's own width (u16 for bf16), for values carried across a loop: a
// 32-bit copy of a 16-bit load is a zero-extension, which the compiler performs before the
// loop's back edge, where it waits for the load; carried in its own width, the value is
// widened only where it is used (as_f32 shifts the low half up, ignoring the rest).
template <typename T>
using Bits = std::conditional_t<sizeof(T) == 2, uint16_t, uint32_t>;
template <typename T>
__device__ __forceinline__ Bits<T> ldr(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(T) == 2)
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  else
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
// An element widened to fp32 at the load (for loads consumed soon after).
template <typename T>
__device__ __forceinline__ float ldf(T* tag, __amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return as_f32<T>(ldb(tag, r, voff, soff));
}

// The lane's index in its wave, formed anew where it is called (v_mbcnt; the asm keeps the
// compiler from hoisting it): per-lane LDS addresses inside the tile loop are rebuilt from it
// and the wave's first thread id (an SGPR) instead of being kept in a VGPR across the loop,
// where at the register limit they were spilled and their reload waited for every load in
// flight (vmcnt(0)), the next tile's included.
__device__ __forceinline__ int lane_in_wave() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Map the linear workgroup id to a channel group so that neighbouring groups (which share
// 128-byte lines of u, delta, z and y) land on the same XCD (workgroups are dealt to the 8
// XCDs round-robin) and are dispatched close together.
__device__ __forceinline__ int64_t group_of(int64_t bid, int64_t ngroups) {
  if (ngroups % 8 != 0) return bid;
  return (bid % 8) * (ngroups / 8) + bid / 8;
}

template <int TC>
struct TileIn {  // raw element bits of one lane's chunk (as_f32 widens them)
  uint32_t raw[TC], uu[TC], zz[TC], vb[TC], vc[TC];
  // Wait for this tile's loads here and give every register a definition that is not a
  // load. For the first tile, before the tile loop: inside the loop the tile registers are
  // copies of the prefetched ones, and a load on one path into the loop makes the compiler
  // wait conservatively, at the loop's start, for loads issued in the loop.
  __device__ __forceinline__ void settle() {
#pragma unroll
    for (int j = 0; j < TC; ++j) asm volatile("" : "+v"(raw[j]), "+v"(uu[j]), "+v"(zz[j]), "+v"(vb[j]), "+v"(vc[j]));
  }
};

// ROWS chunks of TC tokens form one tile (16 for a workgroup tile, 4 for a wave-tile).
template <typename T, bool GATE, int TC, int ROWS>
struct TileLoader {
  const FwdArgs& a;
  int64_t b, c0, L, dim;
  int k, i;
  uint32_t tok_off, bc_off;  // lane byte offsets of token j = 0 of its chunk within a tile
  uint32_t tok_row, bc_row;  // bytes per token of (.., dim) and (.., 16) rows

  __device__ TileLoader(const FwdArgs& args, int64_t b_, int64_t c0_, int k_, int i_, int64_t cc)
      : a(args), b(b_), c0(c0_), L(args.seqlen), dim(args.dim), k(k_), i(i_) {
    tok_row = static_cast<uint32_t>(dim * sizeof(T));
    bc_row = 16 * sizeof(T);
    tok_off = static_cast<uint32_t>(k * TC) * tok_row + static_cast<uint32_t>((cc - c0) * sizeof(T));
    bc_off = static_cast<uint32_t>(k * TC) * bc_row + static_cast<uint32_t>(i * sizeof(T));
  }

  // Request the inputs of the tile starting at t0: load_full for a tile inside the sequence
  // (fixed per-lane offsets, the token step in the SGPR offset), load_tail for the sequence's
  // last, partial tile, whose tokens past the end re-read the last token (their step is
  // forced to 0 where they are used).
  __device__ __forceinline__ void load_full(TileIn<TC>& x, int64_t t0) const { load<true>(x, t0); }
  __device__ __forceinline__ void load_tail(TileIn<TC>& x, int64_t t0) const { load<false>(x, t0); }

  // Token by token: the resources of the full tile at t0 (rsrcs), then the loads of token j
  // (load_token), issued while the previous tile is being consumed.
  struct Rsrcs {
    __amdgpu_buffer_rsrc_t rd, ru, rz, rB, rC;
    uint32_t tr;  // the token step (opaque copy, as in load)
  };
  __device__ __forceinline__ Rsrcs rsrcs(int64_t t0) const {
    const int64_t tok0 = (b * L + t0) * dim + c0;
    const int64_t bc0 = (b * L + t0) * 16;
    Rsrcs r;
    r.rd = rsrc_tile(static_cast<const T*>(a.delta) + tok0);
    r.ru = rsrc_tile(static_cast<const T*>(a.u) + tok0);
    r.rz = rsrc_tile(GATE ? static_cast<const T*>(a.z) + tok0 : static_cast<const T*>(a.u));
    r.rB = rsrc_tile(static_cast<const T*>(a.B) + bc0);
    r.rC = rsrc_tile(static_cast<const T*>(a.C) + bc0);
    r.tr = tok_row;
    asm volatile("" : "+s"(r.tr));
    return r;
  }
  __device__ __forceinline__ void load_token(TileIn<TC>& x, const Rsrcs& r, int j) const {
    T* tag = nullptr;
    x.raw[j] = ldb(tag, r.rd, tok_off, j * r.tr);
    x.uu[j] = ldb(tag, r.ru, tok_off, j * r.tr);
    if (GATE) x.zz[j] = ldb(tag, r.rz, tok_off, j * r.tr);
    x.vb[j] = ldb(tag, r.rB, bc_off, j * bc_row);
    x.vc[j] = ldb(tag, r.rC, bc_off, j * bc_row);
  }

  template <bool FULL>
  __device__ __forceinline__ void load(TileIn<TC>& x, int64_t t0) const {
    // (every access below is in bounds: a tail tile re-reads its last token instead of
    // reading past the sequence, and a lane past the last channel reads channel dim - 1)
    const int64_t tok0 = (b * L + t0) * dim + c0;
    const int64_t bc0 = (b * L + t0) * 16;
    const auto rd = rsrc_tile(static_cast<const T*>(a.delta) + tok0);
    const auto ru = rsrc_tile(static_cast<const T*>(a.u) + tok0);
    const auto rz = rsrc_tile(GATE ? static_cast<const T*>(a.z) + tok0 : static_cast<const T*>(a.u));
    const auto rB = rsrc_tile(static_cast<const T*>(a.B) + bc0);
    const auto rC = rsrc_tile(static_cast<const T*>(a.C) + bc0);
    T* tag = nullptr;
    if (FULL) {
      // (the token steps j * tok_row are formed here at every call from an opaque copy of the
      // stride, so they occupy SGPRs only while the loads issue instead of across the loop)
      uint32_t tr = tok_row;
      asm volatile("" : "+s"(tr));
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        x.raw[j] = ldb(tag, rd, tok_off, j * tr);
        x.uu[j] = ldb(tag, ru, tok_off, j * tr);
        if (GATE) x.zz[j] = ldb(tag, rz, tok_off, j * tr);
        x.vb[j] = ldb(tag, rB, bc_off, j * bc_row);
        x.vc[j] = ldb(tag, rC, bc_off, j * bc_row);
      }
    } else {
      const int last = static_cast<int>(L - 1 - t0);
      const uint32_t col = tok_off - static_cast<uint32_t>(k * TC) * tok_row;
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        const uint32_t tt = static_cast<uint32_t>(min(k * TC + j, last));
        const uint32_t to = tt * tok_row + col;
        const uint32_t bo = tt * bc_row + static_cast<uint32_t>(i * sizeof(T));
        x.raw[j] = ldb(tag, rd, to, 0);
        x.uu[j] = ldb(tag, ru, to, 0);
        if (GATE) x.zz[j] = ldb(tag, rz, to, 0);
        x.vb[j] = ldb(tag, rB, bo, 0);
        x.vc[j] = ldb(tag, rC, bo, 0);
      }
    }
  }
};


}  // namespace chunk
}  // namespace ss
