// ss_kernels.h -- host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// Validated arguments of one ss_fwd call (device pointers, element counts).
struct FwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // may be null
  const void* z;            // may be null
  const float* delta_bias;  // may be null
  float* y;
  float* last_state;        // may be null
  int64_t batch, seqlen, dim, dstate;
  int dtype;
  int softplus;
  const float* h0;          // may be null: zero initial state
  int zoh;                  // input term: 0 dt*B, 1 exact zero-order hold (e^{dt A} - 1)/A * B
  // conv prologue (kconv > 0): u is x, and the scan uses silu(conv_b + conv_w * x) instead
  int kconv;                // 0 (no prologue) or 1..4 taps
  const float* conv_w;      // (dim, kconv)
  const float* conv_b;      // (dim), may be null
  const float* conv_state;  // (batch, dim, kconv - 1) inputs before t = 0, may be null
  float* u_out;             // (batch, seqlen, dim) the prologue output, may be null
  // sequence split of the chunked kernel (parts > 1): the sequence of every channel group is
  // cut into parts of part_len tokens; workgroups take work items (part q, group g) from a
  // counter in split_ws in that order, and part q > 0 starts from the state part q - 1
  // publishes there (so the groups' work spreads evenly over the CUs)
  int parts;                // 0 or 1: one workgroup per channel group over the whole sequence
  int64_t part_len;         // tokens per part, a multiple of the tile; parts * part_len >= seqlen
  uint32_t* split_ws;       // split::region_bytes(split_cap) of device memory whose header and
                            // flags were cleared (split::clear) on the kernel's stream
  int64_t split_cap;        // published-state slots of split_ws, >= (batch * groups) * (parts - 1)
  int split_wait_limit;     // polls before a hand-off wait gives up: 0 the default, < 0 none
};

// Validated arguments of one ss_step call.
struct StepArgs {
  float* state;
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* delta_bias;
  float* y;
  int64_t batch, dim, dstate;
  int dtype;
  int softplus;
  int zoh;                  // as FwdArgs::zoh
};

// Validated arguments of one ss_bwd call. Workspace regions (fp32): ckpt
// (batch, ntiles, ngroups*16, 16), part_bc (2, batch, ngroups, seqlen, dstate),
// part_ch (batch, ngroups*16, 18).
struct BwdArgs {
  const void* u;
  const void* delta;
  const float* A;
  const void* B;
  const void* C;
  const float* D;           // may be null
  const void* z;            // may be null
  const float* delta_bias;  // may be null
  const float* h0;          // may be null
  const float* dy;
  const float* dlast;       // may be null
  float* du;
  float* ddelta;
  float* dz;                // required iff z
  float* dh0;               // may be null
  float* dA;
  float* dB;
  float* dC;
  float* dD;                // may be null
  float* dbias;             // may be null
  float* ckpt;
  float* part_bc;
  float* part_ch;
  int64_t batch, seqlen, dim, dstate;
  int64_t ngroups;          // channel groups of 16 per batch row
  int64_t ntiles;           // checkpoint intervals of bwd_tile_tokens() tokens
  int dtype;
  int softplus;
  int rows;                 // time chunks per workgroup tile: 16 (4 waves) or 32 (8 waves)
  // sequence split (parts > 1) of the reverse kernel (ss_split.h): parts of part_len tokens
  // (whole tiles of both kernels); part_ch then holds one (batch, ngroups*16, 18) block per
  // part. The checkpoint kernel, which holds more workgroups per CU, has its own ckpt_parts
  // of ckpt_part_len tokens. Both kernels use the one workspace, one after the other.
  int parts;
  int64_t part_len;
  uint32_t* split_ws;
  int64_t split_cap;
  int ckpt_parts;
  int64_t ckpt_part_len;
  int split_wait_limit;     // as FwdArgs::split_wait_limit
};

constexpr int kBwdMaxParts = 8;  // sequence parts of the backward split at most

constexpr int kBwdChunk = 2;  // tokens per lane and chunk in the backward kernels

// Validated arguments of one ss_proj call (all token arrays and weights in one dtype).
struct ProjArgs {
  const void* u;            // (tokens, dim)
  const void* W_x;          // (rank + 2 dstate, dim)
  const void* W_dt;         // (dim, rank)
  void* delta_raw;          // (tokens, dim)
  void* B;                  // (tokens, dstate)
  void* C;                  // (tokens, dstate)
  int64_t tokens, dim, dstate, rank;
  int dtype;
  int64_t seqlen;           // tokens per sequence (the convolution restarts at each)
  int kconv;                // 0: u is given; 1..4: u = silu(conv(x) + conv_b) with kconv taps
  const float* conv_w;      // (dim, kconv)
  const float* conv_b;      // (dim,) or null
  const float* conv_state;  // (tokens / seqlen, dim, kconv - 1) or null (zeros)
};

hipError_t fwd_seq(const FwdArgs& a, hipStream_t s);
bool fwd_state_supported(const FwdArgs& a);
hipError_t fwd_state(const FwdArgs& a, hipStream_t s);
bool fwd_chunked_supported(const FwdArgs& a);
// Tile shape of the time-chunked forward: chunk_len tokens per lane (4 or 8) and rows time
// chunks per workgroup (16, or 12 with chunk_len 4).
struct ChunkPlan {
  int chunk_len;
  int rows;
};
hipError_t fwd_chunked(const FwdArgs& a, ChunkPlan plan, hipStream_t s);
ChunkPlan fwd_chunked_pick(const FwdArgs& a, int cus);
// Parts per sequence for the split (1: no split) and the bytes of its workspace.
int fwd_split_parts(const FwdArgs& a, ChunkPlan plan, int cus);
int64_t fwd_split_part_len(int64_t seqlen, ChunkPlan plan, int parts);
int64_t fwd_split_items(int64_t groups, int parts);  // published states of one call
// Bytes of the fixed per-device scratch array of the allocation-free forward entry point,
// and its device address on the current device (looked up on first use, then kept).
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;
hipError_t noalloc_scratch_ptr(uint32_t** out);
hipError_t proj(const ProjArgs& a, int cus, hipStream_t s);
int proj_step_tiles(int64_t rank, int dtype);
hipError_t step(const StepArgs& a, hipStream_t s);
int64_t bwd_tile_tokens();
int bwd_rows(int64_t groups, int64_t seqlen, int cus);  // the tile rows for these channel groups
// Parts per sequence of the backward split for this tile plan (1: none) and their length,
// for the reverse kernel or (ckpt) the checkpoint kernel.
int bwd_split_parts(int64_t groups, int rows, bool ckpt, int64_t seqlen, int cus);
int64_t bwd_split_part_len(int64_t seqlen, int rows, int parts);
size_t bwd_workspace_bytes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);
hipError_t bwd(const BwdArgs& a, hipStream_t s);

}  // namespace ss
