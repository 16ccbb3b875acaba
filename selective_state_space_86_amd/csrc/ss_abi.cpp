// ss_abi.cpp -- the extern "C" entry points of libss: argument validation, device check,
// dispatch to the gfx950 kernels on the caller's stream. See include/ss.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>

#include "../../include/ss.h"
#include "ss_kernels.h"
#include "ss_split.h"

static_assert(ss::kNoallocScratchBytes == SS_NOALLOC_SCRATCH_BYTES, "the scratch size the header states");

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_device_cus[kMaxDevices];

// Is the current device a gfx950? The answer (and the CU count) is cached per device id.
int check_device(int* cus) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SS_ERR_HIP;
  if (dev < kMaxDevices) {
    const int c = g_device_ok[dev].load(std::memory_order_acquire);
    if (c == 1) {
      *cus = g_device_cus[dev].load(std::memory_order_relaxed);
      return SS_OK;
    }
    if (c == 2) return SS_ERR_DEVICE;
  }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) return SS_ERR_HIP;
  const bool ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
  *cus = p.multiProcessorCount > 0 ? p.multiProcessorCount : 256;
  if (dev < kMaxDevices) {
    g_device_cus[dev].store(*cus, std::memory_order_relaxed);
    g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_release);
  }
  return ok ? SS_OK : SS_ERR_DEVICE;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_size(int dtype) { return dtype == SS_DTYPE_BF16 ? 2 : 4; }

// batch * seqlen * dim < 2^62 without overflow
bool product_ok(int64_t a, int64_t b, int64_t c) {
  const int64_t lim = int64_t(1) << 62;
  if (a > 0 && b > lim / a) return false;
  const int64_t ab = a * b;
  if (ab > 0 && c > lim / ab) return false;
  return true;
}

}  // namespace

namespace {

struct ConvArgs {
  int64_t kconv;
  const float* conv_w;
  const float* conv_b;
  const float* conv_state;
  float* u_out;
};

// Sizes and options of a forward call, validated without touching any pointer.
int check_fwd_sizes(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int in_dtype,
                    const ss_fwd_options* opt) {
  if (in_dtype != SS_DTYPE_F32 && in_dtype != SS_DTYPE_BF16) return SS_ERR_BAD_DTYPE;
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 0) return SS_ERR_BAD_SHAPE;
  if (dstate > SS_MAX_DSTATE) return SS_ERR_UNSUPPORTED_N;
  if (!product_ok(batch, seqlen, dim) || !product_ok(batch, seqlen, dstate) ||
      !product_ok(batch, dim, dstate))
    return SS_ERR_BAD_SHAPE;
  if (batch * ((dim + 15) / 16) > 0x7fffffffLL) return SS_ERR_BAD_SHAPE;
  const int kernel = opt ? opt->kernel : 0;
  const int chunk = opt ? opt->chunk_len : 0;
  const int disc = opt ? opt->discretization : SS_DISC_DT;
  const int rows = opt ? opt->chunk_rows : 0;
  const int split_parts = opt ? opt->split_parts : 0;
  if (kernel < 0 || kernel > 3 || !(chunk == 0 || chunk == 4 || chunk == 8)) return SS_ERR_BAD_SHAPE;
  if (split_parts < 0 || split_parts > 16) return SS_ERR_BAD_SHAPE;
  if (!(rows == 0 || rows == 16 || rows == 12 || rows == 32) || (rows == 12 && chunk == 8)) return SS_ERR_BAD_SHAPE;
  // (a tile of 32 rows of 8 tokens spans 256 tokens of the (.., dim) arrays from 32-bit offsets)
  if (rows == 32 && 256 * dim * 4 >= (1LL << 31)) return SS_ERR_BAD_SHAPE;
  if (disc != SS_DISC_DT && disc != SS_DISC_ZOH) return SS_ERR_BAD_SHAPE;
  if (kernel == 2 && dstate != 16) return SS_ERR_UNSUPPORTED_N;
  return SS_OK;
}

// The kernel a forward call runs, and for the time-chunked kernel its tile plan and split.
struct FwdPlan {
  int kind;              // 1 sequential, 2 time-chunked, 3 state-parallel
  ss::ChunkPlan chunk;   // kind 2
  int parts;             // kind 2: sequence parts (1: none)
  int64_t part_len;      // with parts > 1
  size_t split_bytes;    // workspace the split needs (0: none)
};

// Plan a forward call (sizes validated) on a device with `cus` CUs. The time-chunked kernel
// addresses a tile of R rows of TC tokens of the (.., dim) arrays from 32-bit offsets, so a
// plan whose tile spans 2^31 bytes or more of fp32 rows is not taken (an explicit choice of
// it is an error); the state-parallel kernel spans 16 tokens of the input rows.
int plan_fwd(ss::FwdArgs& a, const ss_fwd_options* opt, int cus, FwdPlan* pl) {
  const int kernel = opt ? opt->kernel : 0;
  const int chunk = opt ? opt->chunk_len : 0;
  const int rows = opt ? opt->chunk_rows : 0;
  const int split_parts = opt ? opt->split_parts : 0;
  const int64_t groups = a.batch * ((a.dim + 15) / 16);
  const int64_t es = elem_size(a.dtype);
  auto tile_fits = [&](const ss::ChunkPlan& p) {
    return static_cast<int64_t>(p.rows) * p.chunk_len * a.dim * 4 < (1LL << 31);
  };
  const bool state_fits = 16 * a.dim * es < (1LL << 31);
  *pl = FwdPlan{1, {4, 16}, 1, 0, 0};
  if (a.seqlen == 0) return SS_OK;  // the sequential kernel writes the final state (h0 or zero)
  if (kernel == 3) {
    if (!ss::fwd_state_supported(a) || !state_fits) return SS_ERR_BAD_SHAPE;
    pl->kind = 3;
    return SS_OK;
  }
  if (kernel == 1) return SS_OK;
  auto split_plan = [&](const ss::ChunkPlan& plan) {
    int parts = split_parts == 0 ? ss::fwd_split_parts(a, plan, cus) : split_parts;
    if (parts > 1) {  // whole tiles per part: a short sequence gets fewer parts
      pl->part_len = ss::fwd_split_part_len(a.seqlen, plan, parts);
      parts = static_cast<int>((a.seqlen + pl->part_len - 1) / pl->part_len);
      if (groups * parts > 0x7fffffffLL) parts = 1;
    }
    pl->parts = parts;
    if (parts > 1) pl->split_bytes = ss::split::region_bytes(ss::fwd_split_items(groups, parts));
  };
  const bool chunked = kernel == 2 || (kernel == 0 && ss::fwd_chunked_supported(a));
  if (chunked) {
    // explicit choices override the automatic plan; 12 rows exist only with 4-token chunks
    ss::ChunkPlan plan = ss::fwd_chunked_pick(a, cus);
    if (chunk != 0) plan.chunk_len = chunk;
    if (rows != 0) plan.rows = rows;
    if (plan.rows == 12 && plan.chunk_len != 4) {
      if (rows == 12) plan.chunk_len = 4;  // rows asked for, chunk length automatic
      else plan.rows = 16;                 // chunk length 8 asked for, rows automatic
    }
    if (!tile_fits(plan)) {
      if (kernel == 2 && (chunk != 0 || rows != 0)) return SS_ERR_BAD_SHAPE;
      plan = ss::ChunkPlan{4, 16};
      if (!tile_fits(plan)) {
        if (kernel == 2) return SS_ERR_BAD_SHAPE;
        return SS_OK;  // the sequential kernel, which takes 64-bit addresses
      }
    }
    pl->kind = 2;
    pl->chunk = plan;
    split_plan(plan);
    return SS_OK;
  }
  if (kernel == 0 && ss::fwd_state_supported(a) && state_fits) pl->kind = 3;  // dstate != 16
  return SS_OK;
}

// Bytes at the start of ss_bwd's workspace that hold the split region (header, flags and
// states for up to ss::kBwdMaxParts parts of every channel group), rounded to 256 bytes.
size_t bwd_split_region(int64_t batch, int64_t dim) {
  const int64_t groups = batch * ((dim + 15) / 16);
  return (ss::split::region_bytes(groups * (ss::kBwdMaxParts - 1)) + 255) / 256 * 256;
}

int fwd_common(const void* u, const void* delta, const float* A, const void* B, const void* C,
               const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
               float* last_state, const float* h0, int64_t batch, int64_t seqlen, int64_t dim,
               int64_t dstate, int in_dtype, const ss_fwd_options* opt, const ConvArgs& cv,
               void* stream, bool noalloc = false) {
  // with seqlen == 0 no token is read or written: the per-token arrays may be NULL
  if (!A || (seqlen != 0 && (!u || !delta || !B || !C || !y))) return SS_ERR_NULL_ARG;
  const int sv = check_fwd_sizes(batch, seqlen, dim, dstate, in_dtype, opt);
  if (sv != SS_OK) return sv;
  const size_t es = elem_size(in_dtype);
  void* ws = (opt && !noalloc) ? opt->workspace : nullptr;
  size_t ws_bytes = (opt && !noalloc) ? opt->workspace_bytes : 0;
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || !aligned(y, 4) ||
      (last_state && !aligned(last_state, 4)) || (h0 && !aligned(h0, 4)) || !aligned(cv.conv_w, 4) ||
      (cv.conv_b && !aligned(cv.conv_b, 4)) || (cv.conv_state && !aligned(cv.conv_state, 4)) ||
      (cv.u_out && !aligned(cv.u_out, 4)) || !aligned(ws, 16))
    return SS_ERR_MISALIGNED;
  int cus = 0;
  const int dv = check_device(&cus);
  if (dv != SS_OK) return dv;
  if (noalloc) {  // the fixed per-device scratch array stands in for the workspace
    uint32_t* p = nullptr;
    if (ss::noalloc_scratch_ptr(&p) != hipSuccess) return SS_ERR_HIP;
    ws = p;
    ws_bytes = ss::kNoallocScratchBytes;
  }

  ss::FwdArgs a{u, delta, A, B, C, D, z, delta_bias, y, last_state,
                batch, seqlen, dim, dstate, in_dtype, softplus_flag ? 1 : 0, h0,
                (opt && opt->discretization == SS_DISC_ZOH) ? 1 : 0, static_cast<int>(cv.kconv), cv.conv_w,
                cv.conv_b, cv.conv_state, cv.u_out};
  FwdPlan pl;
  const int pv = plan_fwd(a, opt, cus, &pl);
  if (pv != SS_OK) return pv;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (pl.kind == 2) {
    if (pl.parts > 1 && (!ws || ws_bytes < pl.split_bytes)) {
      // the split needs the caller's workspace: without one an explicit split is an error and
      // the automatic plan runs unsplit
      if (opt && opt->split_parts > 1) return SS_ERR_WORKSPACE;
      pl.parts = 1;
    }
    if (pl.parts > 1) {
      a.parts = pl.parts;
      a.part_len = pl.part_len;
      a.split_ws = static_cast<uint32_t*>(ws);
      a.split_cap = ss::fwd_split_items(batch * ((dim + 15) / 16), pl.parts);
      a.split_wait_limit = opt ? opt->split_wait_limit : 0;
      e = ss::split::clear(a.split_ws, a.split_cap, s);
      if (e != hipSuccess) return SS_ERR_HIP;
    }
    e = ss::fwd_chunked(a, pl.chunk, s);
  } else {
    e = pl.kind == 3 ? ss::fwd_state(a, s) : ss::fwd_seq(a, s);
  }
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace

extern "C" {

int ss_abi_version(void) { return SS_ABI_VERSION; }

const char* ss_status_string(int s) {
  switch (s) {
    case SS_OK: return "ok";
    case SS_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case SS_ERR_BAD_SHAPE: return "a size argument is out of range";
    case SS_ERR_BAD_DTYPE: return "unknown input dtype";
    case SS_ERR_UNSUPPORTED_N: return "dstate exceeds the supported maximum of 16";
    case SS_ERR_MISALIGNED: return "a pointer is not aligned to its element size";
    case SS_ERR_HIP: return "a HIP runtime call or kernel launch failed";
    case SS_ERR_DEVICE: return "the current device is not a gfx950 GPU";
    case SS_ERR_WORKSPACE: return "the workspace is NULL or smaller than the size query returns";
    case SS_ERR_SPLIT_WAIT: return "a sequence-split hand-off wait gave up: the affected outputs are NaN";
    default: return "unknown status code";
  }
}

int ss_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
              const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
              float* last_state, const float* h0, int64_t batch, int64_t seqlen, int64_t dim,
              int64_t dstate, int in_dtype, const ss_fwd_options* opt, void* stream) {
  return fwd_common(u, delta, A, B, C, D, z, delta_bias, softplus_flag, y, last_state, h0, batch, seqlen,
                    dim, dstate, in_dtype, opt, ConvArgs{0, nullptr, nullptr, nullptr, nullptr}, stream);
}

int ss_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
                   float* last_state, const float* h0, int64_t batch, int64_t seqlen, int64_t dim,
                   int64_t dstate, int in_dtype, const ss_fwd_options* opt, void* stream) {
  return fwd_common(u, delta, A, B, C, D, z, delta_bias, softplus_flag, y, last_state, h0, batch, seqlen,
                    dim, dstate, in_dtype, opt, ConvArgs{0, nullptr, nullptr, nullptr, nullptr}, stream, true);
}

int ss_fwd_conv(const void* x, const float* conv_w, const float* conv_b, const float* conv_state,
                int64_t kconv, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
                float* last_state, const float* h0, float* u_out, int64_t batch, int64_t seqlen,
                int64_t dim, int64_t dstate, int in_dtype, const ss_fwd_options* opt, void* stream) {
  if (!conv_w) return SS_ERR_NULL_ARG;
  if (kconv < 1 || kconv > 4) return SS_ERR_BAD_SHAPE;
  return fwd_common(x, delta, A, B, C, D, z, delta_bias, softplus_flag, y, last_state, h0, batch, seqlen,
                    dim, dstate, in_dtype, opt, ConvArgs{kconv, conv_w, conv_b, conv_state, u_out}, stream);
}

int ss_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
           const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
           float* last_state, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
           int in_dtype, void* stream) {
  return ss_fwd_ex(u, delta, A, B, C, D, z, delta_bias, softplus_flag, y, last_state, nullptr, batch,
                   seqlen, dim, dstate, in_dtype, nullptr, stream);
}

int ss_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int in_dtype,
                          const ss_fwd_options* opt, size_t* bytes) {
  if (!bytes) return SS_ERR_NULL_ARG;
  *bytes = 0;
  const int sv = check_fwd_sizes(batch, seqlen, dim, dstate, in_dtype, opt);
  if (sv != SS_OK) return sv;
  int cus = 0;
  const int dv = check_device(&cus);
  if (dv != SS_OK) return dv;
  ss::FwdArgs a{};
  a.batch = batch;
  a.seqlen = seqlen;
  a.dim = dim;
  a.dstate = dstate;
  a.dtype = in_dtype;
  a.zoh = (opt && opt->discretization == SS_DISC_ZOH) ? 1 : 0;
  FwdPlan pl;
  const int pv = plan_fwd(a, opt, cus, &pl);
  if (pv != SS_OK) return pv;
  *bytes = pl.kind == 2 && pl.parts > 1 ? pl.split_bytes : 0;
  return SS_OK;
}

int ss_workspace_status(const void* workspace, size_t workspace_bytes, uint32_t* giveups, void* stream) {
  if (!workspace || !giveups) return SS_ERR_NULL_ARG;
  if (!aligned(workspace, 16) || !aligned(giveups, 4)) return SS_ERR_MISALIGNED;
  if (workspace_bytes < static_cast<size_t>(ss::split::kHeader) * 4) return SS_ERR_WORKSPACE;
  const uint32_t* word = static_cast<const uint32_t*>(workspace) + ss::split::kGiveUpWord;
  // (hipMemcpyDefault: *giveups may be device memory or pinned host memory)
  if (hipMemcpyAsync(giveups, word, sizeof(uint32_t), hipMemcpyDefault, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return SS_ERR_HIP;
  return SS_OK;
}

int ss_step_ex(float* state, const void* u, const void* delta, const float* A, const void* B,
               const void* C, const float* D, const void* z, const float* delta_bias,
               int softplus_flag, float* y, int64_t batch, int64_t dim, int64_t dstate,
               int in_dtype, int discretization, void* stream) {
  if (!state || !u || !delta || !A || !B || !C || !y) return SS_ERR_NULL_ARG;
  if (in_dtype != SS_DTYPE_F32 && in_dtype != SS_DTYPE_BF16) return SS_ERR_BAD_DTYPE;
  if (batch < 1 || dim < 1 || dstate < 1) return SS_ERR_BAD_SHAPE;
  if (discretization != SS_DISC_DT && discretization != SS_DISC_ZOH) return SS_ERR_BAD_SHAPE;
  if (dstate > SS_MAX_DSTATE) return SS_ERR_UNSUPPORTED_N;
  if (!product_ok(batch, dim, dstate)) return SS_ERR_BAD_SHAPE;
  if ((batch * dim + 255) / 256 > 0x7fffffffLL) return SS_ERR_BAD_SHAPE;
  const size_t es = elem_size(in_dtype);
  if (!aligned(state, 4) || !aligned(u, es) || !aligned(delta, es) || !aligned(B, es) ||
      !aligned(C, es) || (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || !aligned(y, 4))
    return SS_ERR_MISALIGNED;
  int cus = 0;
  const int dv = check_device(&cus);
  if (dv != SS_OK) return dv;

  ss::StepArgs a{state, u, delta, A, B, C, D, z, delta_bias, y,
                 batch, dim, dstate, in_dtype, softplus_flag ? 1 : 0,
                 discretization == SS_DISC_ZOH ? 1 : 0};
  const hipError_t e = ss::step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

int ss_step(float* state, const void* u, const void* delta, const float* A, const void* B,
            const void* C, const float* D, const void* z, const float* delta_bias,
            int softplus_flag, float* y, int64_t batch, int64_t dim, int64_t dstate, int in_dtype,
            void* stream) {
  return ss_step_ex(state, u, delta, A, B, C, D, z, delta_bias, softplus_flag, y, batch, dim, dstate,
                    in_dtype, SS_DISC_DT, stream);
}

namespace {

int proj_common(const void* u, const void* W_x, const void* W_dt, void* delta_raw, void* B, void* C,
                int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t rank, int in_dtype,
                int64_t kconv, const float* conv_w, const float* conv_b, const float* conv_state,
                void* stream) {
  if (!W_x || !W_dt || (seqlen != 0 && (!u || !delta_raw || !B || !C))) return SS_ERR_NULL_ARG;
  if (in_dtype != SS_DTYPE_F32 && in_dtype != SS_DTYPE_BF16) return SS_ERR_BAD_DTYPE;
  if (batch < 1 || seqlen < 0 || dim < 8 || dstate < 1 || dim % 8 != 0 || dim > (1 << 20)) return SS_ERR_BAD_SHAPE;
  if (rank < 8 || rank > 256 || rank % 8 != 0) return SS_ERR_BAD_SHAPE;
  if (dstate > SS_MAX_DSTATE) return SS_ERR_UNSUPPORTED_N;
  if (!product_ok(batch, seqlen, dim) || !product_ok(batch, seqlen, dstate)) return SS_ERR_BAD_SHAPE;
  if ((batch * seqlen + 31) / 32 > 0x7fffffffLL) return SS_ERR_BAD_SHAPE;
  const size_t es = elem_size(in_dtype);
  if (!aligned(u, 16) || !aligned(W_x, 16) || !aligned(W_dt, 16) || !aligned(delta_raw, 16) ||
      !aligned(B, es) || !aligned(C, es) || !aligned(conv_w, 4) || (conv_b && !aligned(conv_b, 4)) ||
      (conv_state && !aligned(conv_state, 4)))
    return SS_ERR_MISALIGNED;
  int cus = 0;
  const int dv = check_device(&cus);
  if (dv != SS_OK) return dv;
  if (seqlen == 0) return SS_OK;
  const ss::ProjArgs a{u,      W_x,   W_dt,     delta_raw, B,      C,      batch * seqlen, dim, dstate, rank,
                       in_dtype, seqlen, static_cast<int>(kconv), conv_w, conv_b, conv_state};
  const hipError_t e = ss::proj(a, cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // namespace

int ss_proj(const void* u, const void* W_x, const void* W_dt, void* delta_raw, void* B, void* C,
            int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t rank, int in_dtype,
            void* stream) {
  return proj_common(u, W_x, W_dt, delta_raw, B, C, batch, seqlen, dim, dstate, rank, in_dtype, 0, nullptr,
                     nullptr, nullptr, stream);
}

int ss_proj_conv(const void* x, const float* conv_w, const float* conv_b, const float* conv_state,
                 int64_t kconv, const void* W_x, const void* W_dt, void* delta_raw, void* B, void* C,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t rank, int in_dtype,
                 void* stream) {
  if (!conv_w) return SS_ERR_NULL_ARG;
  if (kconv < 1 || kconv > 4) return SS_ERR_BAD_SHAPE;
  return proj_common(x, W_x, W_dt, delta_raw, B, C, batch, seqlen, dim, dstate, rank, in_dtype, kconv, conv_w,
                     conv_b, conv_state, stream);
}

size_t ss_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate) {
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 0 || dstate > SS_MAX_DSTATE) return 0;
  if (!product_ok(batch, seqlen, dim) || !product_ok(batch, seqlen, 16 * dstate)) return 0;
  return bwd_split_region(batch, dim) + ss::bwd_workspace_bytes(batch, seqlen, dim, dstate);
}

int ss_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
           const float* D, const void* z, const float* delta_bias, int softplus_flag,
           const float* h0, const float* dy, const float* dlast_state, float* du, float* ddelta,
           float* dA, float* dB, float* dC, float* dD, float* dz, float* ddelta_bias, float* dh0,
           void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
           int64_t dstate, int in_dtype, void* stream) {
  if (!A || !dA) return SS_ERR_NULL_ARG;
  if (seqlen != 0 && (!u || !delta || !B || !C || !dy || !du || !ddelta || !dB || !dC || (z && !dz)))
    return SS_ERR_NULL_ARG;
  if (in_dtype != SS_DTYPE_F32 && in_dtype != SS_DTYPE_BF16) return SS_ERR_BAD_DTYPE;
  if (batch < 1 || dim < 1 || dstate < 1 || seqlen < 0) return SS_ERR_BAD_SHAPE;
  if (dstate > SS_MAX_DSTATE) return SS_ERR_UNSUPPORTED_N;
  if (!product_ok(batch, seqlen, dim) || !product_ok(batch, seqlen, 16 * dstate) ||
      !product_ok(batch, dim, dstate))
    return SS_ERR_BAD_SHAPE;
  const int64_t ngroups = (dim + 15) / 16;
  if (batch * ngroups > 0x7fffffffLL) return SS_ERR_BAD_SHAPE;
  if (batch * seqlen * dstate + dim * (dstate + 2) > 0x7fffffffLL * 256LL) return SS_ERR_BAD_SHAPE;
  const size_t es = elem_size(in_dtype);
  if (!aligned(u, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) ||
      (z && !aligned(z, es)) || !aligned(A, 4) || (D && !aligned(D, 4)) ||
      (delta_bias && !aligned(delta_bias, 4)) || (h0 && !aligned(h0, 4)) || !aligned(dy, 4) ||
      (dlast_state && !aligned(dlast_state, 4)) || !aligned(du, 4) || !aligned(ddelta, 4) ||
      !aligned(dA, 4) || !aligned(dB, 4) || !aligned(dC, 4) || (dD && !aligned(dD, 4)) ||
      (dz && !aligned(dz, 4)) || (ddelta_bias && !aligned(ddelta_bias, 4)) || (dh0 && !aligned(dh0, 4)) ||
      !aligned(workspace, 4))
    return SS_ERR_MISALIGNED;
  const size_t split_region = bwd_split_region(batch, dim);
  const size_t need = split_region + ss::bwd_workspace_bytes(batch, seqlen, dim, dstate);
  if (!workspace || workspace_bytes < need) return SS_ERR_WORKSPACE;
  int cus = 0;
  const int dv = check_device(&cus);
  if (dv != SS_OK) return dv;

  const int64_t ntiles = seqlen > 0 ? (seqlen + ss::bwd_tile_tokens() - 1) / ss::bwd_tile_tokens() : 0;
  float* ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + split_region);
  float* ckpt = ws;
  float* part_bc = ckpt + batch * ntiles * ngroups * 16 * 16;
  float* part_ch = part_bc + 2 * batch * ngroups * seqlen * dstate;
  ss::BwdArgs a{u, delta, A, B, C, D, z, delta_bias, h0, dy, dlast_state,
                du, ddelta, z ? dz : nullptr, dh0, dA, dB, dC, dD, ddelta_bias,
                ckpt, part_bc, part_ch, batch, seqlen, dim, dstate, ngroups, ntiles,
                in_dtype, softplus_flag ? 1 : 0, ss::bwd_rows(batch * ngroups, seqlen, cus)};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t groups = batch * ngroups;
  int parts = ss::bwd_split_parts(groups, a.rows, false, seqlen, cus);
  int ckpt_parts = ss::bwd_split_parts(groups, a.rows, true, seqlen, cus);
  if (groups * ss::kBwdMaxParts > 0x7fffffffLL) parts = ckpt_parts = 1;
  if (parts > 1 || ckpt_parts > 1) {  // one split region for both kernels, used one after the other
    a.split_ws = static_cast<uint32_t*>(workspace);
    a.split_cap = groups * (ss::kBwdMaxParts - 1);
  }
  if (parts > 1) {
    a.parts = parts;
    a.part_len = ss::bwd_split_part_len(seqlen, a.rows, parts);
  }
  if (ckpt_parts > 1) {
    a.ckpt_parts = ckpt_parts;
    a.ckpt_part_len = ss::bwd_split_part_len(seqlen, a.rows, ckpt_parts);
  }
  const hipError_t e = ss::bwd(a, s);
  return e == hipSuccess ? SS_OK : SS_ERR_HIP;
}

}  // extern "C"
