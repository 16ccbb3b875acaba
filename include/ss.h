/*
 * ss.h -- C ABI of libss, the gfx950 (MI355X) selective state-space scan (S6).
 *
 * The operation (for every batch row b, channel d and state n):
 *
 *   dt        = softplus(delta[b,t,d] + delta_bias[d])   (or without softplus)
 *   abar      = exp(dt * A[d,n])
 *   h[n]      = abar * h[n] + (dt * B[b,t,n]) * u[b,t,d]      (ss_discretization: or
 *               the exact zero-order-hold coefficient in place of dt)
 *   y[b,t,d]  = (sum_n C[b,t,n] * h[n] + D[d] * u[b,t,d]) * silu(z[b,t,d])
 *
 * Sources: "Mamba：选择性状态空间的线性时间序列建模" (wiki note on arXiv 2312.00752),
 * table "算法对比（核心直觉）" row S6 -- B and C are input-dependent with shape
 * (batch, L, N) and the step is tau(Delta + s_Delta(x)); section "第二个创新：硬件感知
 * 算法" -- the scan runs as one fused kernel whose expanded state never reaches HBM.
 * "Mamba：选择性状态空间模型入门教程" (jindou-blog tutorial), sections
 * "状态空间模型（SSM）的直觉" (h = A h + B x, y = C h + D x) and "Mamba 的关键创新：
 * 选择性机制" (softplus step, discretised A and B, y read from the updated state).
 * "架构变体：Mamba/SSM" (aiqz.cc), section "离散化" (zero-order hold with step Delta).
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers on the current HIP device, owned by the
 *    caller. The library allocates and frees nothing, keeps no state between calls (beyond
 *    a cache of each device's architecture and CU count), never blocks in an enqueueing
 *    call, and is safe to call from several host threads. Scratch memory comes from the
 *    caller as a workspace argument (ss_fwd_options.workspace, ss_bwd's workspace).
 *  - Tensors are dense, row-major, with no padding or strides.
 *  - in_dtype selects the element type of u, delta, z, B and C (all the same);
 *    A, D, delta_bias, y and the state are always fp32.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null stream).
 *    Arguments are validated before anything is enqueued; on a validation error the
 *    call returns the code and writes nothing. A launch failure returns SS_ERR_HIP.
 *    Faults during execution surface at the caller's next synchronisation.
 *  - Outputs must not alias inputs. NaN and Inf propagate unchecked.
 */
#ifndef SS_H_
#define SS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SS_ABI_VERSION 12
#define SS_MAX_DSTATE 16

typedef enum {
  SS_OK = 0,
  SS_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
  SS_ERR_BAD_SHAPE = 2,     /* a size is < 1 (batch, dim, dstate) or < 0 (seqlen), or too large */
  SS_ERR_BAD_DTYPE = 3,     /* in_dtype is not one of ss_dtype */
  SS_ERR_UNSUPPORTED_N = 4, /* dstate > SS_MAX_DSTATE */
  SS_ERR_MISALIGNED = 5,    /* a pointer is not aligned to its element size */
  SS_ERR_HIP = 6,           /* a HIP runtime call or kernel launch failed */
  SS_ERR_DEVICE = 7,        /* the current device is not a gfx950 GPU */
  SS_ERR_WORKSPACE = 8,     /* workspace NULL or smaller than its size query returns */
  SS_ERR_SPLIT_WAIT = 9     /* a sequence-split hand-off wait gave up (the count that
                               ss_workspace_status delivers is nonzero) */
} ss_status;

typedef enum {
  SS_DTYPE_F32 = 0,  /* IEEE binary32 */
  SS_DTYPE_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} ss_dtype;

/* Discretised input term bbar in h = abar h + (bbar B) u. ss_fwd and ss_step use the
 * first; the _ex entry points take either. Both hold the decay abar = exp(dt A). */
typedef enum {
  SS_DISC_DT = 0, /* bbar = dt (the simplified input term) */
  SS_DISC_ZOH = 1 /* bbar = (exp(dt A) - 1) / A, the exact zero-order hold of the
                     continuous input ("架构变体：Mamba/SSM", section "离散化"); its
                     A -> 0 limit dt is used where A == 0 */
} ss_discretization;

/* SS_ABI_VERSION of the built library. */
int ss_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* ss_status_string(int status);

/*
 * ss_fwd -- selective-scan forward over a whole sequence, from a zero initial state.
 *
 *   u, delta, z   (batch, seqlen, dim)     in_dtype. delta is the raw step before bias.
 *                                          z may be NULL: no SiLU gate.
 *   A             (dim, dstate)            fp32, the diagonal state matrix per channel
 *                                          (normally negative; any finite value is used as is).
 *   B, C          (batch, seqlen, dstate)  in_dtype, shared by all channels of a batch row.
 *   D             (dim)                    fp32, may be NULL: no skip term.
 *   delta_bias    (dim)                    fp32, may be NULL: zero bias. Added before softplus.
 *   softplus_flag                          non-zero: dt = softplus(delta + bias); else dt = delta + bias.
 *   y             (batch, seqlen, dim)     fp32 output.
 *   last_state    (batch, dim, dstate)     fp32 output, may be NULL: the state after the last token.
 *   seqlen == 0 is allowed: no token is read, y is not written, last_state is set to
 *   zero; u, delta, z, B, C and y may then be NULL (A is still required).
 * Limits: dstate <= 16; batch * seqlen * dim < 2^62; for dstate == 16, 64 * dim * 4 < 2^31
 * (dim below 8,388,608: the time-chunked kernel addresses a tile of 64 tokens of the fp32
 * rows from 32-bit offsets; larger plans are taken only where their tile fits too).
 * ss_fwd takes no workspace and so never splits the sequences (ss_fwd_options.split_parts);
 * ss_fwd_ex with a workspace does where the automatic plan splits.
 */
int ss_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
           const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
           float* last_state, int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
           int in_dtype, void* stream);

/* Options of ss_fwd_ex. A zero-initialised struct (or a NULL pointer) means ss_fwd's
 * behaviour. kernel and chunk_len are for tuning and testing. */
typedef struct {
  int kernel;         /* 0: automatic; 1: one lane per channel, sequential in t (any dstate);
                         2: time-chunked (dstate == 16 only, else SS_ERR_UNSUPPORTED_N);
                         3: one lane per (channel, state), sequential in t (default input
                            term, no conv prologue, else SS_ERR_BAD_SHAPE); automatic picks
                            2 for dstate == 16, else 3 when it applies, else 1 */
  int chunk_len;      /* tokens per lane and tile for kernel 2: 0 (automatic), 4 or 8 */
  int discretization; /* an ss_discretization value */
  int chunk_rows;     /* time chunks per workgroup tile for kernel 2: 0 (automatic), 16, 12 or
                         32; 12 needs chunk_len 0 or 4 (else SS_ERR_BAD_SHAPE) and is never
                         chosen automatically; 32 (8 waves) is chosen for at most 2 groups of
                         16 channels per CU and needs 256 * dim * 4 < 2^31 (else
                         SS_ERR_BAD_SHAPE); otherwise 16 */
  int split_parts;    /* kernel 2 only: cut every sequence into this many parts of whole tiles
                         (fewer when it is too short), processed by successive workgroups
                         that hand the chunk state on (the associative combine of
                         "架构变体：Mamba/SSM", section "硬件感知算法", one level above the
                         tiles). 0: automatic (split when the channel groups leave part of the
                         last round of resident workgroups empty and outnumber the resident
                         slots, e.g. 320 groups on 256 CUs, and the workspace below is large
                         enough; otherwise run unsplit); 1: never; 2..16: that many (else
                         SS_ERR_BAD_SHAPE; SS_ERR_WORKSPACE without a large enough
                         workspace). The parts start on tile boundaries, so the results are
                         bit-identical to the unsplit kernel's. */
  void* workspace;    /* device memory for the split's work queue, flags and hand-off states,
                         owned by the caller, 16-byte aligned, or NULL (no split). Its size for
                         a call: ss_fwd_workspace_size (about 1 KiB per channel group and part
                         after the first: 1 MB at batch 1, dim 5120, 4 parts). Its contents on
                         entry do not matter: the call first enqueues a small kernel on `stream`
                         that clears what must start at zero (no memset, so the call can be
                         captured in a graph). Calls that use one workspace must not overlap:
                         give each stream its own, or order the streams. */
  size_t workspace_bytes; /* bytes at workspace */
  int split_wait_limit; /* testing the failure path: 0 (default) bounds each hand-off wait at
                           about two seconds of polling; n > 0 at n polls; < 0 makes every
                           wait give up at once. A wait that gives up continues its part from a
                           NaN state, so that part's outputs (and those of the later parts of
                           its channel group, and last_state) are NaN, and counts itself in the
                           workspace: see ss_workspace_status. Every kernel still ends. */
} ss_fwd_options;

/*
 * ss_fwd_workspace_size -- the workspace bytes (*bytes) an ss_fwd_ex / ss_fwd_conv call with
 * these sizes, in_dtype and options would use on the current device: nonzero when its plan
 * splits the sequences, else 0 (opt->workspace and workspace_bytes are ignored here; opt may
 * be NULL). Errors: SS_ERR_NULL_ARG (bytes NULL), the size and option errors of ss_fwd_ex,
 * SS_ERR_DEVICE, SS_ERR_HIP. Enqueues nothing.
 */
int ss_fwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int in_dtype,
                          const ss_fwd_options* opt, size_t* bytes);

/*
 * ss_workspace_status -- enqueue on `stream` a copy of the number of sequence-split hand-off
 * waits that gave up in the most recent split call that used this workspace (the workspace
 * given to ss_fwd_ex / ss_fwd_conv, or to ss_bwd) into *giveups. Waits hold until the previous
 * part has published its state, which it always does; the count reports the bounded wait's
 * safety net (or split_wait_limit < 0): 0, or the number of waits that gave up, whose parts
 * ran from a NaN state. Asynchronous like every other call: *giveups (4 bytes, 4-byte aligned;
 * device memory, or pinned host memory for a copy that does not block) holds the count once
 * `stream` has reached this point. A caller that reports the give-up as a status uses
 * SS_ERR_SPLIT_WAIT. Errors: SS_ERR_NULL_ARG (workspace or giveups NULL), SS_ERR_MISALIGNED
 * (workspace not 16-byte or giveups not 4-byte aligned), SS_ERR_WORKSPACE (workspace_bytes <
 * 1024), SS_ERR_HIP (the copy could not be enqueued).
 */
int ss_workspace_status(const void* workspace, size_t workspace_bytes, uint32_t* giveups, void* stream);

/*
 * ss_fwd_ex -- ss_fwd from a given initial state, with a choice of input term and kernel.
 * Same arguments, layouts, ownership and errors as ss_fwd, plus:
 *   h0   (batch, dim, dstate) fp32 initial state, may be NULL (zero state, as ss_fwd).
 *        With h0 = the last_state of a call over tokens [0, t0), a call over [t0, L)
 *        continues that scan (chunked prefill; the update is associative, "架构变体：
 *        Mamba/SSM" section "硬件感知算法"); with seqlen == 0, last_state = h0.
 *   opt  options, may be NULL (automatic kernel, bbar = dt, no workspace). Every kernel
 *        choice computes the same result up to fp32 rounding order. An out-of-range option
 *        returns SS_ERR_BAD_SHAPE; a misaligned workspace SS_ERR_MISALIGNED.
 */
int ss_fwd_ex(const void* u, const void* delta, const float* A, const void* B, const void* C,
              const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
              float* last_state, const float* h0, int64_t batch, int64_t seqlen, int64_t dim,
              int64_t dstate, int in_dtype, const ss_fwd_options* opt, void* stream);

/*
 * ss_fwd_noalloc -- ss_fwd_ex for callers that cannot allocate device memory and have no
 * workspace to give: code under graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results and errors as ss_fwd_ex, except that the sequence
 * split takes its work queue, flags and hand-off states from a fixed array of
 * SS_NOALLOC_SCRATCH_BYTES that the library holds in device memory on every device it runs
 * on (from the first call on that device until the process ends); opt->workspace and
 * workspace_bytes are ignored. Nothing is allocated or freed. The automatic plan splits only
 * when the split fits the array (about 4000 hand-off slots of channel group x part after the
 * first: 320 groups in 4 parts use 960); an explicit split_parts that does not fit returns
 * SS_ERR_WORKSPACE. Every call on a device shares that device's array and first clears
 * what must start at zero, on `stream`: calls that overlap on one device (on different
 * streams, or from several host threads) race and must be ordered by the caller.
 */
#define SS_NOALLOC_SCRATCH_BYTES (4u << 20)
int ss_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B, const void* C,
                   const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
                   float* last_state, const float* h0, int64_t batch, int64_t seqlen, int64_t dim,
                   int64_t dstate, int in_dtype, const ss_fwd_options* opt, void* stream);

/*
 * ss_fwd_conv -- ss_fwd_ex with the block's prologue fused into the scan: the scan's input
 * u is computed from x as silu(causal depthwise conv1d(x) + conv_b), the short causal
 * convolution and SiLU that precede the SSM in the Mamba block ("Mamba：选择性状态空间的
 * 线性时间序列建模", section "架构：极简设计"):
 *   u[b,t,d] = silu(conv_b[d] + sum_{m=0}^{kconv-1} conv_w[d,m] * x[b, t-(kconv-1)+m, d])
 * and y = (C h + D u) silu(z) uses that u. u never has to be written unless asked for.
 *   x             (batch, seqlen, dim)       in_dtype, in place of ss_fwd's u.
 *   conv_w        (dim, kconv) fp32; kconv in 1..4 (else SS_ERR_BAD_SHAPE).
 *   conv_b        (dim) fp32, may be NULL (zero).
 *   conv_state    (batch, dim, kconv - 1) fp32, may be NULL (zeros): the kconv - 1 inputs x
 *                 before t = 0, oldest first (the last inputs of a previous call continue it).
 *   u_out         (batch, seqlen, dim) fp32, may be NULL: receives u (for a backward pass).
 * Everything else (delta .. h0, opt, errors) as in ss_fwd_ex.
 */
int ss_fwd_conv(const void* x, const float* conv_w, const float* conv_b, const float* conv_state,
                int64_t kconv, const void* delta, const float* A, const void* B, const void* C,
                const float* D, const void* z, const float* delta_bias, int softplus_flag, float* y,
                float* last_state, const float* h0, float* u_out, int64_t batch, int64_t seqlen,
                int64_t dim, int64_t dstate, int in_dtype, const ss_fwd_options* opt, void* stream);

/*
 * ss_step -- one decode step: the same update for a single token, with the state
 * carried across calls and updated in place (streaming inference, O(1) per token:
 * "Mamba：选择性状态空间模型入门教程", table "Mamba vs Transformer vs RNN").
 *
 *   state         (batch, dim, dstate)     fp32, read and written in place.
 *   u, delta, z   (batch, dim)             in_dtype; z may be NULL.
 *   B, C          (batch, dstate)          in_dtype.
 *   A, D, delta_bias, softplus_flag        as in ss_fwd.
 *   y             (batch, dim)             fp32 output.
 * Running ss_step for t = 0..L-1 from a zero state gives the same y and final state as
 * ss_fwd over the L tokens, up to fp32 rounding.
 */
int ss_step(float* state, const void* u, const void* delta, const float* A, const void* B,
            const void* C, const float* D, const void* z, const float* delta_bias,
            int softplus_flag, float* y, int64_t batch, int64_t dim, int64_t dstate, int in_dtype,
            void* stream);

/*
 * ss_step_ex -- ss_step with a choice of input term: discretization is an
 * ss_discretization value (anything else returns SS_ERR_BAD_SHAPE). A decode stream must
 * use the discretization of the ss_fwd_ex prefill whose last_state it continues.
 */
int ss_step_ex(float* state, const void* u, const void* delta, const float* A, const void* B,
               const void* C, const float* D, const void* z, const float* delta_bias,
               int softplus_flag, float* y, int64_t batch, int64_t dim, int64_t dstate,
               int in_dtype, int discretization, void* stream);

/*
 * ss_bwd_workspace_size -- bytes of device workspace ss_bwd needs for these sizes
 * (about 4/(16*2) * 16 bytes per (b, t, d) of tile-start states plus 8 bytes per
 * (b, t, n) per group of 16 channels of partial sums, plus 8 * 72 bytes per (b, d) for
 * the partial sums of up to 8 sequence parts, plus the sequence split's region at the
 * start: about 7 KiB per group of 16 channels; see ss_bwd). 0 for invalid sizes.
 */
size_t ss_bwd_workspace_size(int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate);

/*
 * ss_bwd -- backward of ss_fwd_ex with the default input term (bbar = dt): the gradients
 * of a loss L given dL/dy and, optionally, dL/d(last_state), by the chain rule of the
 * recurrence run in reverse time. The expanded (batch, L, dim, N) state is never stored:
 * the states are recomputed tile by tile from checkpoints kept in the workspace, as the
 * pages prescribe for the backward ("Mamba：选择性状态空间的线性时间序列建模", section
 * "第二个创新：硬件感知算法": recomputation instead of storing intermediate states).
 *
 *   u, delta, A, B, C, D, z, delta_bias, softplus_flag, h0
 *                 the forward's inputs, as in ss_fwd_ex (h0 may be NULL: zero state).
 *   dy            (batch, seqlen, dim) fp32: dL/dy.
 *   dlast_state   (batch, dim, dstate) fp32, may be NULL (zero): dL/d(last_state).
 * Outputs (fp32, written, never accumulated into):
 *   du, ddelta    (batch, seqlen, dim); ddelta is dL/d(delta) (before the bias).
 *   dz            (batch, seqlen, dim); required when z is given, ignored otherwise.
 *   dA            (dim, dstate).
 *   dB, dC        (batch, seqlen, dstate).
 *   dD, ddelta_bias (dim), may be NULL (not computed). With D or delta_bias NULL they are
 *                 the gradients at D = 0 / bias = 0.
 *   dh0           (batch, dim, dstate), may be NULL: dL/dh0 (of the zero state if h0 is NULL).
 *   workspace     device memory of at least ss_bwd_workspace_size() bytes, 4-byte
 *                 aligned, owned by the caller; its contents on entry do not matter and
 *                 are undefined on return (ss_workspace_status reads its split region).
 * seqlen == 0 is allowed (the per-token arrays may then be NULL): dh0 = dlast_state and
 * dA, dD, ddelta_bias are zero. Sums over channels, tokens and batch rows have a fixed
 * order, so the result is deterministic. Errors as ss_fwd, plus SS_ERR_WORKSPACE.
 * With fewer channel groups of 16 than twice the CUs the kernels run 8-wave workgroups (one
 * per CU), else 4-wave ones (two per CU). When the groups fill those resident slots in more
 * than one round and leave part of the last round empty, they also split every sequence into
 * parts (as ss_fwd_options.split_parts describes; the reverse pass hands the adjoint from
 * each part to the one before it), with the hand-off in the split region at the start of
 * the workspace.
 */
int ss_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
           const float* D, const void* z, const float* delta_bias, int softplus_flag,
           const float* h0, const float* dy, const float* dlast_state, float* du, float* ddelta,
           float* dA, float* dB, float* dC, float* dD, float* dz, float* ddelta_bias, float* dh0,
           void* workspace, size_t workspace_bytes, int64_t batch, int64_t seqlen, int64_t dim,
           int64_t dstate, int in_dtype, void* stream);

/*
 * ss_proj -- the input projections that give the scan its step, B and C: linear maps of
 * each token's input vector ("Mamba：选择性状态空间模型入门教程", section "Mamba 的关键创新：
 * 选择性机制": B, C and the step are linear functions of x_t; "Mamba：选择性状态空间的线性
 * 时间序列建模", table "算法对比（核心直觉）", row S6: s_B(x_t), s_C(x_t) of shape (B, L, N),
 * step tau(Delta + s_Delta(x_t))). The step map is low-rank, W_dt W_x[0:rank] (rank = dim
 * expresses any full map). For every token t (b, t flattened):
 *   xp_t          = W_x u_t                       rank + 2*dstate outputs
 *   delta_raw_t   = W_dt xp_t[0 : rank]           dim outputs (ss_fwd adds delta_bias, softplus)
 *   B_t           = xp_t[rank : rank + dstate]
 *   C_t           = xp_t[rank + dstate : rank + 2*dstate]
 *
 *   u          (batch, seqlen, dim)          in_dtype, device, read
 *   W_x        (rank + 2*dstate, dim)        in_dtype, device, read (out x in, row-major)
 *   W_dt       (dim, rank)                   in_dtype, device, read
 *   delta_raw  (batch, seqlen, dim)          in_dtype, device, written
 *   B, C       (batch, seqlen, dstate)       in_dtype, device, written
 * The products run on the matrix cores with fp32 accumulation; bf16 outputs are rounded to
 * nearest even. Requirements: dim % 8 == 0 and dim <= 2^20; rank % 8 == 0 and
 * 8 <= rank <= 256; 1 <= dstate <= 16; u, W_x, W_dt, delta_raw 16-byte aligned, B and C
 * element aligned. seqlen == 0 writes nothing (the token arrays may then be NULL).
 * Errors: SS_ERR_NULL_ARG, SS_ERR_BAD_DTYPE, SS_ERR_BAD_SHAPE (sizes, the divisibility
 * above), SS_ERR_UNSUPPORTED_N (dstate > 16), SS_ERR_MISALIGNED, SS_ERR_DEVICE, SS_ERR_HIP.
 * Nothing is allocated; the work is enqueued on stream.
 */
int ss_proj(const void* u, const void* W_x, const void* W_dt, void* delta_raw, void* B, void* C,
            int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t rank, int in_dtype,
            void* stream);

/*
 * ss_proj_conv -- ss_proj with the block's prologue fused into the input loads: the
 * projections take u = silu(causal depthwise conv1d(x) + conv_b) ("Mamba：选择性状态空间的
 * 线性时间序列建模", section "架构：极简设计"), formed per token in fp32 and never written, so
 * x -> ss_proj_conv -> ss_fwd_conv runs the block's SSM path from its input without u in
 * memory:
 *   u[b,t,d] = silu(conv_b[d] + sum_{m=0}^{kconv-1} conv_w[d,m] * x[b, t-(kconv-1)+m, d])
 *   x             (batch, seqlen, dim)       in_dtype, in place of ss_proj's u (16-byte aligned).
 *   conv_w        (dim, kconv) fp32; kconv in 1..4 (else SS_ERR_BAD_SHAPE; NULL: SS_ERR_NULL_ARG).
 *   conv_b        (dim) fp32, may be NULL (zero).
 *   conv_state    (batch, dim, kconv - 1) fp32, may be NULL (zeros): the kconv - 1 inputs x
 *                 before t = 0, oldest first.
 * With bf16 x the fp32 u enters the matrix cores as a bf16 hi part and a bf16 remainder, so
 * the products see u to about 2^-17 relative. Everything else (W_x .. C, requirements,
 * errors) as in ss_proj.
 */
int ss_proj_conv(const void* x, const float* conv_w, const float* conv_b, const float* conv_state,
                 int64_t kconv, const void* W_x, const void* W_dt, void* delta_raw, void* B, void* C,
                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t rank, int in_dtype,
                 void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SS_H_ */
