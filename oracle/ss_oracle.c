/*
 * ss_oracle.c -- plain fp64 CPU oracle for the selective state-space scan (S6).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark may load this library. It shares no code, header or table with the
 * GPU library, and never calls it.
 *
 * What it computes (one independent recurrence per batch row b and channel d):
 *
 *   x      = delta[b,t,d] + bias[d]                        (bias absent -> 0)
 *   dt     = softplus(x) if softplus_flag else x
 *   for each state n:
 *     abar = exp(dt * A[d,n])                               (zero-order-hold decay)
 *     bbar = dt                       by default (first-order input term), or
 *          = (exp(dt A[d,n]) - 1) / A[d,n]  with zoh set (exact zero-order hold; the
 *            A -> 0 limit of that quotient is dt)
 *     h[n] = abar * h[n] + (bbar * B[b,t,n]) * u[b,t,d]
 *   y[b,t,d] = (sum_n C[b,t,n] * h[n] + D[d] * u[b,t,d]) * silu(z[b,t,d])
 *   last_state[b,d,n] = h[n] after the last step
 *
 * Sources (web pages on the Mamba selective SSM):
 *  - "Mamba：选择性状态空间模型入门教程" (jindou-blog tutorial), section
 *    "状态空间模型（SSM）的直觉": recurrence h = A h + B x, output y = C h + D x;
 *    section "Mamba 的关键创新：选择性机制": B, C and the step size are functions of
 *    the input, the step size passes through softplus, the state is discretised with
 *    the step and y is read from the updated state.
 *  - "Mamba：选择性状态空间的线性时间序列建模" (wiki note on arXiv 2312.00752),
 *    table "算法对比（核心直觉）", row S6: B_t and C_t have shape (batch, L, N) and the
 *    step is tau(Delta + s_Delta(x_t)), i.e. the bias is added before softplus;
 *    section "架构：极简设计": the SSM branch is multiplied by a SiLU branch.
 *  - "架构变体：Mamba/SSM" (aiqz.cc), section "离散化": zero-order hold with step Delta;
 *    section "Python 演示": state starts at zero.
 * Readings where the pages are silent or disagree (all in the design notes):
 *  - the default discretised input term is dt * B; the exact zero-order-hold term
 *    (exp(dt A) - 1)/A * B of "架构变体：Mamba/SSM" section "离散化" is the zoh option;
 *  - y reads the post-update state; the D term is included; the SiLU gate multiplies
 *    the whole output including the D term; the bias is added before softplus;
 *  - A is a diagonal (dim, dstate) array; B and C carry no channel index.
 *
 * The backward (ss_oracle_bwd, below) is the chain rule of the same loop, run in reverse.
 * ss_oracle_conv_silu is the causal-convolution + SiLU prologue that produces u from x.
 *
 * Arithmetic: every input is converted exactly to double (bf16 -> fp32 -> fp64 is
 * exact), all arithmetic is IEEE double with libm exp/expm1/log1p, compiled without fast
 * math. Work is split over (b, d) channels with OpenMP; each channel runs the plain
 * sequential loop above, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* element types of u, delta, z, B and C (fp64 lets a caller feed values that are not
   representable in fp32, e.g. the output of the conv prologue below) */
#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_F64 2

static int dtype_ok(int dtype) {
  return dtype == ORACLE_F32 || dtype == ORACLE_BF16 || dtype == ORACLE_F64;
}

static double in_at(const void* p, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)p)[i];
  if (dtype == ORACLE_F64) return ((const double*)p)[i];
  uint32_t w = (uint32_t)((const uint16_t*)p)[i] << 16; /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* softplus(x) = log(1 + e^x), written so that neither branch overflows */
static double softplus(double x) {
  if (x > 0.0) return x + log1p(exp(-x));
  return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) */
static double silu(double z) {
  if (z >= 0.0) return z / (1.0 + exp(-z));
  double e = exp(z);
  return z * e / (1.0 + e);
}

/* One channel (b, d) over t in [0, seqlen). h holds the state on entry and exit.
   y_out[t * y_stride] receives y[b,t,d]. */
static void scan_channel(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* bias,
                         int softplus_flag, int zoh, int64_t b, int64_t d, int64_t seqlen,
                         int64_t dim, int64_t dstate, int dtype, double* h, double* y_out,
                         int64_t y_stride) {
  const double bias_d = bias ? (double)bias[d] : 0.0;
  const double D_d = D ? (double)D[d] : 0.0;
  for (int64_t t = 0; t < seqlen; ++t) {
    const int64_t e = (b * seqlen + t) * dim + d;  /* index into (batch, seqlen, dim) */
    const int64_t bc = (b * seqlen + t) * dstate;  /* row of (batch, seqlen, dstate) */
    const double x = in_at(delta, dtype, e) + bias_d;
    const double dt = softplus_flag ? softplus(x) : x;
    const double uv = in_at(u, dtype, e);
    double acc = 0.0;
    for (int64_t n = 0; n < dstate; ++n) {
      const double a_dn = (double)A[d * dstate + n];
      const double abar = exp(dt * a_dn);
      const double bbar = !zoh ? dt : (a_dn != 0.0 ? expm1(dt * a_dn) / a_dn : dt);
      h[n] = abar * h[n] + (bbar * in_at(B, dtype, bc + n)) * uv;
      acc += in_at(C, dtype, bc + n) * h[n];
    }
    double yv = acc + D_d * uv;
    if (z) yv *= silu(in_at(z, dtype, e));
    if (y_out) y_out[t * y_stride] = yv;
  }
}

/*
 * Full forward over every (b, d), or over a listed subset of channels.
 *   zoh         0: input term dt * B; 1: exact zero-order hold (exp(dt A) - 1)/A * B.
 *   h0          optional (batch, dim, dstate) initial state; NULL means zeros.
 *   nchan == 0  all channels: y is (batch, seqlen, dim), last_state is (batch, dim, dstate).
 *   nchan  > 0  only the channels (chan_b[i], chan_d[i]): y is (nchan, seqlen) and
 *               last_state is (nchan, dstate); h0 is still indexed as (batch, dim, dstate).
 * y and last_state may be NULL. Returns 0, or -1 on a bad argument.
 */
int ss_oracle_fwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                  int zoh, const double* h0, double* y, double* last_state, int64_t batch,
                  int64_t seqlen, int64_t dim, int64_t dstate, int dtype, const int64_t* chan_b,
                  const int64_t* chan_d, int64_t nchan, int nthreads) {
  if (!u || !delta || !A || !B || !C) return -1;
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || nchan < 0) return -1;
  if (!dtype_ok(dtype)) return -1;
  if (nchan > 0 && (!chan_b || !chan_d)) return -1;
  const int64_t njobs = nchan > 0 ? nchan : batch * dim;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t j = 0; j < njobs; ++j) {
    const int64_t b = nchan > 0 ? chan_b[j] : j / dim;
    const int64_t d = nchan > 0 ? chan_d[j] : j % dim;
    if (b < 0 || b >= batch || d < 0 || d >= dim) { bad = 1; continue; }
    double* h = (double*)calloc((size_t)dstate, sizeof(double));
    if (!h) { bad = 1; continue; }
    if (h0)
      for (int64_t n = 0; n < dstate; ++n) h[n] = h0[(b * dim + d) * dstate + n];
    double* yo = NULL;
    int64_t ys = 0;
    if (y) {
      if (nchan > 0) { yo = y + j * seqlen; ys = 1; }
      else { yo = y + b * seqlen * dim + d; ys = dim; }
    }
    scan_channel(u, delta, A, B, C, D, z, delta_bias, softplus_flag, zoh, b, d, seqlen, dim,
                 dstate, dtype, h, yo, ys);
    if (last_state) {
      double* dst = nchan > 0 ? last_state + j * dstate : last_state + (b * dim + d) * dstate;
      for (int64_t n = 0; n < dstate; ++n) dst[n] = h[n];
    }
    free(h);
  }
  return bad ? -1 : 0;
}

/*
 * One decode step for every (b, d): the loop body above for a single time index,
 * with the state carried in place (fp64). u, delta, z, y are (batch, dim);
 * B and C are (batch, dstate); state is (batch, dim, dstate).
 */
int ss_oracle_step(double* state, const void* u, const void* delta, const float* A, const void* B,
                   const void* C, const float* D, const void* z, const float* delta_bias,
                   int softplus_flag, int zoh, double* y, int64_t batch, int64_t dim,
                   int64_t dstate, int dtype, int nthreads) {
  if (!state || !u || !delta || !A || !B || !C) return -1;
  if (batch < 0 || dim < 0 || dstate < 1) return -1;
  if (!dtype_ok(dtype)) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < batch * dim; ++j) {
    const int64_t b = j / dim, d = j % dim;
    /* a step is a length-1 sequence: (batch, 1, dim) and (batch, 1, dstate) index the
       same memory as (batch, dim) and (batch, dstate) */
    scan_channel(u, delta, A, B, C, D, z, delta_bias, softplus_flag, zoh, b, d, 1, dim, dstate,
                 dtype, state + j * dstate, y ? y + j : NULL, 1);
  }
  return 0;
}

/* ----------------------------------------------------------------------------------------
 * Backward: the reverse-mode derivative of the forward above (input term dt * B), written
 * out by the chain rule for one channel. With lam_t[n] = dL/dh_t[n] and
 * mu_t[n] = abar_t[n] lam_t[n] (what token t passes back to h_{t-1}):
 *   s_t = sum_n C_t[n] h_t[n] + D u_t,  g_t = silu(z_t) (1 without z),  ds_t = dy_t g_t
 *   dz_t = dy_t s_t silu'(z_t),  dD += ds_t u_t,  du_t = ds_t D + sum_n lam_t[n] dt_t B_t[n]
 *   lam_t[n] = ds_t C_t[n] + mu_{t+1}[n]                   (mu_L = dL/dlast_state)
 *   dC_t[n] += ds_t h_t[n];  dB_t[n] += lam_t[n] dt_t u_t
 *   ddt_t = sum_n lam_t[n] (B_t[n] u_t + A[n] abar_t[n] h_{t-1}[n])
 *   dA[n] += lam_t[n] abar_t[n] h_{t-1}[n] dt_t
 *   ddelta_t = ddt_t sigmoid(x_t) with softplus (its derivative), ddt_t without; dbias += it
 *   dh0 = mu_0
 * The backward of the pages' method ("Mamba：选择性状态空间的线性时间序列建模", section
 * "第二个创新：硬件感知算法") recomputes the states instead of storing them; this
 * reference simply keeps every state of the channel it is differentiating.
 */

static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/* d silu(z) / dz = sigmoid(z) (1 + z (1 - sigmoid(z))) */
static double dsilu(double z) {
  double s = sigmoid(z);
  return s * (1.0 + z * (1.0 - s));
}

/* One channel (b, d). hs: (seqlen + 1) * dstate scratch, mu: dstate scratch. du, dd, dz
   receive element t at index t * stride; dA_ch, dD_ch, dbias_ch are accumulated (+=),
   dh0_ch written; dB and dC ((batch, seqlen, dstate)) are accumulated. */
static void grad_channel(const void* u, const void* delta, const float* A, const void* B,
                         const void* C, const float* D, const void* z, const float* bias,
                         int softplus_flag, const double* h0_ch, const float* dy,
                         const float* dlast_ch, int64_t b, int64_t d, int64_t seqlen, int64_t dim,
                         int64_t dstate, int dtype, double* hs, double* mu, double* du, double* dd,
                         double* dz, int64_t stride, double* dA_ch, double* dD_ch, double* dbias_ch,
                         double* dh0_ch, double* dB, double* dC) {
  const double bias_d = bias ? (double)bias[d] : 0.0;
  const double D_d = D ? (double)D[d] : 0.0;
  /* forward, keeping every state: hs[(t + 1) * dstate + n] = h_t[n], hs[n] = h_{-1}[n] */
  for (int64_t n = 0; n < dstate; ++n) hs[n] = h0_ch ? h0_ch[n] : 0.0;
  for (int64_t t = 0; t < seqlen; ++t) {
    const int64_t e = (b * seqlen + t) * dim + d;
    const int64_t bc = (b * seqlen + t) * dstate;
    const double x = in_at(delta, dtype, e) + bias_d;
    const double dt = softplus_flag ? softplus(x) : x;
    const double uv = in_at(u, dtype, e);
    const double* hp = hs + t * dstate;
    double* ht = hs + (t + 1) * dstate;
    for (int64_t n = 0; n < dstate; ++n) {
      const double abar = exp(dt * (double)A[d * dstate + n]);
      ht[n] = abar * hp[n] + (dt * in_at(B, dtype, bc + n)) * uv;
    }
  }
  /* reverse */
  for (int64_t n = 0; n < dstate; ++n) mu[n] = dlast_ch ? (double)dlast_ch[n] : 0.0;
  for (int64_t t = seqlen - 1; t >= 0; --t) {
    const int64_t e = (b * seqlen + t) * dim + d;
    const int64_t bc = (b * seqlen + t) * dstate;
    const double x = in_at(delta, dtype, e) + bias_d;
    const double dt = softplus_flag ? softplus(x) : x;
    const double uv = in_at(u, dtype, e);
    const double* hp = hs + t * dstate;
    const double* ht = hs + (t + 1) * dstate;
    double acc = 0.0;
    for (int64_t n = 0; n < dstate; ++n) acc += in_at(C, dtype, bc + n) * ht[n];
    const double st = acc + D_d * uv;
    const double dyv = (double)dy[e];
    double ds = dyv;
    if (z) {
      const double zv = in_at(z, dtype, e);
      ds = dyv * silu(zv);
      dz[t * stride] = dyv * st * dsilu(zv);
    }
    *dD_ch += ds * uv;
    double du_t = ds * D_d;
    double ddt = 0.0;
    for (int64_t n = 0; n < dstate; ++n) {
      const double a_dn = (double)A[d * dstate + n];
      const double abar = exp(dt * a_dn);
      const double Bv = in_at(B, dtype, bc + n);
      const double lam = ds * in_at(C, dtype, bc + n) + mu[n];
      dC[bc + n] += ds * ht[n];
      dB[bc + n] += lam * dt * uv;
      du_t += lam * dt * Bv;
      const double g_abar = lam * hp[n]; /* dL/dabar_t[n] */
      ddt += lam * Bv * uv + g_abar * abar * a_dn;
      dA_ch[n] += g_abar * abar * dt;
      mu[n] = abar * lam;
    }
    du[t * stride] = du_t;
    const double dx = softplus_flag ? ddt * sigmoid(x) : ddt;
    dd[t * stride] = dx;
    *dbias_ch += dx;
  }
  if (dh0_ch)
    for (int64_t n = 0; n < dstate; ++n) dh0_ch[n] = mu[n];
}

/*
 * Backward of ss_oracle_fwd (input term dt * B) for the loss L with dL/dy = dy and
 * dL/dlast_state = dlast (NULL: 0). dy and dlast are fp32; h0 is fp64 (NULL: zeros).
 *   nchan == 0: du, ddelta, dz (batch, seqlen, dim); dA (dim, dstate); dD, dbias (dim);
 *               dh0 (batch, dim, dstate); dB, dC (batch, seqlen, dstate).
 *   nchan  > 0: only the listed (b, d) channels: du, ddelta, dz (nchan, seqlen);
 *               dA (nchan, dstate), dD, dbias (nchan) and dh0 (nchan, dstate) are that
 *               channel's own terms; dB, dC (batch, seqlen, dstate) sum the listed channels.
 * dz is required when z is given (else ignored), dh0 may be NULL; every other output is
 * required. Sums over channels go through per-thread buffers (static schedule) added in
 * thread order, so a result depends on the thread count only through rounding.
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int ss_oracle_bwd(const void* u, const void* delta, const float* A, const void* B, const void* C,
                  const float* D, const void* z, const float* delta_bias, int softplus_flag,
                  const double* h0, const float* dy, const float* dlast, double* du,
                  double* ddelta, double* dA, double* dB, double* dC, double* dD, double* dz,
                  double* dbias, double* dh0, int64_t batch, int64_t seqlen, int64_t dim,
                  int64_t dstate, int dtype, const int64_t* chan_b, const int64_t* chan_d,
                  int64_t nchan, int nthreads) {
  if (!u || !delta || !A || !B || !C || !dy) return -1;
  if (!du || !ddelta || !dA || !dB || !dC || !dD || !dbias || (z && !dz)) return -1;
  if (batch < 0 || seqlen < 0 || dim < 0 || dstate < 1 || nchan < 0) return -1;
  if (!dtype_ok(dtype)) return -1;
  if (nchan > 0 && (!chan_b || !chan_d)) return -1;
  const int64_t bln = batch * seqlen * dstate;
  const int64_t njobs = nchan > 0 ? nchan : dim;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  const int nth = omp_get_max_threads();
#else
  (void)nthreads;
  const int nth = 1;
#endif
  double** part = (double**)calloc((size_t)nth, sizeof(double*));
  if (!part) return -1;
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
#ifdef _OPENMP
    const int tid = omp_get_thread_num();
#else
    const int tid = 0;
#endif
    double* acc = (double*)calloc((size_t)(2 * bln + (seqlen + 2) * dstate + 1), sizeof(double));
    part[tid] = acc;
    if (!acc) bad = 1;
#pragma omp for schedule(static)
    for (int64_t j = 0; j < njobs; ++j) {
      if (!acc) continue;
      double* hs = acc + 2 * bln;
      double* mu = hs + (seqlen + 1) * dstate;
      const int64_t b_lo = nchan > 0 ? chan_b[j] : 0;
      const int64_t b_hi = nchan > 0 ? chan_b[j] + 1 : batch;
      const int64_t d = nchan > 0 ? chan_d[j] : j;
      if (b_lo < 0 || b_hi > batch || d < 0 || d >= dim) { bad = 1; continue; }
      double* dA_ch = nchan > 0 ? dA + j * dstate : dA + d * dstate;
      double* dD_ch = nchan > 0 ? dD + j : dD + d;
      double* dbias_ch = nchan > 0 ? dbias + j : dbias + d;
      for (int64_t n = 0; n < dstate; ++n) dA_ch[n] = 0.0;
      *dD_ch = 0.0;
      *dbias_ch = 0.0;
      for (int64_t b = b_lo; b < b_hi; ++b) {
        const int64_t o = nchan > 0 ? j * seqlen : b * seqlen * dim + d;
        const int64_t stride = nchan > 0 ? 1 : dim;
        double* dh0_ch = !dh0 ? NULL : (nchan > 0 ? dh0 + j * dstate : dh0 + (b * dim + d) * dstate);
        grad_channel(u, delta, A, B, C, D, z, delta_bias, softplus_flag,
                     h0 ? h0 + (b * dim + d) * dstate : NULL, dy,
                     dlast ? dlast + (b * dim + d) * dstate : NULL, b, d, seqlen, dim, dstate, dtype,
                     hs, mu, du + o, ddelta + o, z ? dz + o : NULL, stride, dA_ch, dD_ch, dbias_ch,
                     dh0_ch, acc, acc + bln);
      }
    }
  }
  if (!bad) {
    for (int64_t i = 0; i < bln; ++i) {
      double sb = 0.0, sc = 0.0;
      for (int k = 0; k < nth; ++k) {
        if (!part[k]) continue;
        sb += part[k][i];
        sc += part[k][bln + i];
      }
      dB[i] = sb;
      dC[i] = sc;
    }
  }
  for (int k = 0; k < nth; ++k) free(part[k]);
  free(part);
  return bad ? -1 : 0;
}

/* ----------------------------------------------------------------------------------------
 * Prologue: causal depthwise convolution over time, then SiLU, per channel
 * ("Mamba：选择性状态空间的线性时间序列建模", section "架构：极简设计": in the SSM branch
 * of the block the input passes a short causal convolution and a SiLU before the scan;
 * "Mamba：选择性状态空间模型入门教程", section "Mamba 的关键创新：选择性机制", uses the
 * same order).
 *   pre[b,t,d] = conv_b[d] + sum_{m=0}^{K-1} conv_w[d,m] * x[b, t-(K-1)+m, d]
 *   u[b,t,d]   = silu(pre[b,t,d])
 * x before t = 0 is conv_state[b,d,j] for t-(K-1)+m = j-(K-1) (the K-1 inputs preceding
 * the sequence, oldest first), or 0 when conv_state is NULL. conv_b may be NULL (0).
 * x is u_dtype (f32 / bf16 / f64); conv_w, conv_b and conv_state are fp32; u is fp64
 * (batch, seqlen, dim). Returns 0, or -1 on a bad argument.
 */
int ss_oracle_conv_silu(const void* x, const float* conv_w, const float* conv_b,
                        const float* conv_state, int64_t kconv, double* u, int64_t batch,
                        int64_t seqlen, int64_t dim, int dtype, int nthreads) {
  if (!x || !conv_w || !u || kconv < 1 || batch < 0 || seqlen < 0 || dim < 0) return -1;
  if (!dtype_ok(dtype)) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < batch * dim; ++j) {
    const int64_t b = j / dim, d = j % dim;
    for (int64_t t = 0; t < seqlen; ++t) {
      double pre = conv_b ? (double)conv_b[d] : 0.0;
      for (int64_t m = 0; m < kconv; ++m) {
        const int64_t tau = t - (kconv - 1) + m;
        double xv;
        if (tau >= 0) xv = in_at(x, dtype, (b * seqlen + tau) * dim + d);
        else xv = conv_state ? (double)conv_state[(b * dim + d) * (kconv - 1) + (kconv - 1) + tau] : 0.0;
        pre += (double)conv_w[d * kconv + m] * xv;
      }
      u[(b * seqlen + t) * dim + d] = silu(pre);
    }
  }
  return 0;
}

/* ----------------------------------------------------------------------------------------
 * Input-dependent projections: B_t, C_t and the step come from linear maps of the token's
 * input vector u_t ("Mamba：选择性状态空间模型入门教程", section "Mamba 的关键创新：选择性
 * 机制": B, C and the step are linear functions of x_t; "Mamba：选择性状态空间的线性时间
 * 序列建模", table "算法对比（核心直觉）", row S6: s_B(x_t), s_C(x_t) have shape (B, L, N)
 * and the step is tau(Delta + s_Delta(x_t)), the bias added afterwards by the scan). The
 * pages give no rank for the step map; it is taken as the low-rank product W_dt W_x[0:rank]
 * (rank = dim expresses any full map):
 *   xp[o]             = sum_d W_x[o, d] * u[b,t,d]          o < rank + 2 dstate
 *   delta_raw[b,t,d]  = sum_r W_dt[d, r] * xp[r]             r < rank
 *   B[b,t,n]          = xp[rank + n]
 *   C[b,t,n]          = xp[rank + dstate + n]
 * u is u_dtype (f32 / bf16 / f64, (batch, seqlen, dim)); W_x (rank + 2 dstate, dim) and
 * W_dt (dim, rank) are w_dtype (f32 / bf16); outputs fp64. Sums run in index order in
 * double. Returns 0, or -1 on a bad argument.
 */
int ss_oracle_proj(const void* u, const void* W_x, const void* W_dt, int u_dtype, int w_dtype,
                   int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate, int64_t rank,
                   double* delta_raw, double* B, double* C, int nthreads) {
  if (!u || !W_x || !W_dt || !delta_raw || !B || !C) return -1;
  if (batch < 0 || seqlen < 0 || dim < 1 || dstate < 1 || rank < 1) return -1;
  if (!dtype_ok(u_dtype) || (w_dtype != ORACLE_F32 && w_dtype != ORACLE_BF16)) return -1;
  const int64_t nx = rank + 2 * dstate;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double* xp = (double*)malloc((size_t)nx * sizeof(double));
    if (!xp) bad = 1;
#pragma omp for schedule(static)
    for (int64_t bt = 0; bt < batch * seqlen; ++bt) {
      if (!xp) continue;
      const int64_t ub = bt * dim;
      for (int64_t o = 0; o < nx; ++o) {
        double acc = 0.0;
        for (int64_t d = 0; d < dim; ++d) acc += in_at(W_x, w_dtype, o * dim + d) * in_at(u, u_dtype, ub + d);
        xp[o] = acc;
      }
      for (int64_t d = 0; d < dim; ++d) {
        double acc = 0.0;
        for (int64_t r = 0; r < rank; ++r) acc += in_at(W_dt, w_dtype, d * rank + r) * xp[r];
        delta_raw[ub + d] = acc;
      }
      for (int64_t n = 0; n < dstate; ++n) {
        B[bt * dstate + n] = xp[rank + n];
        C[bt * dstate + n] = xp[rank + dstate + n];
      }
    }
    free(xp);
  }
  return bad ? -1 : 0;
}

int ss_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
