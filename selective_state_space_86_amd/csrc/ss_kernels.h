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

hipError_t fwd_seq(const FwdArgs& a, hipStream_t s);
bool fwd_chunked_supported(const FwdArgs& a);
hipError_t fwd_chunked(const FwdArgs& a, int chunk_len, hipStream_t s);
int fwd_chunked_pick(const FwdArgs& a, int cus);
hipError_t step(const StepArgs& a, hipStream_t s);

}  // namespace ss
