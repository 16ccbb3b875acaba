// ss_split.h -- the work queue and state hand-off of the sequence split (gfx950).
//
// A scan over a sequence can be cut into parts: the chunk state one part ends with is the
// carry the next part starts from (the associative combine of "架构变体：Mamba/SSM", section
// "硬件感知算法", one level above a kernel's tiles). When the channel groups do not fill the
// resident workgroup slots in whole rounds, every group's sequence is cut into `parts` parts
// and each workgroup takes one work item (part, group) from a counter, in the order in which
// the chain runs (part-major, first parts first). A part waits until its predecessor in the
// chain has published the state it starts from. The predecessor always holds a smaller
// counter value, so it was taken by a workgroup that is already running and whose own wait is
// on an even earlier item: every wait ends. The wait is bounded all the same, and a wait that
// hits the bound is counted in the workspace (it would leave a wrong carry).
//
// Queues: workgroup ids are dealt to the 8 XCDs round-robin, and neighbouring groups share
// 128-byte lines of the (.., dim) arrays in an XCD's L2, so when the groups divide by 8 the
// workgroups with id = x (mod 8) take items from queue x, which holds the parts of the x-th
// eighth of the groups (a contiguous slice, as the unsplit kernels give XCD x). Each queue
// gets exactly as many workgroups as it has items, and an item's predecessor is in the same
// queue with a smaller counter value; a workgroup's queue is a function of its id alone, so
// results never depend on where it runs. (One queue for the whole chip scattered neighbouring
// groups over the XCDs and ran 12% slower.)
//
// Hand-off: agent-scope atomic loads and stores (coherent across the XCDs' separate L2s by
// themselves) for the flags and the states; the producer waits until its state stores have
// completed before it stores the flag, and the consumer loads the states only after it has
// seen the flag. (Agent-scope acquire/release fences do the same with a write-back and an
// invalidation of the XCD's whole L2 at every hand-off, which cost more than the split saved
// on short parts.)
//
// Workspace (32-bit words) of `cap` slots: the counter of queue x at word 32 x (x < 8), the
// count of waits that hit the bound at word 255, then from word kHeader one flag per slot
// (padded to 64 words), then the published states, 16 x 16 fp32 per slot ([state n][channel
// i]). The state crossing the boundary after part q of group gi goes through slot
// q * groups + gi. The layout depends on the capacity only, never on the call, so a flag word
// is never a state word of another call. The last workgroup to take an item of a queue resets
// its counter and every consumer resets the flag it waited on, so counters and flags are zero
// again when a kernel ends (the states are left as they are): kernels on one stream can share
// one workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {
namespace split {

constexpr int64_t kHeader = 256;
constexpr uint32_t kSpinLimit = 1u << 22;  // several seconds of polling

__host__ __device__ inline int64_t flag_words(int64_t cap) { return (cap + 63) / 64 * 64; }
__host__ __device__ inline size_t ws_bytes(int64_t cap) {
  return static_cast<size_t>(kHeader + flag_words(cap) + cap * 256) * 4;
}
__device__ inline float* states(uint32_t* ws, int64_t cap) {
  return reinterpret_cast<float*>(ws + kHeader + flag_words(cap));
}

// Thread 0 only: take this workgroup's work item; returns part * groups + gi.
__device__ inline uint32_t take(uint32_t* ws, int64_t groups, int parts) {
  const bool by_xcd = groups % 8 == 0;
  const uint32_t qx = by_xcd ? blockIdx.x % 8 : 0;
  const uint32_t slice = static_cast<uint32_t>(by_xcd ? groups / 8 : groups);  // groups per queue
  uint32_t* counter = ws + 32 * qx;
  const uint32_t t = atomicAdd(counter, 1u);
  if (t == slice * static_cast<uint32_t>(parts) - 1)  // every item of the queue is taken
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (t / slice) * static_cast<uint32_t>(groups) + qx * slice + t % slice;
}

// Every thread of the workgroup: wait until slot `slot` is published. Then each thread loads
// its states with load_state(); afterwards (after a barrier) thread 0 calls clear().
__device__ inline void wait(uint32_t* ws, int64_t slot) {
  uint32_t* flag = ws + kHeader + slot;
  uint32_t spins = 0;
  while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
    if (++spins == kSpinLimit) {
      if ((threadIdx.x & 63) == 0) atomicAdd(ws + 255, 1u);
      break;
    }
    __builtin_amdgcn_s_sleep(8);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // (the state loads stay after the flag)
}
__device__ inline float load_state(uint32_t* ws, int64_t cap, int64_t slot, int n, int i) {
  return __hip_atomic_load(states(ws, cap) + slot * 256 + n * 16 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void clear(uint32_t* ws, int64_t slot) {
  __hip_atomic_store(ws + kHeader + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread stores its states with store_state(), then all call finish_stores(); after a
// barrier thread 0 calls publish().
__device__ inline void store_state(uint32_t* ws, int64_t cap, int64_t slot, int n, int i, float v) {
  __hip_atomic_store(states(ws, cap) + slot * 256 + n * 16 + i, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void finish_stores() {
  // this wave's state stores have completed (agent-coherent) before the flag can be stored
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ inline void publish(uint32_t* ws, int64_t slot) {
  __hip_atomic_store(ws + kHeader + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace split
}  // namespace ss
