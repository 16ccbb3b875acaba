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
// on an even earlier item: every wait ends. The wait is bounded all the same. A wait that
// reaches the bound is counted in the region's header and the waiting part continues from a
// NaN state, so its outputs (and every later part's) are NaN rather than silently wrong.
//
// Queues: workgroup ids are dealt to the 8 XCDs round-robin, and neighbouring groups share
// 128-byte lines of the (.., dim) arrays in an XCD's L2, so when the groups divide by 8 the
// workgroups with id = x (mod 8) take items from queue x, which holds the parts of the x-th
// eighth of the groups (a contiguous slice, as the unsplit kernels give XCD x). Each queue
// gets exactly as many workgroups as it has items, and an item's predecessor is in the same
// queue with a smaller counter value; a workgroup's queue is a function of its id alone, so
// results never depend on where it runs.
//
// Hand-off: agent-scope atomic loads and stores (coherent across the XCDs' separate L2s by
// themselves) for the flags and the states; the producer waits until its state stores have
// completed before it stores the flag; in the consumer, thread 0 polls the flag and the other
// threads load the states only after the workgroup barrier that follows the poll.
//
// Region (32-bit words), owned by the caller, of `cap` slots: the counter of queue x at word
// 32 x (x < 8), the count of waits that reached the bound at word kGiveUpWord, then from word
// kHeader one flag per slot (padded to 64 words), then the published states, 16 x 16 fp32 per
// slot ([state n][channel i]). The state crossing the boundary after part q of group gi goes
// through slot q * groups + gi. Before every split launch the host enqueues clear() of the
// header and the flags on the same stream, so no flag or count of an earlier call survives
// into a later one, whatever that call did.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {
namespace split {

constexpr int64_t kHeader = 256;
constexpr int kGiveUpWord = 255;
constexpr uint32_t kSpinLimit = 1u << 22;  // polls of ~8 x 64 cycles: about two seconds

__host__ __device__ inline int64_t flag_words(int64_t cap) { return (cap + 63) / 64 * 64; }
// bytes of a region with cap slots, and the words the clear before a launch zeroes
__host__ __device__ inline size_t region_bytes(int64_t cap) {
  return static_cast<size_t>(kHeader + flag_words(cap) + cap * 256) * 4;
}
__host__ __device__ inline int64_t clear_words(int64_t cap) { return kHeader + flag_words(cap); }
__device__ inline float* states(uint32_t* ws, int64_t cap) {
  return reinterpret_cast<float*>(ws + kHeader + flag_words(cap));
}

// Thread 0 only: take this workgroup's work item; returns part * groups + gi.
__device__ inline uint32_t take(uint32_t* ws, int64_t groups) {
  const bool by_xcd = groups % 8 == 0;
  const uint32_t qx = by_xcd ? blockIdx.x % 8 : 0;
  const uint32_t slice = static_cast<uint32_t>(by_xcd ? groups / 8 : groups);  // groups per queue
  const uint32_t t = atomicAdd(ws + 32 * qx, 1u);
  return (t / slice) * static_cast<uint32_t>(groups) + qx * slice + t % slice;
}

// Thread 0 only: poll until slot `slot` is published, at most `limit` polls (limit < 0: do not
// poll at all, a testing mode in which every wait gives up). Returns false when it gave up,
// after counting that in the header.
__device__ inline bool poll(uint32_t* ws, int64_t slot, int limit) {
  uint32_t* flag = ws + kHeader + slot;
  const uint32_t lim = limit > 0 ? static_cast<uint32_t>(limit) : kSpinLimit;
  bool seen = false;
  if (limit >= 0) {
    for (uint32_t spins = 0; spins < lim; ++spins) {
      if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        seen = true;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  if (!seen) atomicAdd(ws + kGiveUpWord, 1u);
  return seen;
}
__device__ inline float load_state(uint32_t* ws, int64_t cap, int64_t slot, int n, int i) {
  return __hip_atomic_load(states(ws, cap) + slot * 256 + n * 16 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Host: enqueue the zeroing of the header and flags of a region of cap slots on stream s (a
// fill kernel, so a captured graph holds no memset node).
hipError_t clear(uint32_t* ws, int64_t cap, hipStream_t s);

}  // namespace split
}  // namespace ss
