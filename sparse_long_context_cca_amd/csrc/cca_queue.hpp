// Tail queues: the work items of a launch that are not given out by block id.
//
// A kernel whose items are ordered longest first gives items 0 .. n_static-1
// one to a workgroup by block id, and the last n_tail (the shortest) to one
// extra workgroup per compute unit, dispatched after all the others, that
// takes them one at a time from eight per-XCD queues: queue x holds tail
// items n_static + x, + 8, + 16, ...  When the item count is a multiple of 8
// (as in the XCD-aware orders) n_static is too, so an item keeps the XCD its
// block id would have given it; otherwise only the locality is lost.  A queue
// workgroup draws from its
// own XCD's queue first, then from the others in turn, so that an XCD that
// runs faster ends up with more of the tail and the XCDs finish together.
//
// The counters live in a __device__ array of the kernel's source file, one
// slot of 16 words per launch in flight (words 0..7: positions taken from the
// eight queues; word 8: queue workgroups finished).  The launcher takes the
// next slot for every launch; the launch's last queue workgroup clears its
// slot, so a later launch (or graph replay) on that slot finds it zeroed, as
// device memory starts.  Launches in flight at once on one GPU must stay
// below kQueueSlots.  Only lane 0 of a workgroup calls the device functions.
#pragma once

#include <hip/hip_runtime.h>

namespace cca {

constexpr int kQueueSlots = 64;

// Items that go to the queues: the shortest quarter (a multiple of 8) when
// there are at least 8 items per compute unit, none otherwise.
inline int tail_items(long items, int cus) {
  return items >= 8L * cus ? (int)(items / 4) & ~7 : 0;
}

// The next tail item for this workgroup, or -1 once every queue is empty.  cq
// (the queue in use, starting at the XCD's own) and dead (queues found empty)
// carry over between calls.
__device__ __forceinline__ int tail_claim(unsigned* slot, int& cq, int& dead, int n_static, int n_tail) {
  while (dead < 8) {
    const unsigned s = __hip_atomic_fetch_add(slot + cq, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const long pos = cq + 8L * s;
    if (pos < n_tail) return n_static + (int)pos;
    cq = (cq + 1) & 7;
    ++dead;
  }
  return -1;
}

// A kernel's arguments (of type T), read afresh from the kernarg segment:
// the empty asm hides the pointer's value, so loads through it stay where
// they are written.  A kernel that runs its item code in two places (a static
// item, the queue loop) reads its arguments this way; arguments hoisted out of
// both would stay live across the tile loops and spill.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* kernel_args() {
  const __attribute__((address_space(4))) char* p =
      (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return reinterpret_cast<const __attribute__((address_space(4))) T*>(p);
}

// The XCD this workgroup runs on (its first queue).
__device__ __forceinline__ int tail_home_queue() {
  return (int)(__builtin_amdgcn_s_getreg((31 << 11) | 20) & 7u);  // XCC id
}

// A queue workgroup is done; the last of the n_workers clears the slot.
__device__ __forceinline__ void tail_done(unsigned* slot, unsigned n_workers) {
  const unsigned done = __hip_atomic_fetch_add(slot + 8, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (done == n_workers - 1)
    for (int x = 0; x < 9; ++x) __hip_atomic_store(slot + x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace cca
