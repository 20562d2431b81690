// Ready flags between workgroups of one launch: a producer workgroup stores
// its results with device-scope stores, waits until they are acknowledged
// and raises a flag; a consumer polls the flags it depends on with
// device-scope loads, then reads the results with device-scope loads.
//
// On gfx950 a device-scope access (cache-policy field SC1) is performed at
// the level where all XCDs of the GPU see the same data: a store is
// acknowledged once it is visible there, and a load never returns a copy
// that an XCD's L2 holds from before.  So once a consumer has read a raised
// flag, every result store its producer made before raising it is visible to
// the consumer's later device-scope loads, whichever XCDs the two run on.
//
// A flag holds a value unique to the launch (chain_tag), so flags left by
// earlier launches never read as raised and need no clearing -- replays of a
// captured HIP graph included, since every replay enqueues new dispatches.
//
// Progress: consumers are placed after all their producers in the grid, and
// producers never wait.  Workgroups are handed to the XCDs round-robin and
// dispatched in id order within each XCD, so a waiting consumer never holds
// CU resources that a not yet dispatched producer needs.  Every wait is
// bounded all the same (kMaxPolls; MOE_DEV_CHAIN_TIMEOUT when exceeded).
#pragma once

#include "common.hpp"

namespace qrmoe {

// The LLVM intrinsic behind the kernel dispatch id (the index of the
// launch's packet in its hardware queue), which clang exposes under no
// builtin name.
extern "C" __device__ unsigned long long qrmoe_dispatch_id() __asm("llvm.amdgcn.dispatch.id");

// Flag value of this launch: the queue's address in the high 24 bits, the
// dispatch id + 1 in the low 40 (never 0).
__device__ __forceinline__ unsigned long long chain_tag() {
    const unsigned long long q = reinterpret_cast<uintptr_t>(__builtin_amdgcn_queue_ptr());
    return ((q >> 12) << 40) ^ (qrmoe_dispatch_id() + 1ull);
}

// Cache-policy field of a device-scope global -> LDS load (SC1).
constexpr int kAuxDevice = 16;

// Polls per wave before a wait gives up: about a third of a second.
constexpr int kMaxPolls = 1 << 18;

// Polls before giving up: kMaxPolls, unless workspace header word
// kChainPollWord holds w != 0, which sets the limit to w - 1 (w = 1: give
// up at once without reading a flag).  A test of the timeout path sets it
// from the host; moe_workspace_init clears it.
__device__ __forceinline__ int chain_poll_limit(const uint32_t* header) {
    if (!header) return kMaxPolls;
    const uint32_t v = header[kChainPollWord];
    return v != 0u && v <= static_cast<uint32_t>(kMaxPolls) ? static_cast<int>(v) - 1 : kMaxPolls;
}

// Waits until flags[0 .. n) all hold `tag` (lane i polls flags i, i + 64,
// ...), polling each at most max_polls times.  False if it gave up.
__device__ __forceinline__ bool wait_flags(const unsigned long long* flags, int n, unsigned long long tag,
                                           int max_polls = kMaxPolls) {
    if (max_polls <= 0) return false;
    const int lane = threadIdx.x & 63;
    for (int base = 0; base < n; base += kWave) {
        const int i = base + lane;
        for (int polls = 0;; ++polls) {
            const unsigned long long v =
                i < n ? __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : tag;
            if (__all(v == tag)) break;
            if (polls >= max_polls) return false;
            __builtin_amdgcn_s_sleep(8);
        }
    }
    return true;
}

// Producer side, called by every thread of the workgroup after its last
// device-scope result store: waits for the acknowledgement of its own
// stores, then one thread raises the flag.
__device__ __forceinline__ void raise_flag(unsigned long long* flag, unsigned long long tag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qrmoe
