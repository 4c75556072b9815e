// Device side of the projection hand-off between the workgroups of one launch (internal).
//
// The shared projection R travels as (fp32 value, tag) pairs, each written with one 64-bit store
// and read with one coherent 64-bit load; a pair is current when its tag equals the call's
// epoch + 1 (the epoch word sits in the workspace header).  Every workgroup reads the epoch as its
// first load and then arrives once (slot counters, then a counter over the slots); the launch's
// last arrival resets the counters and advances the epoch, so stale pairs never match and no
// memset is needed between calls.  Producers (the lowest workgroup ids) never wait; consumers
// poll with a bounded wait that raises the workspace error word when it expires.
#pragma once

#include "glowq_internal.h"

namespace glowq {

typedef unsigned long long u64;

__device__ __forceinline__ const _Float16* pick_bp(const ForwardArgs& a, int i) {
    const _Float16* b = a.b[0];
#pragma unroll
    for (int k = 1; k < kMaxModules; ++k)
        if (k == i) b = a.b[k];
    return b;
}

// Number of workgroup ids b in [0, n) with b % kArriveSlots == s.
__device__ __forceinline__ int count_slot(int n, int s) {
    return s < n ? (n - 1 - s) / kArriveSlots + 1 : 0;
}

__device__ __forceinline__ uint32_t load_epoch(const ForwardArgs& a) {
    return (uint32_t)__hip_atomic_load(a.sync + kSyncEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_pair(u64* p, float v, uint32_t tag) {
    const u64 w = ((u64)tag << 32) | (u64)__builtin_bit_cast(uint32_t, v);
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (bounded) until pair p carries `tag`, then return its value.
__device__ __forceinline__ float load_pair(const ForwardArgs& a, const u64* p, uint32_t tag) {
    u64 w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    while ((uint32_t)(w >> 32) != tag) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(a.sync + kSyncError, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return __builtin_bit_cast(float, (uint32_t)w);
}

// Hand-off arrival of this workgroup (thread 0), made after its epoch read has completed.
__device__ __forceinline__ int arrive(const ForwardArgs& a) {
    return __hip_atomic_fetch_add(a.sync + kSyncDone + 16 * (blockIdx.x % kArriveSlots), 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// With the result of arrive(): the last arrival of its slot resets the slot's counter and counts
// the slot; returns the previous slot count, or -1 for every other workgroup.
__device__ __forceinline__ int arrive_slot(const ForwardArgs& a, int prev) {
    const int sl = blockIdx.x % kArriveSlots;
    if (prev != count_slot(a.n_prod + a.n_tiles, sl) - 1) return -1;
    __hip_atomic_store(a.sync + kSyncDone + 16 * sl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __hip_atomic_fetch_add(a.sync + kSyncTop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// With the result of arrive_slot(): the launch's very last arrival resets the top counter and
// advances the epoch (read as `epoch` by this thread), skipping 2^32 - 1 so that the tag epoch + 1
// is never 0.  Every workgroup read the epoch before arriving, so no one in this launch sees the
// new value.
__device__ __forceinline__ void finish(const ForwardArgs& a, int top_prev, uint32_t epoch) {
    const int grid = a.n_prod + a.n_tiles;
    if (top_prev != (grid < kArriveSlots ? grid : kArriveSlots) - 1) return;
    const uint32_t next = epoch + 1u == 0xFFFFFFFFu ? 0u : epoch + 1u;
    __hip_atomic_store(a.sync + kSyncTop, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.sync + kSyncEpoch, (int32_t)next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace glowq
