// Hand-off protocol probe (libglowq_probe.so): the decode kernel's projection hand-off -- the
// epoch read, the two-level arrival, the tagged (value, tag) pairs with their bounded wait and the
// last arrival's epoch advance, all from handoff.h -- run on its own with producers that the host
// can slow down or silence.
//
// Producer workgroups (the lowest ids, as in the decode kernel) read the epoch, sleep, arrive and
// then publish their slice of the pairs (value salt + k for pair k); consumer workgroups read the
// epoch, arrive, count their slot and then read every pair through the bounded wait, counting
// values that differ from salt + k.  Producers arrive late, so the slot and launch counting and
// the consumers' waits all run while the pairs of the previous launch (one tag behind) are still
// in memory: a tag, counter or epoch mistake shows up as a mismatch, as an expired wait (the
// workspace error word) or as an epoch that did not advance by exactly one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glowq_probe.h"
#include "handoff.h"

namespace {

constexpr int kNth = 256;
constexpr int64_t kMaxDelay = 4096;   // sleeps of ~8128 clocks: at most ~14 ms, below the shortest wait
constexpr int32_t kMaxPairs = 65536;

__global__ __launch_bounds__(kNth) void handoff_probe_kernel(glowq::ForwardArgs a, int32_t n_pairs, int64_t delay,
                                                             int32_t publish, float salt, int32_t* counts) {
    __shared__ uint32_t tag_lds;
    __shared__ int bad_lds, seen_lds;
    glowq::u64* R = reinterpret_cast<glowq::u64*>(a.R);
    const int b = blockIdx.x;
    uint32_t epoch0 = 0;
    if (threadIdx.x == 0) {
        epoch0 = glowq::load_epoch(a);
        bad_lds = 0;
        seen_lds = 0;
    }
    int arrived = 0;
    if (b < a.n_prod) {
        if (threadIdx.x == 0) {
            // producer p arrives delay * (p + 1) / n_prod sleeps late: staggered, the last one latest
            const int64_t mine = delay * (b + 1) / a.n_prod;
            for (int64_t i = 0; i < mine; ++i) __builtin_amdgcn_s_sleep(127);
            tag_lds = epoch0 + 1u;
        }
        __syncthreads();  // the arrival below follows the epoch's use
        if (threadIdx.x == 0) arrived = glowq::arrive(a);
        const uint32_t tag = tag_lds;
        if (publish) {
            const int per = (n_pairs + a.n_prod - 1) / a.n_prod;
            const int k0 = b * per, k1 = min(k0 + per, n_pairs);
            for (int k = k0 + (int)threadIdx.x; k < k1; k += kNth) glowq::store_pair(R + k, salt + (float)k, tag);
        }
        if (threadIdx.x == 0) glowq::finish(a, glowq::arrive_slot(a, arrived), epoch0);
        return;
    }
    if (threadIdx.x == 0) tag_lds = epoch0 + 1u;
    __syncthreads();
    int top_prev = -1;
    if (threadIdx.x == 0) {
        arrived = glowq::arrive(a);
        top_prev = glowq::arrive_slot(a, arrived);
    }
    const uint32_t tag = tag_lds;
    int bad = 0, seen = 0;
    for (int k = threadIdx.x; k < n_pairs; k += kNth) {
        const float v = glowq::load_pair(a, R + k, tag);
        bad += v != salt + (float)k;
        ++seen;
    }
    if (bad) atomicAdd(&bad_lds, bad);
    atomicAdd(&seen_lds, seen);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (bad_lds) atomicAdd(counts, bad_lds);
        atomicAdd(counts + 1, seen_lds);
        glowq::finish(a, top_prev, epoch0);
    }
}

}  // namespace

extern "C" int glowq_probe_handoff(void* workspace, size_t workspace_bytes, int32_t n_prod, int32_t n_cons,
                                   int32_t n_pairs, int64_t delay, int32_t publish, float salt, int32_t* counts_dev,
                                   hipStream_t stream) {
    if (workspace == nullptr || counts_dev == nullptr) return -1;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0 || (reinterpret_cast<uintptr_t>(counts_dev) & 15) != 0)
        return -1;
    if (n_prod < 1 || n_prod > 1024 || n_cons < 1 || n_cons > 65536) return -1;
    if (n_pairs < 1 || n_pairs > kMaxPairs || delay < 0 || delay > kMaxDelay) return -1;
    if (publish != 0 && publish != 1) return -1;
    if (!publish && (n_pairs > kNth || n_cons > 64)) return -1;  // every waiting thread expires once
    if (workspace_bytes < glowq::kWsHeader + (size_t)n_pairs * 8u) return -1;
    glowq::ForwardArgs a{};
    a.sync = static_cast<int32_t*>(workspace);
    a.R = static_cast<uint8_t*>(workspace) + glowq::kWsHeader;
    a.n_prod = n_prod;
    a.n_tiles = n_cons;
    hipLaunchKernelGGL(handoff_probe_kernel, dim3((unsigned)(n_prod + n_cons)), dim3(kNth), 0, stream, a, n_pairs,
                       delay, publish, salt, counts_dev);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
