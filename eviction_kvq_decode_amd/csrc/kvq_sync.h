// kvq_sync.h -- batch-order counts across the workgroups of one launch.
//
// The append (pops) and the eviction (pushes) serve the free stacks in
// batch order: sequence b's ids sit at an offset given by the counts of
// sequences 0 .. b-1.  One workgroup per sequence publishes its count per
// pool in a word of its own, tagged with the call's epoch (SyncWs); a
// workgroup that needs its offset sums the words of the sequences before it,
// waiting for the ones not yet in.  Workgroups only wait on earlier ones,
// which are dispatched first and never wait on later ones, and every wait is
// bounded.  The last workgroup sums every word, moves the stack tops and
// then stores the epoch, which the next call starts from.
//
// Ordering without fences: a word carries all the data it passes, so it is
// stored and loaded as a relaxed device-scope atomic (no cache write-back or
// invalidate, which an acquire / release would cost).  What must precede a
// publish -- the workgroup's read of the stack tops and of the epoch -- is
// completed with a wait that is also a compiler barrier (wait_loads_done).
#pragma once
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {

constexpr int SYNC_SPINS = 1 << 22;   // polls of one word before giving up
constexpr int SYNC_UNROLL = 4;        // words a lane loads before checking them

// Every load this thread issued has returned, and the compiler moves no
// memory access across this point.
__device__ inline void wait_loads_done() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// This call's epoch, one past the last call's (skipping 0).  Read by one wave
// (the value is the same in every lane).
__device__ inline uint32_t sync_epoch(const SyncWs &s) {
    const uint32_t last = __hip_atomic_load(s.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_amdgcn_readfirstlane(last == 0xffffffffu ? 1u : last + 1u);
}

__device__ inline void sync_publish(const SyncWs &s, int B, int b, int pool, uint32_t epoch, uint32_t count) {
    __hip_atomic_store(s.words + (size_t)pool * B + b, ((unsigned long long)epoch << 32) | count,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last workgroup, once it has every word of the call.
__device__ inline void sync_close(const SyncWs &s, uint32_t epoch) {
    __hip_atomic_store(s.epoch, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of the counts of sequences [0, n) for each pool in pmask (bit p: pool
// p; other pools give 0), by one whole wave; every lane gets the sums.
// False if a word did not come within the spin bound (its count taken as 0).
__device__ inline bool sync_counts_before(const SyncWs &s, int B, int n, uint32_t epoch, uint32_t pmask,
                                          int cnt[3]) {
    const int lane = threadIdx.x & 63;
    // the selected pools in order; word j of the walk is sequence j % n of
    // the (j / n)-th of them
    const int np = __popc(pmask & 7u);
    const int p0 = __builtin_ctz(pmask | 8u);
    const int p1 = __builtin_ctz((pmask & ~(1u << p0)) | 8u);
    const int p2 = 2;
    const int total = np * n;
    int a0 = 0, a1 = 0, a2 = 0;
    bool ok = true;
    for (int j0 = 0; j0 < total; j0 += 64 * SYNC_UNROLL) {
        unsigned long long v[SYNC_UNROLL];
        const unsigned long long *w[SYNC_UNROLL];
        int pool[SYNC_UNROLL];
#pragma unroll
        for (int u = 0; u < SYNC_UNROLL; ++u) {
            const int j = j0 + 64 * u + lane;
            pool[u] = -1;
            w[u] = nullptr;
            v[u] = 0;
            if (j < total) {
                const int k = j / n;
                pool[u] = k == 0 ? p0 : (k == 1 ? p1 : p2);
                w[u] = s.words + (size_t)pool[u] * B + (j - k * n);
                v[u] = __hip_atomic_load(w[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
#pragma unroll
        for (int u = 0; u < SYNC_UNROLL; ++u) {
            if (pool[u] < 0) continue;
            int spins = 0;
            while ((uint32_t)(v[u] >> 32) != epoch) {
                if (++spins > SYNC_SPINS) {
                    ok = false;
                    v[u] = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
                v[u] = __hip_atomic_load(w[u], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            const int cv = (int)(uint32_t)v[u];
            a0 += pool[u] == 0 ? cv : 0;
            a1 += pool[u] == 1 ? cv : 0;
            a2 += pool[u] == 2 ? cv : 0;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        a0 += __shfl_xor(a0, off);
        a1 += __shfl_xor(a1, off);
        a2 += __shfl_xor(a2, off);
    }
    cnt[0] = a0;
    cnt[1] = a1;
    cnt[2] = a2;
    return __ballot(!ok) == 0;
}

}  // namespace kvq
