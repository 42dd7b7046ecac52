// The per-request hand-off of the launches that finish a request's scores
// one wave (or workgroup) per pair: the last one of a request, found by a
// device counter, takes the request's path.  Values cross workgroups as
// agent-scope atomic stores and loads (coherent across the chip's L2 caches
// without a cache write-back), and a wave counts itself in only after its
// stores have completed.
#pragma once

#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

// A wave counts itself into its request's counter once its stores have
// completed (the stores of what the last wave reads are agent-scope atomics:
// coherent across the chip's L2 caches without a cache write-back).  True in
// the request's last wave.  The counters are zeroed by the launch before.
__device__ __forceinline__ bool pair_last_of_request(int* cnt, int req, int B) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores are complete
    asm volatile("" ::: "memory");
    int done = 0;
    if (lane_id() == 0)
        done = __hip_atomic_fetch_add(cnt + static_cast<int64_t>(req) * kCntStride, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    return __shfl(done, 0, 64) == B - 2;
}

// The prefix-first walk of the request's last wave from the pairs' row
// argmaxes best[pair][a] (K <= 16): lane q < B - 1 holds best[q][.] packed
// four bits per entry, the chain k_1 = 0, k_{p+1} = best[p][k_p] follows by
// readlane, and lanes s < B write choice and tokens.
__device__ __forceinline__ void pair_walk(const int32_t* best, int req, int B, int K,
                                          const int32_t* __restrict__ ids, int32_t* __restrict__ tokens,
                                          int32_t* __restrict__ choice) {
    const int l = lane_id();
    uint64_t row = 0;
    {
        // all K loads issued before any is used (entries past K repeat the
        // last, and are not read by the chain)
        const int q = min(l, B - 2);
        const int32_t* bq = best + (static_cast<int64_t>(req) * (B - 1) + q) * K;
        int32_t bt[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) bt[j] = __hip_atomic_load(bq + min(j, K - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int j = 0; j < 16; ++j) row |= static_cast<uint64_t>(bt[j] & 15) << (4 * j);
    }
    const uint32_t lo = static_cast<uint32_t>(row), hi = static_cast<uint32_t>(row >> 32);
    int k = 0, mych = 0;   // lane s < B keeps choice[s]
    for (int q = 0; q + 1 < B; ++q) {
        const uint32_t w = k < 8 ? __builtin_amdgcn_readlane(lo, q) : __builtin_amdgcn_readlane(hi, q);
        k = (w >> (4 * (k & 7))) & 15;
        if (l == q + 1) mych = k;
    }
    if (l < B) {
        const int64_t s = static_cast<int64_t>(req) * B + l;
        if (choice) choice[s] = mych;
        tokens[s] = ids[s * K + mych];
    }
}

}  // namespace

}  // namespace corr
