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

// One wave's share of a pair's K x K scores (K = 4, 8 or 16): lane l < K^2 / 4
// holds the four consecutive scores e = 4l .. 4l + 3 of row aa = e / K,
// columns b0 .. b0 + 3 (lanes past K^2 / 4 repeat the last four, not stored).
struct PairRow4 {
    float4 sv;
    int aa, b0, nv;
};

// Four consecutive partials; kAtomic: with agent-scope atomic loads (written
// by other workgroups of the same launch).
template <bool kAtomic>
__device__ __forceinline__ float4 load_part4(const float* p) {
    if (!kAtomic) return *reinterpret_cast<const float4*>(p);
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float4(__uint_as_float(static_cast<uint32_t>(lo)), __uint_as_float(static_cast<uint32_t>(lo >> 32)),
                       __uint_as_float(static_cast<uint32_t>(hi)), __uint_as_float(static_cast<uint32_t>(hi >> 32)));
}

// The scores of pair `pair` from the MLP's partials: the nblk 64-unit blocks
// in block order (or, with sub, nblk 16-unit partials added four at a time in
// the 64-unit form's tree (P0 + P1) + (P2 + P3), a missing one counting as
// +0, then the 64-unit blocks in order), + b2, + l_{p+1}(b); successors
// b >= m at -inf.
template <bool kAtomic>
__device__ __forceinline__ PairRow4 pair_scores4(const float* part, int nblk, int sub, int m, const float* vals,
                                                 float b2, int B, int K, int pair) {
    const int KK = K * K;
    const int req = pair / (B - 1), p = pair - req * (B - 1);
    const int l = lane_id();
    PairRow4 r;
    r.nv = KK / 4;                            // float4 of the pair: 4, 16 or 64
    const int i4 = min(l, r.nv - 1);
    const int e = 4 * i4;
    r.aa = e / K;
    r.b0 = e - r.aa * K;
    const float* src = part + static_cast<int64_t>(pair) * nblk * KK + e;
    float4 t[kMaxMlpBlocks];
    int nb64 = nblk;
    if (sub) {
        nb64 = (nblk + 3) / 4;
        float4 u[4 * kMaxMlpBlocks];
#pragma unroll
        for (int b = 0; b < 4 * kMaxMlpBlocks; ++b)
            u[b] = b < nblk ? load_part4<kAtomic>(src + b * KK) : make_float4(0.f, 0.f, 0.f, 0.f);
        auto add = [](float4 x, float4 y) { return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w); };
#pragma unroll
        for (int g = 0; g < kMaxMlpBlocks; ++g) t[g] = add(add(u[4 * g], u[4 * g + 1]), add(u[4 * g + 2], u[4 * g + 3]));
    } else {
#pragma unroll
        for (int b = 0; b < kMaxMlpBlocks; ++b) t[b] = load_part4<kAtomic>(src + (b < nblk ? b : nblk - 1) * KK);
    }
    const float4 lv = *reinterpret_cast<const float4*>(vals + (static_cast<int64_t>(req) * B + p + 1) * K + r.b0);
    float4 acc = t[0];
#pragma unroll
    for (int b = 1; b < kMaxMlpBlocks; ++b)
        if (b < nb64) acc = make_float4(acc.x + t[b].x, acc.y + t[b].y, acc.z + t[b].z, acc.w + t[b].w);
    r.sv = make_float4(lv.x + (acc.x + b2), lv.y + (acc.y + b2), lv.z + (acc.z + b2), lv.w + (acc.w + b2));
    if (m < K)   // successors b >= m are not scored
        r.sv = make_float4(r.b0 < m ? r.sv.x : -INFINITY, r.b0 + 1 < m ? r.sv.y : -INFINITY,
                           r.b0 + 2 < m ? r.sv.z : -INFINITY, r.b0 + 3 < m ? r.sv.w : -INFINITY);
    return r;
}

// The prefix-first walk's end of the per-pair finishing step, by one wave:
// the pair's scores written, each row's argmax (the lane's four in index
// order with a strict compare, then across the K / 4 lanes of the row, ties
// to the lower index) to best[pair][aa], the pair counted into its request,
// and the request's last pair walks.
__device__ __forceinline__ void pair_walk_finish(const PairRow4& r, float* scores, int32_t* best, int* cnt,
                                                 const int32_t* __restrict__ ids, int32_t* __restrict__ tokens,
                                                 int32_t* __restrict__ choice, int B, int K, int pair) {
    const int l = lane_id();
    const int req = pair / (B - 1);
    const float4 sv = r.sv;
    if (l < r.nv) reinterpret_cast<float4*>(scores + static_cast<int64_t>(pair) * K * K)[l] = sv;
    float bv = sv.x;
    int bi = r.b0;
    if (sv.y > bv) { bv = sv.y; bi = r.b0 + 1; }
    if (sv.z > bv) { bv = sv.z; bi = r.b0 + 2; }
    if (sv.w > bv) { bv = sv.w; bi = r.b0 + 3; }
    for (int sh = 1; sh < K / 4; sh <<= 1) {
        const float ov = __shfl_xor(bv, sh, 64);
        const int oi = __shfl_xor(bi, sh, 64);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (l < r.nv && r.b0 == 0)
        __hip_atomic_store(best + static_cast<int64_t>(pair) * K + r.aa, bi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!pair_last_of_request(cnt, req, B)) return;
    pair_walk(best, req, B, K, ids, tokens, choice);
}

}  // namespace

}  // namespace corr
