// The cosine transition scores (LiLiCorr section 3.2, Eq. 1, with the
// drafter's successor logit added as in the DCOCO score), the prefix-first
// walk (DCOCO method details step (5); LiLiCorr section 3.5, Eq. 8), and small
// copy kernels used to expose intermediates.
#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

// One workgroup per pair: S[a][b] = l_{p+1}(b) + sigma * <o_p^a, i_{p+1}^b>,
// the vectors already unit-normalised; fp32 dot products in index order.
__global__ __launch_bounds__(256) void cosine_kernel(CosArgs a) {
    const int pair = blockIdx.x;
    const int B = a.B, K = a.K, dv = a.dvec;
    const int req = pair / (B - 1), p = pair % (B - 1);
    const int64_t tp = static_cast<int64_t>(req) * B + p, tq = tp + 1;
    for (int idx = threadIdx.x; idx < K * K; idx += blockDim.x) {
        const int ia = idx / K, ib = idx % K;
        const float* o = a.vout + (tp * K + ia) * dv;
        const float* v = a.vin + (tq * K + ib) * dv;
        float acc = 0.f;
        for (int c = 0; c < dv; ++c) acc += o[c] * v[c];
        a.scores[static_cast<int64_t>(pair) * K * K + idx] = a.vals[tq * K + ib] + a.sigma * acc;
    }
}

// The prefix-first walk of one request by one wave over its scores `src`
// ([B-1][K][K], LDS or memory): choice[0] = 0 (rank 0 is the drafter argmax of
// the first drafted slot); then each step takes the largest score in the row
// of the chosen predecessor, ties to the lowest successor index.
__device__ void walk_wave(const float* src, const int32_t* __restrict__ ids, int req, int B, int K,
                          int32_t* __restrict__ tokens, int32_t* __restrict__ choice) {
    const int l = lane_id();
    int k = 0;
    int mych = 0;  // lane s < B keeps choice[s]
    for (int p = 0; p + 1 < B; ++p) {
        const float* row = src + (static_cast<int64_t>(p) * K + k) * K;
        k = wave_argmax_lowest(l < K ? row[l] : 0.f, K);
        if (l == p + 1) mych = k;
    }
    // tokens[s] = ids[s][choice[s]]: one gather per lane after the walk
    if (l < B) {
        const int64_t s = static_cast<int64_t>(req) * B + l;
        if (choice) choice[s] = mych;
        tokens[s] = ids[s * K + mych];
    }
}

// The walk of one request from its scores held in LDS (sS, [B-1][K][K]) by
// the whole workgroup: first every row's argmax at once (one row per thread,
// scanning in index order with a strict compare, so ties go to the lowest
// successor index) into best[p][a]; then one lane follows the chain
// k_1 = 0, k_{p+1} = best[p][k_p] (B - 1 dependent byte reads); then lanes
// s < B write choice[s] and gather tokens[s] = ids[s][k_s].  Every thread of
// the workgroup calls it.
__device__ void walk_block(const float* sS, uint8_t* best, int* chain, const int32_t* __restrict__ ids, int req,
                           int B, int K, int32_t* __restrict__ tokens, int32_t* __restrict__ choice) {
    const int nrows = (B - 1) * K;
    for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
        const float* row = sS + r * K;
        float bv = row[0];
        int bi = 0;
        if ((K & 3) == 0) {   // rows are 16-byte aligned
            for (int b4 = 0; b4 < K / 4; ++b4) {
                const float4 v = reinterpret_cast<const float4*>(row)[b4];
                if (v.x > bv) { bv = v.x; bi = 4 * b4; }
                if (v.y > bv) { bv = v.y; bi = 4 * b4 + 1; }
                if (v.z > bv) { bv = v.z; bi = 4 * b4 + 2; }
                if (v.w > bv) { bv = v.w; bi = 4 * b4 + 3; }
            }
        } else {
            for (int b = 1; b < K; ++b)
                if (row[b] > bv) { bv = row[b]; bi = b; }
        }
        best[r] = static_cast<uint8_t>(bi);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int k = 0;
        chain[0] = 0;
        for (int p = 0; p + 1 < B; ++p) {
            k = best[p * K + k];
            chain[p + 1] = k;
        }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < B; t += blockDim.x) {
        const int64_t s = static_cast<int64_t>(req) * B + t;
        const int ch = chain[t];
        if (choice) choice[s] = ch;
        tokens[s] = ids[s * K + ch];
    }
}

// LDS layout of a walk with its scores in LDS: the scores, then best
// ([B-1][K] bytes), then chain ([B] ints, 4-byte aligned).
__host__ __device__ inline size_t walk_best_offset(int B, int K) {
    return static_cast<size_t>(B - 1) * K * K * sizeof(float);
}
__host__ __device__ inline size_t walk_chain_offset(int B, int K) {
    return (walk_best_offset(B, K) + static_cast<size_t>(B - 1) * K + 3) / 4 * 4;
}

// Walk over precomputed scores, one wave per request.  When the request's
// scores fit (use_lds) they are first copied into LDS with coalesced 16-byte
// loads, all issued before any is used, so the dependent steps read LDS.
__global__ __launch_bounds__(64) void walk_kernel(const float* __restrict__ scores,
                                                  const int32_t* __restrict__ ids, int n, int B,
                                                  int K, int32_t* __restrict__ tokens,
                                                  int32_t* __restrict__ choice, int use_lds) {
    extern __shared__ __attribute__((aligned(16))) float sl[];
    const int req = blockIdx.x;
    const int l = lane_id();
    if (req >= n) return;
    const int64_t per = static_cast<int64_t>(B - 1) * K * K;
    const float* base = scores + req * per;
    if (use_lds) {
        if ((per & 3) == 0 && (reinterpret_cast<uintptr_t>(base) & 15) == 0) {
            const int64_t nv = per / 4;
            for (int64_t i0 = 0; i0 < nv; i0 += 8 * kWave) {
                float4 t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t i = min(i0 + u * kWave + l, nv - 1);  // clamped: always in bounds
                    t[u] = reinterpret_cast<const float4*>(base)[i];
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t i = i0 + u * kWave + l;
                    if (i < nv) reinterpret_cast<float4*>(sl)[i] = t[u];
                }
            }
        } else {
            for (int64_t i = l; i < per; i += kWave) sl[i] = base[i];
        }
        wave_lds_sync();
    }
    if (use_lds) {
        walk_block(sl, reinterpret_cast<uint8_t*>(reinterpret_cast<char*>(sl) + walk_best_offset(B, K)),
                   reinterpret_cast<int*>(reinterpret_cast<char*>(sl) + walk_chain_offset(B, K)), ids, req, B, K,
                   tokens, choice);
        return;
    }
    walk_wave(base, ids, req, B, K, tokens, choice);
}

// One workgroup per request: S = l_{p+1}(b) + (sum of the hidden-block partial
// Deltas in block order + b2) for all of the request's pairs, written to
// `scores` (and kept in LDS when it fits); then, with tokens given, the walk.
__global__ __launch_bounds__(256) void finish_kernel(FinishArgs a, int use_lds) {
    extern __shared__ __attribute__((aligned(16))) float sS[];
    const int req = blockIdx.x;
    const int B = a.B, K = a.K;
    const int KK = K * K;
    const int64_t per = static_cast<int64_t>(B - 1) * KK;
    const float b2 = a.b2[0];
    const int per32 = static_cast<int>(per);   // (B-1) K^2 < 2^31: 32-bit index math
    const float* part_req = a.part + static_cast<int64_t>(req) * (B - 1) * a.nblk * KK;
    const float* vals_req = a.vals + static_cast<int64_t>(req) * B * K;
    float* scores_req = a.scores + static_cast<int64_t>(req) * per;
    if ((K & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.scores) | reinterpret_cast<uintptr_t>(a.vals)) & 15) == 0) {
        // four consecutive elements (one pair, one row a) per float4; four
        // float4 per thread per round, all loads issued before any is used
        const int per4 = per32 / 4;
        for (int i0 = 0; i0 < per4; i0 += 4 * 256) {
            float4 d[4], lv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i4 = min(i0 + u * 256 + static_cast<int>(threadIdx.x), per4 - 1);  // clamped: in bounds
                const int idx = i4 * 4;
                const int p = idx / KK, e = idx - p * KK;
                const float* src = part_req + (p * a.nblk) * KK + e;
                float4 t[kMaxMlpBlocks];
#pragma unroll
                for (int b = 0; b < kMaxMlpBlocks; ++b)
                    t[b] = *reinterpret_cast<const float4*>(src + (b < a.nblk ? b : a.nblk - 1) * KK);
                float4 acc = t[0];
#pragma unroll
                for (int b = 1; b < kMaxMlpBlocks; ++b)
                    if (b < a.nblk) acc = make_float4(acc.x + t[b].x, acc.y + t[b].y, acc.z + t[b].z, acc.w + t[b].w);
                d[u] = acc;
                lv[u] = *reinterpret_cast<const float4*>(vals_req + (p + 1) * K + e % K);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i4 = i0 + u * 256 + static_cast<int>(threadIdx.x);
                if (i4 < per4) {
                    const float4 sv = make_float4(lv[u].x + (d[u].x + b2), lv[u].y + (d[u].y + b2),
                                                  lv[u].z + (d[u].z + b2), lv[u].w + (d[u].w + b2));
                    reinterpret_cast<float4*>(scores_req)[i4] = sv;
                    if (use_lds) reinterpret_cast<float4*>(sS)[i4] = sv;
                }
            }
        }
    } else
    // 8 elements per thread per round, all loads issued before any is used
    for (int i0 = 0; i0 < per32; i0 += 8 * 256) {
        float d[8], lv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = min(i0 + u * 256 + static_cast<int>(threadIdx.x), per32 - 1);  // clamped: in bounds
            const int p = idx / KK, e = idx - p * KK;
            d[u] = sum_strided<kMaxMlpBlocks>(part_req + (p * a.nblk) * KK + e, KK, a.nblk);
            lv[u] = vals_req[(p + 1) * K + e % K];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = i0 + u * 256 + static_cast<int>(threadIdx.x);
            if (idx < per32) {
                const float sv = lv[u] + (d[u] + b2);
                scores_req[idx] = sv;
                if (use_lds) sS[idx] = sv;
            }
        }
    }
    if (!a.tokens) return;
    __syncthreads();
    if (use_lds) {
        walk_block(sS, reinterpret_cast<uint8_t*>(reinterpret_cast<char*>(sS) + walk_best_offset(B, K)),
                   reinterpret_cast<int*>(reinterpret_cast<char*>(sS) + walk_chain_offset(B, K)), a.ids, req, B,
                   K, a.tokens, a.choice);
        return;
    }
    if ((threadIdx.x >> 6) != 0) return;
    walk_wave(a.scores + req * per, a.ids, req, B, K, a.tokens, a.choice);
}

// z = hi + lo for each node row of the [hi | lo] layout.
__global__ void zhl_to_f32_kernel(const uint16_t* __restrict__ zhl, float* __restrict__ z,
                                  int64_t nodes, int r) {
    const int64_t count = nodes * r;
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t node = i / r, c = i % r;
        z[i] = bf16_to_f32(zhl[node * 2 * r + c]) + bf16_to_f32(zhl[node * 2 * r + r + c]);
    }
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst,
                                int64_t count) {
    for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < count;
         i += static_cast<int64_t>(gridDim.x) * blockDim.x)
        dst[i] = src[i];
}

unsigned grid_for(int64_t count) {
    const int64_t g = (count + 255) / 256;
    return static_cast<unsigned>(g < 4096 ? (g < 1 ? 1 : g) : 4096);
}

}  // namespace

hipError_t launch_cosine(const CosArgs& a, hipStream_t stream) {
    return launch(cosine_kernel, dim3(static_cast<unsigned>(a.n * (a.B - 1))), 256, 0, stream, a);
}

// Dynamic LDS of a walk that holds the request's scores (and the walk's
// best and chain arrays), or 0 when they do not fit and the walk reads memory.
static size_t walk_lds_bytes(int B, int K) {
    if (B < 2) return 0;
    const size_t bytes = walk_chain_offset(B, K) + sizeof(int) * B;
    return bytes <= 60 * 1024 ? bytes : 0;
}

hipError_t launch_walk(const float* scores, const int32_t* ids, int n, int B, int K,
                       int32_t* tokens, int32_t* choice, hipStream_t stream) {
    const size_t lds = walk_lds_bytes(B, K);
    return launch(walk_kernel, dim3(static_cast<unsigned>(n)), 64, static_cast<uint32_t>(lds), stream, scores,
                  ids, n, B, K, tokens, choice, lds > 0);
}

hipError_t launch_finish(const FinishArgs& a, hipStream_t stream) {
    const size_t lds = walk_lds_bytes(a.B, a.K);
    return launch(finish_kernel, dim3(static_cast<unsigned>(a.n)), 256, static_cast<uint32_t>(lds), stream, a,
                  lds > 0);
}

hipError_t launch_zhl_to_f32(const uint16_t* zhl, float* z, int64_t nodes, int r, hipStream_t stream) {
    return launch(zhl_to_f32_kernel, dim3(grid_for(nodes * r)), 256, 0, stream, zhl, z, nodes, r);
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t count, hipStream_t stream) {
    return launch(copy_f32_kernel, dim3(grid_for(count)), 256, 0, stream, src, dst, count);
}

}  // namespace corr
