// Step (5) and the cosine variant's scores:
//   - the prefix-first walk (DCOCO method details step (5); LiLiCorr section
//     3.5, Eq. 8) and the Global-Sum path (LiLiCorr appendix E, Eq. 12: the
//     path with the largest summed score, by dynamic programming);
//   - the cosine transition scores (LiLiCorr section 3.2, Eq. 1, with the
//     drafter's successor logit added as in the DCOCO score);
//   - the finishing reduction of the MLP's hidden-block partials;
//   - small copy kernels used to expose intermediates.
#include "common.h"
#include "handoff.h"
#include "kernels.h"

namespace corr {

namespace {

// The prefix-first walk of one request by one wave over its scores `src`
// ([B-1][K][K], LDS or memory): choice[0] = 0 (rank 0 is the drafter argmax of
// the first drafted slot); then each step takes the largest score in the row
// of the chosen predecessor, ties to the lowest successor index.
__device__ __forceinline__ void walk_wave(const float* src, const int32_t* __restrict__ ids, int req, int B, int K,
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
__device__ __forceinline__ void walk_block(const float* sS, uint8_t* best, int* chain, const int32_t* __restrict__ ids, int req,
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

// The Global-Sum path of one request by one wave over its scores `src`
// ([B-1][K][K], LDS or memory).  best[b] is the best score of a path ending at
// candidate b of the current slot (slot 1: 0 at rank 0 and -inf elsewhere, as
// the walk fixes slot 1 at the drafter's argmax); it lives in LDS (vb, K
// floats, 16-byte aligned), written by lanes b < K and read back by every lane
// as broadcast float4 loads.  Each pair step takes, for every b (one per
// lane), the largest best[a] + S_p(a, b) over a: the predecessors go in groups
// of 16, whose column of S is read first and reduced by a (value, index) tree
// in which the right operand (higher indices) wins only if strictly greater,
// so ties go to the lowest a; the argmax a goes to from[p][b] (LDS).  The last
// slot's largest best (lowest index on ties) is traced back through `from` by
// one lane into chain[] (LDS), and lanes s < B write choice[s] and gather
// tokens[s] = ids[s][chain[s]].
__device__ __forceinline__ void viterbi_wave(const float* src, uint8_t* from, int* chain, float* vb,
                                             const int32_t* __restrict__ ids, int req, int B, int K, float lam,
                                             int32_t* __restrict__ tokens, int32_t* __restrict__ choice) {
    const int l = lane_id();
    const int bl = min(l, K - 1);   // lanes past K mirror the last candidate (never used)
    float bv = l == 0 ? 0.f : -INFINITY;
    float wp = 1.f;                  // lam^p (1 for the Global-Sum rule: fmaf(1, s, b) is b + s)
    for (int p = 0; p + 1 < B; ++p, wp *= lam) {
        if (l < K) vb[l] = bv;
        wave_lds_sync();
        const float* Sp = src + static_cast<int64_t>(p) * K * K;
        float v = -INFINITY;
        int arg = 0;
        for (int a0 = 0; a0 < K; a0 += 16) {
            float w[16];
            float4 pv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)   // vb has room for the whole group (K rounded up to 16)
                pv[q] = *reinterpret_cast<const float4*>(vb + a0 + 4 * q);
#pragma unroll
            for (int u = 0; u < 16; ++u) w[u] = Sp[min(a0 + u, K - 1) * K + bl];   // clamped: past K unused
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const float4 q4 = pv[u / 4];
                const float pb = (u & 3) == 0 ? q4.x : ((u & 3) == 1 ? q4.y : ((u & 3) == 2 ? q4.z : q4.w));
                w[u] = a0 + u < K ? fmaf(wp, w[u], pb) : -INFINITY;
            }
            // The group's maximum, then the lowest predecessor that reaches it
            // (a select sweep over constant indices: no index array to carry).
            float m = w[0];
#pragma unroll
            for (int u = 1; u < 16; ++u) m = fmaxf(m, w[u]);
            int a = 0;
#pragma unroll
            for (int u = 15; u >= 0; --u) a = w[u] == m ? u : a;
            if (a0 == 0 || m > v) {
                v = m;
                arg = a0 + a;
            }
        }
        if (l < K) from[p * K + l] = static_cast<uint8_t>(arg);
        bv = l < K ? v : -INFINITY;
        wave_lds_sync();   // every lane has read vb before the next step rewrites it
    }
    int k = wave_argmax_lowest(bv, K);
    wave_lds_sync();
    if (l == 0) {
        for (int t = B - 1; t >= 1; --t) {
            chain[t] = k;
            k = from[(t - 1) * K + k];
        }
        chain[0] = 0;
    }
    wave_lds_sync();
    if (l < B) {
        const int64_t s_ = static_cast<int64_t>(req) * B + l;
        const int ch = chain[l];
        if (choice) choice[s_] = ch;
        tokens[s_] = ids[s_ * K + ch];
    }
}

// The same dynamic program for K <= 16 with all 64 lanes at work: lane l
// takes successor b = l / 4 and the four predecessors a = 4g .. 4g + 3 of its
// group g = l % 4, so the four groups of a successor share a quad.  Each lane
// forms its four fmaf(lam^p, S_p(a, b), best[a]) (the same float32
// operations as viterbi_wave), their fmaxf and the lowest a reaching it; two
// quad exchanges (DPP, lanes l ^ 1 and l ^ 2) take the fmaxf of the groups'
// values and the lowest a among the groups that reach it.  Every b thus ends
// with viterbi_wave's maximum and predecessor, bit for bit.  best stays in LDS
// (vb), which the one wave writes after it has read it, in program order; a
// step reads it first and then loads the next pair's scores, which arrive
// while the step is reduced.
__device__ __forceinline__ void viterbi16_wave(const float* src, uint8_t* from, int* chain, float* vb,
                                               const int32_t* __restrict__ ids, int req, int B, int K, float lam,
                                               int32_t* __restrict__ tokens, int32_t* __restrict__ choice) {
    const int l = lane_id();
    const int g = l & 3;
    const int b = min(l >> 2, K - 1);
    const bool head = (l & 3) == 0 && (l >> 2) < K;   // one lane per successor writes
    if (l < 16) vb[l] = l == 0 ? 0.f : -INFINITY;   // slot 1: the drafter's argmax
    float s[4];
    auto load = [&](int p, float (&t)[4]) {
        const float* Sp = src + static_cast<int64_t>(p) * K * K;
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = Sp[min(4 * g + i, K - 1) * K + b];   // clamped: past K unused
    };
    if (B > 1) load(0, s);
    float wp = 1.f;
    for (int p = 0; p + 1 < B; ++p, wp *= lam) {
        wave_lds_sync();
        const float4 v4 = *reinterpret_cast<const float4*>(vb + 4 * g);
        float sn[4];
        load(min(p + 1, B - 2), sn);
        const float pv[4] = {v4.x, v4.y, v4.z, v4.w};
        float c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = 4 * g + i < K ? fmaf(wp, s[i], pv[i]) : -INFINITY;
        float m = fmaxf(fmaxf(c[0], c[1]), fmaxf(c[2], c[3]));
        // the lowest a whose value is the maximum (64: none in this group)
        int arg = c[3] == m ? 4 * g + 3 : 64;
        arg = c[2] == m ? 4 * g + 2 : arg;
        arg = c[1] == m ? 4 * g + 1 : arg;
        arg = c[0] == m ? 4 * g : arg;
        {
            const float om = dpp_f<kDppXor1>(m);
            const int oa = __builtin_amdgcn_update_dpp(0, arg, kDppXor1, 0xF, 0xF, false);
            const float mm = fmaxf(m, om);
            arg = min(m == mm ? arg : 64, om == mm ? oa : 64);
            m = mm;
        }
        {
            const float om = dpp_f<kDppXor2>(m);
            const int oa = __builtin_amdgcn_update_dpp(0, arg, kDppXor2, 0xF, 0xF, false);
            const float mm = fmaxf(m, om);
            arg = min(m == mm ? arg : 64, om == mm ? oa : 64);
            m = mm;
        }
        if (head) {
            from[p * K + (l >> 2)] = static_cast<uint8_t>(arg == 64 ? 0 : arg);
            vb[l >> 2] = m;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = sn[i];
    }
    wave_lds_sync();
    const float fin = l < K ? vb[l] : -INFINITY;   // best of the last slot (slot 1 when B = 1)
    int k = wave_argmax_lowest(fin, K);
    wave_lds_sync();
    if (l == 0) {
        for (int t = B - 1; t >= 1; --t) {
            chain[t] = k;
            k = from[(t - 1) * K + k];
        }
        chain[0] = 0;
    }
    wave_lds_sync();
    if (l < B) {
        const int64_t s_ = static_cast<int64_t>(req) * B + l;
        const int ch = chain[l];
        if (choice) choice[s_] = ch;
        tokens[s_] = ids[s_ * K + ch];
    }
}

// LDS of a path over scores held in LDS: the scores, then from/best
// ([B-1][K] bytes), then chain ([B] ints), then vb (K rounded up to 16
// floats, 16-byte aligned); without the scores, the last three alone.
__host__ __device__ inline size_t path_aux_offset(int B, int K, bool scores_in_lds) {
    return scores_in_lds ? walk_best_offset(B, K) : 0;
}
__host__ __device__ inline size_t path_chain_offset(int B, int K, bool scores_in_lds) {
    return (path_aux_offset(B, K, scores_in_lds) + static_cast<size_t>(B > 1 ? B - 1 : 0) * K + 3) / 4 * 4;
}
__host__ __device__ inline size_t path_vb_offset(int B, int K, bool scores_in_lds) {
    return (path_chain_offset(B, K, scores_in_lds) + sizeof(int) * static_cast<size_t>(B) + 15) / 16 * 16;
}
__host__ __device__ inline size_t path_beam_offset(int B, int K, bool scores_in_lds) {
    return path_vb_offset(B, K, scores_in_lds) + sizeof(float) * static_cast<size_t>((K + 15) / 16 * 16);
}
// the beam's backpointers: [B-1][4] (parent, successor) byte pairs
__host__ __device__ inline size_t path_lds_end(int B, int K, bool scores_in_lds) {
    return path_beam_offset(B, K, scores_in_lds) + static_cast<size_t>(B > 1 ? B - 1 : 0) * 8;
}

// Largest value over the wave, the same in every lane.
__device__ __forceinline__ float wave_max_all(float v) {
    const float m = row16_max(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48))));
}

// Beam search of width W (1..4) by one wave over the request's scores `src`
// ([B-1][K][K], LDS or memory): the beam starts as the single path (rank 0)
// with score 0; at pair p, extension c = i*K + b of beam path i by successor
// b scores g_i + S_p(last_i, b) (one float32 addition), lane l holding
// extensions l, l + 64, l + 128, l + 192; W rounds each take the largest
// remaining score, the lowest c among equals (beam index, then successor), so
// the kept paths are ordered as the rounds found them.  Beam scores and last
// candidates are wave-uniform registers; the (parent, successor) of every
// kept path goes to LDS (bp, [B-1][4][2] bytes) and the first path of the
// last step is traced back through it.
__device__ __forceinline__ void beam_wave(const float* src, uint8_t* bp, int* chain, const int32_t* __restrict__ ids,
                                          int req, int B, int K, int W, int32_t* __restrict__ tokens,
                                          int32_t* __restrict__ choice) {
    const int l = lane_id();
    float g[4] = {0.f, 0.f, 0.f, 0.f};
    int last[4] = {0, 0, 0, 0};
    int nb = 1;
    for (int p = 0; p + 1 < B; ++p) {
        const float* Sp = src + static_cast<int64_t>(p) * K * K;
        const int nc = nb * K;
        float cv[4];
        bool ok[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = j * kWave + l;
            const int i = (c >= K) + (c >= 2 * K) + (c >= 3 * K);
            const int b = c - i * K;
            ok[j] = c < nc;
            const float gi = i == 0 ? g[0] : (i == 1 ? g[1] : (i == 2 ? g[2] : g[3]));
            const int li = i == 0 ? last[0] : (i == 1 ? last[1] : (i == 2 ? last[2] : last[3]));
            cv[j] = ok[j] ? gi + Sp[li * K + b] : -INFINITY;
        }
        const int keep = min(W, nc);
        float ng[4] = {0.f, 0.f, 0.f, 0.f};
        int nl[4] = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r >= keep) break;
            // this lane's best remaining extension (the lowest j among equals)
            float bs = -INFINITY;
            int bj = -1;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (ok[j] && (bj < 0 || cv[j] > bs)) {
                    bs = cv[j];
                    bj = j;
                }
            const float M = wave_max_all(bs);
            // the lowest c = j*64 + lane whose score is M: the lowest j first
            int wj = 0, wl = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint64_t m = ballot(bj == j && bs == M);
                if (m) {
                    wj = j;
                    wl = __ffsll(static_cast<unsigned long long>(m)) - 1;
                    break;
                }
            }
            const int wc = wj * kWave + wl;
            const int wi = (wc >= K) + (wc >= 2 * K) + (wc >= 3 * K);
            const int wb = wc - wi * K;
            ng[r] = M;
            nl[r] = wb;
            if (l == 0) {
                bp[(p * 4 + r) * 2] = static_cast<uint8_t>(wi);
                bp[(p * 4 + r) * 2 + 1] = static_cast<uint8_t>(wb);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (j == wj && l == wl) ok[j] = false;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            g[r] = ng[r];
            last[r] = nl[r];
        }
        nb = keep;
    }
    wave_lds_sync();
    if (l == 0) {
        int r = 0;
        for (int p = B - 2; p >= 0; --p) {
            chain[p + 1] = bp[(p * 4 + r) * 2 + 1];
            r = bp[(p * 4 + r) * 2];
        }
        chain[0] = 0;
    }
    wave_lds_sync();
    if (l < B) {
        const int64_t s_ = static_cast<int64_t>(req) * B + l;
        const int ch = chain[l];
        if (choice) choice[s_] = ch;
        tokens[s_] = ids[s_ * K + ch];
    }
}

// The same beam search for K <= 16, where the nb * K <= 64 extensions of a
// pair fit one per lane (extension c = lane): each of the W rounds takes the
// wave's largest remaining score and the lowest lane holding it, which is
// beam_wave's choice (its lanes hold only their first extension here), so
// the kept paths are the same, bit for bit.
__device__ __forceinline__ void beam16_wave(const float* src, uint8_t* bp, int* chain, const int32_t* __restrict__ ids,
                                            int req, int B, int K, int W, int32_t* __restrict__ tokens,
                                            int32_t* __restrict__ choice) {
    const int l = lane_id();
    const int i = (l >= K) + (l >= 2 * K) + (l >= 3 * K);   // the lane's beam path
    const int b = min(l - i * K, K - 1);                    // and successor (clamped past 4K: unused)
    float g0 = 0.f, g1 = 0.f, g2 = 0.f, g3 = 0.f;
    int t0 = 0, t1 = 0, t2 = 0, t3 = 0;
    int nb = 1;
    for (int p = 0; p + 1 < B; ++p) {
        const float* Sp = src + static_cast<int64_t>(p) * K * K;
        const int nc = nb * K;
        const float gi = i == 0 ? g0 : (i == 1 ? g1 : (i == 2 ? g2 : g3));
        const int ti = i == 0 ? t0 : (i == 1 ? t1 : (i == 2 ? t2 : t3));
        bool alive = l < nc;
        const float cv = alive ? gi + Sp[ti * K + b] : -INFINITY;
        const int keep = min(W, nc);
        float ng[4] = {0.f, 0.f, 0.f, 0.f};
        int nt[4] = {0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (r >= keep) break;
            const float M = wave_max_all(alive ? cv : -INFINITY);
            const uint64_t win = ballot(alive && cv == M);
            const int wl = win ? __ffsll(static_cast<unsigned long long>(win)) - 1 : 0;
            const int wi = (wl >= K) + (wl >= 2 * K) + (wl >= 3 * K);
            const int wb = wl - wi * K;
            ng[r] = M;
            nt[r] = wb;
            if (l == 0) {
                bp[(p * 4 + r) * 2] = static_cast<uint8_t>(wi);
                bp[(p * 4 + r) * 2 + 1] = static_cast<uint8_t>(wb);
            }
            alive = alive && l != wl;
        }
        g0 = ng[0]; g1 = ng[1]; g2 = ng[2]; g3 = ng[3];
        t0 = nt[0]; t1 = nt[1]; t2 = nt[2]; t3 = nt[3];
        nb = keep;
    }
    wave_lds_sync();
    if (l == 0) {
        int r = 0;
        for (int p = B - 2; p >= 0; --p) {
            chain[p + 1] = bp[(p * 4 + r) * 2 + 1];
            r = bp[(p * 4 + r) * 2];
        }
        chain[0] = 0;
    }
    wave_lds_sync();
    if (l < B) {
        const int64_t s_ = static_cast<int64_t>(req) * B + l;
        const int ch = chain[l];
        if (choice) choice[s_] = ch;
        tokens[s_] = ids[s_ * K + ch];
    }
}

// The request's path from scores in LDS (every thread of the workgroup
// calls it): the greedy walk uses the whole workgroup, the Global-Sum
// dynamic program its first wave.
__device__ __forceinline__ void path_from_lds(int rule, float lam, int beam, float* sS, const int32_t* __restrict__ ids, int req,
                                              int B, int K, int32_t* __restrict__ tokens,
                                              int32_t* __restrict__ choice) {
    uint8_t* aux = reinterpret_cast<uint8_t*>(reinterpret_cast<char*>(sS) + path_aux_offset(B, K, true));
    int* chain = reinterpret_cast<int*>(reinterpret_cast<char*>(sS) + path_chain_offset(B, K, true));
    if (rule == kPathBeam) {
        uint8_t* bp = reinterpret_cast<uint8_t*>(reinterpret_cast<char*>(sS) + path_beam_offset(B, K, true));
        if ((threadIdx.x >> 6) == 0) {
            if (K <= 16)
                beam16_wave(sS, bp, chain, ids, req, B, K, beam, tokens, choice);
            else
                beam_wave(sS, bp, chain, ids, req, B, K, beam, tokens, choice);
        }
        return;
    }
    if (rule != kPathGreedy) {
        float* vb = reinterpret_cast<float*>(reinterpret_cast<char*>(sS) + path_vb_offset(B, K, true));
        const float w = rule == kPathGeometric ? lam : 1.f;
        if ((threadIdx.x >> 6) == 0) {
            if (K <= 16)
                viterbi16_wave(sS, aux, chain, vb, ids, req, B, K, w, tokens, choice);
            else
                viterbi_wave(sS, aux, chain, vb, ids, req, B, K, w, tokens, choice);
        }
        return;
    }
    walk_block(sS, aux, chain, ids, req, B, K, tokens, choice);
}

// A path over precomputed scores, one wave per request.  When the request's
// scores fit (use_lds) they are first copied into LDS with coalesced 16-byte
// loads, all issued before any is used.
__global__ __launch_bounds__(64) void path_kernel(const float* __restrict__ scores, const int32_t* __restrict__ ids,
                                                  int n, int B, int K, int rule, float lam, int beam,
                                                  int32_t* __restrict__ tokens, int32_t* __restrict__ choice,
                                                  int use_lds) {
    extern __shared__ __attribute__((aligned(16))) float sl[];
    const int req = blockIdx.x;
    const int l = lane_id();
    if (req >= n) return;
    const int64_t per = static_cast<int64_t>(B > 1 ? B - 1 : 0) * K * K;
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
        path_from_lds(rule, lam, beam, sl, ids, req, B, K, tokens, choice);
        return;
    }
    if (rule == kPathBeam) {
        int* chain = reinterpret_cast<int*>(reinterpret_cast<char*>(sl) + path_chain_offset(B, K, false));
        uint8_t* bp = reinterpret_cast<uint8_t*>(reinterpret_cast<char*>(sl) + path_beam_offset(B, K, false));
        if (K <= 16)
            beam16_wave(base, bp, chain, ids, req, B, K, beam, tokens, choice);
        else
            beam_wave(base, bp, chain, ids, req, B, K, beam, tokens, choice);
        return;
    }
    if (rule != kPathGreedy) {
        uint8_t* from = reinterpret_cast<uint8_t*>(sl);
        int* chain = reinterpret_cast<int*>(reinterpret_cast<char*>(sl) + path_chain_offset(B, K, false));
        float* vb = reinterpret_cast<float*>(reinterpret_cast<char*>(sl) + path_vb_offset(B, K, false));
        const float w = rule == kPathGeometric ? lam : 1.f;
        if (K <= 16)
            viterbi16_wave(base, from, chain, vb, ids, req, B, K, w, tokens, choice);
        else
            viterbi_wave(base, from, chain, vb, ids, req, B, K, w, tokens, choice);
        return;
    }
    walk_wave(base, ids, req, B, K, tokens, choice);
}

// The cosine scores of one request per workgroup (one wave per job, up to 16):
//   S_p(a,b) = l_{p+1}(b) + sigma * <o_p^a, i_{p+1}^b>
// with the unit vectors o (W_out z) and i (W_in z).  Each wave takes (pair,
// 16 x 16 tile) jobs and forms the tile's dot products on fp32 MFMA
// (v_mfma_f32_16x16x4_f32): lane group g = lane / 16 covers the dvec / 4
// consecutive components g*dvec/4 .. of its rows, one component per step,
// loaded as float4.  The scores go to memory and, when they fit, to LDS; with
// tokens given the request's path follows from LDS.
__global__ __launch_bounds__(1024) void cosine_kernel(CosArgs a, int use_lds) {
    extern __shared__ __attribute__((aligned(16))) float sS[];
    const int req = blockIdx.x;
    const int B = a.B, K = a.K, dv = a.dvec;
    const int KK = K * K;
    const int l = lane_id();
    const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int g = l >> 4, r16 = l & 15;
    const int nt = (K + 15) / 16;
    const int kper = dv / 4;   // dvec is a multiple of 16 and at most 128: kper in {4, 8, ..., 32}
    const int njobs = (B - 1) * nt * nt;
    for (int job = wave; job < njobs; job += nwaves) {
        const int p = job / (nt * nt), ta = (job / nt) % nt, tb = job % nt;
        const int64_t tp = static_cast<int64_t>(req) * B + p, tq = tp + 1;
        const float* orow = a.vout + (tp * K + min(ta * 16 + r16, K - 1)) * dv + g * kper;  // clamped rows unused
        const float* irow = a.vin + (tq * K + min(tb * 16 + r16, K - 1)) * dv + g * kper;
        // every load of the tile is issued before the first MFMA (steps past
        // kper re-read the last four components and are not used)
        float4 o4[8], i4[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = min(4 * u, kper - 4);
            o4[u] = *reinterpret_cast<const float4*>(orow + j);
            i4[u] = *reinterpret_cast<const float4*>(irow + j);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (4 * u >= kper) break;
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].x, i4[u].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].y, i4[u].y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].z, i4[u].z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].w, i4[u].w, acc, 0, 0, 0);
        }
        // lane l holds D[4g + i][r16]: predecessor a = ta*16 + 4g + i, successor b = tb*16 + r16
        const int bb = tb * 16 + r16;
        if (bb < K) {
            const float lb = a.vals[tq * K + bb];
            float* srow = a.scores + (static_cast<int64_t>(req) * (B - 1) + p) * KK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int aa = ta * 16 + 4 * g + i;
                if (aa < K) {
                    const float sv = bb < a.m ? lb + a.sigma * acc[i] : -INFINITY;
                    srow[aa * K + bb] = sv;
                    if (use_lds) sS[p * KK + aa * K + bb] = sv;
                }
            }
        }
    }
    if (!a.tokens || !use_lds) return;
    __syncthreads();
    path_from_lds(a.rule, a.lam, a.beam, sS, a.ids, req, B, K, a.tokens, a.choice);
}

// The Global-Sum, Geometric or beam path of the request's last wave: the
// request's (B - 1) K^2 scores (stored with agent-scope atomics by the pairs'
// waves) into LDS, 64 bits per load, all of a round's loads issued before any
// is used, then the rule as the one-workgroup-per-request kernels run it.
__device__ __forceinline__ void pair_rule(float* sS, const float* scores, int req, int B, int K, int rule, float lam,
                                          int beam, const int32_t* __restrict__ ids, int32_t* __restrict__ tokens,
                                          int32_t* __restrict__ choice) {
    const int l = lane_id();
    const int n2 = (B - 1) * K * K / 2;
    const uint64_t* src2 = reinterpret_cast<const uint64_t*>(scores + static_cast<int64_t>(req) * (B - 1) * K * K);
    uint64_t* s2 = reinterpret_cast<uint64_t*>(sS);
    for (int i0 = 0; i0 < n2; i0 += 32 * kWave) {
        uint64_t t[32];
#pragma unroll
        for (int u = 0; u < 32; ++u)
            t[u] = __hip_atomic_load(src2 + min(i0 + u * kWave + l, n2 - 1), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);   // clamped: in bounds
#pragma unroll
        for (int u = 0; u < 32; ++u)
            if (i0 + u * kWave + l < n2) s2[i0 + u * kWave + l] = t[u];
    }
    wave_lds_sync();
    path_from_lds(rule, lam, beam, sS, ids, req, B, K, tokens, choice);
}

// The cosine scores split by pair (K = 4, 8 or 16), as the MLP's finishing
// step is split: one wave per pair forms its 16 x 16 tile exactly as
// cosine_kernel does (the same loads and fp32 MFMA sequence, then
// l_{p+1}(b) + sigma * dot) and writes it; the request's last wave takes the
// path.  A request's out and in vectors are thus read by B - 1 CUs at once
// instead of one.  kWalk: the prefix-first walk from the rows' argmaxes
// (lane l holds rows 4 (l / 16) + i of column l % 16, so a row's 16 columns
// share a DPP row: four (value, index) reductions, ties to the lower
// column); else the other rules over the scores read back into LDS.
template <bool kWalk>
__global__ __launch_bounds__(64) void cosine_pair_kernel(CosArgs a) {
    extern __shared__ __attribute__((aligned(16))) float sS[];
    const int B = a.B, K = a.K, dv = a.dvec, KK = K * K;
    const int pair = blockIdx.x;
    const int req = pair / (B - 1), p = pair - req * (B - 1);
    const int l = lane_id();
    const int g = l >> 4, r16 = l & 15;
    const int kper = dv / 4;
    const int64_t tp = static_cast<int64_t>(req) * B + p, tq = tp + 1;
    const float* orow = a.vout + (tp * K + min(r16, K - 1)) * dv + g * kper;  // clamped rows unused
    const float* irow = a.vin + (tq * K + min(r16, K - 1)) * dv + g * kper;
    float4 o4[8], i4[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int j = min(4 * u, kper - 4);
        o4[u] = *reinterpret_cast<const float4*>(orow + j);
        i4[u] = *reinterpret_cast<const float4*>(irow + j);
    }
    const float lb = a.vals[tq * K + min(r16, K - 1)];
    // every load lands before the first MFMA (else the compiler sinks each
    // pair of loads behind the break below: eight dependent round trips)
#pragma unroll
    for (int u = 0; u < 8; ++u)
        asm volatile("" ::"v"(o4[u].x), "v"(o4[u].y), "v"(o4[u].z), "v"(o4[u].w), "v"(i4[u].x), "v"(i4[u].y),
                     "v"(i4[u].z), "v"(i4[u].w));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        if (4 * u >= kper) break;
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].x, i4[u].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].y, i4[u].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].z, i4[u].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(o4[u].w, i4[u].w, acc, 0, 0, 0);
    }
    // lane l holds D[4g + i][r16]: predecessor 4g + i, successor r16
    const bool col = r16 < K;
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = r16 < a.m ? lb + a.sigma * acc[i] : -INFINITY;
    float* srow = a.scores + static_cast<int64_t>(pair) * KK;
    if (!kWalk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (col && 4 * g + i < K)
                __hip_atomic_store(reinterpret_cast<uint32_t*>(srow) + (4 * g + i) * K + r16, __float_as_uint(sv[i]),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!pair_last_of_request(a.cnt, req, B)) return;
        pair_rule(sS, a.scores, req, B, K, a.rule, a.lam, a.beam, a.ids, a.tokens, a.choice);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (col && 4 * g + i < K) srow[(4 * g + i) * K + r16] = sv[i];
        float bv = col ? sv[i] : -INFINITY;
        int bi = col ? r16 : 64;
        auto take = [&](float ov, int oi) {
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        };
        take(dpp_f<kDppXor1>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppXor1, 0xF, 0xF, false));
        take(dpp_f<kDppXor2>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppXor2, 0xF, 0xF, false));
        take(dpp_f<kDppHalfMirror>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppHalfMirror, 0xF, 0xF, false));
        take(dpp_f<kDppMirror>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppMirror, 0xF, 0xF, false));
        if (r16 == 0 && 4 * g + i < K)
            __hip_atomic_store(a.best + static_cast<int64_t>(pair) * K + 4 * g + i, bi, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!pair_last_of_request(a.cnt, req, B)) return;
    pair_walk(a.best, req, B, K, a.ids, a.tokens, a.choice);
}

// One workgroup per request: S = l_{p+1}(b) + (sum of the hidden-block partial
// Deltas in block order + b2) for all of the request's pairs, written to
// `scores` (and kept in LDS when it fits); then, with tokens given (only when
// the scores fit LDS), the request's path by the handle's rule.
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
            int bq[4];   // successor of each float4's first element
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
                bq[u] = e % K;
                lv[u] = *reinterpret_cast<const float4*>(vals_req + (p + 1) * K + bq[u]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i4 = i0 + u * 256 + static_cast<int>(threadIdx.x);
                if (i4 < per4) {
                    float4 sv = make_float4(lv[u].x + (d[u].x + b2), lv[u].y + (d[u].y + b2),
                                            lv[u].z + (d[u].z + b2), lv[u].w + (d[u].w + b2));
                    if (a.m < K) {   // successors b >= m are not scored (K % 4 == 0 here)
                        const int b0 = bq[u];
                        sv = make_float4(b0 < a.m ? sv.x : -INFINITY, b0 + 1 < a.m ? sv.y : -INFINITY,
                                         b0 + 2 < a.m ? sv.z : -INFINITY, b0 + 3 < a.m ? sv.w : -INFINITY);
                    }
                    reinterpret_cast<float4*>(scores_req)[i4] = sv;
                    if (use_lds) reinterpret_cast<float4*>(sS)[i4] = sv;
                }
            }
        }
    } else
    // 8 elements per thread per round, all loads issued before any is used
    for (int i0 = 0; i0 < per32; i0 += 8 * 256) {
        float d[8], lv[8];
        int bq[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = min(i0 + u * 256 + static_cast<int>(threadIdx.x), per32 - 1);  // clamped: in bounds
            const int p = idx / KK, e = idx - p * KK;
            d[u] = sum_strided<kMaxMlpBlocks>(part_req + (p * a.nblk) * KK + e, KK, a.nblk);
            bq[u] = e % K;
            lv[u] = vals_req[(p + 1) * K + bq[u]];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int idx = i0 + u * 256 + static_cast<int>(threadIdx.x);
            if (idx < per32) {
                const float sv = bq[u] < a.m ? lv[u] + (d[u] + b2) : -INFINITY;
                scores_req[idx] = sv;
                if (use_lds) sS[idx] = sv;
            }
        }
    }
    if (!a.tokens || !use_lds) return;
    __syncthreads();
    path_from_lds(a.rule, a.lam, a.beam, sS, a.ids, req, B, K, a.tokens, a.choice);
}

// The finishing step split by pair for the Global-Sum, Geometric and beam
// rules (K = 4, 8 or 16): one wave per pair forms its K x K scores exactly as
// finish_kernel does (block partials in block order, + b2, + l_{p+1}(b); with
// the MLP's 16-unit partials (a.sub) first added four at a time in the
// 64-unit form's tree) and stores them with agent-scope atomic stores; the
// last wave of a request to finish (by the request's count, which the MLP
// launch zeroed, one cache line per request) reads the request's scores back
// into LDS (dynamic, path_lds_bytes) and runs the rule there, as
// finish_kernel does.  A request's partials are thus read by B - 1 CUs at
// once instead of one.  (With the prefix-first walk the same per-pair step
// runs inside the MLP's launch.)
__global__ __launch_bounds__(64) void finish_pair_kernel(FinishArgs a) {
    extern __shared__ __attribute__((aligned(16))) float sS[];
    const int B = a.B, K = a.K, KK = K * K;
    const int pair = blockIdx.x;
    const int req = pair / (B - 1);
    const int l = lane_id();
    const PairRow4 r = pair_scores4<false>(a.part, a.nblk, a.sub, a.m, a.vals, a.b2[0], B, K, pair);
    // read back by the request's last wave, on any XCD
    const float4 sv = r.sv;
    uint64_t* dst = reinterpret_cast<uint64_t*>(a.scores + static_cast<int64_t>(pair) * KK) + 2 * l;
    const uint64_t lo = static_cast<uint64_t>(__float_as_uint(sv.x)) | static_cast<uint64_t>(__float_as_uint(sv.y)) << 32;
    const uint64_t hi = static_cast<uint64_t>(__float_as_uint(sv.z)) | static_cast<uint64_t>(__float_as_uint(sv.w)) << 32;
    if (l < r.nv) {
        __hip_atomic_store(dst, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(dst + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!pair_last_of_request(a.cnt, req, B)) return;
    pair_rule(sS, a.scores, req, B, K, a.rule, a.lam, a.beam, a.ids, a.tokens, a.choice);
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

// Dynamic LDS of a path kernel that holds the request's scores (plus its byte
// and chain arrays), or 0 when they do not fit and the path reads memory.
static size_t path_lds_bytes(int B, int K) {
    if (B < 2) return 0;
    const size_t bytes = path_lds_end(B, K, true);
    return bytes <= 60 * 1024 ? bytes : 0;
}

bool path_fits_lds(int B, int K) { return path_lds_bytes(B, K) > 0; }

bool cosine_by_pair(const CosArgs& a) {
    return a.tokens && a.best && a.cnt && (reinterpret_cast<uintptr_t>(a.scores) & 7) == 0 &&
           finish_split(a.B, a.K, a.rule);
}

hipError_t launch_cosine(const CosArgs& a, hipStream_t stream) {
    if (cosine_by_pair(a)) {
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.n) * (a.B - 1)));
        if (a.rule == kPathGreedy) return launch(cosine_pair_kernel<true>, grid, 64, 0, stream, a);
        return launch(cosine_pair_kernel<false>, grid, 64, static_cast<uint32_t>(path_lds_bytes(a.B, a.K)), stream, a);
    }
    const size_t lds = path_lds_bytes(a.B, a.K);
    const int nt = (a.K + 15) / 16;
    const int jobs = (a.B - 1) * nt * nt;
    const int waves = jobs < 1 ? 1 : (jobs > 16 ? 16 : jobs);
    return launch(cosine_kernel, dim3(static_cast<unsigned>(a.n)), 64 * waves, static_cast<uint32_t>(lds), stream,
                  a, lds > 0);
}

hipError_t launch_path(const float* scores, const int32_t* ids, int n, int B, int K, int rule, float lam, int beam,
                       int32_t* tokens, int32_t* choice, hipStream_t stream) {
    const size_t wl = path_lds_bytes(B, K);
    const size_t lds = wl ? wl : path_lds_end(B, K, false);
    return launch(path_kernel, dim3(static_cast<unsigned>(n)), 64, static_cast<uint32_t>(lds), stream, scores,
                  ids, n, B, K, rule, lam, beam, tokens, choice, wl > 0);
}

bool finish_split(int B, int K, int rule) {
    return B > 1 && (K == 4 || K == 8 || K == 16) && (rule == kPathGreedy || path_fits_lds(B, K));
}

bool finish_by_pair(const FinishArgs& a) {
    const bool aligned =
        ((reinterpret_cast<uintptr_t>(a.scores) | reinterpret_cast<uintptr_t>(a.vals) | reinterpret_cast<uintptr_t>(a.part)) &
         15) == 0;
    return a.tokens && a.best && a.cnt && aligned && finish_split(a.B, a.K, a.rule);
}

hipError_t launch_finish(const FinishArgs& a, hipStream_t stream) {
    if (finish_by_pair(a)) {
        // the walk's per-pair step runs inside the MLP's launch (fin_walk)
        if (a.rule == kPathGreedy) return hipErrorInvalidValue;
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.n) * (a.B - 1)));
        return launch(finish_pair_kernel, grid, 64, static_cast<uint32_t>(path_lds_bytes(a.B, a.K)), stream, a);
    }
    if (a.sub) return hipErrorInvalidValue;   // 16-unit partials are finished by pair only
    const size_t lds = path_lds_bytes(a.B, a.K);
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
