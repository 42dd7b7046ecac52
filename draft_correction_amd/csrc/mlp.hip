// Step (4) of the DCOCO method details: the transition scores
//   S_p(a,b) = l_{p+1}(b) + w2 . GELU(W1 [s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)] + b1) + b2
// for every adjacent drafted-slot pair p and candidate pair (a, b).
//
// Layer 1 is evaluated through the exact column-block identity
//   W1 x = (W1_s s_p + b1 + W1_za z_p^a + w_la l_p(a)) + (W1_zb z_{p+1}^b + w_lb l_{p+1}(b))
//        =              P_p[a]                        +            Q_p[b]
// so the K^2 x (3r+2) x h product collapses to per-candidate products
// U = W1_za z and V = W1_zb z, the per-pair c_p = W1_s s_p (float32 dot
// products, a quarter of r per thread), and a K x K broadcast add.  Each
// candidate's U (for the pair it starts) and V (for the pair it ends) over a
// block of hidden units is needed by one workgroup only, so the workgroup
// forms them itself on MFMA, from z as bf16 hi | lo rows (float32
// accuracy), then forms P and Q and runs the epilogue: the GELU over all
// K^2 x h pre-activations and the h -> 1 dot with w2, one (a, b) per thread.
//
// Work is split into (pair, block of 64 hidden units) workgroups; each block
// writes its partial Delta and the finishing kernel adds the blocks in order,
// adds b2 and l_{p+1}(b) and walks.  Every sum runs in a fixed order with no
// atomics: bit-reproducible.
#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

// GELU(x) = x Phi(x) = max(x, 0) - t Phi(-t), t = |x|, with Phi(-t) from
// Abramowitz & Stegun 26.2.16: Phi(-t) = phi(t) (a1 k + a2 k^2 + a3 k^3),
// k = 1 / (1 + p t), p = 0.33267, |error| < 1e-5.  Two exact rewrites
// shorten it:
//   * t k = (1 - k) / p, so t Phi(-t) = exp(-t^2/2) R(k) with the cubic
//     R(k) = (1 - k)(a1 + a2 k + a3 k^2) / (p sqrt(2 pi));
//   * with y = alpha x, alpha = sqrt(log2(e) / 2), exp(-x^2/2) = 2^(-y^2) and
//     alpha GELU(x) = max(y, 0) - 2^(-y^2) alpha R(k), k = 1 / (1 + (p/alpha)|y|).
// The kernel keeps P and Q (so x) scaled by alpha and w2 scaled by 1/alpha,
// so w2 . GELU(x) = (w2/alpha) . gelu_scaled(alpha x).  Evaluated in float32
// this is within 2.7e-5 of the exact erf form on [-12, 12] (11 vector
// instructions per evaluation with the add of P and Q and the w2 multiply-add).
constexpr float kGeluAlpha = 0.849321800f;      // sqrt(log2(e) / 2)
__device__ __forceinline__ float gelu_scaled(float y) {
    const float t = fabsf(y);
    const float k = __builtin_amdgcn_rcpf(fmaf(0.391688992f, t, 1.0f));  // p / alpha
    float r = fmaf(k, -0.954654864f, 1.07704772f);   // alpha R(k), Horner from k^3
    r = fmaf(k, r, -0.566653699f);
    r = fmaf(k, r, 0.444260838f);
    const float e = __builtin_amdgcn_exp2f(-(y * y));
    return fmaf(-e, r, fmaxf(y, 0.0f));
}

// Hidden units of one block (a multiple of 16).
constexpr int kJB = 64;
static_assert(256 / kJB <= kMaxMlpBlocks, "the finishing kernel sums at most kMaxMlpBlocks blocks");
constexpr int kPS = kJB + 4;        // LDS row stride of P / Q (floats)
// Workgroups of one launch, at most: one per CU, each running a contiguous
// share of the pairs of one block of hidden units.
constexpr int kMlpGrid = 256;

typedef __attribute__((address_space(3))) void* mlp_lds_ptr;
typedef __attribute__((address_space(1))) void* mlp_global_ptr;

// A staged z row holds its 2r bf16 values unpadded; segment s (16 bytes) of
// row a sits at position s ^ (a & mask), mask = min(7, segments - 1), so the
// eight rows one fragment read touches at a time sit in distinct banks
// (r >= 32) while every segment stays inside its row.
template <int ZSEG>
__device__ __forceinline__ int zpos(int a, int s) { return s ^ (a & (ZSEG < 8 ? ZSEG - 1 : 7)); }

// Shapes of one instance: K <= 16 KT candidates, NT threads, chunks of at
// most C pairs (their z rows, P, Q and results fill the LDS).
template <int R, int KT>
struct MlpShape {
    static constexpr int NT = KT == 1 ? 1024 : 512;
    static constexpr int KMAX = 16 * KT;
    static constexpr int C = KT == 1 ? 7 : (KT == 2 ? 3 : 1);
};

// The transition MLP for K > 16.  The G workgroups form nj equal groups, one per block
// of 64 hidden units; workgroup w of group jb = w / (G / nj) takes a
// contiguous run of the pairs, in chunks of at most C consecutive pairs of
// one request (slots t0 .. t0 + np).  For each chunk:
//   1. the z rows of the np + 1 slots (bf16 [hi | lo], float32 accuracy),
//      the pair states and the slots' logits go straight into LDS;
//   2. c_p[j] = W1_s[j] s_p for every pair (float32 dots, an eighth of r
//      per thread), then on MFMA U[a][j] = W1_za[j] z_p^a (waves with
//      (w / 4) even) and V[b][j] = W1_zb[j] z_{p+1}^b (odd), each wave one
//      16-unit column tile, the pairs split between the groups of eight
//      waves, and from them
//        P[a][j] = c_p[j] + b1[j] + w_la[j] l_p(a) + U[a][j]
//        Q[b][j] = w_lb[j] l_{p+1}(b) + V[b][j];
//   3. GELU(P[a] + Q[b]) and the dot with w2 over the block for every pair
//      and K x m candidate pairs (successors b < m), eight threads per
//      (a, b, b + 1), each over 8 units, their sums added in a fixed order;
//   4. the partial Deltas go to part[pair][block][a][b] and the finishing
//      kernel adds the blocks in order.
template <int R, int KT>
__global__ __launch_bounds__((MlpShape<R, KT>::NT), 1) void mlp_chunk_kernel(MlpArgs a) {
    using S = MlpShape<R, KT>;
    constexpr int NT = S::NT, KMAX = S::KMAX, C = S::C;
    constexpr int KS = 2 * R / 32;              // 32-wide k-steps over [hi | lo]
    constexpr int KD = R >= 32 ? R / 32 : 1;    // distinct W1 fragments (hi and lo share them)
    constexpr int ZSEG = 2 * R / 8;             // 16-byte segments per z row
    constexpr int NW = NT / 64;                 // waves
    static_assert(NW >= 8, "two groups of four column-tile waves");
    // z rows of the chunk's slots, then P and Q of its pairs, then results
    __shared__ __attribute__((aligned(16))) uint16_t zbuf[(C + 1) * KMAX * 2 * R];
    __shared__ __attribute__((aligned(16))) float pq[C * 2 * KMAX * kPS];
    __shared__ __attribute__((aligned(16))) float res[C * KMAX * KMAX];
    __shared__ __attribute__((aligned(16))) float sp[C * R];
    __shared__ __attribute__((aligned(16))) float lv[(C + 1) * KMAX];
    __shared__ __attribute__((aligned(16))) float w2s[kJB];
    __shared__ float cps[C][8][kJB];

    const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
    const int B = a.B, K = a.K, h = a.h;
    const int nj = (h + kJB - 1) / kJB;
    const int P = a.n * (B - 1);
    // this workgroup's block and run of pairs [q_lo, q_hi) (pairs per call < 2^24)
    const int per = gridDim.x / nj;             // workgroups per block
    const int jb = blockIdx.x / per, wi = blockIdx.x - jb * per;
    const int q_lo = static_cast<int>(static_cast<int64_t>(wi) * P / per);
    const int q_hi = static_cast<int>(static_cast<int64_t>(wi + 1) * P / per);
    if (jb >= nj || q_lo >= q_hi) return;
    const int j0 = jb * kJB, jn = min(kJB, h - j0);
    const int ms = a.m;
    const int mh = (ms + 1) / 2;
    const int TP = K * mh * 8;                  // GELU tasks per pair
    const int nin = 3 * R + 2;

    // ---- the block's W1 slices in registers, for the whole run:
    //   MFMA waves: wave w takes column tile g = w % 4 (units 16 g .. 16 g + 15)
    //   of U (w / 4 even) or V (odd), for the pairs i with i % NG == w / 8
    //   (NG groups of eight waves)
    constexpr int NG = NW / 8;
    const int g = wave & 3;
    const bool isu = ((wave >> 2) & 1) == 0;
    const int ph = wave >> 3;
    const bool mfma_wave = 16 * g < jn;
    const int jl = min(16 * g + (l & 15), jn - 1);   // the lane's unit (clamped: not stored)
    u32x4 bw[KD];
    {
        const uint16_t* wr = a.w1 + static_cast<int64_t>(j0 + jl) * nin + (isu ? R : 2 * R);
        const int kq = 8 * (l >> 4);
#pragma unroll
        for (int d = 0; d < KD; ++d) bw[d] = load16(wr + ((d * 32 + kq) % R));
    }
    const float wl = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + jl) * nin + 3 * R + (isu ? 0 : 1)]);
    const float b1j = a.b1[j0 + jl];
    // c_p: thread (unit jj, eighth e8 of r, pair parity cq) dots W1_s row
    // j0 + jj with s_p over columns e8 R/8 .. e8 R/8 + R/8 - 1, read as
    // 32-bit words of two columns
    const int jj = tid & (kJB - 1), e8 = (tid >> 6) & 7, cq = tid >> 9;
    constexpr int NCQ = NT / 512;               // pair parities of the c_p threads
    uint32_t ws[R / 16];
    {
        const uint32_t* wsr = reinterpret_cast<const uint32_t*>(a.w1 + static_cast<int64_t>(j0 + min(jj, jn - 1)) * nin +
                                                                e8 * (R / 8));
#pragma unroll
        for (int q = 0; q < R / 16; ++q) ws[q] = wsr[q];
    }
    if (tid < kJB) w2s[tid] = tid < jn ? a.w2[j0 + tid] * (1.0f / kGeluAlpha) : 0.f;   // see gelu_scaled

    for (int c0 = q_lo; c0 < q_hi;) {
        // the chunk: pairs c0 .. c0 + np - 1 of one request, slots t0 .. t0 + np
        const int req = c0 / (B - 1), p0 = c0 - req * (B - 1);
        const int np = min(min(C, q_hi - c0), B - 1 - p0);
        const int64_t t0 = static_cast<int64_t>(req) * B + p0;
        // ---- 1. direct loads into LDS: each wave instruction fills 64
        // consecutive 16-byte (or 4-byte) positions; lanes past the end take
        // no part
        {
            const uint16_t* zsrc = a.zhl + t0 * K * (2 * R);
            const int nseg = (np + 1) * K * ZSEG;
            for (int s0 = wave * 64; s0 < nseg; s0 += NT) {
                const int sg = s0 + l;
                if (sg < nseg) {
                    const int row = sg / ZSEG, pos = sg - row * ZSEG;
                    __builtin_amdgcn_global_load_lds((mlp_global_ptr)(zsrc + row * (2 * R) + zpos<ZSEG>(row, pos) * 8),
                                                     (mlp_lds_ptr)(zbuf + s0 * 8), 16, 0, 0);
                }
            }
            const int nsp = np * (R / 4);       // pair states: consecutive pairs are contiguous
            for (int s0 = wave * 64; s0 < nsp; s0 += NT)
                if (s0 + l < nsp)
                    __builtin_amdgcn_global_load_lds(
                        (mlp_global_ptr)(a.s + static_cast<int64_t>(c0) * R + 4 * (s0 + l)), (mlp_lds_ptr)(sp + 4 * s0),
                        16, 0, 0);
            const int nl = (np + 1) * K;        // the slots' logits
            for (int s0 = wave * 64; s0 < nl; s0 += NT)
                if (s0 + l < nl)
                    __builtin_amdgcn_global_load_lds((mlp_global_ptr)(a.vals + t0 * K + s0 + l), (mlp_lds_ptr)(lv + s0),
                                                     4, 0, 0);
        }
        __syncthreads();   // every load has landed (and the previous chunk's results are stored)

        // ---- 2. c_p partial dots of every pair, column order
        for (int i = cq; i < np; i += NCQ) {
            float c = 0.f;
#pragma unroll
            for (int q = 0; q < R / 16; ++q) {
                const float2 sv = *reinterpret_cast<const float2*>(&sp[i * R + e8 * (R / 8) + 2 * q]);
                c = fmaf(__uint_as_float(ws[q] << 16), sv.x, c);
                c = fmaf(__uint_as_float(ws[q] & 0xFFFF0000u), sv.y, c);
            }
            cps[i][e8][jj] = c;
        }
        __syncthreads();
        // U | V column tiles (lane l holds rows 4 (l / 16) + e, unit 16 g + l % 16)
        // and P | Q from them, kept scaled by alpha (see gelu_scaled)
        if (mfma_wave) {
            const int kq = 8 * (l >> 4);
            const int jc = 16 * g + (l & 15);
            for (int i = ph; i < np; i += NG) {
                float cp = 0.f;
                if (isu)
                    cp = (((cps[i][0][jl] + cps[i][1][jl]) + (cps[i][2][jl] + cps[i][3][jl])) +
                          ((cps[i][4][jl] + cps[i][5][jl]) + (cps[i][6][jl] + cps[i][7][jl]))) + b1j;
                const int slot = isu ? i : i + 1;
                const int dst = (2 * i + (isu ? 0 : 1)) * KMAX * kPS;
#pragma unroll
                for (int rt = 0; rt < KT; ++rt) {
                    if (rt * 16 >= K) break;
                    // fragment rows past K repeat row K - 1 (not stored)
                    const int ar = slot * K + min(rt * 16 + (l & 15), K - 1);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int sgi = (ks * 32 + kq) / 8;
                        const u32x4 zf = *reinterpret_cast<const u32x4*>(&zbuf[(ar * ZSEG + zpos<ZSEG>(ar, sgi)) * 8]);
                        acc = mfma16x16x32(zf, bw[ks % KD], acc);
                    }
                    if (jc < jn) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int m = rt * 16 + 4 * (l >> 4) + e;
                            if (m < K) {
                                constexpr float al = kGeluAlpha;
                                const float lm = lv[slot * K + m];
                                pq[dst + static_cast<int>(__umul24(m, kPS)) + jc] =
                                    isu ? al * (cp + fmaf(wl, lm, acc[e])) : al * fmaf(wl, lm, acc[e]);
                            }
                        }
                    }
                }
            }
        }
        __syncthreads();

        // ---- 3. GELU and the dot with w2: task t is (pair i, predecessor a,
        // successors b and b + 1, eighth t % 8 of the block's units); the
        // eight partial sums meet in a fixed order within each aligned group
        // of eight lanes.  (24-bit products for the small index arithmetic:
        // the 64-bit multiply-add the compiler otherwise picks reads a
        // second, unrelated register.)
        const int T = np * TP;
#pragma unroll 1
        for (int t = tid; t < T; t += NT) {
            const int i = t / TP, r8 = t - static_cast<int>(__umul24(i, TP));
            const int q = r8 & 7, rest = r8 >> 3;
            const int aa = rest / mh, bb = 2 * (rest - static_cast<int>(__umul24(aa, mh)));
            const bool two = bb + 1 < ms;
            const int j = 8 * q;
            float d0 = 0.f, d1 = 0.f, e0 = 0.f, e1 = 0.f;
            if (j < jn) {
                const int pb = static_cast<int>(__umul24(2 * i, KMAX * kPS));
                const int pr = pb + static_cast<int>(__umul24(aa, kPS)) + j;
                const int qr = pb + static_cast<int>(__umul24(KMAX + bb, kPS)) + j;
                const int qs = qr + (two ? kPS : 0);
                const float4 pv0 = *reinterpret_cast<const float4*>(&pq[pr]);
                const float4 pv1 = *reinterpret_cast<const float4*>(&pq[pr + 4]);
                const float4 wv0 = *reinterpret_cast<const float4*>(&w2s[j]);
                const float4 wv1 = *reinterpret_cast<const float4*>(&w2s[j + 4]);
                const float4 qv0 = *reinterpret_cast<const float4*>(&pq[qr]);
                const float4 qv1 = *reinterpret_cast<const float4*>(&pq[qr + 4]);
                const float4 sv0 = *reinterpret_cast<const float4*>(&pq[qs]);
                const float4 sv1 = *reinterpret_cast<const float4*>(&pq[qs + 4]);
                d0 = fmaf(wv0.x, gelu_scaled(pv0.x + qv0.x), d0);
                d1 = fmaf(wv0.y, gelu_scaled(pv0.y + qv0.y), d1);
                d0 = fmaf(wv0.z, gelu_scaled(pv0.z + qv0.z), d0);
                d1 = fmaf(wv0.w, gelu_scaled(pv0.w + qv0.w), d1);
                d0 = fmaf(wv1.x, gelu_scaled(pv1.x + qv1.x), d0);
                d1 = fmaf(wv1.y, gelu_scaled(pv1.y + qv1.y), d1);
                d0 = fmaf(wv1.z, gelu_scaled(pv1.z + qv1.z), d0);
                d1 = fmaf(wv1.w, gelu_scaled(pv1.w + qv1.w), d1);
                e0 = fmaf(wv0.x, gelu_scaled(pv0.x + sv0.x), e0);
                e1 = fmaf(wv0.y, gelu_scaled(pv0.y + sv0.y), e1);
                e0 = fmaf(wv0.z, gelu_scaled(pv0.z + sv0.z), e0);
                e1 = fmaf(wv0.w, gelu_scaled(pv0.w + sv0.w), e1);
                e0 = fmaf(wv1.x, gelu_scaled(pv1.x + sv1.x), e0);
                e1 = fmaf(wv1.y, gelu_scaled(pv1.y + sv1.y), e1);
                e0 = fmaf(wv1.z, gelu_scaled(pv1.z + sv1.z), e0);
                e1 = fmaf(wv1.w, gelu_scaled(pv1.w + sv1.w), e1);
            }
            float v = d0 + d1, w = e0 + e1;
            v += dpp_f<kDppXor1>(v);
            w += dpp_f<kDppXor1>(w);
            v += dpp_f<kDppXor2>(v);
            w += dpp_f<kDppXor2>(w);
            v += dpp_f<kDppHalfMirror>(v);
            w += dpp_f<kDppHalfMirror>(w);
            if (q == 0) {
                const int o = static_cast<int>(__umul24(i, KMAX * KMAX)) + static_cast<int>(__umul24(aa, K)) + bb;
                res[o] = v;
                if (two) res[o + 1] = w;
            }
        }
        __syncthreads();
        // ---- 4. the chunk's partial Deltas, each pair's K x K contiguous
        for (int e = tid; e < np * K * K; e += NT) {
            const int i = e / (K * K), r = e - i * K * K;
            if (r % K < ms)
                a.part[(static_cast<int64_t>(c0 + i) * nj + jb) * K * K + r] = res[i * KMAX * KMAX + r];
        }
        c0 += np;
    }
}

// ------------------------------------------------------------- K <= 16 --
// The transition MLP for K <= 16, with a workgroup's waves split by role.
// Work assignment and arithmetic are those of mlp_chunk_kernel (nj equal
// groups of workgroups, one per block of 64 hidden units, each a contiguous
// run of pairs), but the run is streamed one pair at a time:
//   - waves 12-15 (producers) load the next pair's z rows, pair state and
//     logits into registers (coalesced 16-byte loads) while they finish the
//     current one, write them to LDS, form c_p and the U | V tiles (each
//     producer wave one 16-unit column tile of both, its lanes splitting
//     the c_p dots of the tile's units in quarters of r) and write P | Q
//     into one of kRing LDS buffers;
//   - waves 0-11 (consumers) run each pair's GELU loop as soon as its buffer
//     is ready and store its partial Deltas.
// The two sides meet through LDS counters (the generation written into a
// buffer, and how many consumer waves are done with it), so the loads and
// matrix products of later pairs overlap the vector-ALU work of earlier
// ones.  No workgroup barrier is used after the roles split; every wait on
// a counter is bounded (kSpinLimit sleeps), so the workgroup always ends.
constexpr int kRing = 3;            // P | Q buffers
constexpr int kProd = 4;            // producer waves
constexpr int kCons = 12;           // consumer waves
constexpr int kWsThreads = 64 * (kProd + kCons);
constexpr unsigned kSpinLimit = 1u << 22;

// Waits until the LDS counter reaches `target` (counters only grow).  The
// pointer is typed as LDS so the poll is a ds_read, not a flat load (which
// would also wait for every global load of the wave).
typedef __attribute__((address_space(3))) volatile int lds_counter;
__device__ __forceinline__ void spin_until(lds_counter* c, int target) {
    for (unsigned n = 0; n < kSpinLimit && *c < target; ++n) __builtin_amdgcn_s_sleep(1);
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ lds_counter* as_lds(int* p) { return (lds_counter*)(p); }

template <int R>
__global__ __launch_bounds__(kWsThreads, 1) void mlp_ws_kernel(MlpArgs a) {
    constexpr int KMAX = 16;
    constexpr int KS = 2 * R / 32;              // 32-wide k-steps over [hi | lo]
    constexpr int ZSEG = 2 * R / 8;             // 16-byte segments per z row
    constexpr int PT = 64 * kProd;              // producer threads
    constexpr int ZPT = (2 * KMAX * ZSEG + PT - 1) / PT;   // z segments per producer thread, at most
    constexpr int PQ = 2 * KMAX * kPS;          // floats of one P | Q buffer
    static_assert(2 * KMAX <= PT && R / 4 <= PT, "one logit and one s_p segment per producer thread");
    __shared__ __attribute__((aligned(16))) uint16_t zbuf[2 * KMAX * 2 * R];
    __shared__ __attribute__((aligned(16))) float ring[kRing * PQ];
    __shared__ __attribute__((aligned(16))) float sp[R];
    __shared__ float lv[2 * KMAX];
    __shared__ __attribute__((aligned(16))) float w2s[kJB];
    // the block's W1_s rows as 32-bit words of two columns, rows padded
    constexpr int WSW = R / 2 + 4;
    __shared__ __attribute__((aligned(16))) uint32_t wsl[kJB * WSW];
    // the block's W1_za and W1_zb rows (bf16), rows padded by 16 bytes
    constexpr int WZ = R + 8;
    __shared__ __attribute__((aligned(16))) uint16_t wza[kJB * WZ];
    __shared__ __attribute__((aligned(16))) uint16_t wzb[kJB * WZ];
    __shared__ int ready[kRing];                // generation (unit index + 1) of each buffer's contents
    __shared__ int freed[kRing];                // consumer waves done with each buffer, cumulative
    __shared__ int pbar;                        // producer-wave barrier count

    const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
    const int B = a.B, K = a.K, h = a.h;
    const int nj = (h + kJB - 1) / kJB;
    const int P = a.n * (B - 1);
    const int per = gridDim.x / nj;
    const int jb = blockIdx.x / per, wi = blockIdx.x - jb * per;
    const int q_lo = static_cast<int>(static_cast<int64_t>(wi) * P / per);
    const int q_hi = static_cast<int>(static_cast<int64_t>(wi + 1) * P / per);
    if (jb >= nj || q_lo >= q_hi) return;
    const int n = q_hi - q_lo;
    const int j0 = jb * kJB, jn = min(kJB, h - j0);
    const int nin = 3 * R + 2;

    // a pair's coordinates (pair number, slot row of its predecessor), stepped
    struct Coord {
        int pair, p, t0;
    };
    auto first = [&](int pair) {
        Coord c;
        c.pair = pair;
        const int req = pair / (B - 1);
        c.p = pair - req * (B - 1);
        c.t0 = req * B + c.p;
        return c;
    };
    auto step = [&](Coord c) {
        ++c.pair;
        ++c.p;
        ++c.t0;
        if (c.p == B - 1) {
            c.p = 0;
            ++c.t0;
        }
        return c;
    };
    // the producers' registers for the next pair's z rows (2K contiguous
    // rows of zhl), pair state and logits; the first pair's loads are issued
    // before the block's weights are staged, so the two latencies overlap
    const int pt = tid - 64 * kCons;            // producer thread 0 .. PT - 1 (negative: consumer)
    const int nseg = 2 * K * ZSEG;
    u32x4 zr[ZPT];
    float4 spr;
    float lvr;
    auto fetch = [&](const Coord& c) {
        const uint16_t* zsrc = a.zhl + static_cast<int64_t>(c.t0) * K * (2 * R);
#pragma unroll
        for (int i = 0; i < ZPT; ++i) zr[i] = load16(zsrc + min(pt + i * PT, nseg - 1) * 8);   // clamped: not written
        spr = *reinterpret_cast<const float4*>(a.s + static_cast<int64_t>(c.pair) * R + 4 * min(pt, R / 4 - 1));
        lvr = a.vals[static_cast<int64_t>(c.t0) * K + min(pt, 2 * K - 1)];
    };
    if (wave >= kCons) fetch(first(q_lo));

    if (tid < kJB) w2s[tid] = tid < jn ? a.w2[j0 + tid] * (1.0f / kGeluAlpha) : 0.f;   // see gelu_scaled
    for (int idx = tid; idx < kJB * (R / 2); idx += kWsThreads) {
        const int jj = idx / (R / 2), w = idx - jj * (R / 2);
        wsl[jj * WSW + w] =
            reinterpret_cast<const uint32_t*>(a.w1 + static_cast<int64_t>(j0 + min(jj, jn - 1)) * nin)[w];
    }
    for (int idx = tid; idx < kJB * (R / 8); idx += kWsThreads) {   // 16-byte pieces
        const int jj = idx / (R / 8), w = idx - jj * (R / 8);
        const uint16_t* row = a.w1 + static_cast<int64_t>(j0 + min(jj, jn - 1)) * nin;
        *reinterpret_cast<u32x4*>(&wza[jj * WZ + 8 * w]) = load16(row + R + 8 * w);
        *reinterpret_cast<u32x4*>(&wzb[jj * WZ + 8 * w]) = load16(row + 2 * R + 8 * w);
    }
    if (tid < kRing) {
        ready[tid] = 0;
        freed[tid] = 0;
    }
    if (tid == 0) pbar = 0;
    __syncthreads();

    if (wave >= kCons) {
        // ================================================= producers ==
        // The producer waves issue ahead of the consumer waves that share
        // their SIMDs, so the chain of loads, products and barriers that
        // feeds the ring is not slowed to a quarter of the issue rate.
        __builtin_amdgcn_s_setprio(3);
        const int pw = pt >> 6;                 // producer wave: column tile 16 pw .. 16 pw + 15
        int gen = 0;                            // producer barriers passed
        auto pbarrier = [&]() {
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
            asm volatile("" ::: "memory");
            ++gen;
            if (l == 0) atomicAdd(&pbar, 1);
            spin_until(as_lds(&pbar), kProd * gen);
        };
        // the block's W1 slices: U and V fragments of the wave's 16 units,
        // and for c_p (thread: unit pt % 64, quarter pt / 64 of r) W1_s words
        const bool tile_on = 16 * pw < jn;
        const int jl = min(16 * pw + (l & 15), jn - 1);
        const float wla = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + jl) * nin + 3 * R]);
        const float wlb = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + jl) * nin + 3 * R + 1]);
        const float b1j = a.b1[j0 + jl];
        Coord c = first(q_lo);
        for (int u = 0; u < n; ++u) {
            const int slot = u % kRing;
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this pair's loads have landed
#pragma unroll
            for (int i = 0; i < ZPT; ++i) {
                const int sg = pt + i * PT;
                if (sg < nseg) {
                    const int row = sg / ZSEG, pos = sg - row * ZSEG;
                    *reinterpret_cast<u32x4*>(&zbuf[(row * ZSEG + zpos<ZSEG>(row, pos)) * 8]) = zr[i];
                }
            }
            if (pt < R / 4) *reinterpret_cast<float4*>(&sp[4 * pt]) = spr;
            if (pt < 2 * K) lv[pt] = lvr;
            pbarrier();                           // z rows, s_p and logits in LDS
            if (u + 1 < n) {
                c = step(c);
                fetch(c);
            }
            // c_p of the lane's unit 16 pw + l % 16 (zero past jn is not
            // stored): a quarter l / 16 of r per lane, column order, then the
            // four quarters added in a fixed order across lanes l, l ^ 16,
            // l ^ 32, l ^ 48 (every lane gets the same sum)
            float cp;
            {
                constexpr int WQ = R / 8;           // words of a quarter of r
                const int e4 = l >> 4;
                uint32_t wv[WQ];
                if constexpr (WQ % 4 == 0) {
#pragma unroll
                    for (int q4 = 0; q4 < WQ / 4; ++q4) {
                        const u32x4 w4 = *reinterpret_cast<const u32x4*>(&wsl[jl * WSW + e4 * WQ + 4 * q4]);
#pragma unroll
                        for (int q = 0; q < 4; ++q) wv[4 * q4 + q] = w4[q];
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < WQ; ++q) wv[q] = wsl[jl * WSW + e4 * WQ + q];
                }
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < WQ; ++q) {
                    const float2 sv = *reinterpret_cast<const float2*>(&sp[e4 * (R / 4) + 2 * q]);
                    acc = fmaf(__uint_as_float(wv[q] << 16), sv.x, acc);
                    acc = fmaf(__uint_as_float(wv[q] & 0xFFFF0000u), sv.y, acc);
                }
                acc += __shfl_xor(acc, 16, 64);
                acc += __shfl_xor(acc, 32, 64);
                cp = acc + b1j;
            }
            // U (slot 0 rows) and V (slot 1 rows) of the wave's column tile;
            // fragment rows past K repeat row K - 1 (not stored)
            f32x4 au = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
            if (tile_on) {
                const int kq = 8 * (l >> 4);
                const int ra = min(l & 15, K - 1), rb = K + ra;
                const int wrow = (16 * pw + (l & 15)) * WZ;   // the lane's unit (rows past jn are not stored)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int sgi = (ks * 32 + kq) / 8;
                    const int wcol = (ks * 32 + kq) % R;       // the hi and lo halves meet the same columns
                    const u32x4 za = *reinterpret_cast<const u32x4*>(&zbuf[(ra * ZSEG + zpos<ZSEG>(ra, sgi)) * 8]);
                    const u32x4 zb = *reinterpret_cast<const u32x4*>(&zbuf[(rb * ZSEG + zpos<ZSEG>(rb, sgi)) * 8]);
                    const u32x4 bu = *reinterpret_cast<const u32x4*>(&wza[wrow + wcol]);
                    const u32x4 bv = *reinterpret_cast<const u32x4*>(&wzb[wrow + wcol]);
                    au = mfma16x16x32(za, bu, au);
                    av = mfma16x16x32(zb, bv, av);
                }
            }
            // the buffer is free once every consumer wave is done with its
            // previous contents (pair u - kRing)
            spin_until(as_lds(&freed[slot]), kCons * (u / kRing));
            // P and Q, kept scaled by alpha (see gelu_scaled)
            const int jc = 16 * pw + (l & 15);
            if (tile_on && jc < jn) {
                float* buf = ring + slot * PQ;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = 4 * (l >> 4) + e;
                    if (m < K) {
                        constexpr float al = kGeluAlpha;
                        buf[static_cast<int>(__umul24(m, kPS)) + jc] = al * (cp + fmaf(wla, lv[m], au[e]));
                        buf[static_cast<int>(__umul24(KMAX + m, kPS)) + jc] = al * fmaf(wlb, lv[K + m], av[e]);
                    }
                }
            }
            pbarrier();                           // P | Q written and z rows read by every producer wave
            if (pt == 0) *as_lds(&ready[slot]) = u + 1;
        }
    } else {
        // ================================================= consumers ==
        // task t of a pair: (predecessor a, successors b and b + 1, eighth
        // t % 8 of the block's units); the eight partial sums meet in a fixed
        // order within each aligned group of eight lanes.  (24-bit products
        // for the small index arithmetic: the 64-bit multiply-add the
        // compiler otherwise picks reads a second, unrelated register.)
        const int ms = a.m;
        const int mh = (ms + 1) / 2;
        const int T = K * mh * 8;               // at most 16 * 8 * 8 = 1024: two tasks per thread
        constexpr int CT = 64 * kCons;
        static_assert(2 * CT >= KMAX * (KMAX / 2) * 8, "two tasks per consumer thread");
        // the thread's tasks, decoded once: LDS offsets of its P row, Q rows
        // and w2, and its output offset (o < 0: no task)
        int tpr[2], tqr[2], tqs[2], tj[2], to[2];
        bool ttwo[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int t = tid + k * CT;
            const int q = t & 7, rest = t >> 3;
            const int aa = rest / mh, bb = 2 * (rest - static_cast<int>(__umul24(aa, mh)));
            ttwo[k] = bb + 1 < ms;
            tj[k] = 8 * q;
            tpr[k] = static_cast<int>(__umul24(aa, kPS)) + tj[k];
            tqr[k] = static_cast<int>(__umul24(KMAX + bb, kPS)) + tj[k];
            tqs[k] = tqr[k] + (ttwo[k] ? kPS : 0);
            to[k] = t < T ? (q == 0 ? static_cast<int>(__umul24(aa, K)) + bb : 1 << 30) : -1;
        }
        Coord c = first(q_lo);
        for (int u = 0; u < n; ++u) {
            const int slot = u % kRing;
            spin_until(as_lds(&ready[slot]), u + 1);
            const float* buf = ring + slot * PQ;
            float* out = a.part + (static_cast<int64_t>(c.pair) * nj + jb) * K * K;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                if (to[k] < 0) break;   // uniform over each aligned group of eight lanes (T % 8 == 0)
                const bool two = ttwo[k];
                const int j = tj[k];
                float d0 = 0.f, d1 = 0.f, e0 = 0.f, e1 = 0.f;
                if (j < jn) {
                    const int pr = tpr[k], qr = tqr[k], qs = tqs[k];
                    const float4 pv0 = *reinterpret_cast<const float4*>(&buf[pr]);
                    const float4 pv1 = *reinterpret_cast<const float4*>(&buf[pr + 4]);
                    const float4 wv0 = *reinterpret_cast<const float4*>(&w2s[j]);
                    const float4 wv1 = *reinterpret_cast<const float4*>(&w2s[j + 4]);
                    const float4 qv0 = *reinterpret_cast<const float4*>(&buf[qr]);
                    const float4 qv1 = *reinterpret_cast<const float4*>(&buf[qr + 4]);
                    const float4 sv0 = *reinterpret_cast<const float4*>(&buf[qs]);
                    const float4 sv1 = *reinterpret_cast<const float4*>(&buf[qs + 4]);
                    d0 = fmaf(wv0.x, gelu_scaled(pv0.x + qv0.x), d0);
                    d1 = fmaf(wv0.y, gelu_scaled(pv0.y + qv0.y), d1);
                    d0 = fmaf(wv0.z, gelu_scaled(pv0.z + qv0.z), d0);
                    d1 = fmaf(wv0.w, gelu_scaled(pv0.w + qv0.w), d1);
                    d0 = fmaf(wv1.x, gelu_scaled(pv1.x + qv1.x), d0);
                    d1 = fmaf(wv1.y, gelu_scaled(pv1.y + qv1.y), d1);
                    d0 = fmaf(wv1.z, gelu_scaled(pv1.z + qv1.z), d0);
                    d1 = fmaf(wv1.w, gelu_scaled(pv1.w + qv1.w), d1);
                    e0 = fmaf(wv0.x, gelu_scaled(pv0.x + sv0.x), e0);
                    e1 = fmaf(wv0.y, gelu_scaled(pv0.y + sv0.y), e1);
                    e0 = fmaf(wv0.z, gelu_scaled(pv0.z + sv0.z), e0);
                    e1 = fmaf(wv0.w, gelu_scaled(pv0.w + sv0.w), e1);
                    e0 = fmaf(wv1.x, gelu_scaled(pv1.x + sv1.x), e0);
                    e1 = fmaf(wv1.y, gelu_scaled(pv1.y + sv1.y), e1);
                    e0 = fmaf(wv1.z, gelu_scaled(pv1.z + sv1.z), e0);
                    e1 = fmaf(wv1.w, gelu_scaled(pv1.w + sv1.w), e1);
                }
                float v = d0 + d1, w = e0 + e1;
                v += dpp_f<kDppXor1>(v);
                w += dpp_f<kDppXor1>(w);
                v += dpp_f<kDppXor2>(v);
                w += dpp_f<kDppXor2>(w);
                v += dpp_f<kDppHalfMirror>(v);
                w += dpp_f<kDppHalfMirror>(w);
                if (to[k] < (1 << 30)) {   // the group's first lane stores
                    out[to[k]] = v;
                    if (two) out[to[k] + 1] = w;
                }
            }
            // this wave is done reading the buffer
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            asm volatile("" ::: "memory");
            if (l == 0) atomicAdd(&freed[slot], 1);
            c = step(c);
        }
    }
}

}  // namespace

int mlp_blocks(int h) { return (h + kJB - 1) / kJB; }

template <int R>
hipError_t launch_mlp_r(const MlpArgs& a, dim3 grid, hipStream_t stream) {
    if (a.K <= 16) return launch(mlp_ws_kernel<R>, grid, kWsThreads, 0, stream, a);
    if (a.K <= 32) return launch(mlp_chunk_kernel<R, 2>, grid, MlpShape<R, 2>::NT, 0, stream, a);
    return launch(mlp_chunk_kernel<R, 4>, grid, MlpShape<R, 4>::NT, 0, stream, a);
}

hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream) {
    if (a.B < 2 || a.n < 1) return hipSuccess;
    // nj equal groups of workgroups, one per block of hidden units, each
    // workgroup a run of at least one pair
    const int nj = mlp_blocks(a.h);
    const int64_t pairs = static_cast<int64_t>(a.n) * (a.B - 1);
    int64_t per = kMlpGrid / nj;
    if (per > pairs) per = pairs;
    const dim3 grid(static_cast<unsigned>(per * nj));
    switch (a.r) {
        case 16: return launch_mlp_r<16>(a, grid, stream);
        case 32: return launch_mlp_r<32>(a, grid, stream);
        case 64: return launch_mlp_r<64>(a, grid, stream);
        case 128: return launch_mlp_r<128>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace corr
