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
// Work is split by (pairs, block of 64 hidden units): for K <= 16 each
// workgroup streams a run of pairs through a producer / consumer split of its
// waves (mlp_ws_kernel), or, for calls with few pairs, takes one pair and 16
// units (mlp_pair16_kernel); for larger K each takes two adjacent pairs
// (mlp_kernel).  Each block writes its partial Delta and the finishing kernel
// adds the blocks in order, adds b2 and l_{p+1}(b) and walks.  Every sum runs
// in a fixed order, and no value is accumulated with atomics (they only
// count): bit-reproducible.
#include "common.h"
#include "handoff.h"
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
// Workgroups of a launch for K <= 16: one per CU, each running a contiguous
// share of the pairs of one block of hidden units (more when a share would
// exceed kMaxRun pairs).
constexpr int kMlpGrid = 256;

typedef __attribute__((address_space(3))) void* mlp_lds_ptr;
typedef __attribute__((address_space(1))) void* mlp_global_ptr;

// A staged z row holds its 2r bf16 values unpadded; segment s (16 bytes) of
// row a sits at position s ^ (a & mask), mask = min(7, segments - 1), so the
// eight rows one fragment read touches at a time sit in distinct banks
// (r >= 32) while every segment stays inside its row.
template <int ZSEG>
__device__ __forceinline__ int zpos(int a, int s) { return s ^ (a & (ZSEG < 8 ? ZSEG - 1 : 7)); }

// ------------------------------------------------------------- K > 16 --
static_assert(256 == 4 * kJB, "four r quarters per hidden unit in the c_p dot of mlp_kernel");

// One workgroup per (NP adjacent pairs p0 .. p0 + NP - 1 of a request, block
// of up to 64 hidden units); the last group of a request may hold fewer.  For
// each pair p of the group:
//   U_p[a][j] = W1_za[j] z_p^a,  V_{p+1}[b][j] = W1_zb[j] z_{p+1}^b   (MFMA)
//   P[a][j] = c_p[j] + b1[j] + w_la[j] l_p(a) + U_p[a][j]
//   Q[b][j] = w_lb[j] l_{p+1}(b) + V_{p+1}[b][j]
// with c_p = W1_s s_p formed here too, then GELU and the dot with w2 over the
// K x m candidate pairs (successors b < m; m = K unless sparsified), one
// (a, b) per thread; each pair's partial Delta for the block goes to
// part[pair][block][a][b].  With two pairs per group they share the W1
// fragments and the z rows of their middle slot; one pair per group gives
// twice the workgroups, which spread the GELU work evenly over the CUs.  U and V are accumulated exactly as a 16 x 16
// tile product over the 2r values [hi(z) | lo(z)] in k order, the hi and lo
// halves meeting the same W1 columns.
template <int R, int KT, int NP>
__global__ __launch_bounds__(256, KT > 2 ? 4 : (NP == 1 ? 7 : 5)) void mlp_kernel(MlpArgs a) {
    constexpr int KS = 2 * R / 32;          // 32-wide k-steps over [hi | lo]
    constexpr int KD = R >= 32 ? R / 32 : 1;  // distinct W1 fragments (hi and lo share them)
    constexpr int ZSEG = 2 * R / 8;         // 16-byte segments per z row
    const int tid = threadIdx.x;
    const int B = a.B, K = a.K, h = a.h;
    const int nj = (h + kJB - 1) / kJB;
    const int G = (B - 1 + NP - 1) / NP;    // pair groups per request
    // Consecutive workgroup numbers go to different XCDs (round-robin over 8):
    // the hidden blocks of one group are numbered 8 apart so they share an XCD.
    const int lin = blockIdx.x;
    const int xcd = lin % 8, i8 = lin / 8;
    const int jblk = i8 % nj;
    const int grp = (i8 / nj) * 8 + xcd;
    if (grp >= a.n * G) return;
    const int req = grp / G, p0 = NP * (grp % G);
    const int np = min(NP, B - 1 - p0);     // pairs in this group
    const int pair0 = req * (B - 1) + p0;
    const int64_t t0 = static_cast<int64_t>(req) * B + p0;   // slot row of the first pair's predecessor
    const int j0 = jblk * kJB;
    const int jn = min(kJB, h - j0);
    constexpr int PS = kJB + 4;     // LDS row stride of P / Q (floats)
    const int nin = 3 * R + 2;
    const int l = tid & 63, wave = tid >> 6;

    __shared__ __attribute__((aligned(16))) float w2s[kJB];
    __shared__ __attribute__((aligned(16))) float sps[NP][R];   // the pair states s_p
    __shared__ float cps4[NP][4][kJB];  // c_p partial dots, one per quarter of r
    __shared__ float lv[3 * 64];        // the candidates' logits l of slots t0 .. t0 + np (K <= 64)
    // First the z rows of the group's slots t0 .. t0 + np ([(np + 1) K][2r]
    // bf16, segments permuted by zpos); once the U | V products are formed,
    // the same memory holds P [NP][K][PS] and Q [NP][K][PS].
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    uint16_t* zs = reinterpret_cast<uint16_t*>(dyn);
    float* Pb = dyn;
    float* Qb = dyn + NP * K * PS;

    // ---- z rows straight into LDS (no registers held while in flight):
    // the slots' rows are contiguous in zhl.  A wave instruction moves 64
    // segments to 64 consecutive LDS positions; lanes past the last take no
    // part.  Then the pair states s_p, r / 4 segments each.
    {
        const int nseg = (np + 1) * K * ZSEG;
        for (int s0 = wave * 64; s0 < nseg; s0 += 4 * 64) {
            const int sg = s0 + l;
            if (sg < nseg) {
                const int row = sg / ZSEG, pos = sg % ZSEG;
                const uint16_t* src = a.zhl + (t0 * K + row) * (2 * R) + zpos<ZSEG>(row, pos) * 8;
                __builtin_amdgcn_global_load_lds((mlp_global_ptr)(src), (mlp_lds_ptr)(zs + s0 * 8), 16, 0, 0);
            }
        }
        if (wave >= 4 - np && l < R / 4) {
            const int i = 3 - wave;   // wave 3: the first pair, wave 2: the second
            __builtin_amdgcn_global_load_lds((mlp_global_ptr)(a.s + static_cast<int64_t>(pair0 + i) * R + 4 * l),
                                             (mlp_lds_ptr)(sps[i]), 16, 0, 0);
        }
        // the slots' logits, 4 bytes per lane (waves 0 and 1, 64 values each)
        const int nl = (np + 1) * K;
        if (wave < 2 && wave * 64 < nl && wave * 64 + l < nl)
            __builtin_amdgcn_global_load_lds((mlp_global_ptr)(a.vals + t0 * K + wave * 64 + l),
                                             (mlp_lds_ptr)(lv + wave * 64), 4, 0, 0);
        if (nl > 128 && wave == 2 && 128 + l < nl)
            __builtin_amdgcn_global_load_lds((mlp_global_ptr)(a.vals + t0 * K + 128 + l),
                                             (mlp_lds_ptr)(lv + 128), 4, 0, 0);
    }

    // ---- per-lane operands of the U | V tiles: wave w owns hidden units
    // j0 + 16 w .. + 15 of the block (columns past jn are formed from the
    // last valid unit and not stored)
    const int jl = min(16 * wave + (l & 15), jn - 1);   // this lane's unit within the block
    const bool wave_on = 16 * wave < jn;
    // W1_za | W1_zb fragments of this lane's unit (shared by both pairs)
    u32x4 bu[KD], bv[KD];
    {
        const uint16_t* wr = a.w1 + static_cast<int64_t>(j0 + jl) * nin;
        const int kq = 8 * (l >> 4);
#pragma unroll
        for (int d = 0; d < KD; ++d) {
            bu[d] = load16(wr + R + ((d * 32 + kq) % R));
            bv[d] = load16(wr + 2 * R + ((d * 32 + kq) % R));
        }
    }
    const float wla = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + jl) * nin + 3 * R]);
    const float wlb = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + jl) * nin + 3 * R + 1]);
    const float b1j = a.b1[j0 + jl];
    if (tid < kJB) w2s[tid] = tid < jn ? a.w2[j0 + tid] * (1.0f / kGeluAlpha) : 0.f;   // see gelu_scaled
    // c_p = W1_s s_p for the block's units: thread (jj, kq) dots row j0 + jj
    // of W1_s with s_p over the quarter kq of its r columns, in column order.
    // W1 rows are 3r + 2 bf16 long (4-byte aligned: r is a multiple of 16),
    // so they are read in 32-bit words of two columns each; s_p is read from
    // LDS once every load of the workgroup has landed.
    const int jj = tid & (kJB - 1), kqc = tid / kJB;
    constexpr int kw = R / 4;
    constexpr int kG = kw / 4;
    uint32_t wv[2 * kG];
    {
        const uint32_t* wr = reinterpret_cast<const uint32_t*>(
            a.w1 + static_cast<int64_t>(min(j0 + jj, h - 1)) * nin + kqc * kw);
#pragma unroll
        for (int g = 0; g < 2 * kG; ++g) wv[g] = wr[g];
    }
    __syncthreads();   // every load has landed: z rows and s_p in LDS
    for (int i = 0; i < np; ++i) {
        const float* sp = sps[i] + kqc * kw;
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const float4 sv = *reinterpret_cast<const float4*>(sp + 4 * g);
            acc = fmaf(__uint_as_float(wv[2 * g] << 16), sv.x, acc);
            acc = fmaf(__uint_as_float(wv[2 * g] & 0xFFFF0000u), sv.y, acc);
            acc = fmaf(__uint_as_float(wv[2 * g + 1] << 16), sv.z, acc);
            acc = fmaf(__uint_as_float(wv[2 * g + 1] & 0xFFFF0000u), sv.w, acc);
        }
        cps4[i][kqc][jj] = acc;
    }

    // ---- U | V tiles on MFMA (lane l holds rows 4 (l/16) + i, unit l % 16
    // of a 16 x 16 tile): U of pair i from slot t0 + i, V from slot t0 + i + 1
    f32x4 accu[NP][KT], accv[NP][KT];
    if (wave_on) {
        const int kq = 8 * (l >> 4);
#pragma unroll
        for (int i = 0; i < NP; ++i)
#pragma unroll
            for (int rt = 0; rt < KT; ++rt) {
                accu[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                accv[i][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (i < np && rt * 16 < K) {
                    // fragment rows past K repeat row K - 1 (not stored)
                    const int ar = i * K + min(rt * 16 + (l & 15), K - 1);
                    const int br = ar + K;
                    // one k-step's z fragments in registers at a time (the
                    // compiler barrier keeps the reads from being hoisted together)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const int sgi = (ks * 32 + kq) / 8;
                        const u32x4 zu = *reinterpret_cast<const u32x4*>(zs + (ar * ZSEG + zpos<ZSEG>(ar, sgi)) * 8);
                        const u32x4 zv = *reinterpret_cast<const u32x4*>(zs + (br * ZSEG + zpos<ZSEG>(br, sgi)) * 8);
                        accu[i][rt] = mfma16x16x32(zu, bu[ks % KD], accu[i][rt]);
                        accv[i][rt] = mfma16x16x32(zv, bv[ks % KD], accv[i][rt]);
                        asm volatile("" ::: "memory");
                    }
                }
            }
    }
    __syncthreads();   // the z rows are no longer read; P / Q take their place

    // ---- P and Q in the tiles' lane layout
    if (wave_on) {
        const int jc = 16 * wave + (l & 15);            // column in P / Q
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i >= np) break;
            const float cp = ((cps4[i][0][jl] + cps4[i][1][jl]) + (cps4[i][2][jl] + cps4[i][3][jl])) + b1j;
            float* P = Pb + i * K * PS;
            float* Q = Qb + i * K * PS;
#pragma unroll
            for (int rt = 0; rt < KT; ++rt) {
                if (rt * 16 >= K || jc >= jn) break;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = rt * 16 + 4 * (l >> 4) + e;
                    if (m < K) {   // kept scaled by alpha (see gelu_scaled)
                        constexpr float al = kGeluAlpha;
                        const float lp = lv[i * K + m], lq = lv[(i + 1) * K + m];
                        P[m * PS + jc] = al * (cp + fmaf(wla, lp, accu[i][rt][e]));
                        Q[m * PS + jc] = al * fmaf(wlb, lq, accv[i][rt][e]);
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- GELU and the dot with w2: each thread takes successors b and b + 1
    // of one predecessor a of one pair, so the P row and w2 are read once for
    // both (each sum keeps its own order)
    const int ms = a.m;
    const int mh = (ms + 1) / 2;
    const int per = K * mh;
    for (int idx = tid; idx < np * per; idx += 256) {
        const int i = idx / per, r = idx - i * per;
        const int aa = r / mh, bb = 2 * (r - aa * mh);
        const bool two = bb + 1 < ms;
        const float* pr = Pb + i * K * PS + aa * PS;
        const float* qr = Qb + i * K * PS + bb * PS;
        const float* qs = Qb + i * K * PS + (two ? bb + 1 : bb) * PS;
        float d0 = 0.f, d1 = 0.f, e0 = 0.f, e1 = 0.f;
        for (int j = 0; j < jn; j += 8) {
            const float4 pv0 = *reinterpret_cast<const float4*>(pr + j);
            const float4 pv1 = *reinterpret_cast<const float4*>(pr + j + 4);
            const float4 wv0 = *reinterpret_cast<const float4*>(w2s + j);
            const float4 wv1 = *reinterpret_cast<const float4*>(w2s + j + 4);
            const float4 qv0 = *reinterpret_cast<const float4*>(qr + j);
            const float4 qv1 = *reinterpret_cast<const float4*>(qr + j + 4);
            const float4 sv0 = *reinterpret_cast<const float4*>(qs + j);
            const float4 sv1 = *reinterpret_cast<const float4*>(qs + j + 4);
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
        float* out = a.part + (static_cast<int64_t>(pair0 + i) * nj + jblk) * K * K + aa * K + bb;
        out[0] = d0 + d1;
        if (two) out[1] = e0 + e1;
    }
}

// ------------------------------------------------------------- K <= 16 --
// The transition MLP for K <= 16, with a workgroup's waves split by role.
// The launch's workgroups form nj equal groups, one per block of 64 hidden
// units; each workgroup takes a contiguous run of at most kMaxRun pairs (256
// workgroups, one per CU, unless the runs would be longer) and streams it one
// pair at a time:
//   - waves 12-15 (producers) load the next pair's z rows and logits into
//     registers (coalesced 16-byte loads) while they finish the current one,
//     write them to LDS, form the U | V tiles (each producer wave one 16-unit
//     column tile of both, its W1 fragments held in registers) and write
//     P | Q into one of kRing LDS buffers;
//   - waves 0-11 (consumers) first form c_p + b1 of every pair of the run,
//     in pair order (the producers wait for a pair's before writing its P),
//     then run each pair's GELU loop as soon as its buffer is ready and
//     store its partial Deltas.
// The two sides meet through LDS counters (the generation written into a
// buffer, and how many consumer waves are done with it), so the loads and
// matrix products of later pairs overlap the vector-ALU work of earlier
// ones.  No workgroup barrier is used after the roles split (the producers
// meet through an LDS counter of their own); every wait on a counter is
// bounded (kSpinLimit sleeps), so the workgroup always ends.
constexpr int kRing = 3;            // P | Q buffers
constexpr int kMaxRun = 64;         // pairs per workgroup, at most (their c_p are formed up front)
constexpr int kProd = 4;            // producer waves
constexpr int kCons = 12;           // consumer waves
constexpr int kWsThreads = 64 * (kProd + kCons);
static_assert(kCons % 4 == 0 && kProd == 4, "a wave's units (16 (wave % 4) ..) are the same in every c_p job and P | Q tile");
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

// kFin: the finishing step and the walk in the same launch (MlpArgs
// fin_walk): the consumers store their partials with agent-scope atomic
// stores; once the workgroup's run is done (one barrier), wave i counts pair
// i of the run into the pair's counter, and the last of the pair's nj block
// workgroups forms its scores, row argmaxes and count with the per-pair
// finishing code of handoff.h (agent-scope loads of the partials); the
// request's last pair walks.
template <int R, bool kFin>
__global__ __launch_bounds__(kWsThreads, 1) void mlp_ws_kernel(MlpArgs a) {
    constexpr int KMAX = 16;
    constexpr int KS = 2 * R / 32;              // 32-wide k-steps over [hi | lo]
    constexpr int ZSEG = 2 * R / 8;             // 16-byte segments per z row
    constexpr int PT = 64 * kProd;              // producer threads
    constexpr int ZPT = (2 * KMAX * ZSEG + PT - 1) / PT;   // z segments per producer thread, at most
    constexpr int PQ = 2 * KMAX * kPS;          // floats of one P | Q buffer
    static_assert(2 * KMAX <= PT, "one logit per producer thread");
    __shared__ __attribute__((aligned(16))) uint16_t zbuf[2 * KMAX * 2 * R];
    __shared__ __attribute__((aligned(16))) float ring[kRing * PQ];
    __shared__ float cpr[kMaxRun][kJB];         // c_p + b1 of every pair of the run
    __shared__ __attribute__((aligned(16))) float spa[kMaxRun * R];   // the run's pair states
    __shared__ float lv[2 * KMAX];
    __shared__ __attribute__((aligned(16))) float w2s[kJB];
    // the block's W1_s rows as 32-bit words of two columns, rows padded
    constexpr int WSW = R / 2 + 4;
    __shared__ __attribute__((aligned(16))) uint32_t wsl[kJB * WSW];
    __shared__ int ready[kRing];                // generation (pair index in the run + 1) of each buffer's contents
    __shared__ int freed[kRing];                // consumer waves done with each buffer, cumulative
    __shared__ int pbar;                        // producer-wave barrier count
    __shared__ int cpn[kMaxRun];                // consumer waves done with each pair's c_p (4 when formed)

    const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
    if (!kFin && a.zero_cnt && blockIdx.x == 0)   // the finishing launch's per-request counts
        for (int i = tid; i < a.n; i += kWsThreads) a.zero_cnt[static_cast<int64_t>(i) * kCntStride] = 0;
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
    float lvr;
    auto fetch = [&](const Coord& c) {
        const uint16_t* zsrc = a.zhl + static_cast<int64_t>(c.t0) * K * (2 * R);
#pragma unroll
        for (int i = 0; i < ZPT; ++i) zr[i] = load16(zsrc + min(pt + i * PT, nseg - 1) * 8);   // clamped: not written
        lvr = a.vals[static_cast<int64_t>(c.t0) * K + min(pt, 2 * K - 1)];
    };
    // the run's pair states (consecutive pairs are contiguous) straight into
    // LDS, for the c_p of every pair below
    {
        const int nsp = n * (R / 4);
        const float* ssrc = a.s + static_cast<int64_t>(q_lo) * R;
        for (int s0 = wave * 64; s0 < nsp; s0 += kWsThreads)
            if (s0 + l < nsp)
                __builtin_amdgcn_global_load_lds((mlp_global_ptr)(ssrc + 4 * (s0 + l)), (mlp_lds_ptr)(spa + 4 * s0), 16,
                                                 0, 0);
    }
    if (wave >= kCons) fetch(first(q_lo));

    // the block's W1_s slice straight into LDS as well, one instruction per
    // row (its r bf16 at column 0, r / 2 four-byte words; rows are 4-byte
    // aligned: nin is even), so every load of the prologue is in flight at
    // once; rows past jn repeat row jn - 1 and are not used
    for (int jj = wave; jj < kJB; jj += kWsThreads / 64) {
        const uint16_t* src = a.w1 + static_cast<int64_t>(j0 + min(jj, jn - 1)) * nin;
        if (l < R / 2)
            __builtin_amdgcn_global_load_lds((mlp_global_ptr)(src + 2 * l), (mlp_lds_ptr)(&wsl[jj * WSW]), 4, 0, 0);
    }
    const float w2v = a.w2[j0 + min(tid, jn - 1)];   // loaded unconditionally: no wait inside a branch
    // b1 of the lane's unit in the c_p jobs below (a consumer wave's jobs all
    // cover units 16 (wave % 4) .. + 15), and the logit columns w_la, w_lb of
    // a producer lane's unit
    const int ju = min(16 * (wave & 3) + (l & 15), jn - 1);
    const float b1v = a.b1[j0 + ju];
    const float wla = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + ju) * nin + 3 * R]);
    const float wlb = bf16_to_f32(a.w1[static_cast<int64_t>(j0 + ju) * nin + 3 * R + 1]);
    // a producer wave's W1_za and W1_zb fragments (its 16 units), the same
    // for every pair (the [hi | lo] halves of z meet the same R / 32 column
    // fragments), loaded straight into registers
    constexpr int KD = R >= 32 ? R / 32 : 1;
    u32x4 bu[KD], bv[KD];
    if (wave >= kCons) {
        const uint16_t* wrow = a.w1 + static_cast<int64_t>(j0 + ju) * nin;
        const int kq = 8 * (l >> 4);
#pragma unroll
        for (int d = 0; d < KD; ++d) {
            const int wcol = (d * 32 + kq) % R;
            bu[d] = load16(wrow + R + wcol);
            bv[d] = load16(wrow + 2 * R + wcol);
        }
    }
    if (tid < kRing) {
        ready[tid] = 0;
        freed[tid] = 0;
    }
    if (tid < kMaxRun) cpn[tid] = 0;
    if (tid == 0) pbar = 0;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every direct load (and the first pair's z rows) has landed
    if (tid < kJB) w2s[tid] = tid < jn ? w2v * (1.0f / kGeluAlpha) : 0.f;   // see gelu_scaled
    __syncthreads();

    // ---- c_p + b1 of every pair of the run (n <= kMaxRun), formed by the
    // consumer waves, in pair order, while the producers stage and multiply
    // the first pairs: job (pair i, group ug of 16 units) per wave; lane l
    // dots a quarter l / 16 of r of unit 16 ug + l % 16 (W1_s words and s_p
    // from LDS), column order, and the four quarters are added in a fixed
    // order across lanes l, l ^ 16, l ^ 32, l ^ 48.  cpn[i] counts the jobs
    // of pair i done; the producers wait for 4 before writing its P.
    for (int job = wave; wave < kCons && job < n * (kJB / 16); job += kCons) {
        const int i = job >> 2, ug = job & 3;
        const int jl = min(16 * ug + (l & 15), jn - 1);   // clamped: past jn not used
        constexpr int WQ = R / 8;           // words of a quarter of r
        const int e4 = l >> 4;
        const float* sq = spa + i * R + e4 * (R / 4);
        float acc = 0.f;
        if constexpr (WQ % 2 == 0) {
#pragma unroll
            for (int q2 = 0; q2 < WQ / 2; ++q2) {
                const float4 sv = *reinterpret_cast<const float4*>(sq + 4 * q2);
                const uint32_t w0 = wsl[jl * WSW + e4 * WQ + 2 * q2], w1 = wsl[jl * WSW + e4 * WQ + 2 * q2 + 1];
                acc = fmaf(__uint_as_float(w0 << 16), sv.x, acc);
                acc = fmaf(__uint_as_float(w0 & 0xFFFF0000u), sv.y, acc);
                acc = fmaf(__uint_as_float(w1 << 16), sv.z, acc);
                acc = fmaf(__uint_as_float(w1 & 0xFFFF0000u), sv.w, acc);
            }
        } else {
#pragma unroll
            for (int q = 0; q < WQ; ++q) {
                const float2 sv = *reinterpret_cast<const float2*>(sq + 2 * q);
                const uint32_t w = wsl[jl * WSW + e4 * WQ + q];
                acc = fmaf(__uint_as_float(w << 16), sv.x, acc);
                acc = fmaf(__uint_as_float(w & 0xFFFF0000u), sv.y, acc);
            }
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        if (l < 16) cpr[i][16 * ug + l] = acc + b1v;
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the c_p are in LDS
        asm volatile("" ::: "memory");
        if (l == 0) atomicAdd(&cpn[i], 1);
    }

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
            if (pt < 2 * K) lv[pt] = lvr;
            pbarrier();                           // z rows and logits in LDS
            if (u + 1 < n) {
                c = step(c);
                fetch(c);
            }
            // U (slot 0 rows) and V (slot 1 rows) of the wave's column tile;
            // fragment rows past K repeat row K - 1 (not stored)
            f32x4 au = {0.f, 0.f, 0.f, 0.f}, av = {0.f, 0.f, 0.f, 0.f};
            if (tile_on) {
                const int kq = 8 * (l >> 4);
                const int ra = min(l & 15, K - 1), rb = K + ra;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int sgi = (ks * 32 + kq) / 8;
                    const u32x4 za = *reinterpret_cast<const u32x4*>(&zbuf[(ra * ZSEG + zpos<ZSEG>(ra, sgi)) * 8]);
                    const u32x4 zb = *reinterpret_cast<const u32x4*>(&zbuf[(rb * ZSEG + zpos<ZSEG>(rb, sgi)) * 8]);
                    au = mfma16x16x32(za, bu[ks % KD], au);
                    av = mfma16x16x32(zb, bv[ks % KD], av);
                }
            }
            // the buffer is free once every consumer wave is done with its
            // previous contents (pair u - kRing), and P needs the pair's c_p:
            // both counters and the lane's c_p are read in one round (LDS
            // requests of a wave complete in order, so a c_p read issued
            // after a count of 4 was read returns the formed value)
            float cp = 0.f;
            for (unsigned it = 0; it < kSpinLimit; ++it) {
                const int fr = *as_lds(&freed[slot]);
                const int cn = *as_lds(&cpn[u]);
                cp = *(__attribute__((address_space(3))) volatile float*)(&cpr[u][16 * pw + (l & 15)]);
                if (fr >= kCons * (u / kRing) && cn >= kJB / 16) break;
                __builtin_amdgcn_s_sleep(1);
            }
            asm volatile("" ::: "memory");
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
                    if (kFin) {
                        uint32_t* o = reinterpret_cast<uint32_t*>(out + to[k]);
                        __hip_atomic_store(o, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (two)
                            __hip_atomic_store(o + 1, __float_as_uint(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    } else {
                        out[to[k]] = v;
                        if (two) out[to[k] + 1] = w;
                    }
                }
            }
            // this wave is done reading the buffer
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            asm volatile("" ::: "memory");
            if (l == 0) atomicAdd(&freed[slot], 1);
            c = step(c);
        }
    }
    if (!kFin) return;
    // ---- the run's pairs counted in; each pair's last block workgroup
    // finishes it (every wave of both roles reaches this barrier: every wait
    // above is bounded)
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's partial stores have completed
    __syncthreads();
    for (int i = wave; i < n; i += kWsThreads / 64) {
        const int pair = q_lo + i;
        int done = 0;
        if (l == 0)
            done = __hip_atomic_fetch_add(a.pcnt + static_cast<int64_t>(pair) * kCntStride, 1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        if (__shfl(done, 0, 64) != nj - 1) continue;   // another block of the pair is still running
        const PairRow4 r = pair_scores4<true>(a.part, nj, 0, a.m, a.vals, a.b2[0], B, K, pair);
        pair_walk_finish(r, a.scores, a.best, a.rcnt, a.ids, a.tokens, a.choice, B, K, pair);
    }
}

// ------------------------------------------------- K <= 16, few pairs --
// For calls with few pairs: one workgroup of 256 threads per (pair, block of
// 16 hidden units), so that a pair's work and its W1 rows spread over
// (h / 16) CUs.  Every value is formed exactly as in mlp_ws_kernel: U and V
// by the same MFMA sequence (z fragments read from memory instead of LDS),
// c_p + b1 by the same quarter dots and shuffles, P and Q by the same
// expressions, and each GELU task (predecessor a, successors b and b + 1,
// eight units) by the same loop.  The ws kernel then adds the eight tasks of
// a 64-unit block in the tree ((q0 + q1) + (q2 + q3)) + ((q4 + q5) + (q6 + q7))
// (DPP xor 1, xor 2, half-row mirror); here each workgroup stops after the
// first level and writes (q0 + q1) of its sixteen units, and the finishing
// step adds the four of a 64-unit block in the same tree.  The scores are
// therefore identical to the ws kernel's.
// kFin: the finishing step and the walk in the same launch (MlpArgs
// fin_walk): the partials go out as agent-scope atomic stores, the last of a
// pair's workgroups reads them back the same way and forms the pair's scores
// and row argmaxes as the per-pair finishing code does (one score per thread; a row's
// K columns share a DPP row, quad or half-row), and the last pair of a
// request walks.
template <int R, bool kFin>
__global__ __launch_bounds__(256) void mlp_pair16_kernel(MlpArgs a) {
    constexpr int KMAX = 16;
    constexpr int KS = 2 * R / 32;              // 32-wide k-steps over [hi | lo]
    constexpr int KD = R >= 32 ? R / 32 : 1;    // distinct W1 fragments
    constexpr int PQ = 2 * KMAX * kPS;
    __shared__ __attribute__((aligned(16))) float pq[PQ];
    __shared__ float cps[16];
    __shared__ float lv[2 * KMAX];
    __shared__ __attribute__((aligned(16))) float w2s[16];
    __shared__ int s_count;
    const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
    if (!kFin && a.zero_cnt && blockIdx.x == 0)  // the finishing launch's per-request counts
        for (int i = tid; i < a.n; i += 256) a.zero_cnt[static_cast<int64_t>(i) * kCntStride] = 0;
    const int B = a.B, K = a.K;
    const int nb = a.h / 16;                     // blocks of 16 units (h is a multiple of 16)
    const int pair = blockIdx.x / nb, blk = blockIdx.x - pair * nb;
    const int req = pair / (B - 1), p = pair - req * (B - 1);
    const int64_t t0 = static_cast<int64_t>(req) * B + p;   // slot row of the predecessor
    const int j0 = 16 * blk;
    const int nin = 3 * R + 2;
    const int ju = j0 + (l & 15);                // the lane's unit (every block is full)
    const uint16_t* wrow = a.w1 + static_cast<int64_t>(ju) * nin;
    // every load first: the U (wave 0) or V (wave 1) operands, c_p's W1_s
    // words and pair state (wave 2), logits, w2
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int kq = 8 * (l >> 4);
    if (wave < 2) {
        const int row = min(l & 15, K - 1);      // rows past K repeat row K - 1 (not stored)
        const uint16_t* zr = a.zhl + ((t0 + wave) * K + row) * (2 * R) + kq;
        const uint16_t* wz = wrow + (1 + wave) * R;
        u32x4 zf[KS], wf[KD];
#pragma unroll
        for (int d = 0; d < KD; ++d) wf[d] = load16(wz + (d * 32 + kq) % R);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) zf[ks] = load16(zr + ks * 32);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(zf[ks], wf[ks % KD], acc);
    } else if (wave == 2) {
        // lane l: quarter l / 16 of r of unit ju, column order, the quarters
        // added across lanes l ^ 16 and l ^ 32
        constexpr int WQ = R / 8;                // words of a quarter
        const int e4 = l >> 4;
        const uint32_t* ws = reinterpret_cast<const uint32_t*>(wrow) + e4 * WQ;
        const float* sq = a.s + static_cast<int64_t>(pair) * R + e4 * (R / 4);
        float cacc = 0.f;
#pragma unroll
        for (int q2 = 0; q2 < WQ / 2; ++q2) {
            const float4 sv = *reinterpret_cast<const float4*>(sq + 4 * q2);
            const uint32_t w0 = ws[2 * q2], w1 = ws[2 * q2 + 1];
            cacc = fmaf(__uint_as_float(w0 << 16), sv.x, cacc);
            cacc = fmaf(__uint_as_float(w0 & 0xFFFF0000u), sv.y, cacc);
            cacc = fmaf(__uint_as_float(w1 << 16), sv.z, cacc);
            cacc = fmaf(__uint_as_float(w1 & 0xFFFF0000u), sv.w, cacc);
        }
        cacc += __shfl_xor(cacc, 16, 64);
        cacc += __shfl_xor(cacc, 32, 64);
        if (l < 16) cps[l] = cacc + a.b1[ju];
    } else {
        if (l < 2 * K) lv[l] = a.vals[t0 * K + l];
        if (l >= 32 && l < 48) w2s[l - 32] = a.w2[j0 + l - 32] * (1.0f / kGeluAlpha);   // see gelu_scaled
    }
    __syncthreads();
    // P (wave 0) and Q (wave 1), kept scaled by alpha
    if (wave < 2) {
        const int jc = l & 15;
        const float wl = bf16_to_f32(wrow[3 * R + wave]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 4 * (l >> 4) + e;
            if (m < K) {
                constexpr float al = kGeluAlpha;
                if (wave == 0)
                    pq[static_cast<int>(__umul24(m, kPS)) + jc] = al * (cps[jc] + fmaf(wl, lv[m], acc[e]));
                else
                    pq[static_cast<int>(__umul24(KMAX + m, kPS)) + jc] = al * fmaf(wl, lv[K + m], acc[e]);
            }
        }
    }
    __syncthreads();
    // one task per thread: (predecessor a, successors b and b + 1, eighth
    // t % 2 of the sixteen units), as in mlp_ws_kernel
    const int ms = a.m;
    const int mh = (ms + 1) / 2;
    const int T = K * mh * 2;
    const int q = tid & 1, rest = tid >> 1;
    const int aa = rest / mh, bb = 2 * (rest - static_cast<int>(__umul24(aa, mh)));
    const bool two = bb + 1 < ms;
    const int j = 8 * q;
    float d0 = 0.f, d1 = 0.f, e0 = 0.f, e1 = 0.f;
    if (tid < T) {
        const int pr = static_cast<int>(__umul24(aa, kPS)) + j;
        const int qr = static_cast<int>(__umul24(KMAX + bb, kPS)) + j;
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
    if (tid < T && q == 0) {
        float* out = a.part + (static_cast<int64_t>(pair) * nb + blk) * K * K + static_cast<int>(__umul24(aa, K)) + bb;
        if (kFin) {
            __hip_atomic_store(reinterpret_cast<uint32_t*>(out), __float_as_uint(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            if (two)
                __hip_atomic_store(reinterpret_cast<uint32_t*>(out) + 1, __float_as_uint(w), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        } else {
            out[0] = v;
            if (two) out[1] = w;
        }
    }
    if (!kFin) return;
    // ---- the pair's last workgroup: its scores and row argmaxes
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are complete
    __syncthreads();
    if (tid == 0)
        s_count = __hip_atomic_fetch_add(a.pcnt + static_cast<int64_t>(pair) * kCntStride, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_count != nb - 1) return;        // another block of the pair is still running
    const int KK = K * K;
    if (wave * 64 < KK) {                 // whole waves: the row reductions below use DPP
        const int e = min(tid, KK - 1);   // threads past K^2 repeat the last score (not stored)
        const int ra = e / K, cb = e - ra * K;
        const float* src = a.part + static_cast<int64_t>(pair) * nb * KK + e;
        // 16-unit partials: a 64-unit block's value is (P0 + P1) + (P2 + P3),
        // a missing one counting as +0; the blocks then in order
        float u[4 * kMaxMlpBlocks];
#pragma unroll
        for (int b = 0; b < 4 * kMaxMlpBlocks; ++b)
            u[b] = b < nb ? __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(src + b * KK),
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                          : 0.f;
        const float lvb = a.vals[(t0 + 1) * K + cb];
        float t4[kMaxMlpBlocks];
#pragma unroll
        for (int g = 0; g < kMaxMlpBlocks; ++g) t4[g] = (u[4 * g] + u[4 * g + 1]) + (u[4 * g + 2] + u[4 * g + 3]);
        const int nb64 = (nb + 3) / 4;
        float acc = t4[0];
#pragma unroll
        for (int g = 1; g < kMaxMlpBlocks; ++g)
            if (g < nb64) acc += t4[g];
        float sv = lvb + (acc + a.b2[0]);
        if (cb >= a.m) sv = -INFINITY;    // successors b >= m are not scored
        if (tid < KK) a.scores[static_cast<int64_t>(pair) * KK + e] = sv;
        // row ra's argmax over its K lanes, ties to the lower index
        float bv = tid < KK ? sv : -INFINITY;
        int bi = tid < KK ? cb : 64;
        auto take = [&](float ov, int oi) {
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        };
        take(dpp_f<kDppXor1>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppXor1, 0xF, 0xF, false));
        take(dpp_f<kDppXor2>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppXor2, 0xF, 0xF, false));
        if (K > 4)
            take(dpp_f<kDppHalfMirror>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppHalfMirror, 0xF, 0xF, false));
        if (K > 8) take(dpp_f<kDppMirror>(bv), __builtin_amdgcn_update_dpp(0, bi, kDppMirror, 0xF, 0xF, false));
        if (tid < KK && cb == 0)
            __hip_atomic_store(a.best + static_cast<int64_t>(pair) * K + ra, bi, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores are complete
    __syncthreads();
    if (tid == 0)
        s_count = __hip_atomic_fetch_add(a.rcnt + static_cast<int64_t>(req) * kCntStride, 1, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_count != B - 2 || wave != 0) return;   // not the request's last pair
    pair_walk(a.best, req, B, K, a.ids, a.tokens, a.choice);
}

}  // namespace

int mlp_blocks(int h) { return (h + kJB - 1) / kJB; }

// Pairs per workgroup of the K > 16 kernel.
constexpr int kMlpPairs = 2;

// Dynamic LDS of the K > 16 kernel: the z rows of the group's slots, or P and
// Q of its pairs, whichever is larger.
static size_t mlp_lds_bytes(int K, int r) {
    const size_t z = static_cast<size_t>(kMlpPairs + 1) * K * 2 * r * sizeof(uint16_t);
    const size_t pq = static_cast<size_t>(2 * kMlpPairs) * K * (kJB + 4) * sizeof(float);
    return z > pq ? z : pq;
}

template <int R>
hipError_t launch_mlp_r(const MlpArgs& a, hipStream_t stream) {
    const int nj = mlp_blocks(a.h);
    if (a.K <= 16) {
        // nj equal groups of workgroups, one per block of hidden units, each
        // workgroup a run of at least one pair
        const int64_t pairs = static_cast<int64_t>(a.n) * (a.B - 1);
        int64_t per = kMlpGrid / nj;
        if (per * kMaxRun < pairs) per = (pairs + kMaxRun - 1) / kMaxRun;   // runs of at most kMaxRun pairs
        if (per > pairs) per = pairs;
        if (a.fin_walk)
            return launch(mlp_ws_kernel<R, true>, dim3(static_cast<unsigned>(per * nj)), kWsThreads, 0, stream, a);
        return launch(mlp_ws_kernel<R, false>, dim3(static_cast<unsigned>(per * nj)), kWsThreads, 0, stream, a);
    }
    // one workgroup per (group of kMlpPairs pairs, block); groups rounded up to
    // eight so that the blocks of a group share an XCD
    const int groups = a.n * ((a.B - 1 + kMlpPairs - 1) / kMlpPairs);
    const dim3 grid(static_cast<unsigned>((groups + 7) / 8 * 8 * nj));
    const uint32_t lds = static_cast<uint32_t>(mlp_lds_bytes(a.K, a.r));
    if (a.K <= 32) return launch(mlp_kernel<R, 2, kMlpPairs>, grid, 256, lds, stream, a);
    return launch(mlp_kernel<R, 4, kMlpPairs>, grid, 256, lds, stream, a);
}

hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream) {
    if (a.B < 2 || a.n < 1) return hipSuccess;
    if (a.fin_walk && ((a.K != 4 && a.K != 8 && a.K != 16) || a.zero_cnt || !a.pcnt || !a.rcnt || !a.best ||
                       !a.tokens || !a.scores ||
                       ((reinterpret_cast<uintptr_t>(a.scores) | reinterpret_cast<uintptr_t>(a.vals) |
                         reinterpret_cast<uintptr_t>(a.part)) & 15)))
        return hipErrorInvalidValue;
    if (a.units16) {
        if (a.K > 16 || a.h % 16) return hipErrorInvalidValue;
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.n) * (a.B - 1) * (a.h / 16)));
        if (a.fin_walk) {
            switch (a.r) {
                case 16: return launch(mlp_pair16_kernel<16, true>, grid, 256, 0, stream, a);
                case 32: return launch(mlp_pair16_kernel<32, true>, grid, 256, 0, stream, a);
                case 64: return launch(mlp_pair16_kernel<64, true>, grid, 256, 0, stream, a);
                case 128: return launch(mlp_pair16_kernel<128, true>, grid, 256, 0, stream, a);
                default: return hipErrorInvalidValue;
            }
        }
        switch (a.r) {
            case 16: return launch(mlp_pair16_kernel<16, false>, grid, 256, 0, stream, a);
            case 32: return launch(mlp_pair16_kernel<32, false>, grid, 256, 0, stream, a);
            case 64: return launch(mlp_pair16_kernel<64, false>, grid, 256, 0, stream, a);
            case 128: return launch(mlp_pair16_kernel<128, false>, grid, 256, 0, stream, a);
            default: return hipErrorInvalidValue;
        }
    }
    switch (a.r) {
        case 16: return launch_mlp_r<16>(a, stream);
        case 32: return launch_mlp_r<32>(a, stream);
        case 64: return launch_mlp_r<64>(a, stream);
        case 128: return launch_mlp_r<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace corr
