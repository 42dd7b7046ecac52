// Steps (2) and (3) of the DCOCO method details: the LayerNorm-projected
// candidate representations and the per-slot halves of the pair state.
//
//   gemm   a tiled MFMA GEMM used for (i) hproj: the drafter hidden states h
//          [rows][d] against the stacked [W_ctx; W_pair[:, :d]; W_pair[:, d:]]
//          ([3r][d]): each slot's hidden row is read once and yields W_ctx h
//          (for g), the left half W_pair,L h (for pairs that start at the
//          slot) and the right half W_pair,R h (for pairs that end at it); and
//          (ii) the folded table E W_cand^T over the whole vocabulary, and
//          reduction is split over a fixed number of workgroups per shape;
//          consumers add the partials in split order.
//          (iii) u = W_cand E[c] over the gathered embedding rows of all
//          candidates.
//   cand   one workgroup per 32 candidates: b = LN(u) (non-affine),
//          g = LN(W_ctx h) from hproj,
//          y = W_fuse [b; g] on MFMA, z = gamma * LN(y) + beta, stored as
//          bf16 hi | lo halves (the MLP kernel forms its layer-1 products
//          from them); the cosine variant also forms unit(W_out z) and
//          unit(W_in z).  MFMA operands that are not already bf16 (b, g, z)
//          are split into hi + lo bf16 parts multiplied by the same weight
//          columns, so those products carry float32 accuracy.
// All LayerNorm statistics are fp32 over the r features, biased variance.
#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace corr {

namespace {

// Two problems per launch: workgroups [0, nblk0) run j0, the rest j1 (the
// body is instantiated once per problem so each reads its own arguments).
__global__ __launch_bounds__(256) void gemm_kernel(GemmJob j0, GemmJob j1, int64_t nblk0) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kGemmSmem];
    const int64_t b = blockIdx.x;
    if (b < nblk0)
        gemm_any_body(j0, b, smem);
    else
        gemm_any_body(j1, b - nblk0, smem);
}

// ------------------------------------------------------------ gather gemm --
// The candidate projection u = W_cand E[c]: 128 x 128 output tiles of one
// k-split per 512-thread workgroup (8 waves, 4 along m x 2 along n, each
// 32 x 64 as 2 x 4 v_mfma_f32_16x16x32_bf16).  The gathered embedding rows
// and the W rows go from memory straight into LDS (global_load_lds_dwordx4:
// no registers held while they are in flight) through a ring of four
// [A | W] stages of 64-deep k-slabs; three slabs are in flight while one is
// multiplied, and one workgroup barrier per slab orders the ring.  Each
// output is accumulated in the same k order as gemm_body (slab by slab, the
// two 32-wide halves of a slab in turn), so the two give identical partials.

constexpr int kGM = 128, kGN = 128, kGK = 64;    // tile rows, columns, slab depth
constexpr int kGThreads = 512;
constexpr int kGStage = kGM * kGK;               // bf16 per A (= per W) stage
constexpr int kGStages = 4;
static_assert(kGM == kGN, "A and W stages share one size");

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// Segment p (16 bytes) of stage row r holds k-segment p ^ gswz(r), so the
// 8 (or 16) rows that one fragment read touches at a time sit in distinct
// LDS banks; a load instruction still covers whole 128-byte row pieces.
__device__ __forceinline__ int gswz(int r) { return ((r >> 1) + 4 * (r & 1)) & 7; }

// One 16-byte load per lane from g into LDS at lds + 16 * lane (lds is the
// same for the whole wave).
__device__ __forceinline__ void lds_dma16(const uint16_t* g, uint16_t* lds) {
    __builtin_amdgcn_global_load_lds((global_void_ptr)(g), (lds_void_ptr)(lds), 16, 0, 0);
}

// s_waitcnt vmcnt(n) with the other counters unconstrained.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0xF70);
}

// The candidate projection in its small form: workgroups of two waves, each
// wave one 16 x 16 output tile of one k-split (split fastest), the two tiles
// side by side (columns), as gemm_small_body, but with every k-step of a
// round of up to kSmallRound loaded at once straight into LDS
// (global_load_lds_dwordx4: the lanes' A and W fragments of a k-step, 1 KB
// each, land lane-linearly, which is also the layout the MFMA reads back,
// bank-conflict free), so a wave waits for memory once per round instead of
// once per few k-steps.  The two waves share the round's A fragments (each
// loads half of them), so a CU takes in three fragments per k-step for two
// tiles instead of four.  Same MFMA sequence per output: identical partials.
constexpr int kSmallRound = 32;   // k-steps per round (96 KB of LDS)

__global__ __launch_bounds__(128) void gemm_small_kernel(GemmJob J) {
    // [A | W of wave 0 | W of wave 1], kSmallRound k-steps of 512 bf16 each
    __shared__ __attribute__((aligned(1024))) uint16_t st[3 * kSmallRound * 512];
    const GemmA& A = J.A;
    const GemmW& W = J.W;
    const int64_t M = J.M;
    const int N = J.N, kdim = J.kdim, splits = J.splits;
    const int l = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int kper = ((kdim / 32 + splits - 1) / splits) * 32;
    const int ntn = (N + 15) / 16;
    const int ncp = (ntn + 1) / 2;                // column-tile pairs
    const int64_t t = blockIdx.x;
    const int split = static_cast<int>(t % splits);
    const int64_t rest = t / splits;
    const int ct = static_cast<int>(rest % ncp) * 2 + wave;   // ct == ntn: no tile (odd ntn), loads clamped
    const int n0 = min(ct, ntn - 1) * 16;
    const int64_t m0 = (rest / ncp) * 16;
    if (m0 >= M) return;   // whole workgroup
    const int k_lo = split * kper;
    const int k_hi = min(kdim, k_lo + kper);
    const int nks = k_lo < k_hi ? (k_hi - k_lo) / 32 : 0;
    const int kq = 8 * (l >> 4);
    // rows past M or N repeat the last row (their results are not stored)
    const uint16_t* ap = a_row(A, min(m0 + (l & 15), M - 1)) + k_lo + kq;
    const int nn = min(n0 + (l & 15), N - 1);
    const int b = nn / W.nb;
    const uint16_t* wb = b == 0 ? W.base[0] : (b == 1 ? W.base[1] : W.base[2]);
    const int64_t wld = b == 0 ? W.ld[0] : (b == 1 ? W.ld[1] : W.ld[2]);
    const uint16_t* wp = wb + static_cast<int64_t>(nn % W.nb) * wld + k_lo + kq;
    uint16_t* sa = st;
    uint16_t* sw = st + (1 + wave) * kSmallRound * 512;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nks; c0 += kSmallRound) {
        const int nc = min(kSmallRound, nks - c0);
        // both waves are done reading the previous round before its LDS is refilled
        __syncthreads();
        for (int i = wave; i < nc; i += 2) lds_dma16(ap + 32 * (c0 + i), sa + i * 512);
        for (int i = 0; i < nc; ++i) lds_dma16(wp + 32 * (c0 + i), sw + i * 512);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's loads of the round have landed
        __syncthreads();                       // and the other wave's half of A
        // eight k-steps' fragments read at a time (reads past the round's
        // last k-step stay inside the buffer and are not used)
        for (int i0 = 0; i0 < nc; i0 += 8) {
            u32x4 a[8], w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = min(i0 + j, kSmallRound - 1);
                a[j] = *reinterpret_cast<const u32x4*>(sa + i * 512 + 8 * l);
                w[j] = *reinterpret_cast<const u32x4*>(sw + i * 512 + 8 * l);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (i0 + j < nc) acc = mfma16x16x32(a[j], w[j], acc);
        }
    }
    if (ct >= ntn) return;
    // lane l holds rows 4 (l / 16) + e of column l % 16
    float* out = J.C + static_cast<int64_t>(split) * M * N;
    const int c = n0 + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t r = m0 + 4 * (l >> 4) + e;
        if (r < M && c < N) out[r * N + c] = acc[e];
    }
}

__global__ __launch_bounds__(kGThreads) void gemm_gather_kernel(GemmJob J) {
    // the ring: stage s is [A slab | W slab]; after the loop the first
    // 72 KB stage the output tiles
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kGStages * 2 * kGStage];
    const GemmA& A = J.A;
    const GemmW& W = J.W;
    const int64_t M = J.M;
    const int N = J.N, kdim = J.kdim, splits = J.splits;
    const int tid = threadIdx.x, l = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // split fastest, as in gemm_body: consecutive workgroups (spread over the
    // XCDs) take different k-slices
    const int64_t lin = blockIdx.x;
    const int split = static_cast<int>(lin % splits);
    const int64_t rest = lin / splits;
    const int ntn = (N + kGN - 1) / kGN;
    const int n0 = static_cast<int>(rest % ntn) * kGN;
    const int64_t m0 = (rest / ntn) * kGM;
    const int kper = ((kdim / 32 + splits - 1) / splits) * 32;
    const int k_lo = split * kper;
    const int k_hi = min(kdim, k_lo + kper);
    const int nslab = k_lo < k_hi ? (k_hi - k_lo + kGK - 1) / kGK : 0;

    // Wave w fills 8-row blocks 2w and 2w + 1 of each stage's A and W slabs,
    // one instruction per block: lane l takes row 8b + l/8 and places its
    // 16 bytes at position l % 8 of that row, i.e. k-segment
    // (l % 8) ^ gswz(row).  Rows past M or N repeat the last row (their
    // results are not stored).
    const uint16_t* ga[2];
    const uint16_t* gw[2];
    int segk[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (2 * wave + i) * 8 + (l >> 3);
        segk[i] = ((l & 7) ^ gswz(row)) * 8;
        ga[i] = a_row(A, min(m0 + row, M - 1));
        const int nn = min(n0 + row, N - 1);
        const int b = nn / W.nb;
        const uint16_t* wb = b == 0 ? W.base[0] : (b == 1 ? W.base[1] : W.base[2]);
        const int64_t wld = b == 0 ? W.ld[0] : (b == 1 ? W.ld[1] : W.ld[2]);
        gw[i] = wb + static_cast<int64_t>(nn % W.nb) * wld;
    }
    auto stage_a = [&](int st) { return smem + st * 2 * kGStage; };
    auto stage_w = [&](int st) { return smem + st * 2 * kGStage + kGStage; };
    // k ranges are multiples of 32, so only a split's last slab can be half
    // valid; its loads then re-read the valid half (in bounds) and only the
    // first 32-wide half is multiplied.
    auto issue = [&](int s) {
        const int k0 = k_lo + s * kGK;
        const bool half = k0 + kGK > k_hi;
        uint16_t* sa = stage_a(s % kGStages);
        uint16_t* sw = stage_w(s % kGStages);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int ko = k0 + (half ? (segk[i] & 31) : segk[i]);
            lds_dma16(ga[i] + ko, sa + (2 * wave + i) * 8 * kGK);
            lds_dma16(gw[i] + ko, sw + (2 * wave + i) * 8 * kGK);
        }
    };
    // Fragments: lane l reads row l % 16 of a 16-row tile, k-segment
    // 4 ks + l / 16 of the slab, at position (4 ks + l / 16) ^ gswz(l % 16).
    const int q = l >> 4;
    const int sz = gswz(l & 15);
    const int off[2] = {(l & 15) * kGK + ((q ^ sz) * 8), (l & 15) * kGK + (((4 + q) ^ sz) * 8)};
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto lds_addr = [](const uint16_t* p) {
        return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint16_t*)(p)));
    };
    // The fragment reads are written as inline assembly, so the compiler sees
    // no LDS read that it would have to order after the direct loads still in
    // flight (it would wait for all of them, later slabs included); the
    // per-slab vmcnt waits and the barrier order them instead.
    auto mma_half = [&](uint32_t ab, uint32_t wb) {
        u32x4 af0, af1, wf0, wf1, wf2, wf3;
        asm volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %6 offset:2048\n\t"
            "ds_read_b128 %2, %7\n\t"
            "ds_read_b128 %3, %7 offset:2048\n\t"
            "ds_read_b128 %4, %7 offset:4096\n\t"
            "ds_read_b128 %5, %7 offset:6144\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(af0), "=&v"(af1), "=&v"(wf0), "=&v"(wf1), "=&v"(wf2), "=&v"(wf3)
            : "v"(ab), "v"(wb));
        const u32x4 af[2] = {af0, af1}, wf[4] = {wf0, wf1, wf2, wf3};
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], wf[j], acc[i][j]);
    };
    for (int s = 0; s < kGStages - 1 && s < nslab; ++s) issue(s);
    for (int s = 0; s < nslab; ++s) {
        // this wave's loads of slab s have landed once no more than those of
        // the slabs issued after it (four instructions each) are pending
        switch (min(kGStages - 2, nslab - 1 - s)) {
            case 0: wait_vmcnt<0>(); break;
            case 1: wait_vmcnt<4>(); break;
            default: wait_vmcnt<8>(); break;
        }
        // workgroup barrier without a memory fence (a fence would wait for
        // every load in flight): every wave's slab s has landed, and every
        // wave has finished reading slab s - 1, whose stage is refilled next
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (s + kGStages - 1 < nslab) issue(s + kGStages - 1);
        const uint32_t ab = lds_addr(stage_a(s % kGStages) + wm * 32 * kGK);
        const uint32_t wb = lds_addr(stage_w(s % kGStages) + wn * 64 * kGK);
        mma_half(ab + 2 * off[0], wb + 2 * off[0]);
        if (k_lo + s * kGK + kGK <= k_hi) mma_half(ab + 2 * off[1], wb + 2 * off[1]);
    }
    // Output: each wave stages its 32 x 64 tile (9 KB) once every wave has
    // finished its reads, then writes whole rows; the partials are written
    // nontemporally (read once, by the next kernel).
    __syncthreads();
    constexpr int kRS = 64 + 4;                  // staging row stride (floats)
    float* cs = reinterpret_cast<float*>(smem + wave * 4608);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) cs[(i * 16 + 4 * q + e) * kRS + j * 16 + (l & 15)] = acc[i][j][e];
    __builtin_amdgcn_wave_barrier();
    float* out = J.C + static_cast<int64_t>(split) * M * N;
    const int64_t r0 = m0 + wm * 32;
    const int c0 = n0 + wn * 64 + (l & 15) * 4;
    f32x4 v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = *reinterpret_cast<const f32x4*>(cs + (t * 4 + q) * kRS + (l & 15) * 4);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t r = r0 + t * 4 + q;
        if (r < M && c0 + 3 < N) {
            __builtin_nontemporal_store(v[t], reinterpret_cast<f32x4*>(out + r * N + c0));
        } else {
            for (int e = 0; e < 4; ++e)
                if (r < M && c0 + e < N) out[r * N + c0 + e] = v[t][e];
        }
    }
}

// ------------------------------------------------------------------- cand --

constexpr int kCR = 32;                 // candidate rows per workgroup
constexpr int kCRSmall = 4;             // the same for calls with few candidates (see launch_cand),
constexpr int kCRMid = 8;               // and with somewhat more
constexpr int kCT = 512;                // threads of a candidate workgroup
constexpr int kCW = kCT / kWave;        // its waves
constexpr int kCRows = 4 * kCW;         // 16-lane rows it processes at a time

// LayerNorm of one row of R values held by the 16 lanes of a DPP row, R/16
// consecutive values per lane; statistics in float32, biased variance.
template <int R>
__device__ __forceinline__ void row16_layernorm(float (&v)[R / 16], float eps) {
    constexpr int VPL = R / 16;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) s += v[i];
    const float mean = row16_sum(s) * (1.0f / R);
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        v[i] -= mean;
        q += v[i] * v[i];
    }
    const float inv = 1.0f / sqrtf(row16_sum(q) * (1.0f / R) + eps);
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] *= inv;
}

__host__ __device__ inline int cand_us(int r, int dvec) { return (dvec > r ? dvec : r) + 4; }
// Distinct slots a group of cr consecutive candidates can touch.
__host__ __device__ inline int cand_slots(int K, int cr) {
    const int s = (cr - 1) / K + 2;
    return s < cr ? s : cr;
}
__host__ __device__ inline int cand_as(int r) { return 4 * r + 8; }

// acc = A (16 rows of LDS bf16 [hi | lo], 2 * KIN wide) x W^T for one 16-column
// tile of W ([*][ldw] bf16, rows w_row0 + 0..15, columns 0..KIN-1).  The hi and
// lo halves of A meet the same W columns, so acc ~ A_fp32 x W^T.  All W
// fragments are loaded before the first MFMA.  Rows past M read row M - 1
// (every fragment read is unconditional, so they are issued together); their
// results are not used, and a row's results depend on that row only.
template <int KIN>
__device__ __forceinline__ f32x4 mfma_hilo_tile(const uint16_t* abuf, int as, int M, const uint16_t* W,
                                                int ldw, int w_row0) {
    constexpr int KS = (2 * KIN + 31) / 32;
    const int l = lane_id();
    const int kq = 8 * (l >> 4);
    const int m = l & 15;
    const uint16_t* wp = W + static_cast<int64_t>(w_row0 + m) * ldw;
    u32x4 bv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bv[ks] = load16(wp + ((ks * 32 + kq) % KIN));
    const uint16_t* arow = abuf + min(m, M - 1) * as + kq;
    u32x4 av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) av[ks] = *reinterpret_cast<const u32x4*>(arow + ks * 32);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(av[ks], bv[ks], acc);
    return acc;
}

// As mfma_hilo_tile, with the W fragments already in registers.
template <int KIN>
__device__ __forceinline__ f32x4 mfma_hilo_tile_w(const uint16_t* abuf, int as, int M,
                                                  const u32x4 (&bv)[(2 * KIN + 31) / 32]) {
    constexpr int KS = (2 * KIN + 31) / 32;
    const int l = lane_id();
    const int kq = 8 * (l >> 4);
    const int m = l & 15;
    const uint16_t* arow = abuf + min(m, M - 1) * as + kq;
    u32x4 av[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) av[ks] = *reinterpret_cast<const u32x4*>(arow + ks * 32);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(av[ks], bv[ks], acc);
    return acc;
}

// Splits N float32 values into bf16 hi and lo parts (v ~ hi + lo to 2^-16).
template <int N>
__device__ __forceinline__ void split_hilo(const float (&v)[N], uint16_t (&hi)[N], uint16_t (&lo)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        hi[i] = f32_to_bf16(v[i]);
        lo[i] = f32_to_bf16(v[i] - bf16_to_f32(hi[i]));
    }
}

// Stores N consecutive bf16 values with the widest aligned stores (N * 2
// bytes; dst is aligned to that size or to 16 bytes).
template <int N>
__device__ __forceinline__ void store_bf16s(uint16_t* dst, const uint16_t (&v)[N]) {
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int j = 0; j < N / 8; ++j) {
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                w[q] = static_cast<uint32_t>(v[8 * j + 2 * q]) | (static_cast<uint32_t>(v[8 * j + 2 * q + 1]) << 16);
            *reinterpret_cast<u32x4*>(dst + 8 * j) = w;
        }
    } else if constexpr (N == 4) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(static_cast<uint32_t>(v[0]) | (static_cast<uint32_t>(v[1]) << 16),
                                                   static_cast<uint32_t>(v[2]) | (static_cast<uint32_t>(v[3]) << 16));
    } else if constexpr (N == 2) {
        *reinterpret_cast<uint32_t*>(dst) = static_cast<uint32_t>(v[0]) | (static_cast<uint32_t>(v[1]) << 16);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = v[i];
    }
}

// One workgroup per CR consecutive candidates (nodes) of the [rows][K] list:
//   u = W_cand E[c]   the candidate GEMM's split partials summed in order (or
//                     a row of the folded table when one is given)
//   b = LN(u), g = LN(W_ctx h) for the candidate's slot (from hproj)
//   z = gamma * LN(W_fuse [b; g]) + beta, W_fuse on MFMA over [b; g] hi | lo
//   stored as bf16 z hi | lo; cosine: unit(W_out z), unit(W_in z).
// Loops over r are compile-time so each phase issues all of its loads at once.
// Every candidate's values are computed the same way whatever CR is (each row
// of an MFMA tile, and each LayerNorm, depends on its own row only), so the
// two group sizes give identical results.
template <int R, int CR>
__global__ __launch_bounds__(kCT) void cand_kernel(CandArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    constexpr int NCT = R / 16;
    const int tid = threadIdx.x;
    const int l = lane_id();
    const int wave = tid >> 6;
    const int64_t nodes = a.rows * a.K;
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * CR;
    const int M = static_cast<int>(min(static_cast<int64_t>(CR), nodes - n0));
    if (a.zero_cnt && blockIdx.x == 0)   // the cosine launch's per-request counts
        for (int i = tid; i < a.zero_n; i += kCT) a.zero_cnt[static_cast<int64_t>(i) * kCntStride] = 0;
    const int us = cand_us(R, a.vout ? a.dvec : 0);
    const int as = cand_as(R);
    float* ubuf = reinterpret_cast<float*>(smem_raw);                     // [CR][us]
    uint16_t* abuf = reinterpret_cast<uint16_t*>(smem_raw + CR * us * 4);  // [CR][as]
    float* gs = reinterpret_cast<float*>(smem_raw + CR * us * 4 + CR * as * 2);  // [cand_slots(K, CR)][R]

    // ---- W_fuse fragments of this wave's column tiles (ct = wave + kCW c),
    // issued first so they arrive with the u loads below
    constexpr int KSF = (2 * (2 * R) + 31) / 32;
    constexpr int CPW = (NCT + kCW - 1) / kCW;
    u32x4 wfr[CPW][KSF];
    {
        const int kq = 8 * (l >> 4);
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int ct = min(wave + kCW * c, NCT - 1);  // clamped tiles are not used
            const uint16_t* wp = a.w_fuse + static_cast<int64_t>(ct * 16 + (l & 15)) * (2 * R);
#pragma unroll
            for (int ks = 0; ks < KSF; ++ks) wfr[c][ks] = load16(wp + ((ks * 32 + kq) % (2 * R)));
        }
    }

    // nodes < 2^30 (rows <= 2^24, K <= 64): 32-bit slot arithmetic
    const int n0i = static_cast<int>(n0);
    const int t0 = n0i / a.K;
    const int nslot = (n0i + M - 1) / a.K - t0 + 1;
    const int64_t hs = a.rows * a.hstride;

    // ---- u: a row of the folded table, or the candidate GEMM's split
    // partials (four consecutive columns per thread and load).  The loads are
    // only issued here; they are summed after the slot-state loads below have
    // been issued too, so all of the prologue's memory latency overlaps.
    constexpr int PER4 = (CR * R / 4 + kCT - 1) / kCT;
    float4 ut[PER4][kMaxUSplits];
#pragma unroll
    for (int q = 0; q < PER4; ++q) {
        const int e = (tid + kCT * q) * 4;
        const int m = min(e / R, M - 1), c = e % R;  // rows past M are not stored
        if (a.table) {
            int64_t tok = a.ids[n0 + m];
            tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
            ut[q][0] = *reinterpret_cast<const float4*>(a.table + tok * R + c);
        } else {
            const float* base = a.upart + (n0 + m) * R + c;
#pragma unroll
            for (int i = 0; i < kMaxUSplits; ++i)
                ut[q][i] = *reinterpret_cast<const float4*>(base + (i < a.usplits ? i : a.usplits - 1) * nodes * R);
        }
    }

    // ---- per-slot state from the hidden-state projection partials, each
    // value summed in split order, spread over all threads: W_ctx h of the
    // group's slots (into gs, normalised below) and, for the slots whose first
    // candidate the group holds, g_t (published below) and the pair state
    // s_t = W_pair,L h_t + W_pair,R h_{t+1}
    for (int idx = tid; idx < nslot * R; idx += kCT) {
        const int sl = idx / R, c = idx % R;
        const int64_t t = t0 + sl;
        const float* hp = a.hproj + t * a.hstride;
        const bool pair = a.s_out && t * a.K >= n0 && (t % a.B) != a.B - 1;
        const float gv = sum_strided<kMaxSplits>(hp + c, hs, a.splits);
        if (pair) {
            const float sv = sum_strided<kMaxSplits>(hp + R + c, hs, a.splits) +
                             sum_strided<kMaxSplits>(hp + a.hstride + 2 * R + c, hs, a.splits);
            a.s_out[((t / a.B) * (a.B - 1) + t % a.B) * R + c] = sv;
        }
        gs[idx] = gv;
    }

    // ---- u sums (split order) into ubuf
#pragma unroll
    for (int q = 0; q < PER4; ++q) {
        const int e = (tid + kCT * q) * 4;
        float4 sum = ut[q][0];
        if (!a.table) {
#pragma unroll
            for (int i = 1; i < kMaxUSplits; ++i)
                if (i < a.usplits)
                    sum = make_float4(sum.x + ut[q][i].x, sum.y + ut[q][i].y, sum.z + ut[q][i].z, sum.w + ut[q][i].w);
        }
        if (e / R < M) *reinterpret_cast<float4*>(ubuf + (e / R) * us + e % R) = sum;
    }
    __syncthreads();

    // Rows are processed 16 lanes each (4 per wave, kCRows per pass of the
    // workgroup): lane c16 = l & 15 holds columns c16*VPL .. c16*VPL+VPL-1.
    constexpr int VPL = R / 16;
    const int c16 = l & 15;
    const int rsub = wave * 4 + (l >> 4);   // 0..kCRows-1
    // ---- g = LN(W_ctx h) of the group's slots, in place; the workgroup
    // holding a slot's first candidate publishes g_t
    for (int sl = rsub; sl < nslot; sl += kCRows) {
        const int64_t t = t0 + sl;
        float gv[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) gv[i] = gs[sl * R + c16 * VPL + i];
        row16_layernorm<R>(gv, a.eps);
        const bool owner = t * a.K >= n0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            gs[sl * R + c16 * VPL + i] = gv[i];
            if (owner) a.g_out[t * R + c16 * VPL + i] = gv[i];
        }
    }
    __syncthreads();

    // ---- b = LN(u) per row; [b; g] as bf16 hi | lo rows in abuf
    for (int m = rsub; m < M; m += kCRows) {
        float bv[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) bv[i] = ubuf[m * us + c16 * VPL + i];
        row16_layernorm<R>(bv, a.eps);
        const int sl = (n0i + m) / a.K - t0;
        float gv[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) gv[i] = gs[sl * R + c16 * VPL + i];
        // row layout [b hi | g hi | b lo | g lo], each R wide
        uint16_t* arow = abuf + m * as + c16 * VPL;
        uint16_t hi[VPL], lo[VPL];
        split_hilo<VPL>(bv, hi, lo);
        store_bf16s<VPL>(arow, hi);
        store_bf16s<VPL>(arow + 2 * R, lo);
        split_hilo<VPL>(gv, hi, lo);
        store_bf16s<VPL>(arow + R, hi);
        store_bf16s<VPL>(arow + 3 * R, lo);
    }
    __syncthreads();

    // ---- y = W_fuse [b; g] (MFMA on the hi / lo split), into ubuf
    const int nrt = (M + 15) / 16;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int ct = wave + kCW * c;
        if (ct >= NCT) break;
        for (int rt = 0; rt < nrt; ++rt) {
            const f32x4 acc = mfma_hilo_tile_w<2 * R>(abuf + rt * 16 * as, as, M - rt * 16, wfr[c]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (CR % 16 == 0 || rt * 16 + 4 * (l >> 4) + i < CR)   // a tile's rows past the group (CR = 4, 8) are not kept
                    ubuf[(rt * 16 + 4 * (l >> 4) + i) * us + ct * 16 + (l & 15)] = acc[i];
        }
    }
    // cosine variant: this wave's W_out and W_in fragments (column tile
    // ct = wave of each map; dvec <= 16 kCW), issued now so that they arrive
    // during the LayerNorm of z
    constexpr int KSV = (2 * R + 31) / 32;
    const int nvt = a.vout ? a.dvec / 16 : 0;
    u32x4 bvm[2][KSV];
    if (wave < nvt) {
        const int kq = 8 * (l >> 4);
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const uint16_t* wp = (which ? a.w_in : a.w_out) + static_cast<int64_t>(wave * 16 + (l & 15)) * R;
#pragma unroll
            for (int ks = 0; ks < KSV; ++ks) bvm[which][ks] = load16(wp + ((ks * 32 + kq) % R));
        }
    }
    __syncthreads();

    // ---- z = gamma * LN(y) + beta; stored as bf16 hi | lo (and kept in abuf)
    for (int m = rsub; m < M; m += kCRows) {
        float zv[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) zv[i] = ubuf[m * us + c16 * VPL + i];
        row16_layernorm<R>(zv, a.eps);
        uint16_t* grow = a.zhl + (n0 + m) * (2 * R) + c16 * VPL;
        uint16_t* arow = abuf + m * as + c16 * VPL;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const int c = c16 * VPL + i;
            zv[i] = fmaf(a.gamma[c], zv[i], a.beta[c]);
        }
        // z as [hi | lo] rows, in memory and in abuf
        uint16_t hi[VPL], lo[VPL];
        split_hilo<VPL>(zv, hi, lo);
        store_bf16s<VPL>(grow, hi);
        store_bf16s<VPL>(grow + R, lo);
        store_bf16s<VPL>(arow, hi);
        store_bf16s<VPL>(arow + R, lo);
    }
    if (!a.vout) return;
    __syncthreads();

    // ---- cosine variant: unit(W_out z) then unit(W_in z), one map at a time;
    // wave w < dvec / 16 forms column tile w of the map over every row tile
    const int dv = a.dvec;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        if (wave < nvt) {
            for (int rt = 0; rt < nrt; ++rt) {
                const f32x4 acc = mfma_hilo_tile_w<R>(abuf + rt * 16 * as, as, M - rt * 16, bvm[which]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (CR % 16 == 0 || rt * 16 + 4 * (l >> 4) + i < CR)   // a tile's rows past the group (CR = 4, 8) are not kept
                        ubuf[(rt * 16 + 4 * (l >> 4) + i) * us + wave * 16 + (l & 15)] = acc[i];
            }
        }
        __syncthreads();
        for (int m = rsub; m < M; m += kCRows) {
            // dv = 16 * (dv / 16) columns, dv / 16 per lane of the row
            const int vpl = dv / 16;
            const float* v = ubuf + m * us + c16 * vpl;
            float q = 0.f;
            for (int i = 0; i < vpl; ++i) q += v[i] * v[i];
            const float inv = 1.0f / fmaxf(sqrtf(row16_sum(q)), 1e-12f);
            float* dst = (which ? a.vin : a.vout) + (n0 + m) * dv + c16 * vpl;
            for (int i = 0; i < vpl; ++i) dst[i] = v[i] * inv;
        }
        __syncthreads();
    }
}

}  // namespace

int64_t gemm_launch_blocks(const GemmJob& j) { return gemm_blocks_256(j); }

static int64_t small_tiles(const GemmJob& j) { return ((j.M + 15) / 16) * ((j.N + 15) / 16) * j.splits; }

void gemm_pick_small(GemmJob& j, int bm, int bn) {
    // operand bytes per CU (256 CUs): a tiled workgroup reads bm + bn rows of
    // its k-range, and the workgroups run in ceil(blocks / 256) rounds; the
    // small form spreads 32 rows of a k-range per 16 x 16 tile over all CUs
    const int64_t kper = ((j.kdim / 32 + j.splits - 1) / j.splits) * 32;
    const int64_t blocks = ((j.M + bm - 1) / bm) * ((j.N + bn - 1) / bn) * j.splits;
    const int64_t tiles = ((j.M + 15) / 16) * ((j.N + 15) / 16) * j.splits;
    const int64_t tiled = (bm + bn) * kper * ((blocks + 255) / 256);
    const int64_t small = (tiles * 32 * kper + 255) / 256;
    j.small = j.M > 0 && small < tiled ? 1 : 0;
}

hipError_t launch_gemm2(const GemmJob& j0, const GemmJob& j1, hipStream_t stream) {
    const int64_t b0 = gemm_launch_blocks(j0);
    return launch(gemm_kernel, dim3(static_cast<unsigned>(b0 + gemm_launch_blocks(j1))), 256, 0, stream, j0, j1, b0);
}

hipError_t launch_gemm_gather(const GemmJob& j, hipStream_t stream) {
    if (j.W.kwrap > 0 || j.kdim % 32 != 0) return hipErrorInvalidValue;
    if (j.small) {
        const int64_t pairs = ((j.M + 15) / 16) * (((j.N + 15) / 16 + 1) / 2) * j.splits;
        return launch(gemm_small_kernel, dim3(static_cast<unsigned>(pairs)), 128, 0, stream, j);
    }
    const int64_t blocks = ((j.M + kGM - 1) / kGM) * ((j.N + kGN - 1) / kGN) * j.splits;
    return launch(gemm_gather_kernel, dim3(static_cast<unsigned>(blocks)), kGThreads, 0, stream, j);
}

hipError_t launch_gemm(const GemmA& A, const GemmW& W, int64_t M, int N, int kdim, int splits, float* C,
                       hipStream_t stream) {
    GemmJob j{A, W, M, N, kdim, splits, C, 0};
    GemmJob none = j;
    none.M = 0;
    return launch_gemm2(j, none, stream);
}

static size_t cand_lds_cr(int r, int dvec, int K, int cr) {
    return sizeof(float) * cr * cand_us(r, dvec) + sizeof(uint16_t) * cr * cand_as(r) +
           sizeof(float) * cand_slots(K, cr) * r;
}

size_t cand_lds_bytes(int r, int dvec, int K) {
    size_t m = cand_lds_cr(r, dvec, K, kCR);
    for (const int cr : {kCRSmall, kCRMid}) {
        const size_t b = cand_lds_cr(r, dvec, K, cr);
        m = b > m ? b : m;
    }
    return m;
}

template <int CR>
static hipError_t launch_cand_cr(const CandArgs& a, int64_t nodes, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((nodes + CR - 1) / CR));
    const size_t lds = cand_lds_cr(a.r, a.vout ? a.dvec : 0, a.K, CR);
    switch (a.r) {
        case 16: return launch(cand_kernel<16, CR>, grid, kCT, lds, stream, a);
        case 32: return launch(cand_kernel<32, CR>, grid, kCT, lds, stream, a);
        case 64: return launch(cand_kernel<64, CR>, grid, kCT, lds, stream, a);
        case 128: return launch(cand_kernel<128, CR>, grid, kCT, lds, stream, a);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_cand(const CandArgs& a, hipStream_t stream) {
    // The smallest group (4, 8, else 32 candidates) that still fits one
    // workgroup per CU: every group reads all of W_fuse, so with few
    // candidates small groups spread those loads over more CUs
    const int64_t nodes = a.rows * a.K;
    if ((nodes + kCRSmall - 1) / kCRSmall <= 256) return launch_cand_cr<kCRSmall>(a, nodes, stream);
    if ((nodes + kCRMid - 1) / kCRMid <= 256) return launch_cand_cr<kCRMid>(a, nodes, stream);
    return launch_cand_cr<kCR>(a, nodes, stream);
}

}  // namespace corr
