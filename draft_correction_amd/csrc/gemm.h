// The tiled MFMA GEMM body shared by the projection launches: one 64 x 128
// output tile of one k-split per 256-thread workgroup, LDS supplied by the
// caller (kernels that also run other work in the same launch carve it from
// one shared buffer).
#pragma once

#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

// ------------------------------------------------------------------- gemm --
// C[split][m][n] = sum over the split's k range of A[m][k] * W[n][k], float32,
// for bf16 A and W stored K-contiguous.  A rows are gathered (embedding rows of
// candidate ids), strided (drafter hidden rows of a slot block) or dense; W
// rows come from up to three blocks of nb rows.  Tile 64 x 128, K slab 64,
// double-buffered in LDS, with the global loads of the next two slabs in
// flight (two register sets) during the MFMAs; 4 waves in 2 x 2, each 32 x 64
// (2 x 4 v_mfma_f32_16x16x32_bf16).

constexpr int kBM = 64, kBN = 128, kBK = 64, kLS = kBK + 8;  // LDS row stride (bf16)
constexpr int kSegs = kBK / 8;                 // 16-byte segments per slab row
constexpr int kNA = kBM * kSegs / 256;         // A segments per thread
constexpr int kNW = kBN * kSegs / 256;         // W segments per thread
constexpr int kCS = kBN + 4;                   // output staging row stride (floats)
constexpr int kSlabBytes = 2 * (kBM + kBN) * kLS * 2;
constexpr int kOutBytes = kBM * kCS * 4;
// LDS bytes a gemm_body workgroup needs.
constexpr int kGemmSmem = kSlabBytes > kOutBytes ? kSlabBytes : kOutBytes;

__device__ __forceinline__ const uint16_t* a_row(const GemmA& A, int64_t m) {
    switch (A.mode) {
        case GEMM_A_GATHER: {
            int64_t id = A.ids[m];
            id = id < 0 ? 0 : (id >= A.V ? A.V - 1 : id);
            return A.base + id * A.lda;
        }
        case GEMM_A_SLOTS:
            return A.base + (m / A.B) * A.rs + (m % A.B) * A.ss;
        default:
            return A.base + m * A.lda;
    }
}

// Workgroups are numbered so that consecutive numbers (which the dispatcher
// spreads round-robin over the 8 XCDs) vary the split fastest: with a split
// count dividing 8 every XCD works on one k-slice, and the k-slice of W and
// of the A rows is fetched into that XCD's L2 only.
__device__ __forceinline__ void gemm_body(const GemmJob J, int64_t lin, unsigned char* smem) {
    const GemmA& A = J.A;
    const GemmW& W = J.W;
    const int64_t M = J.M;
    const int N = J.N, kdim = J.kdim, splits = J.splits;
    float* __restrict__ C = J.C;
    const int kper = ((kdim / 32 + splits - 1) / splits) * 32;
    const int ntn = (N + kBN - 1) / kBN;
    // LDS (smem, kGemmSmem bytes, 16-byte aligned): the double-buffered A and
    // W slabs, reused at the end to stage the float32 output tile for
    // row-contiguous stores
    uint16_t (*As)[kBM * kLS] = reinterpret_cast<uint16_t (*)[kBM * kLS]>(smem);
    uint16_t (*Ws)[kBN * kLS] = reinterpret_cast<uint16_t (*)[kBN * kLS]>(smem + 2 * kBM * kLS * 2);
    const int tid = threadIdx.x;
    const int l = lane_id();
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int split = static_cast<int>(lin % splits);
    const int64_t rest = lin / splits;
    const int n0 = static_cast<int>(rest % ntn) * kBN;
    const int64_t m0 = (rest / ntn) * kBM;
    const int k_lo = split * kper;
    const int k_hi = min(kdim, k_lo + kper);

    // per-thread load assignments: 2 A segments, 4 W segments of 16 bytes.
    // Rows past M or N are clamped to the last row (their results are not
    // stored), so every load is issued unconditionally: the number of loads
    // in flight is then fixed and each wait for a slab is exact.
    const uint16_t* ap[kNA];
    int aoff[kNA];
    int sego[kNA + kNW];  // segment column offset within a slab
#pragma unroll
    for (int i = 0; i < kNA; ++i) {
        const int seg = tid + 256 * i;
        const int r = seg / kSegs;
        aoff[i] = r * kLS + (seg % kSegs) * 8;
        sego[i] = (seg % kSegs) * 8;
        ap[i] = a_row(A, min(m0 + r, M - 1));
    }
    const uint16_t* wp[kNW];
    int woff[kNW];
    const int kmask = W.kwrap > 0 ? W.kwrap - 1 : -1;
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
        const int seg = tid + 256 * i;
        const int r = seg / kSegs;
        const int nn = min(n0 + r, N - 1);
        woff[i] = r * kLS + (seg % kSegs) * 8;
        sego[kNA + i] = (seg % kSegs) * 8;
        const int b = nn / W.nb;
        // block select without indexing the argument arrays (keeps them in registers)
        const uint16_t* wb = b == 0 ? W.base[0] : (b == 1 ? W.base[1] : W.base[2]);
        const int64_t wld = b == 0 ? W.ld[0] : (b == 1 ? W.ld[1] : W.ld[2]);
        wp[i] = wb + static_cast<int64_t>(nn % W.nb) * wld;
    }
    const int nslab = k_lo < k_hi ? (k_hi - k_lo + kBK - 1) / kBK : 0;
    // Slab s covers k_lo + s*kBK .. +kBK-1; k ranges are multiples of 32, so
    // only the last slab can be half valid.  Its upper half re-reads the
    // lower half (in bounds) and is zeroed in LDS after the store.  Slab
    // numbers past the last are clamped to it: those loads are never used.
    auto load = [&](int sl, u32x4* ra, u32x4* rw) {
        const int s2 = min(sl, nslab - 1);
        const int k0 = k_lo + s2 * kBK;
        const bool half = k0 + kBK > k_hi;
#pragma unroll
        for (int i = 0; i < kNA; ++i) ra[i] = load16(ap[i] + k0 + (half ? (sego[i] & 31) : sego[i]));
#pragma unroll
        for (int i = 0; i < kNW; ++i)
            rw[i] = load16(wp[i] + ((k0 + (half ? (sego[kNA + i] & 31) : sego[kNA + i])) & kmask));
    };
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto store = [&](int buf, int sl, const u32x4* ra, const u32x4* rw) {
#pragma unroll
        for (int i = 0; i < kNA; ++i) *reinterpret_cast<u32x4*>(&As[buf][aoff[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < kNW; ++i) *reinterpret_cast<u32x4*>(&Ws[buf][woff[i]]) = rw[i];
        if (k_lo + sl * kBK + kBK > k_hi) {  // half slab: clear its upper 32 columns
#pragma unroll
            for (int i = 0; i < kNA; ++i)
                if (sego[i] >= 32) *reinterpret_cast<u32x4*>(&As[buf][aoff[i]]) = zero;
#pragma unroll
            for (int i = 0; i < kNW; ++i)
                if (sego[kNA + i] >= 32) *reinterpret_cast<u32x4*>(&Ws[buf][woff[i]]) = zero;
        }
    };
    // two register sets of slab data: the slabs one and two ahead of the one
    // being multiplied are in flight while it runs
    u32x4 ra0[kNA], rw0[kNW], ra1[kNA], rw1[kNW];

    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kq = 8 * (l >> 4);
    // All fragments of a slab are read from LDS before its MFMAs, so the
    // reads overlap one another and the MFMAs issue back to back.
    auto compute = [&](int buf) {
        constexpr int NKS = kBK / 32;
        u32x4 af[NKS][2], wf[NKS][4];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[ks][i] =
                    *reinterpret_cast<const u32x4*>(&As[buf][(wm * 32 + i * 16 + (l & 15)) * kLS + ks * 32 + kq]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wf[ks][j] =
                    *reinterpret_cast<const u32x4*>(&Ws[buf][(wn * 64 + j * 16 + (l & 15)) * kLS + ks * 32 + kq]);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[ks][i], wf[ks][j], acc[i][j]);
    };

    if (nslab > 0) {
        load(0, ra0, rw0);
        load(1, ra1, rw1);
        store(0, 0, ra0, rw0);
        load(2, ra0, rw0);
        __syncthreads();
        // slab s sits in LDS buffer s & 1; slab s+1 in register set (s + 1) & 1.
        // Two slabs per iteration, no exit in between; an odd last slab after.
        int s = 0;
        for (; s + 2 <= nslab; s += 2) {
            compute(0);
            store(1, s + 1, ra1, rw1);
            load(s + 3, ra1, rw1);
            __syncthreads();
            compute(1);
            store(0, s + 2, ra0, rw0);
            load(s + 4, ra0, rw0);
            __syncthreads();
        }
        if (s < nslab) compute(0);
    }
    float* out = C + static_cast<int64_t>(split) * M * N;
    // stage the tile in LDS, then write whole rows as float4
    float* Cs = reinterpret_cast<float*>(smem);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Cs[(wm * 32 + i * 16 + 4 * (l >> 4) + e) * kCS + wn * 64 + j * 16 + (l & 15)] = acc[i][j][e];
    __syncthreads();
    if ((N & 3) == 0) {
#pragma unroll
        for (int q = 0; q < kBM * kBN / 4 / 256; ++q) {
            const int f = tid + 256 * q;
            const int r = f / (kBN / 4), c = (f % (kBN / 4)) * 4;
            if (m0 + r < M && n0 + c < N)
                *reinterpret_cast<float4*>(out + (m0 + r) * N + n0 + c) =
                    *reinterpret_cast<const float4*>(Cs + r * kCS + c);
        }
    } else {
        for (int f = tid; f < kBM * kBN; f += 256) {
            const int r = f / kBN, c = f % kBN;
            if (m0 + r < M && n0 + c < N) out[(m0 + r) * N + n0 + c] = Cs[r * kCS + c];
        }
    }
}

// ---------------------------------------------------------------- small --
// The same product for calls with few rows: wave t of the launch computes
// one 16 x 16 output tile of one k-split (split fastest), its A and W
// fragments loaded straight into registers, eight 32-wide k-steps in flight
// while the previous eight are multiplied.  Each output takes the same
// sequence of v_mfma_f32_16x16x32_bf16 over the split's k-steps, on the same
// lane layout, as gemm_body, so the partials are identical.
constexpr int kSmallDepth = 8;

__device__ __forceinline__ int64_t gemm_small_tiles(const GemmJob& J) {
    return ((J.M + 15) / 16) * ((J.N + 15) / 16) * J.splits;
}

__device__ __forceinline__ void gemm_small_body(const GemmJob J, int64_t t) {
    if (t >= gemm_small_tiles(J)) return;
    const GemmA& A = J.A;
    const GemmW& W = J.W;
    const int64_t M = J.M;
    const int N = J.N, kdim = J.kdim, splits = J.splits;
    const int l = lane_id();
    const int kper = ((kdim / 32 + splits - 1) / splits) * 32;
    const int ntn = (N + 15) / 16;
    const int split = static_cast<int>(t % splits);
    const int64_t rest = t / splits;
    const int n0 = static_cast<int>(rest % ntn) * 16;
    const int64_t m0 = (rest / ntn) * 16;
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
    const uint16_t* wp = wb + static_cast<int64_t>(nn % W.nb) * wld;
    const int kmask = W.kwrap > 0 ? W.kwrap - 1 : -1;
    // k-steps past the split's last are clamped to it: loaded, never used
    auto ld = [&](int ks0, u32x4 (&a)[kSmallDepth], u32x4 (&w)[kSmallDepth]) {
#pragma unroll
        for (int i = 0; i < kSmallDepth; ++i) {
            const int ks = min(ks0 + i, nks - 1);
            a[i] = load16(ap + 32 * ks);
            w[i] = load16(wp + ((k_lo + 32 * ks + kq) & kmask));
        }
    };
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (nks > 0) {
        u32x4 a0[kSmallDepth], w0[kSmallDepth], a1[kSmallDepth], w1[kSmallDepth];
        ld(0, a0, w0);
        for (int ks = 0; ks < nks; ks += 2 * kSmallDepth) {
            ld(ks + kSmallDepth, a1, w1);
#pragma unroll
            for (int i = 0; i < kSmallDepth; ++i)
                if (ks + i < nks) acc = mfma16x16x32(a0[i], w0[i], acc);
            if (ks + 2 * kSmallDepth < nks) ld(ks + 2 * kSmallDepth, a0, w0);
#pragma unroll
            for (int i = 0; i < kSmallDepth; ++i)
                if (ks + kSmallDepth + i < nks) acc = mfma16x16x32(a1[i], w1[i], acc);
        }
    }
    // lane l holds rows 4 (l / 16) + e of column l % 16
    float* out = J.C + static_cast<int64_t>(split) * M * N;
    const int c = n0 + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t r = m0 + 4 * (l >> 4) + e;
        if (r < M && c < N) out[r * N + c] = acc[e];
    }
}

// Workgroups of 256 threads a GEMM job occupies in a launch (tiled or small).
// The small form runs one tile per workgroup, on its first wave: the form is
// for calls with few tiles, whose time is set by how many CUs share the loads.
__host__ __device__ inline int64_t gemm_blocks_256(const GemmJob& j) {
    if (j.small) return ((j.M + 15) / 16) * ((j.N + 15) / 16) * j.splits;
    return ((j.M + kBM - 1) / kBM) * ((j.N + kBN - 1) / kBN) * j.splits;
}

// Workgroup lin of a job, tiled or small (256 threads; smem: kGemmSmem bytes).
__device__ __forceinline__ void gemm_any_body(const GemmJob& J, int64_t lin, unsigned char* smem) {
    if (J.small) {
        if (threadIdx.x < 64) gemm_small_body(J, lin);
    }
    else
        gemm_body(J, lin, smem);
}

}  // namespace

}  // namespace corr
