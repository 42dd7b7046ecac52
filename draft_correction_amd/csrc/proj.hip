// Steps (2) and (3) of the DCOCO method details: the LayerNorm-projected
// candidate representations and the per-slot halves of the pair state.
//
//   gemm   a tiled MFMA GEMM used for (i) hproj: the drafter hidden states h
//          [rows][d] against the stacked [W_ctx; W_pair[:, :d]; W_pair[:, d:]]
//          ([3r][d]): each slot's hidden row is read once and yields W_ctx h
//          (for g), the left half W_pair,L h (for pairs that start at the
//          slot) and the right half W_pair,R h (for pairs that end at it); and
//          (ii) u = W_cand E[c] over the gathered embedding rows of all
//          candidates (or over the whole table, to fold it once).  The
//          reduction is split over a fixed number of workgroups per shape;
//          consumers add the partials in split order.
//   cand   one workgroup per drafted slot and group of up to 16 candidates:
//          b = LN(u) (non-affine), g = LN(W_ctx h) from hproj,
//          y = W_fuse [b; g] on MFMA, z = gamma * LN(y) + beta, stored as
//          bf16 hi | lo halves.  The cosine variant also forms unit(W_out z)
//          and unit(W_in z).  MFMA operands that are not already bf16 (b, g,
//          z) are split into hi + lo bf16 parts multiplied by the same weight
//          columns, so those products carry float32 accuracy.
// All LayerNorm statistics are fp32 over the r features, biased variance.
#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

// ------------------------------------------------------------------- gemm --
// C[split][m][n] = sum over the split's k range of A[m][k] * W[n][k], float32,
// for bf16 A and W stored K-contiguous.  A rows are gathered (embedding rows of
// candidate ids), strided (drafter hidden rows of a slot block) or dense; W
// rows come from up to three blocks of nb rows.  Tile 64 x 128, K slab 64,
// double-buffered in LDS with the next slab's global loads in flight during
// the MFMAs; 4 waves in 2 x 2, each 32 x 64 (2 x 4 v_mfma_f32_16x16x32_bf16).

constexpr int kBM = 64, kBN = 128, kBK = 64, kLS = kBK + 8;  // LDS row stride (bf16)

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

__global__ __launch_bounds__(256) void gemm_kernel(GemmA A, GemmW W, int64_t M, int N, int kper, int kdim,
                                                   float* __restrict__ C) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kLS];
    __shared__ __attribute__((aligned(16))) uint16_t Ws[2][kBN * kLS];
    const int tid = threadIdx.x;
    const int l = lane_id();
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = static_cast<int64_t>(blockIdx.x) * kBM;
    const int n0 = blockIdx.y * kBN;
    const int split = blockIdx.z;
    const int k_lo = split * kper;
    const int k_hi = min(kdim, k_lo + kper);

    // per-thread load assignments: 2 A segments, 4 W segments of 16 bytes
    const uint16_t* ap[2];
    bool aok[2];
    int aoff[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int seg = tid + 256 * i;
        const int r = seg >> 3;
        aoff[i] = r * kLS + (seg & 7) * 8;
        aok[i] = m0 + r < M;
        ap[i] = (aok[i] ? a_row(A, m0 + r) : A.base) + (seg & 7) * 8;
    }
    const uint16_t* wp[4];
    bool wok[4];
    int woff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int seg = tid + 256 * i;
        const int r = seg >> 3;
        const int n = n0 + r;
        woff[i] = r * kLS + (seg & 7) * 8;
        wok[i] = n < N;
        const int nn = wok[i] ? n : 0;
        const int b = nn / W.nb;
        wp[i] = W.base[b] + static_cast<int64_t>(nn % W.nb) * W.ld[b] + (seg & 7) * 8;
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 ra[2], rw[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int kk = k0 + ((tid + 256 * i) & 7) * 8;
            ra[i] = (aok[i] && kk < k_hi) ? load16(ap[i] + k0) : zero;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = k0 + ((tid + 256 * i) & 7) * 8;
            rw[i] = (wok[i] && kk < k_hi) ? load16(wp[i] + k0) : zero;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) *reinterpret_cast<u32x4*>(&As[buf][aoff[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&Ws[buf][woff[i]]) = rw[i];
    };

    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (k_lo < k_hi) {
        load(k_lo);
        store(0);
    }
    __syncthreads();
    const int kq = 8 * (l >> 4);
    int buf = 0;
    for (int k0 = k_lo; k0 < k_hi; k0 += kBK) {
        const bool more = k0 + kBK < k_hi;
        if (more) load(k0 + kBK);
#pragma unroll
        for (int ks = 0; ks < kBK; ks += 32) {
            u32x4 af[2], wf[4];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const u32x4*>(&As[buf][(wm * 32 + i * 16 + (l & 15)) * kLS + ks + kq]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                wf[j] = *reinterpret_cast<const u32x4*>(&Ws[buf][(wn * 64 + j * 16 + (l & 15)) * kLS + ks + kq]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], wf[j], acc[i][j]);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    float* out = C + static_cast<int64_t>(split) * M * N;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + (l & 15);
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + wm * 32 + i * 16 + 4 * (l >> 4) + e;
                if (m < M) out[m * N + n] = acc[i][j][e];
            }
        }
}

// ------------------------------------------------------------------- cand --

constexpr int kCandRows = 16;  // candidates per workgroup (one 16-row MFMA tile)

// LayerNorm of one row of m <= 128 floats held in LDS, by one wave; writes
// gamma * y + beta (or y) to dst, which may alias src.
__device__ void wave_layernorm(const float* src, float* dst, int m, float eps,
                               const float* gamma, const float* beta) {
    const int l = lane_id();
    float v0 = l < m ? src[l] : 0.f;
    float v1 = l + 64 < m ? src[l + 64] : 0.f;
    float s = v0 + v1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
    const float mean = s / static_cast<float>(m);
    const float d0 = l < m ? v0 - mean : 0.f;
    const float d1 = l + 64 < m ? v1 - mean : 0.f;
    float q = d0 * d0 + d1 * d1;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o, kWave);
    const float inv = 1.0f / sqrtf(q / static_cast<float>(m) + eps);
    if (l < m) dst[l] = gamma ? gamma[l] * (d0 * inv) + beta[l] : d0 * inv;
    if (l + 64 < m) dst[l + 64] = gamma ? gamma[l + 64] * (d1 * inv) + beta[l + 64] : d1 * inv;
}

// Row stride (floats) of the fp32 staging rows: u / y need r, the cosine
// out and in vectors need 2 * dvec.
__host__ __device__ inline int cand_row_stride(int r, int dvec) {
    return (2 * dvec > r ? 2 * dvec : r) + 4;
}

// Row stride (bf16) of the MFMA operand rows: [x_hi | x_lo] with x = [b; g]
// (4r wide) or z (2r wide).
__host__ __device__ inline int cand_op_stride(int r) { return 4 * r + 8; }

// acc = A (16 rows of LDS bf16 [hi | lo], 2 * kin wide) x W^T for one 16-column
// tile of W ([*][ldw] bf16, rows w_row0 + 0..15, columns 0..kin-1).  The hi and
// lo halves of A meet the same W columns, so acc ~ A_fp32 x W^T.
__device__ f32x4 mfma_hilo_tile(const uint16_t* abuf, int as, int M, const uint16_t* W, int ldw,
                                int w_row0, int kin) {
    const int l = lane_id();
    const int kq = 8 * (l >> 4);
    const int m = l & 15;
    const uint16_t* wp = W + static_cast<int64_t>(w_row0 + m) * ldw;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < 2 * kin; k0 += 32) {
        const int kg = k0 + kq;
        const u32x4 av = m < M ? *reinterpret_cast<const u32x4*>(abuf + m * as + kg) : zero;
        const u32x4 bv = load16(wp + (kg % kin));
        acc = mfma16x16x32(av, bv, acc);
    }
    return acc;
}

__device__ __forceinline__ void split_store(uint16_t* row, int width, int c, float v) {
    const uint16_t hi = f32_to_bf16(v);
    row[c] = hi;
    row[width + c] = f32_to_bf16(v - bf16_to_f32(hi));
}

__global__ __launch_bounds__(256) void cand_kernel(CandArgs a) {
    const int l = lane_id();
    const int wave = threadIdx.x >> 6;
    const int64_t t = blockIdx.x;                 // drafted-slot row
    const int m0 = blockIdx.y * kCandRows;        // first candidate of this group
    const int M = min(kCandRows, a.K - m0);
    const int r = a.r;
    const int nct = r / 16;

    extern __shared__ float smem[];
    const int us = cand_row_stride(r, a.vout ? a.dvec : 0);
    const int as = cand_op_stride(r);
    float* ubuf = smem;                                        // [16][us] fp32
    float* gbuf = ubuf + kCandRows * us;                       // [128]
    uint16_t* abuf = reinterpret_cast<uint16_t*>(gbuf + 128);  // [16][as] bf16

    // ---- u = W_cand E[c]: the GEMM partials summed in split order, or a row of
    // the folded table T = E W_cand^T
    for (int idx = threadIdx.x; idx < M * r; idx += blockDim.x) {
        const int m = idx / r, c = idx % r;
        const int64_t node = t * a.K + m0 + m;
        float u;
        if (a.table) {
            int64_t tok = a.ids[node];
            tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
            u = a.table[tok * r + c];
        } else {
            u = 0.f;
            for (int sk = 0; sk < a.usplits; ++sk) u += a.upart[(sk * a.rows * a.K + node) * r + c];
        }
        ubuf[m * us + c] = u;
    }
    // ---- g pre-activation: the hproj partials summed in split order
    for (int c = threadIdx.x; c < r; c += blockDim.x) {
        float s = 0.f;
        for (int sk = 0; sk < a.splits; ++sk) s += a.hproj[(static_cast<int64_t>(sk) * a.rows + t) * a.hstride + c];
        gbuf[c] = s;
    }
    __syncthreads();

    // ---- b = LN(u), g = LN(g) (non-affine)
    for (int m = wave; m < M; m += 4) wave_layernorm(ubuf + m * us, ubuf + m * us, r, a.eps, nullptr, nullptr);
    if (wave == 0) wave_layernorm(gbuf, gbuf, r, a.eps, nullptr, nullptr);
    __syncthreads();
    // [b; g] as bf16 hi | lo rows, 4r wide
    for (int idx = threadIdx.x; idx < M * r; idx += blockDim.x) {
        const int m = idx / r, c = idx % r;
        split_store(abuf + m * as, 2 * r, c, ubuf[m * us + c]);
        split_store(abuf + m * as, 2 * r, r + c, gbuf[c]);
    }
    if (blockIdx.y == 0)
        for (int c = threadIdx.x; c < r; c += blockDim.x) a.g[t * r + c] = gbuf[c];
    __syncthreads();

    // ---- y = W_fuse [b; g] (MFMA on the hi/lo split, K = 2 x 2r), into ubuf
    for (int ct = wave; ct < nct; ct += 4) {
        const f32x4 acc = mfma_hilo_tile(abuf, as, M, a.w_fuse, 2 * r, ct * 16, 2 * r);
#pragma unroll
        for (int i = 0; i < 4; ++i) ubuf[(4 * (l >> 4) + i) * us + ct * 16 + (l & 15)] = acc[i];
    }
    __syncthreads();

    // ---- z = gamma * LN(y) + beta; store as bf16 hi | lo (also kept in abuf)
    for (int m = wave; m < M; m += 4) wave_layernorm(ubuf + m * us, ubuf + m * us, r, a.eps, a.gamma, a.beta);
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * r; idx += blockDim.x) {
        const int m = idx / r, c = idx % r;
        const float zv = ubuf[m * us + c];
        uint16_t* grow = a.zhl + (t * a.K + m0 + m) * (2 * r);
        const uint16_t hi = f32_to_bf16(zv);
        const uint16_t lo = f32_to_bf16(zv - bf16_to_f32(hi));
        grow[c] = hi;
        grow[r + c] = lo;
        abuf[m * as + c] = hi;
        abuf[m * as + r + c] = lo;
    }
    if (!a.vout) return;
    __syncthreads();

    // ---- cosine variant: o = W_out z, i = W_in z (MFMA on z hi/lo), unit vectors
    const int dv = a.dvec;
    const int nvt = dv / 16;
    for (int job = wave; job < 2 * nvt; job += 4) {
        const int which = job / nvt, ct = job % nvt;
        const f32x4 acc = mfma_hilo_tile(abuf, as, M, which ? a.w_in : a.w_out, r, ct * 16, r);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ubuf[(4 * (l >> 4) + i) * us + which * dv + ct * 16 + (l & 15)] = acc[i];
    }
    __syncthreads();
    for (int job = wave; job < 2 * M; job += 4) {
        const int m = job >> 1, which = job & 1;
        const float* v = ubuf + m * us + which * dv;
        float x0 = l < dv ? v[l] : 0.f;
        float x1 = l + 64 < dv ? v[l + 64] : 0.f;
        float q = x0 * x0 + x1 * x1;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) q += __shfl_xor(q, o, kWave);
        const float inv = 1.0f / fmaxf(sqrtf(q), 1e-12f);
        float* dst = (which ? a.vin : a.vout) + (t * a.K + m0 + m) * dv;
        if (l < dv) dst[l] = x0 * inv;
        if (l + 64 < dv) dst[l + 64] = x1 * inv;
    }
}

}  // namespace

hipError_t launch_gemm(const GemmA& A, const GemmW& W, int64_t M, int N, int kdim, int splits, float* C,
                       hipStream_t stream) {
    const int kper = ((kdim / 32 + splits - 1) / splits) * 32;
    const dim3 grid(static_cast<unsigned>((M + kBM - 1) / kBM), static_cast<unsigned>((N + kBN - 1) / kBN),
                    static_cast<unsigned>(splits));
    gemm_kernel<<<grid, 256, 0, stream>>>(A, W, M, N, kper, kdim, C);
    return hipGetLastError();
}

size_t cand_lds_bytes(int r, int dvec) {
    return sizeof(float) * (kCandRows * cand_row_stride(r, dvec) + 128) +
           sizeof(uint16_t) * kCandRows * cand_op_stride(r);
}

hipError_t launch_cand(const CandArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.rows), static_cast<unsigned>((a.K + kCandRows - 1) / kCandRows));
    cand_kernel<<<grid, 256, cand_lds_bytes(a.r, a.vout ? a.dvec : 0), stream>>>(a);
    return hipGetLastError();
}

}  // namespace corr
