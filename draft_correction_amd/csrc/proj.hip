// Steps (2) and (3) of the DCOCO method details: the LayerNorm-projected
// candidate representations and the per-slot halves of the pair state.
//
//   hproj  one MFMA GEMM over the drafter hidden states h [rows][d] against the
//          stacked [W_ctx; W_pair[:, :d]; W_pair[:, d:]] ([3r][d]): each slot's
//          hidden row is read once and yields W_ctx h (for g), the left half
//          W_pair,L h (for pairs that start at the slot) and the right half
//          W_pair,R h (for pairs that end at it).  The d reduction is split
//          over `splits` workgroups; consumers add the partials in split order.
//   cand   one workgroup per drafted slot and group of up to 16 candidates:
//          gathers the candidates' embedding rows E[c], u = W_cand E[c] on
//          MFMA, b = LN(u) (non-affine), g = LN(W_ctx h) from hproj,
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

// ------------------------------------------------------------------ hproj --
// Grid: x = waves / 4 (wave -> (row tile, 64-column group)), y = d-split.
__global__ __launch_bounds__(256) void hproj_kernel(
    const uint16_t* __restrict__ hidden, int64_t h_req_stride, int64_t h_slot_stride, int B,
    int64_t rows, int d, int r, const uint16_t* __restrict__ w_ctx,
    const uint16_t* __restrict__ w_pair, int kper, float* __restrict__ hproj) {
    const int l = lane_id();
    const int ncols = 3 * r;                      // output row stride
    const int ncomp = w_pair ? 3 * r : r;         // columns computed (no pair state: W_ctx only)
    const int ncg = (ncomp + 63) / 64;
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const int64_t nrt = (rows + 15) / 16;
    if (w >= nrt * ncg) return;
    const int64_t rt = w / ncg;
    const int cg = static_cast<int>(w % ncg);
    const int sk = blockIdx.y;
    const int k_lo = sk * kper;
    const int k_hi = min(d, k_lo + kper);

    const int64_t arow = rt * 16 + (l & 15);
    const bool arow_ok = arow < rows;
    const uint16_t* ap = hidden;
    if (arow_ok) ap = hidden + (arow / B) * h_req_stride + (arow % B) * h_slot_stride;
    const int kq = 8 * (l >> 4);

    const uint16_t* bp[4];
    bool bok[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int col = cg * 64 + ct * 16 + (l & 15);
        bok[ct] = col < ncomp;
        const int c = bok[ct] ? col : 0;
        if (c < r) bp[ct] = w_ctx + static_cast<int64_t>(c) * d;
        else if (c < 2 * r) bp[ct] = w_pair + static_cast<int64_t>(c - r) * (2 * d);
        else bp[ct] = w_pair + static_cast<int64_t>(c - 2 * r) * (2 * d) + d;
    }

    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 zero = {0u, 0u, 0u, 0u};

    for (int k0 = k_lo; k0 < k_hi; k0 += 32) {
        const u32x4 a = arow_ok ? load16(ap + k0 + kq) : zero;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const u32x4 b = bok[ct] ? load16(bp[ct] + k0 + kq) : zero;
            acc[ct] = mfma16x16x32(a, b, acc[ct]);
        }
    }
    float* out = hproj + static_cast<int64_t>(sk) * rows * ncols;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int col = cg * 64 + ct * 16 + (l & 15);
        if (col >= ncomp) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = rt * 16 + 4 * (l >> 4) + i;
            if (row < rows) out[row * ncols + col] = acc[ct][i];
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
    const int kq = 8 * (l >> 4);

    extern __shared__ float smem[];
    const int us = cand_row_stride(r, a.vout ? a.dvec : 0);
    const int as = cand_op_stride(r);
    float* ubuf = smem;                                        // [16][us] fp32
    float* gbuf = ubuf + kCandRows * us;                       // [128]
    uint16_t* abuf = reinterpret_cast<uint16_t*>(gbuf + 128);  // [16][as] bf16

    // ---- u = E[c] W_cand^T (MFMA; E and W_cand are bf16, exact products)
    {
        const int m = l & 15;
        const bool eok = m < M;
        int64_t tok = eok ? a.ids[t * a.K + m0 + m] : 0;
        tok = tok < 0 ? 0 : (tok >= a.V ? a.V - 1 : tok);
        const uint16_t* ep = a.embed + tok * a.de;
        const int ct0 = wave, ct1 = wave + 4;
        const bool c0ok = ct0 < nct, c1ok = ct1 < nct;
        const uint16_t* wp0 = a.w_cand + static_cast<int64_t>((c0ok ? ct0 : 0) * 16 + m) * a.de;
        const uint16_t* wp1 = a.w_cand + static_cast<int64_t>((c1ok ? ct1 : 0) * 16 + m) * a.de;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const u32x4 zero = {0u, 0u, 0u, 0u};
        if (c0ok) {
            for (int k0 = 0; k0 < a.de; k0 += 32) {
                const u32x4 av = eok ? load16(ep + k0 + kq) : zero;
                acc0 = mfma16x16x32(av, load16(wp0 + k0 + kq), acc0);
                if (c1ok) acc1 = mfma16x16x32(av, load16(wp1 + k0 + kq), acc1);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int mm = 4 * (l >> 4) + i;
                ubuf[mm * us + ct0 * 16 + m] = acc0[i];
                if (c1ok) ubuf[mm * us + ct1 * 16 + m] = acc1[i];
            }
        }
    }
    // ---- g pre-activation: the hproj partials summed in split order
    for (int c = threadIdx.x; c < r; c += blockDim.x) {
        float s = 0.f;
        for (int sk = 0; sk < a.splits; ++sk) s += a.hproj[(static_cast<int64_t>(sk) * a.rows + t) * (3 * r) + c];
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

hipError_t launch_hproj(const uint16_t* hidden, int64_t h_req_stride, int64_t h_slot_stride,
                        int B, int64_t rows, int d, int r, const uint16_t* w_ctx,
                        const uint16_t* w_pair, int splits, float* hproj, hipStream_t stream) {
    const int ncg = ((w_pair ? 3 * r : r) + 63) / 64;
    const int64_t waves = ((rows + 15) / 16) * ncg;
    const int kper = ((d / 32 + splits - 1) / splits) * 32;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4), static_cast<unsigned>(splits));
    hproj_kernel<<<grid, 256, 0, stream>>>(hidden, h_req_stride, h_slot_stride, B, rows, d, r,
                                           w_ctx, w_pair, kper, hproj);
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
