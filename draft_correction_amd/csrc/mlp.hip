// Step (4) of the DCOCO method details: the transition scores
//   S_p(a,b) = l_{p+1}(b) + w2 . GELU(W1 [s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)] + b1) + b2
// for every adjacent drafted-slot pair p and candidate pair (a, b).
//
// One workgroup per pair (4 waves).  The pair state s_p = W_pair,L h_p +
// W_pair,R h_{p+1} is assembled once from the hproj partials, and its layer-1
// contribution c_p = W1[:, s-block] s_p + b1 is formed once per pair in fp32
// and shared by all K^2 transitions.  The dense part of layer 1 runs on MFMA
// (v_mfma_f32_16x16x32_bf16) with rows (a, b) = [z_p^a ; z_{p+1}^b] (K = 2r)
// against W1's z columns, which each wave keeps in registers for its 64
// hidden units.  One extra 32-wide K step carries the remaining terms exactly:
// A = [l_p(a) hi, lo, l_{p+1}(b) hi, lo, 1, 1, 0...] against
// B = [w1_la, w1_la, w1_lb, w1_lb, c_p hi, c_p lo, 0...] (hi/lo = bf16 split),
// so the accumulator ends as the full pre-activation.  The epilogue applies
// GELU, the 256 -> 1 dot with w2 (lane, then 16-lane butterfly, then the four
// waves in fixed order) and adds b2 and l_{p+1}(b).  No atomics: results are
// bit-reproducible.
#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16(v);
    lo = f32_to_bf16(v - bf16_to_f32(hi));
}

template <int R>
__global__ __launch_bounds__(256) void mlp_kernel(MlpArgs a) {
    constexpr int KS = 2 * R / 32;  // MFMA K steps over [z_a; z_b]
    constexpr int ZS = R + 8;       // LDS row stride of z tiles (bf16)
    const int l = lane_id();
    const int wave = threadIdx.x >> 6;
    const int tid = threadIdx.x;
    const int B = a.B, K = a.K, h = a.h;
    const int pair = blockIdx.x;
    const int req = pair / (B - 1), p = pair % (B - 1);
    const int64_t tp = static_cast<int64_t>(req) * B + p;  // slot rows of the pair
    const int64_t tq = tp + 1;
    const int64_t nslots = static_cast<int64_t>(a.n) * B;

    __shared__ float sv[128];
    __shared__ float cvec[256];
    __shared__ __attribute__((aligned(16))) uint16_t bx[256][8];
    __shared__ float red[4][256];
    extern __shared__ __attribute__((aligned(16))) uint16_t dyn[];
    uint16_t* zp = dyn;                       // [K][ZS]
    uint16_t* zq = zp + K * ZS;               // [K][ZS]
    float* lp = reinterpret_cast<float*>(zq + K * ZS);  // [K]
    float* lq = lp + K;                                 // [K]

    // ---- pair state and staging
    for (int c = tid; c < R; c += 256) {
        float s = 0.f;
        for (int sk = 0; sk < a.splits; ++sk) s += a.hproj[(sk * nslots + tp) * (3 * R) + R + c];
        for (int sk = 0; sk < a.splits; ++sk) s += a.hproj[(sk * nslots + tq) * (3 * R) + 2 * R + c];
        sv[c] = s;
        if (a.s_out) a.s_out[static_cast<int64_t>(pair) * R + c] = s;
    }
    for (int idx = tid; idx < K * (R / 8); idx += 256) {
        const int m = idx / (R / 8), c8 = (idx % (R / 8)) * 8;
        *reinterpret_cast<u32x4*>(zp + m * ZS + c8) = load16(a.z + (tp * K + m) * R + c8);
        *reinterpret_cast<u32x4*>(zq + m * ZS + c8) = load16(a.z + (tq * K + m) * R + c8);
    }
    for (int m = tid; m < K; m += 256) {
        lp[m] = a.vals[tp * K + m];
        lq[m] = a.vals[tq * K + m];
    }
    __syncthreads();

    // ---- c_p = W1[:, 0:R] s_p + b1 (fp32), and the extra-K-step B rows
    const int nin = 3 * R + 2;
    for (int j = tid; j < h; j += 256) {
        const uint16_t* w = a.w1 + static_cast<int64_t>(j) * nin;
        float acc = a.b1[j];
        for (int c = 0; c < R; ++c) acc += bf16_to_f32(w[c]) * sv[c];
        cvec[j] = acc;
        uint16_t hi, lo;
        split_bf16(acc, hi, lo);
        bx[j][0] = w[3 * R];
        bx[j][1] = w[3 * R];
        bx[j][2] = w[3 * R + 1];
        bx[j][3] = w[3 * R + 1];
        bx[j][4] = hi;
        bx[j][5] = lo;
        bx[j][6] = 0;
        bx[j][7] = 0;
    }
    __syncthreads();

    // ---- this wave's W1 z-column fragments, kept in registers
    const int nct = h / 16;
    const int kq = 8 * (l >> 4);
    u32x4 wf[4][KS];
    u32x4 xf[4];
    float w2c[4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int ct = wave + 4 * q;
        const bool ok = ct < nct;
        const int j = (ok ? ct : 0) * 16 + (l & 15);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(a.w1 + static_cast<int64_t>(j) * nin + R);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int o = (ks * 32 + kq) / 2;   // dword offset; rows are 4-byte aligned
            wf[q][ks] = ok ? u32x4{w[o], w[o + 1], w[o + 2], w[o + 3]} : zero;
        }
        xf[q] = (ok && l < 16) ? *reinterpret_cast<const u32x4*>(&bx[j][0]) : zero;
        w2c[q] = ok ? a.w2[j] : 0.f;
    }

    const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
    const int nrows = K * K;
    const int nrt = (nrows + 15) / 16;
    const float b2 = a.b2[0];
    for (int rb0 = 0; rb0 < nrt; rb0 += 16) {
        const int rb1 = min(nrt, rb0 + 16);
        for (int rt = rb0; rt < rb1; ++rt) {
            const int m = rt * 16 + (l & 15);
            const bool valid = m < nrows;
            const int ia = valid ? m / K : 0, ib = valid ? m % K : 0;
            u32x4 af[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kg = ks * 32 + kq;
                const uint16_t* src = kg < R ? zp + ia * ZS + kg : zq + ib * ZS + (kg - R);
                af[ks] = valid ? *reinterpret_cast<const u32x4*>(src) : zero;
            }
            u32x4 ax = zero;
            if (valid && l < 16) {
                uint16_t ah, al, bh, bl;
                split_bf16(lp[ia], ah, al);
                split_bf16(lq[ib], bh, bl);
                ax = u32x4{static_cast<uint32_t>(ah) | (static_cast<uint32_t>(al) << 16),
                           static_cast<uint32_t>(bh) | (static_cast<uint32_t>(bl) << 16), one2, 0u};
            }
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (wave + 4 * q >= nct) continue;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(af[ks], wf[q][ks], acc);
                acc = mfma16x16x32(ax, xf[q], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) part[i] += w2c[q] * gelu_erf(acc[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) part[i] = wave_sum16(part[i]);
            if ((l & 15) == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wave][(rt - rb0) * 16 + 4 * (l >> 4) + i] = part[i];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < (rb1 - rb0) * 16; idx += 256) {
            const int row = rb0 * 16 + idx;
            if (row < nrows) {
                const float delta = ((red[0][idx] + red[1][idx]) + red[2][idx]) + red[3][idx] + b2;
                const int ib = row % K;
                a.scores[static_cast<int64_t>(pair) * nrows + row] = lq[ib] + delta;
            }
        }
        __syncthreads();
    }
}

}  // namespace

size_t mlp_lds_bytes(int K, int r) {
    return static_cast<size_t>(2) * K * (r + 8) * sizeof(uint16_t) + 2 * K * sizeof(float);
}

hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.n * (a.B - 1)));
    const size_t lds = mlp_lds_bytes(a.K, a.r);
    switch (a.r) {
        case 16: mlp_kernel<16><<<grid, 256, lds, stream>>>(a); break;
        case 32: mlp_kernel<32><<<grid, 256, lds, stream>>>(a); break;
        case 64: mlp_kernel<64><<<grid, 256, lds, stream>>>(a); break;
        case 128: mlp_kernel<128><<<grid, 256, lds, stream>>>(a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace corr
