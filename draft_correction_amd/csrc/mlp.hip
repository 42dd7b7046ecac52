// Step (4) of the DCOCO method details: the transition scores
//   S_p(a,b) = l_{p+1}(b) + w2 . GELU(W1 [s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)] + b1) + b2
// for every adjacent drafted-slot pair p and candidate pair (a, b).
//
// Layer 1 is evaluated through the exact column-block identity
//   W1 x = (W1_s s_p + b1 + W1_za z_p^a + w_la l_p(a)) + (W1_zb z_{p+1}^b + w_lb l_{p+1}(b))
//        =              P_p[a]                        +            Q_p[b]
// so the K^2 x (3r+2) x h product collapses to two K x 2r x h MFMA products
// per pair plus a K x K broadcast add; the pair state s_p enters once per
// pair through c_p = W1_s s_p + b1 (one more MFMA row).  The MFMA inputs are z split into bf16
// hi + lo parts (z = hi + lo to ~2^-16), against the same W1 columns twice, so
// P and Q carry float32 accuracy.  The epilogue is the GELU over all K^2 x h
// pre-activations and the h -> 1 dot with w2, one (a, b) per thread.
//
// Work is split into (pair, block of 64 hidden units) workgroups, so a pass
// has (B-1) * n * h/64 of them to balance over the CUs and each block's W1
// columns are read once per pair.  Each block writes its partial Delta; the
// finishing kernel adds the blocks in order, adds b2 and l_{p+1}(b) and walks.
// Every sum runs in a fixed order with no atomics: bit-reproducible.
#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

// GELU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|), with Phi(-t) from
// Abramowitz & Stegun 26.2.17 (Hastings): Phi(-t) = phi(t) (b1 k + ... + b5 k^5),
// k = 1 / (1 + p t), |error| < 7.5e-8; phi's 1/sqrt(2 pi) is folded into b.
// In float32 the result is within 4e-7 of the exact erf form everywhere.
__device__ __forceinline__ float gelu(float x) {
    const float t = fabsf(x);
    const float k = __builtin_amdgcn_rcpf(fmaf(0.2316419f, t, 1.0f));
    float poly = fmaf(k, 0.530702714f, -0.726576013f);  // b5, b4 (times 1/sqrt(2 pi))
    poly = fmaf(k, poly, 0.710706871f);                 // b3
    poly = fmaf(k, poly, -0.142248368f);                // b2
    poly = fmaf(k, poly, 0.127414796f);                 // b1
    poly *= k;
    const float e = __builtin_amdgcn_exp2f(t * t * -0.72134752f);  // exp(-t^2 / 2)
    return fmaxf(x, 0.0f) - (t * e) * poly;
}

// Hidden units handled by one workgroup (a multiple of 16 and of 8).
constexpr int kJB = 64;

// One 16-column tile of P (which = 0) or Q (which = 1) for hidden units
// j0 .. j0+15: rows are the K candidates of the slot, computed on MFMA from
// z hi | lo; P also carries c_p = W1_s s_p + b1, itself one MFMA row over
// s_p hi | lo (shv).  Written to P/Q in LDS.
template <int R>
__device__ __forceinline__ void pq_tile(const MlpArgs& a, int which, int j0, int64_t zrow0, int K,
                                        const uint16_t* shv, const float* lp, const float* lq, float* dst,
                                        int dcol, int PS) {
    constexpr int KS = 2 * R / 32;
    const int nin = 3 * R + 2;
    const int l = lane_id();
    const int kq = 8 * (l >> 4);
    const int j = j0 + (l & 15);
    const uint32_t* wz = reinterpret_cast<const uint32_t*>(a.w1 + static_cast<int64_t>(j) * nin + (which ? 2 * R : R));
    const uint32_t* ws = reinterpret_cast<const uint32_t*>(a.w1 + static_cast<int64_t>(j) * nin);
    const u32x4 zero = {0u, 0u, 0u, 0u};
    u32x4 bz[KS], bs[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int o = ((ks * 32 + kq) % R) / 2;   // same W1 columns for hi and lo
        bz[ks] = u32x4{wz[o], wz[o + 1], wz[o + 2], wz[o + 3]};
        bs[ks] = which ? zero : u32x4{ws[o], ws[o + 1], ws[o + 2], ws[o + 3]};
    }
    const float wl = bf16_to_f32(a.w1[static_cast<int64_t>(j) * nin + 3 * R + which]);
    const float b1j = which ? 0.f : a.b1[j];
    const int nrt = (K + 15) / 16;
    // z fragments of a row tile (rows past K read row 0 and are zeroed)
    auto zfrag = [&](int rt, u32x4* af) {
        const int m = rt * 16 + (l & 15);
        const uint16_t* zr = a.zhl + (zrow0 + (m < K ? m : 0)) * (2 * R);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 v = load16(zr + ks * 32 + kq);
            af[ks] = m < K ? v : zero;
        }
    };
    u32x4 af[KS];
    zfrag(0, af);  // issued with the weight loads above, before any MFMA
    float cj = 0.f;
    if (!which) {
        // c_p tile: A row 0 = [s_hi | s_lo], other rows zero
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 av = (l & 15) == 0 ? *reinterpret_cast<const u32x4*>(shv + ks * 32 + kq) : zero;
            acc = mfma16x16x32(av, bs[ks], acc);
        }
        cj = __shfl(acc[0], l & 15, kWave) + b1j;   // D[0][col] lives in lanes 0..15
    }
    for (int rt = 0; rt < nrt; ++rt) {
        if (rt > 0) zfrag(rt, af);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mfma16x16x32(af[ks], bz[ks], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int mm = rt * 16 + 4 * (l >> 4) + i;
            if (mm < K) dst[mm * PS + dcol + (l & 15)] = acc[i] + fmaf(wl, which ? lq[mm] : lp[mm], cj);
        }
    }
}

// One workgroup per (pair, block of up to 64 hidden units): P, Q and c_p for
// the block's units on MFMA, then GELU and the dot with w2 over all K^2
// candidate pairs; the block's partial Delta goes to part[pair][block][a][b].
template <int R>
__global__ __launch_bounds__(256) void mlp_kernel(MlpArgs a) {
    const int wave = threadIdx.x >> 6;
    const int tid = threadIdx.x;
    const int B = a.B, K = a.K, h = a.h;
    const int nj = (h + kJB - 1) / kJB;
    // Consecutive workgroup numbers go to different XCDs (round-robin over 8):
    // the hidden blocks of one pair are numbered 8 apart so they share an
    // XCD, and its L2 serves the pair's z rows after the first fetch.
    const int lin = blockIdx.x;
    const int xcd = lin % 8, i8 = lin / 8;
    const int jblk = i8 % nj;
    const int pair = (i8 / nj) * 8 + xcd;
    if (pair >= a.n * (B - 1)) return;
    const int item = pair * nj + jblk;
    const int j0 = jblk * kJB;
    const int jn = min(kJB, h - j0);
    const int req = pair / (B - 1), p = pair % (B - 1);
    const int64_t tp = static_cast<int64_t>(req) * B + p;  // slot rows of the pair
    const int64_t tq = tp + 1;
    constexpr int PS = kJB + 4;     // LDS row stride of P / Q (floats)

    __shared__ __attribute__((aligned(16))) uint16_t shv[2 * 128];  // s_p as bf16 hi | lo
    __shared__ __attribute__((aligned(16))) float w2s[kJB];
    __shared__ float lp[64], lq[64];
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    float* P = dyn;                 // [K][PS]
    float* Q = dyn + K * PS;        // [K][PS]

    // ---- pair state (bf16 hi | lo, computed once per pair), logits, w2
    for (int c = tid; c < 2 * R; c += 256) shv[c] = a.shl[static_cast<int64_t>(pair) * 2 * R + c];
    for (int m = tid; m < K; m += 256) {
        lp[m] = a.vals[tp * K + m];
        lq[m] = a.vals[tq * K + m];
    }
    for (int j = tid; j < kJB; j += 256) w2s[j] = j < jn ? a.w2[j0 + j] : 0.f;
    __syncthreads();

    // ---- P (with c_p) and Q tiles of this block
    const int nct = jn / 16;
    for (int job = wave; job < 2 * nct; job += 4) {
        const int which = job / nct, ct = job % nct;
        pq_tile<R>(a, which, j0 + ct * 16, (which ? tq : tp) * K, K, shv, lp, lq, which ? Q : P, ct * 16, PS);
    }
    __syncthreads();

    // ---- GELU and the dot with w2, one (a, b) per thread
    const int nidx = K * K;
    float* out = a.part + static_cast<int64_t>(item) * nidx;
    for (int idx = tid; idx < nidx; idx += 256) {
        const float* pr = P + (idx / K) * PS;
        const float* qr = Q + (idx % K) * PS;
        float d0 = 0.f, d1 = 0.f;
        for (int j = 0; j < jn; j += 8) {
            const float4 pv0 = *reinterpret_cast<const float4*>(pr + j);
            const float4 qv0 = *reinterpret_cast<const float4*>(qr + j);
            const float4 wv0 = *reinterpret_cast<const float4*>(w2s + j);
            const float4 pv1 = *reinterpret_cast<const float4*>(pr + j + 4);
            const float4 qv1 = *reinterpret_cast<const float4*>(qr + j + 4);
            const float4 wv1 = *reinterpret_cast<const float4*>(w2s + j + 4);
            d0 = fmaf(wv0.x, gelu(pv0.x + qv0.x), d0);
            d1 = fmaf(wv0.y, gelu(pv0.y + qv0.y), d1);
            d0 = fmaf(wv0.z, gelu(pv0.z + qv0.z), d0);
            d1 = fmaf(wv0.w, gelu(pv0.w + qv0.w), d1);
            d0 = fmaf(wv1.x, gelu(pv1.x + qv1.x), d0);
            d1 = fmaf(wv1.y, gelu(pv1.y + qv1.y), d1);
            d0 = fmaf(wv1.z, gelu(pv1.z + qv1.z), d0);
            d1 = fmaf(wv1.w, gelu(pv1.w + qv1.w), d1);
        }
        out[idx] = d0 + d1;
    }
}

}  // namespace

int mlp_blocks(int h) { return (h + kJB - 1) / kJB; }

hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream) {
    const int pairs = a.n * (a.B - 1);
    const dim3 grid(static_cast<unsigned>((pairs + 7) / 8 * 8 * mlp_blocks(a.h)));
    const size_t lds = static_cast<size_t>(2) * a.K * (kJB + 4) * sizeof(float);
    switch (a.r) {
        case 16: return launch(mlp_kernel<16>, grid, 256, lds, stream, a);
        case 32: return launch(mlp_kernel<32>, grid, 256, lds, stream, a);
        case 64: return launch(mlp_kernel<64>, grid, 256, lds, stream, a);
        case 128: return launch(mlp_kernel<128>, grid, 256, lds, stream, a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace corr
