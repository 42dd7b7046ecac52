// Step (4) of the DCOCO method details: the transition scores
//   S_p(a,b) = l_{p+1}(b) + w2 . GELU(W1 [s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)] + b1) + b2
// for every adjacent drafted-slot pair p and candidate pair (a, b).
//
// Layer 1 is evaluated through the exact column-block identity
//   W1 x = (W1_s s_p + b1 + W1_za z_p^a + w_la l_p(a)) + (W1_zb z_{p+1}^b + w_lb l_{p+1}(b))
//        =              P_p[a]                        +            Q_p[b]
// so the K^2 x (3r+2) x h product collapses to per-candidate products
// U = W1_za z and V = W1_zb z (each candidate's z meets the weights once,
// whichever pairs it belongs to; the candidate kernel forms them on MFMA
// with z as bf16 hi | lo rows, so they carry float32 accuracy), the per-pair
// c_p = W1_s s_p (float32 dot products here, a quarter of r per thread), and
// a K x K broadcast add.  This kernel forms P and Q and runs the epilogue:
// the GELU over all K^2 x h pre-activations and the h -> 1 dot with w2, one
// (a, b) per thread.
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
// Abramowitz & Stegun 26.2.17 (Hastings): Phi(-t) = phi(t) (b1 k + ... + b5 k^5),
// k = 1 / (1 + p t), |error| < 7.5e-8.  Two exact rewrites shorten it:
//   * t k = (1 - k) / p, so t Phi(-t) = exp(-t^2/2) R(k) with the degree-5
//     polynomial R(k) = (1 - k)(b1 + b2 k + ... + b5 k^4) / (p sqrt(2 pi));
//   * with y = alpha x, alpha = sqrt(log2(e) / 2), exp(-x^2/2) = 2^(-y^2) and
//     alpha GELU(x) = max(y, 0) - 2^(-y^2) alpha R(k), k = 1 / (1 + (p/alpha)|y|).
// The kernel keeps P and Q (so x) scaled by alpha and w2 scaled by 1/alpha,
// so w2 . GELU(x) = (w2/alpha) . gelu_scaled(alpha x).  Evaluated in float32
// this is within 1.3e-6 of the exact erf form on [-12, 12].
constexpr float kGeluAlpha = 0.849321800f;      // sqrt(log2(e) / 2)
__device__ __forceinline__ float gelu_scaled(float y) {
    const float t = fabsf(y);
    const float k = __builtin_amdgcn_rcpf(fmaf(0.272737495f, t, 1.0f));  // p / alpha
    float r = fmaf(k, -1.94583702f, 4.60984922f);   // alpha R(k), Horner from k^5
    r = fmaf(k, r, -5.26983972f);
    r = fmaf(k, r, 3.12738533f);
    r = fmaf(k, r, -0.988727877f);
    r = fmaf(k, r, 0.467170075f);
    const float e = __builtin_amdgcn_exp2f(-(y * y));
    return fmaf(-e, r, fmaxf(y, 0.0f));
}

// Hidden units handled by one workgroup (a multiple of 16 and of 8).
constexpr int kJB = 64;
static_assert(256 == 4 * kJB, "four r quarters per hidden unit in the c_p dot");
static_assert(256 / kJB <= kMaxMlpBlocks, "the finishing kernel sums at most kMaxMlpBlocks blocks");

// One workgroup per (pair, block of up to 64 hidden units):
//   P[a][j] = c_p[j] + b1[j] + w_la[j] l_p(a) + U_p[a][j]
//   Q[b][j] = w_lb[j] l_{p+1}(b) + V_{p+1}[b][j]
// from the per-candidate products U | V and the pair's c_p (formed here from
// s_p), then GELU and the dot with w2 over the K x m
// candidate pairs (successors b < m; m = K unless sparsified), one (a, b) per
// thread; the block's partial Delta goes to
// part[pair][block][a][b].
__global__ __launch_bounds__(256) void mlp_kernel(MlpArgs a) {
    const int tid = threadIdx.x;
    const int B = a.B, K = a.K, h = a.h;
    const int nj = (h + kJB - 1) / kJB;
    // Consecutive workgroup numbers go to different XCDs (round-robin over 8):
    // the hidden blocks of one pair are numbered 8 apart so they share an XCD.
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
    const int nin = 3 * a.r + 2;

    __shared__ __attribute__((aligned(16))) float w2s[kJB];
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    float* P = dyn;                 // [K][PS]
    float* Q = dyn + K * PS;        // [K][PS]

    __shared__ float cps4[4][kJB];  // c_p partial dots, one per quarter of r

    // ---- operands: thread (rg, cg) forms 4 columns of rows rg, rg + 16, ...;
    // the first row's U, V and logits load here with everything else
    const int cg = tid & 15, rg = tid >> 4;
    const int c = cg * 4;
    const bool colok = c < jn;
    const int cc = colok ? j0 + c : j0;  // clamped columns are not stored
    const int64_t ustride = 2 * static_cast<int64_t>(h);
    const int m0 = min(rg, K - 1);        // rows past K are not stored
    const float4 u0 = *reinterpret_cast<const float4*>(a.uv + (tp * K + m0) * ustride + cc);
    const float4 v0 = *reinterpret_cast<const float4*>(a.uv + (tq * K + m0) * ustride + h + cc);
    const float lp0 = a.vals[tp * K + m0], lq0 = a.vals[tq * K + m0];
    const float4 b1v = *reinterpret_cast<const float4*>(a.b1 + cc);
    float wla[4], wlb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t wrow = static_cast<int64_t>(cc + i) * nin + 3 * a.r;
        wla[i] = bf16_to_f32(a.w1[wrow]);
        wlb[i] = bf16_to_f32(a.w1[wrow + 1]);
    }
    if (tid < kJB) w2s[tid] = tid < jn ? a.w2[j0 + tid] * (1.0f / kGeluAlpha) : 0.f;   // see gelu_scaled
    // c_p = W1_s s_p for the block's units: thread (jj, kq) dots row j0 + jj
    // of W1_s with s_p over the quarter kq of its r columns, in column order.
    // W1 rows are 3r + 2 bf16 long (4-byte aligned: r is a multiple of 16),
    // so they are read in 32-bit words of two columns each.
    {
        const int jj = tid & (kJB - 1), kq = tid / kJB;
        const int kw = a.r / 4;
        const uint32_t* wr = reinterpret_cast<const uint32_t*>(
            a.w1 + static_cast<int64_t>(min(j0 + jj, h - 1)) * nin + kq * kw);
        const float* sp = a.s + static_cast<int64_t>(pair) * a.r + kq * kw;
        // every load is issued before the first is used (r <= 128: at most
        // 8 groups of 4 columns; groups past kw re-read the last and are not
        // summed)
        constexpr int kG = 128 / 4 / 4;
        uint32_t wv[2 * kG];
        float4 sv[kG];
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int k = min(4 * g, kw - 4);
            wv[2 * g] = wr[k / 2];
            wv[2 * g + 1] = wr[k / 2 + 1];
            sv[g] = *reinterpret_cast<const float4*>(sp + k);
        }
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            if (4 * g < kw) {
                acc = fmaf(__uint_as_float(wv[2 * g] << 16), sv[g].x, acc);
                acc = fmaf(__uint_as_float(wv[2 * g] & 0xFFFF0000u), sv[g].y, acc);
                acc = fmaf(__uint_as_float(wv[2 * g + 1] << 16), sv[g].z, acc);
                acc = fmaf(__uint_as_float(wv[2 * g + 1] & 0xFFFF0000u), sv[g].w, acc);
            }
        }
        cps4[kq][jj] = acc;
    }
    __syncthreads();

    // ---- P = c_p + b1 + w_la l_p(a) + U, Q = w_lb l_{p+1}(b) + V
    {
        float cpv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int jj = min(c + i, kJB - 1);
            cpv[i] = ((cps4[0][jj] + cps4[1][jj]) + (cps4[2][jj] + cps4[3][jj]));
        }
        cpv[0] += b1v.x;
        cpv[1] += b1v.y;
        cpv[2] += b1v.z;
        cpv[3] += b1v.w;
        for (int m = rg; m < K; m += 16) {
            float4 u = u0, v = v0;
            float lp = lp0, lq = lq0;
            if (m != rg) {
                const int64_t np = tp * K + m, nq = tq * K + m;
                u = *reinterpret_cast<const float4*>(a.uv + np * ustride + cc);
                v = *reinterpret_cast<const float4*>(a.uv + nq * ustride + h + cc);
                lp = a.vals[np];
                lq = a.vals[nq];
            }
            if (colok) {   // kept scaled by alpha (see gelu_scaled)
                constexpr float al = kGeluAlpha;
                *reinterpret_cast<float4*>(P + m * PS + c) =
                    make_float4(al * (cpv[0] + fmaf(wla[0], lp, u.x)), al * (cpv[1] + fmaf(wla[1], lp, u.y)),
                                al * (cpv[2] + fmaf(wla[2], lp, u.z)), al * (cpv[3] + fmaf(wla[3], lp, u.w)));
                *reinterpret_cast<float4*>(Q + m * PS + c) =
                    make_float4(al * fmaf(wlb[0], lq, v.x), al * fmaf(wlb[1], lq, v.y), al * fmaf(wlb[2], lq, v.z),
                                al * fmaf(wlb[3], lq, v.w));
            }
        }
    }
    __syncthreads();

    // ---- GELU and the dot with w2, one (a, b) per thread
    const int ms = a.m;
    const int nidx = K * ms;
    float* out = a.part + static_cast<int64_t>(item) * K * K;
    for (int idx = tid; idx < nidx; idx += 256) {
        const int aa = idx / ms, bb = idx - aa * ms;
        const float* pr = P + aa * PS;
        const float* qr = Q + bb * PS;
        float d0 = 0.f, d1 = 0.f;
        for (int j = 0; j < jn; j += 8) {
            const float4 pv0 = *reinterpret_cast<const float4*>(pr + j);
            const float4 qv0 = *reinterpret_cast<const float4*>(qr + j);
            const float4 wv0 = *reinterpret_cast<const float4*>(w2s + j);
            const float4 pv1 = *reinterpret_cast<const float4*>(pr + j + 4);
            const float4 qv1 = *reinterpret_cast<const float4*>(qr + j + 4);
            const float4 wv1 = *reinterpret_cast<const float4*>(w2s + j + 4);
            d0 = fmaf(wv0.x, gelu_scaled(pv0.x + qv0.x), d0);
            d1 = fmaf(wv0.y, gelu_scaled(pv0.y + qv0.y), d1);
            d0 = fmaf(wv0.z, gelu_scaled(pv0.z + qv0.z), d0);
            d1 = fmaf(wv0.w, gelu_scaled(pv0.w + qv0.w), d1);
            d0 = fmaf(wv1.x, gelu_scaled(pv1.x + qv1.x), d0);
            d1 = fmaf(wv1.y, gelu_scaled(pv1.y + qv1.y), d1);
            d0 = fmaf(wv1.z, gelu_scaled(pv1.z + qv1.z), d0);
            d1 = fmaf(wv1.w, gelu_scaled(pv1.w + qv1.w), d1);
        }
        out[aa * K + bb] = d0 + d1;
    }
}

}  // namespace

int mlp_blocks(int h) { return (h + kJB - 1) / kJB; }

hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream) {
    const int pairs = a.n * (a.B - 1);
    const dim3 grid(static_cast<unsigned>((pairs + 7) / 8 * 8 * mlp_blocks(a.h)));
    const size_t lds = static_cast<size_t>(2) * a.K * (kJB + 4) * sizeof(float);
    return launch(mlp_kernel, grid, 256, static_cast<uint32_t>(lds), stream, a);
}

}  // namespace corr
