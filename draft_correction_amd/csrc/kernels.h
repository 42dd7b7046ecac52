// Internal launch interface between the C-ABI layer (corrector.hip) and the
// kernel files.  Every launcher enqueues on `stream` and returns the HIP
// launch status; shapes have been validated by the caller.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#define CORR_DT_BF16 0
#define CORR_DT_F32 1

namespace corr {

// Path rules (the values of CORR_PATH_GREEDY / _GLOBAL_SUM / _GEOMETRIC / _BEAM).
constexpr int kPathGreedy = 0;
constexpr int kPathGlobalSum = 1;
constexpr int kPathGeometric = 2;
constexpr int kPathBeam = 3;

// Optional timing events for the next launch made on this thread.  The host
// sequencer sets them around one step; launch() hands them to
// hipExtLaunchKernel, which stamps them with the kernel's own start and end
// times, and marks them used.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
    bool used = false;
};
extern thread_local LaunchTiming g_launch_timing;

template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                  A... args) {
    LaunchTiming& t = g_launch_timing;
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, t.start, t.stop, 0u, static_cast<P>(args)...);
    if (t.start) t.used = true;
    return hipGetLastError();
}

// Upper bounds of the split-K factors of the two projection GEMMs (the hidden-
// state projections and the candidate projection); consumers sum that many
// partials at most.
constexpr int kMaxSplits = 8;
constexpr int kMaxUSplits = 4;

// ---- top-K (topk.hip)
// part [rows][chunks][K]: each chunk's K best as 64-bit composites
// (float32-order value key << 32 | inverted token id; 0 = no element).
// lse_part [rows][chunks] (optional): each chunk's (max, sum of exp(l - max)).
int topk_chunk_elems(int dtype);
hipError_t launch_topk_partial(int dtype, const void* logits, int64_t req_stride,
                               int64_t slot_stride, int B, int64_t V, int K, int chunks,
                               int64_t rows, uint64_t* part, float2* lse_part, hipStream_t stream);
// Confidence scalars per candidate: log-prob, probability, gap, rank, top flag.
constexpr int kConfFields = 5;
// ---- projections (proj.hip)
// Tiled GEMM C[split][m][n] = sum_k A[m][k] W[n][k] (bf16 in, float32 out).
#define GEMM_A_DENSE 0
#define GEMM_A_GATHER 1
#define GEMM_A_SLOTS 2
struct GemmA {
    int mode;
    const uint16_t* base;
    int64_t lda;          // DENSE / GATHER row stride
    const int32_t* ids;   // GATHER: row m is base[clamp(ids[m])]
    int64_t V;
    int B;                // SLOTS: row m is base + (m/B)*rs + (m%B)*ss
    int64_t rs, ss;
};
struct GemmW {
    const uint16_t* base[3];  // row n is base[n / nb] + (n % nb) * ld[n / nb]
    int64_t ld[3];
    int nb;
    int kwrap;                // > 0 (a power of two): column k of W is column k % kwrap, so an
                              // A row [hi | lo] of 2 * kwrap meets the same W columns twice
};
// One GEMM problem; two can share a launch (their workgroups side by side).
struct GemmJob {
    GemmA A;
    GemmW W;
    int64_t M;
    int N;
    int kdim;
    int splits;
    float* C;
    int small;            // 1: one 16 x 16 output tile per wave, operands straight to
                          // registers (few rows); identical partials either way
};
// Sets j.small when the one-wave-per-16x16-tile form moves fewer operand bytes
// per CU than tiles of bm x bn (the launch's tiled form).
void gemm_pick_small(GemmJob& j, int bm, int bn);
hipError_t launch_gemm(const GemmA& A, const GemmW& W, int64_t M, int N, int kdim, int splits, float* C,
                       hipStream_t stream);
hipError_t launch_gemm2(const GemmJob& j0, const GemmJob& j1, hipStream_t stream);
// The same product for one job on 128 x 128 tiles with loads going straight
// to LDS (the candidate projection); identical partials.  W.kwrap must be 0.
hipError_t launch_gemm_gather(const GemmJob& j, hipStream_t stream);
// Workgroups a GEMM job occupies in a launch.
int64_t gemm_launch_blocks(const GemmJob& j);

// The K winners of every row, in order, from the chunks' composites; with
// lse_part given, also logz [rows] and (conf non-null) conf [rows][K][5]; with
// a GEMM job given, its tiles run in the same launch (after the merge waves).
hipError_t launch_topk_merge(int dtype, const uint64_t* part, int chunks, int K, int64_t rows, int32_t* ids,
                             float* vals, const float2* lse_part, float* logz, float* conf, const GemmJob* hj,
                             hipStream_t stream);

// Per drafted slot: b = LN(u) with u = W_cand E[ids], g = LN(W_ctx h) per slot,
// z = gamma * LN(W_fuse [b; g]) + beta stored as bfloat16 hi/lo halves
// zhl [rows][K][2r] = [hi(z) | lo(z)] with z = hi + lo to ~2^-16.
// Cosine: also unit out/in vectors [rows][K][dvec].
struct CandArgs {
    const int32_t* ids;
    int64_t V;
    int K;
    int r;
    int64_t rows;
    const float* upart;     // [usplits][rows*K][r] partials of u = W_cand E[c] ...
    int usplits;
    const float* table;     // ... or, when non-null, the folded table [V][r] = E W_cand^T
    const uint16_t* w_fuse;
    const float* gamma;
    const float* beta;
    float eps;
    // Per-slot state from the hidden-state projection partials hproj
    // [splits][rows][hstride] (W_ctx h in columns [0, r), W_pair,L h in
    // [r, 2r) and W_pair,R h in [2r, 3r) when the variant has pairs): the
    // kernel forms g = LN(W_ctx h) of the slots its candidates belong to and,
    // for each slot t whose first candidate it holds, writes g_t to g_out and
    // (s_out non-null, t not the last drafted slot) the pair state
    // s_t = W_pair,L h_t + W_pair,R h_{t+1} to s_out.
    const float* hproj;
    int hstride;
    int splits;
    int B;                  // drafted slots per request
    float* g_out;           // [rows][r]
    float* s_out;           // [n(B-1)][r], or null
    uint16_t* zhl;          // [rows][K][2r] bf16 [hi | lo] rows of z
    // cosine only (null otherwise)
    const uint16_t* w_out;
    const uint16_t* w_in;
    int dvec;
    float* vout;
    float* vin;
    // with zero_cnt given, workgroup 0 zeroes zero_cnt[i * kCntStride], i < zero_n
    // (the per-request counts of a cosine launch split by pair)
    int* zero_cnt;
    int zero_n;
};
size_t cand_lds_bytes(int r, int dvec, int K);
hipError_t launch_cand(const CandArgs& a, hipStream_t stream);

// ---- transition scores (mlp.hip, cosine.hip)
struct MlpArgs {
    const uint16_t* zhl;    // [n][B][K][2r] bf16: z as [hi | lo] rows (the candidate kernel's output)
    const float* s;         // [n(B-1)][r]: pair state s_p (float32)
    const float* vals;      // [n][B][K]
    int n;
    int B;
    int K;
    int r;
    int h;
    const uint16_t* w1;     // [h][3r+2]
    const float* b1;
    const float* w2;
    float* part;            // [n*(B-1)][blocks][K][K] partial Delta per hidden-unit block (b < m written)
    int m;                  // successors scored per predecessor (b < m; 1..K)
    int* zero_cnt;          // K <= 16 and non-null: n counters (kCntStride apart) the launch sets to 0
                            // (for the per-pair finishing launch)
    int units16;            // K <= 16: one workgroup per (pair, 16 units); part then holds
                            // [pairs][h/16][K][K] partials, each the first level of a 64-unit block's sum
    // With fin_walk set (K = 4, 8 or 16), the finishing step and the
    // prefix-first walk run in the same launch: the last of a pair's block
    // workgroups (by pcnt[pair * kCntStride]) forms the pair's scores exactly
    // as the per-pair finishing step does and its rows' argmaxes (best), and the last
    // pair of a request (by rcnt[req * kCntStride]) walks.  The launch before
    // zeroes both counts; zero_cnt must then be null.
    int fin_walk;
    int* pcnt;
    int* rcnt;
    const float* b2;
    float* scores;          // [n(B-1)][K][K]
    const int32_t* ids;
    int32_t* tokens;
    int32_t* choice;
    int32_t* best;          // [n(B-1)][K]
};
// The finishing step's per-request counters sit kCntStride ints (128 bytes)
// apart, one cache line each, so the requests' counts do not queue on one line.
constexpr int kCntStride = 32;
// Most hidden-unit blocks of the MLP (h <= 256 units in blocks of 64).
constexpr int kMaxMlpBlocks = 4;
// Most (pair, 16-unit block) workgroups for which the MLP takes its 16-unit
// form: about one per CU.
constexpr int64_t kMlp16MaxGroups = 256;
int mlp_blocks(int h);
hipError_t launch_mlp(const MlpArgs& a, hipStream_t stream);

// Sum of the MLP partials in block order + b2 + l_{p+1}(b) -> scores (one
// workgroup per request).
struct FinishArgs {
    const float* part;
    int nblk;
    int m;                  // successors scored (b < m); S = -inf for the others
    const float* vals;
    const float* b2;
    int n;
    int B;
    int K;
    float* scores;
    const int32_t* ids;
    int32_t* tokens;        // with tokens given (only when path_fits_lds), the
    int32_t* choice;        // request's path by `rule` follows in the launch
    int rule;
    float lam;              // the Geometric rule's discount
    int beam;               // the beam rule's width (1..4)
    int sub;                // part holds 16-unit partials (nblk of them), added four at a
                            // time in the 64-unit kernel's tree before the 64-unit blocks' sum
    int32_t* best;          // [n(B-1)][K] row argmaxes and
    int* cnt;               // [n][kCntStride] pairs finished per request (zero at launch): with both
                            // given, K = 4, 8 or 16 and the scores fitting the path's LDS, the
                            // work is split by pair (the request's last pair takes the path); for
                            // the prefix-first walk that split runs inside the MLP's launch
                            // (MlpArgs fin_walk), and launch_finish refuses it
};
hipError_t launch_finish(const FinishArgs& a, hipStream_t stream);
// Whether the finishing step splits the work by pair for this shape and rule
// (it then needs best and cnt), and whether it will for these arguments.
bool finish_split(int B, int K, int rule);
bool finish_by_pair(const FinishArgs& a);

struct CosArgs {
    const float* vout;      // [n][B][K][dvec]
    const float* vin;
    const float* vals;
    int n;
    int B;
    int K;
    int dvec;
    float sigma;
    int m;                  // successors scored (b < m); S = -inf for the others
    float* scores;
    // with tokens given (only when path_fits_lds), the request's path by
    // `rule` follows in the same launch
    const int32_t* ids;
    int32_t* tokens;
    int32_t* choice;
    int rule;
    float lam;
    int beam;
    int32_t* best;          // [n(B-1)][K] row argmaxes and [n][kCntStride] pairs finished per
    int* cnt;               // request (zero at launch): with both given, as for FinishArgs, one
                            // wave per pair
};
hipError_t launch_cosine(const CosArgs& a, hipStream_t stream);
bool cosine_by_pair(const CosArgs& a);

// ---- paths (walk.hip)
// Whether a request's scores (plus the path's small arrays) fit one
// workgroup's LDS; only then do the finishing and cosine kernels run the path
// themselves.
bool path_fits_lds(int B, int K);
// The path of every request over precomputed scores by `rule`
// (kPathGreedy: the prefix-first walk; kPathGlobalSum: the best
// summed score by dynamic programming; kPathGeometric: the same with pair p
// weighted by lam^p; kPathBeam: beam search of width `beam`), one wave per
// request.
hipError_t launch_path(const float* scores, const int32_t* ids, int n, int B, int K, int rule, float lam, int beam,
                       int32_t* tokens, int32_t* choice, hipStream_t stream);

// ---- intermediates (walk.hip)
hipError_t launch_zhl_to_f32(const uint16_t* zhl, float* z, int64_t nodes, int r, hipStream_t stream);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t count, hipStream_t stream);

}  // namespace corr
