// C-ABI of the corrector library: handle, validation, workspace carving and
// launch sequencing.  Every argument is checked on the host before anything is
// enqueued, so a call that returns an error has launched nothing.  The library
// never allocates device memory and never synchronises (except
// corrector_kernel_times, which waits for timing events by design).
#include <math.h>
#include <mutex>
#include <new>
#include <string.h>
#include <unordered_set>

#include "../../include/corrector.h"
#include "kernels.h"

static_assert(corr::kPathGreedy == CORR_PATH_GREEDY && corr::kPathGlobalSum == CORR_PATH_GLOBAL_SUM &&
                  corr::kPathGeometric == CORR_PATH_GEOMETRIC && corr::kPathBeam == CORR_PATH_BEAM,
              "kernel path-rule values match the header");

using namespace corr;

namespace corr {
thread_local LaunchTiming g_launch_timing;
}

namespace {

constexpr int kMaxKernels = 12;
constexpr size_t kAlign = 256;

struct Layout {
    size_t part, lse, ids, vals, hproj, upart, z, g, s, vout, vin, mlp_part, best, cnt, scores, total;
    int chunks, splits, usplits;
};

}  // namespace

struct corrector {
    corrector_desc d;
    corrector_weights w;
    bool timing;
    bool events_ready;
    hipEvent_t ev[2 * kMaxKernels];
    const char* names[kMaxKernels];
    int nk;
    const float* table;  // folded E W_cand^T [V][r], or null
    // Serialises calls that record the timing events (a diagnostic mode);
    // without timing a call touches no mutable handle state.
    std::mutex mu;
};

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int logits_elem_bytes(const corrector_desc& d) { return d.logits_dtype == CORR_DTYPE_BF16 ? 2 : 4; }

// Splits of the two GEMM reductions (over d for the hidden-state projections,
// over d_e for the candidate projection): functions of the widths only, so a
// request's results do not depend on how many requests share the call.
int choose_splits(const corrector_desc& d) {
    int s = d.d_hidden / 512;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : s;
}
// Successors scored per predecessor: the first m of the next slot's top-K.
int succ_m(const corrector_desc& d) { return d.succ_top_m > 0 && d.succ_top_m < d.k ? d.succ_top_m : d.k; }

int choose_usplits(const corrector_desc& d) {
    int s = d.d_embed / 1024;
    if (s > kMaxUSplits) s = kMaxUSplits;
    return s < 1 ? 1 : s;
}


Layout layout(const corrector_desc& d, int32_t n) {
    Layout L{};
    const int64_t rows = static_cast<int64_t>(n) * d.slots;
    const int64_t pairs = static_cast<int64_t>(n) * (d.slots - 1);
    L.chunks = static_cast<int>((d.vocab + topk_chunk_elems(d.logits_dtype) - 1) /
                                topk_chunk_elems(d.logits_dtype));
    L.splits = choose_splits(d);
    L.usplits = choose_usplits(d);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = up(o + bytes); return at; };
    L.part = take(sizeof(uint64_t) * rows * L.chunks * d.k);
    L.lse = take(sizeof(float) * 2 * rows * L.chunks);
    L.ids = take(sizeof(int32_t) * rows * d.k);
    L.vals = take(sizeof(float) * rows * d.k);
    L.hproj = take(sizeof(float) * L.splits * rows * 3 * d.r);
    L.upart = take(sizeof(float) * L.usplits * rows * d.k * d.r);
    L.z = take(sizeof(uint16_t) * rows * d.k * 2 * d.r);
    L.g = take(sizeof(float) * rows * d.r);
    L.s = take(sizeof(float) * pairs * d.r);
    const bool mlp = d.variant == CORR_VARIANT_MLP;
    const bool cos = d.variant == CORR_VARIANT_COSINE;
    // the MLP's finishing launch or the cosine launch split by pair: row
    // argmaxes and per-request counts
    const bool split = (mlp || cos) && finish_split(d.slots, d.k, d.path_rule);
    // the partials of the 64-unit blocks, or those of the 16-unit blocks of
    // mlp_pair16_kernel when a call this size may take that form
    const bool p16 = split && d.k <= 16 && pairs * (d.mlp_hidden / 16) <= kMlp16MaxGroups;
    L.mlp_part = take(mlp ? sizeof(float) * pairs * (p16 ? d.mlp_hidden / 16 : mlp_blocks(d.mlp_hidden)) * d.k * d.k
                          : 0);
    L.best = take(split ? sizeof(int32_t) * pairs * d.k : 0);
    // per-request counts, then (for the MLP launch that also finishes and
    // walks) per-pair counts, each on a 128-byte line of its own
    L.cnt = take(split ? sizeof(int) * kCntStride * (n + pairs) : 0);
    L.vout = take(cos ? sizeof(float) * rows * d.k * d.d_vec : 0);
    L.vin = take(cos ? sizeof(float) * rows * d.k * d.d_vec : 0);
    L.scores = take(sizeof(float) * pairs * d.k * d.k);
    L.total = o;
    return L;
}

template <typename T>
T* at(void* ws, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Handles of live correctors.  A handle is checked against this set before
// anything reads through it, so a destroyed handle is rejected without its
// freed memory being touched.  (A later corrector_create may reuse the
// address; the stale pointer then names the new corrector, as with any
// pointer handle.)
std::mutex g_live_mu;
std::unordered_set<const corrector*>& live_set() {
    static std::unordered_set<const corrector*>* s = new std::unordered_set<const corrector*>();
    return *s;
}

bool live(const corrector* h) {
    if (!h) return false;
    std::lock_guard<std::mutex> lock(g_live_mu);
    return live_set().count(h) != 0;
}

int check_n(const corrector* h, int32_t n) {
    if (!live(h)) return CORR_E_HANDLE;
    if (n < 0 || n > h->d.max_requests) return CORR_E_SHAPE;
    return CORR_OK;
}

int check_ws(const corrector* h, int32_t n, const void* ws, size_t bytes) {
    if (!ws) return CORR_E_NULL;
    if (!aligned(ws, 16)) return CORR_E_ALIGN;
    if (bytes < layout(h->d, n).total) return CORR_E_WORKSPACE;
    return CORR_OK;
}

int check_logits(const corrector* h, const void* logits, int64_t rs, int64_t ss) {
    if (!logits) return CORR_E_NULL;
    if (rs < 0 || ss < 0) return CORR_E_SHAPE;
    const int64_t e = logits_elem_bytes(h->d);
    if (!aligned(logits, 16) || (rs * e) % 16 != 0 || (ss * e) % 16 != 0) return CORR_E_ALIGN;
    return CORR_OK;
}

int check_hidden(const void* hidden, int64_t rs, int64_t ss) {
    if (!hidden) return CORR_E_NULL;
    if (rs < 0 || ss < 0) return CORR_E_SHAPE;
    if (!aligned(hidden, 16) || (rs * 2) % 16 != 0 || (ss * 2) % 16 != 0) return CORR_E_ALIGN;
    return CORR_OK;
}

// Enqueues kernels.  With timing on, each step's launch carries a pair of
// events that take the kernel's own start and end timestamps; a step that
// launched nothing records the pair back to back.
struct Seq {
    corrector* h;
    hipStream_t s;
    hipError_t err = hipSuccess;
    int k = 0;
    template <class F>
    void operator()(const char* name, F&& f) {
        if (err != hipSuccess) return;
        const bool t = h->timing && h->events_ready && k < kMaxKernels;
        if (t) g_launch_timing = LaunchTiming{h->ev[2 * k], h->ev[2 * k + 1], false};
        err = f();
        const bool used = g_launch_timing.used;
        g_launch_timing = LaunchTiming{};
        if (t && err == hipSuccess) {
            if (!used) err = hipEventRecord(h->ev[2 * k], s);
            if (!used && err == hipSuccess) err = hipEventRecord(h->ev[2 * k + 1], s);
            h->names[k] = name;
        }
        ++k;
    }
    void record(hipEvent_t e, hipStream_t st) {
        if (err == hipSuccess) err = hipEventRecord(e, st);
    }
    void wait(hipEvent_t e, hipStream_t st) {
        if (err == hipSuccess) err = hipStreamWaitEvent(st, e, 0);
    }
    int finish() {
        if (h->timing) h->nk = k < kMaxKernels ? k : kMaxKernels;
        return err == hipSuccess ? CORR_OK : CORR_E_HIP;
    }
};

// Step (5) over precomputed scores, by the handle's path rule.
hipError_t launch_path_rule(const corrector* h, const float* scores, const int32_t* ids, int32_t n, int32_t* tokens,
                            int32_t* choice, hipStream_t s) {
    return launch_path(scores, ids, n, h->d.slots, h->d.k, h->d.path_rule, h->d.path_lambda, h->d.beam_width, tokens,
                       choice, s);
}

const char* path_name(const corrector* h) {
    return h->d.path_rule == CORR_PATH_GREEDY ? "walk" : (h->d.path_rule == CORR_PATH_BEAM ? "beam" : "viterbi");
}

// Step (1).  With `hj` given, the hidden-state projection runs in the merge
// launch (it does not depend on the top-K).
// Step (1); with logz given, also the rows' log-normalisers (and, with conf,
// the confidence scalars) from the same pass over the logits.
void enqueue_topk(Seq& q, const corrector* h, const Layout& L, int32_t n, const void* logits,
                  int64_t rs, int64_t ss, int32_t* ids, float* vals, void* ws, const GemmJob* hj,
                  float* logz = nullptr, float* conf = nullptr) {
    const corrector_desc& d = h->d;
    const int64_t rows = static_cast<int64_t>(n) * d.slots;
    uint64_t* part = at<uint64_t>(ws, L.part);
    float2* lse = logz ? at<float2>(ws, L.lse) : nullptr;
    q(logz ? "topk_partial_lse" : "topk_partial", [&] {
        return launch_topk_partial(d.logits_dtype, logits, rs, ss, d.slots, d.vocab, d.k, L.chunks,
                                   rows, part, lse, q.s);
    });
    q(hj ? "topk_merge_hproj" : (logz ? "topk_merge_lse" : "topk_merge"), [&] {
        return launch_topk_merge(d.logits_dtype, part, L.chunks, d.k, rows, ids, vals, lse, logz, conf, hj, q.s);
    });
}

// The hidden-state projection: hproj rows are [W_ctx h | W_pair,L h |
// W_pair,R h] (3r wide); the cosine variant has no pair state and computes the
// W_ctx block alone (r wide).
GemmJob hproj_job(const corrector* h, const Layout& L, int32_t n, const void* hidden, int64_t hrs, int64_t hss,
                  void* ws) {
    const corrector_desc& d = h->d;
    const corrector_weights& w = h->w;
    const bool cos = d.variant == CORR_VARIANT_COSINE;
    GemmJob hj{};
    hj.A.mode = GEMM_A_SLOTS;
    hj.A.base = static_cast<const uint16_t*>(hidden);
    hj.A.B = d.slots;
    hj.A.rs = hrs;
    hj.A.ss = hss;
    hj.W.nb = d.r;
    hj.W.base[0] = static_cast<const uint16_t*>(w.w_ctx);
    hj.W.ld[0] = d.d_hidden;
    if (!cos) {
        hj.W.base[1] = static_cast<const uint16_t*>(w.w_pair);
        hj.W.base[2] = static_cast<const uint16_t*>(w.w_pair) + d.d_hidden;
        hj.W.ld[1] = hj.W.ld[2] = 2 * static_cast<int64_t>(d.d_hidden);
    }
    hj.M = static_cast<int64_t>(n) * d.slots;
    hj.N = cos ? d.r : 3 * d.r;
    hj.kdim = d.d_hidden;
    hj.splits = L.splits;
    hj.C = at<float>(ws, L.hproj);
    gemm_pick_small(hj, 64, 128);
    return hj;
}

// Steps (2)-(4); with tokens given also step (5) (fused into the MLP finish
// for the MLP variant, a walk launch for the cosine variant).  Everything runs
// in order on the call's stream.  When `hproj_done` is false the hidden-state
// projection shares one GEMM launch with the candidate projection; otherwise
// an earlier launch of the call has produced it.
void enqueue_score(Seq& q, const corrector* h, const Layout& L, int32_t n, const int32_t* ids,
                   const float* vals, const void* hidden, int64_t hrs, int64_t hss, float* scores,
                   void* ws, int32_t* tokens, int32_t* choice, bool hproj_done) {
    const corrector_desc& d = h->d;
    const corrector_weights& w = h->w;
    const int64_t rows = static_cast<int64_t>(n) * d.slots;
    float* hproj = at<float>(ws, L.hproj);
    const bool cos = d.variant == CORR_VARIANT_COSINE;
    const GemmJob hj = hproj_job(h, L, n, hidden, hrs, hss, ws);
    const int hn = hj.N;
    const bool mlp_pairs = !cos && d.slots > 1;
    float* upart = at<float>(ws, L.upart);
    if (!h->table) {
        // the candidate projection u = W_cand E[c] first (longer workgroups),
        // the hidden-state projection after it in the same launch
        GemmJob uj{};
        uj.A.mode = GEMM_A_GATHER;
        uj.A.base = static_cast<const uint16_t*>(w.embed);
        uj.A.lda = d.d_embed;
        uj.A.ids = ids;
        uj.A.V = d.vocab;
        uj.W.nb = d.r;
        uj.W.base[0] = static_cast<const uint16_t*>(w.w_cand);
        uj.W.ld[0] = d.d_embed;
        uj.M = rows * d.k;
        uj.N = d.r;
        uj.kdim = d.d_embed;
        uj.splits = L.usplits;
        uj.C = upart;
        gemm_pick_small(uj, hproj_done ? 128 : 64, 128);
        if (hproj_done) {
            q("cand_gemm", [&] { return launch_gemm_gather(uj, q.s); });
        } else {
            q("proj_gemm", [&] { return launch_gemm2(uj, hj, q.s); });
        }
    } else if (!hproj_done) {
        q("hproj", [&] { return launch_gemm(hj.A, hj.W, hj.M, hj.N, hj.kdim, hj.splits, hj.C, q.s); });
    }
    CandArgs ca{};
    ca.ids = ids;
    ca.V = d.vocab;
    ca.K = d.k;
    ca.r = d.r;
    ca.rows = rows;
    ca.upart = upart;
    ca.usplits = L.usplits;
    ca.table = h->table;
    ca.w_fuse = static_cast<const uint16_t*>(w.w_fuse);
    ca.gamma = w.ln_gamma;
    ca.beta = w.ln_beta;
    ca.eps = d.ln_eps;
    ca.hproj = hproj;
    ca.hstride = hn;
    ca.splits = L.splits;
    ca.B = d.slots;
    ca.g_out = at<float>(ws, L.g);
    ca.s_out = mlp_pairs ? at<float>(ws, L.s) : nullptr;
    ca.zhl = at<uint16_t>(ws, L.z);
    if (cos) {
        ca.w_out = static_cast<const uint16_t*>(w.w_out);
        ca.w_in = static_cast<const uint16_t*>(w.w_in);
        ca.dvec = d.d_vec;
        ca.vout = at<float>(ws, L.vout);
        ca.vin = at<float>(ws, L.vin);
    }
    // the cosine launch split by pair counts its pairs per request; the
    // candidate launch zeroes the counts
    const bool cos_split = cos && tokens && d.slots > 1 && finish_split(d.slots, d.k, d.path_rule);
    // the MLP variant's finishing step and walk inside the MLP launch (the
    // walk, with the finishing step splitting by pair): it counts blocks per
    // pair and pairs per request, zeroed by the candidate launch
    const int64_t npairs = static_cast<int64_t>(n) * (d.slots - 1);
    bool mlp_walk = false;
    if (!cos && tokens && d.slots > 1 && d.path_rule == CORR_PATH_GREEDY && path_fits_lds(d.slots, d.k)) {
        FinishArgs pf{};
        pf.part = at<float>(ws, L.mlp_part);
        pf.vals = vals;
        pf.B = d.slots;
        pf.K = d.k;
        pf.scores = scores;
        pf.tokens = tokens;
        pf.rule = d.path_rule;
        pf.best = at<int32_t>(ws, L.best);
        pf.cnt = at<int>(ws, L.cnt);
        mlp_walk = finish_by_pair(pf);   // implies the layout holds best and the counts
    }
    ca.zero_cnt = cos_split || mlp_walk ? at<int>(ws, L.cnt) : nullptr;
    ca.zero_n = mlp_walk ? static_cast<int>(n + npairs) : n;
    q("cand", [&] { return launch_cand(ca, q.s); });
    if (d.slots < 2) {
        if (tokens) q(path_name(h), [&] { return launch_path_rule(h, scores, ids, n, tokens, choice, q.s); });
        return;
    }
    if (cos) {
        CosArgs c{};
        c.vout = ca.vout;
        c.vin = ca.vin;
        c.vals = vals;
        c.n = n;
        c.B = d.slots;
        c.K = d.k;
        c.dvec = d.d_vec;
        c.sigma = d.sigma;
        c.m = succ_m(d);
        c.scores = scores;
        // the path runs inside the cosine launch when the scores fit its LDS
        const bool fused = tokens && path_fits_lds(d.slots, d.k);
        c.ids = ids;
        c.tokens = fused ? tokens : nullptr;
        c.choice = fused ? choice : nullptr;
        c.rule = d.path_rule;
        c.lam = d.path_lambda;
        c.beam = d.beam_width;
        c.best = cos_split ? at<int32_t>(ws, L.best) : nullptr;
        c.cnt = ca.zero_cnt;
        q(fused ? (d.path_rule == CORR_PATH_GREEDY ? "cosine_walk"
                                                    : (d.path_rule == CORR_PATH_BEAM ? "cosine_beam" : "cosine_viterbi"))
                : "cosine",
          [&] { return launch_cosine(c, q.s); });
        if (tokens && !fused)
            q(path_name(h), [&] { return launch_path_rule(h, scores, ids, n, tokens, choice, q.s); });
    } else {
        MlpArgs m{};
        m.zhl = ca.zhl;
        m.s = ca.s_out;
        m.vals = vals;
        m.n = n;
        m.B = d.slots;
        m.K = d.k;
        m.r = d.r;
        m.h = d.mlp_hidden;
        m.w1 = static_cast<const uint16_t*>(w.w1);
        m.b1 = w.b1;
        m.w2 = w.w2;
        m.part = at<float>(ws, L.mlp_part);
        m.m = succ_m(d);
        if (mlp_walk) {
            // few pairs: one workgroup per (pair, 16 units), as below
            m.units16 = npairs * (d.mlp_hidden / 16) <= kMlp16MaxGroups ? 1 : 0;
            m.fin_walk = 1;
            m.rcnt = at<int>(ws, L.cnt);
            m.pcnt = m.rcnt + static_cast<int64_t>(n) * kCntStride;
            m.b2 = w.b2;
            m.scores = scores;
            m.ids = ids;
            m.tokens = tokens;
            m.choice = choice;
            m.best = at<int32_t>(ws, L.best);
            q("mlp_walk", [&] { return launch_mlp(m, q.s); });
            return;
        }
        const bool split = tokens && finish_split(d.slots, d.k, d.path_rule);
        m.zero_cnt = split ? at<int>(ws, L.cnt) : nullptr;
        FinishArgs f{};
        f.part = m.part;
        f.nblk = mlp_blocks(d.mlp_hidden);
        f.m = succ_m(d);
        f.vals = vals;
        f.b2 = w.b2;
        f.n = n;
        f.B = d.slots;
        f.K = d.k;
        f.scores = scores;
        f.ids = ids;
        // the path runs inside the finishing launch when the scores fit its LDS
        const bool fused = tokens && path_fits_lds(d.slots, d.k);
        f.tokens = fused ? tokens : nullptr;
        f.choice = fused ? choice : nullptr;
        f.rule = d.path_rule;
        f.lam = d.path_lambda;
        f.beam = d.beam_width;
        f.best = split ? at<int32_t>(ws, L.best) : nullptr;
        f.cnt = m.zero_cnt;
        // few pairs: one MLP workgroup per (pair, 16 units) when the scores
        // are finished by pair (which adds its 16-unit partials)
        if (finish_by_pair(f) && static_cast<int64_t>(n) * (d.slots - 1) * (d.mlp_hidden / 16) <= kMlp16MaxGroups) {
            m.units16 = 1;
            f.sub = 1;
            f.nblk = d.mlp_hidden / 16;
        }
        q("mlp", [&] { return launch_mlp(m, q.s); });
        q(fused ? (d.path_rule == CORR_PATH_GREEDY ? "finish_walk"
                                                    : (d.path_rule == CORR_PATH_BEAM ? "finish_beam" : "finish_viterbi"))
                : "finish",
          [&] { return launch_finish(f, q.s); });
        if (tokens && !fused)
            q(path_name(h), [&] { return launch_path_rule(h, scores, ids, n, tokens, choice, q.s); });
    }
}

int run_checked(const corrector* hc, int32_t n, const void* logits, int64_t lrs, int64_t lss, const void* hidden,
                int64_t hrs, int64_t hss, int32_t* tokens, int32_t* choice_or_null, int32_t* ids_or_null,
                float* vals_or_null, float* scores_or_null, void* ws, void* stream);

// ---- the workspace of corrector_run_static, for callers that cannot
// allocate.  Each GPU the library runs on holds its own copy of `scratch`
// until the process ends.  In host code the array's name is only a host-side
// stand-in: its device address on a device is looked up once per device
// (hipGetSymbolAddress with that device current) and kept in
// g_scratch_ptr[device]; only that address is ever handed to kernels.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up on its first use).
int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return CORR_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return CORR_E_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CORR_E_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CORR_OK;
}

}  // namespace

extern "C" {

int corrector_create(const corrector_desc* desc, const corrector_weights* wt, corrector** out) {
    if (!out) return CORR_E_NULL;
    *out = nullptr;
    if (!desc || !wt) return CORR_E_NULL;
    const corrector_desc& d = *desc;
    if (d.variant != CORR_VARIANT_MLP && d.variant != CORR_VARIANT_COSINE) return CORR_E_UNSUPPORTED;
    if (d.logits_dtype != CORR_DTYPE_BF16 && d.logits_dtype != CORR_DTYPE_F32) return CORR_E_UNSUPPORTED;
    if (d.path_rule != CORR_PATH_GREEDY && d.path_rule != CORR_PATH_GLOBAL_SUM && d.path_rule != CORR_PATH_GEOMETRIC &&
        d.path_rule != CORR_PATH_BEAM)
        return CORR_E_UNSUPPORTED;
    if (d.path_rule == CORR_PATH_GEOMETRIC && !(d.path_lambda > 0.f && d.path_lambda <= 1.f)) return CORR_E_SHAPE;
    if (d.path_rule == CORR_PATH_BEAM && (d.beam_width < 1 || d.beam_width > 4)) return CORR_E_SHAPE;
    if (d.succ_top_m < 0 || d.succ_top_m > d.k) return CORR_E_SHAPE;
    if (d.vocab < 1 || d.vocab > 0x7FFFFFFF) return CORR_E_SHAPE;
    if (d.slots < 1 || d.slots > 64) return CORR_E_SHAPE;  // the walk keeps one slot per lane
    if (d.k < 1 || d.k > 64 || d.k > d.vocab) return CORR_E_SHAPE;
    if (d.d_hidden < 32 || d.d_hidden % 32 || d.d_hidden > 65536) return CORR_E_SHAPE;
    if (d.d_embed < 32 || d.d_embed % 32 || d.d_embed > 65536) return CORR_E_SHAPE;
    if (d.r != 16 && d.r != 32 && d.r != 64 && d.r != 128) return CORR_E_UNSUPPORTED;
    if (d.max_requests < 1 || static_cast<int64_t>(d.max_requests) * d.slots > (1 << 24)) return CORR_E_SHAPE;
    // chunk numbers of the top-K are 32-bit
    if (static_cast<int64_t>(d.max_requests) * d.slots *
            ((d.vocab + topk_chunk_elems(d.logits_dtype) - 1) / topk_chunk_elems(d.logits_dtype)) >
        0x7FFFFFFF)
        return CORR_E_SHAPE;
    if (!(d.ln_eps > 0.f) || !isfinite(d.ln_eps)) return CORR_E_SHAPE;
    if (d.variant == CORR_VARIANT_MLP) {
        if (d.mlp_hidden < 16 || d.mlp_hidden > 256 || d.mlp_hidden % 16) return CORR_E_UNSUPPORTED;
    } else {
        if (d.d_vec < 16 || d.d_vec > 128 || d.d_vec % 16) return CORR_E_UNSUPPORTED;
        if (!isfinite(d.sigma)) return CORR_E_SHAPE;
    }

    // LDS of the candidate kernel (staging rows for 32 candidates)
    if (cand_lds_bytes(d.r, d.variant == CORR_VARIANT_COSINE ? d.d_vec : 0, d.k) > 64 * 1024)
        return CORR_E_UNSUPPORTED;

    const corrector_weights& w = *wt;
    if (!w.embed || !w.w_cand || !w.w_ctx || !w.w_fuse || !w.ln_gamma || !w.ln_beta) return CORR_E_NULL;
    if (d.variant == CORR_VARIANT_MLP && (!w.w_pair || !w.w1 || !w.b1 || !w.w2 || !w.b2)) return CORR_E_NULL;
    if (d.variant == CORR_VARIANT_COSINE && (!w.w_out || !w.w_in)) return CORR_E_NULL;
    const void* mats[] = {w.embed, w.w_cand, w.w_ctx, w.w_fuse,
                          d.variant == CORR_VARIANT_MLP ? w.w_pair : w.w_out,
                          d.variant == CORR_VARIANT_MLP ? w.w1 : w.w_in};
    for (const void* m : mats)
        if (!aligned(m, 16)) return CORR_E_ALIGN;
    if (!aligned(w.ln_gamma, 4) || !aligned(w.ln_beta, 4)) return CORR_E_ALIGN;

    corrector* h = new (std::nothrow) corrector();
    if (!h) return CORR_E_SHAPE;
    h->d = d;
    h->w = w;
    h->timing = false;
    h->events_ready = false;
    h->nk = 0;
    h->table = nullptr;
    try {
        std::lock_guard<std::mutex> lock(g_live_mu);
        live_set().insert(h);
    } catch (...) {
        delete h;
        return CORR_E_SHAPE;
    }
    *out = h;
    return CORR_OK;
}

void corrector_destroy(corrector* h) {
    if (!h) return;
    {
        // unregister first: a second destroy (or any later call) with this
        // handle is rejected without reading *h
        std::lock_guard<std::mutex> lock(g_live_mu);
        if (live_set().erase(h) == 0) return;
    }
    if (h->events_ready)
        for (hipEvent_t& e : h->ev) (void)hipEventDestroy(e);
    delete h;
}

size_t corrector_workspace_bytes(const corrector* h, int32_t n) {
    if (check_n(h, n) != CORR_OK) return 0;
    return layout(h->d, n).total;
}

int corrector_topk(const corrector* hc, int32_t n, const void* logits, int64_t rs, int64_t ss,
                   int32_t* ids, float* vals, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_n(hc, n);
    if (rc || n == 0) return rc;
    if ((rc = check_logits(hc, logits, rs, ss))) return rc;
    if (!ids || !vals) return CORR_E_NULL;
    if ((rc = check_ws(hc, n, ws, ws_bytes))) return rc;
    corrector* h = const_cast<corrector*>(hc);
    const Layout L = layout(h->d, n);
    std::unique_lock<std::mutex> lock(h->mu, std::defer_lock);
    if (h->timing) lock.lock();
    Seq q{h, static_cast<hipStream_t>(stream)};
    enqueue_topk(q, h, L, n, logits, rs, ss, ids, vals, ws, nullptr);
    return q.finish();
}

int corrector_topk_softmax(const corrector* hc, int32_t n, const void* logits, int64_t rs, int64_t ss,
                           int32_t* ids, float* vals, float* logz, float* conf, void* ws, size_t ws_bytes,
                           void* stream) {
    int rc = check_n(hc, n);
    if (rc || n == 0) return rc;
    if ((rc = check_logits(hc, logits, rs, ss))) return rc;
    if (!ids || !vals || !logz) return CORR_E_NULL;
    if ((rc = check_ws(hc, n, ws, ws_bytes))) return rc;
    corrector* h = const_cast<corrector*>(hc);
    const Layout L = layout(h->d, n);
    std::unique_lock<std::mutex> lock(h->mu, std::defer_lock);
    if (h->timing) lock.lock();
    Seq q{h, static_cast<hipStream_t>(stream)};
    enqueue_topk(q, h, L, n, logits, rs, ss, ids, vals, ws, nullptr, logz, conf);
    return q.finish();
}

int corrector_score(const corrector* hc, int32_t n, const int32_t* ids, const float* vals,
                    const void* hidden, int64_t hrs, int64_t hss, float* scores, void* ws,
                    size_t ws_bytes, void* stream) {
    int rc = check_n(hc, n);
    if (rc || n == 0) return rc;
    if (!ids || !vals) return CORR_E_NULL;
    if ((rc = check_hidden(hidden, hrs, hss))) return rc;
    if (!scores && hc->d.slots > 1) return CORR_E_NULL;
    if ((rc = check_ws(hc, n, ws, ws_bytes))) return rc;
    corrector* h = const_cast<corrector*>(hc);
    const Layout L = layout(h->d, n);
    std::unique_lock<std::mutex> lock(h->mu, std::defer_lock);
    if (h->timing) lock.lock();
    Seq q{h, static_cast<hipStream_t>(stream)};
    enqueue_score(q, h, L, n, ids, vals, hidden, hrs, hss, scores, ws, nullptr, nullptr, false);
    return q.finish();
}

int corrector_walk(const corrector* hc, int32_t n, const float* scores, const int32_t* ids,
                   int32_t* tokens, int32_t* choice, void* stream) {
    int rc = check_n(hc, n);
    if (rc || n == 0) return rc;
    if (!ids || !tokens || (!scores && hc->d.slots > 1)) return CORR_E_NULL;
    corrector* h = const_cast<corrector*>(hc);
    std::unique_lock<std::mutex> lock(h->mu, std::defer_lock);
    if (h->timing) lock.lock();
    Seq q{h, static_cast<hipStream_t>(stream)};
    q(path_name(h), [&] { return launch_path_rule(h, scores, ids, n, tokens, choice, q.s); });
    return q.finish();
}

int corrector_run(const corrector* hc, int32_t n, const void* logits, int64_t lrs, int64_t lss,
                  const void* hidden, int64_t hrs, int64_t hss, int32_t* tokens,
                  int32_t* choice_or_null, int32_t* ids_or_null, float* vals_or_null,
                  float* scores_or_null, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_n(hc, n);
    if (rc || n == 0) return rc;
    if ((rc = check_logits(hc, logits, lrs, lss))) return rc;
    if ((rc = check_hidden(hidden, hrs, hss))) return rc;
    if (!tokens) return CORR_E_NULL;
    if ((rc = check_ws(hc, n, ws, ws_bytes))) return rc;
    return run_checked(hc, n, logits, lrs, lss, hidden, hrs, hss, tokens, choice_or_null, ids_or_null, vals_or_null,
                       scores_or_null, ws, stream);
}

int corrector_run_static(const corrector* hc, int32_t n, const void* logits, int64_t lrs, int64_t lss,
                         const void* hidden, int64_t hrs, int64_t hss, int32_t* tokens, int32_t* choice_or_null,
                         int32_t* ids_or_null, float* vals_or_null, float* scores_or_null, void* stream) {
    int rc = check_n(hc, n);
    if (rc || n == 0) return rc;
    if ((rc = check_logits(hc, logits, lrs, lss))) return rc;
    if ((rc = check_hidden(hidden, hrs, hss))) return rc;
    if (!tokens) return CORR_E_NULL;
    if (layout(hc->d, n).total > kStaticScratchBytes) return CORR_E_WORKSPACE;
    void* ws = nullptr;
    if ((rc = static_scratch(&ws))) return rc;
    return run_checked(hc, n, logits, lrs, lss, hidden, hrs, hss, tokens, choice_or_null, ids_or_null, vals_or_null,
                       scores_or_null, ws, stream);
}

}  // extern "C"

namespace {

// corrector_run after validation: every step on the call's stream, with `ws`
// as the workspace (at least layout(n).total bytes, 16-byte aligned).
int run_checked(const corrector* hc, int32_t n, const void* logits, int64_t lrs, int64_t lss, const void* hidden,
                int64_t hrs, int64_t hss, int32_t* tokens, int32_t* choice_or_null, int32_t* ids_or_null,
                float* vals_or_null, float* scores_or_null, void* ws, void* stream) {
    corrector* h = const_cast<corrector*>(hc);
    const Layout L = layout(h->d, n);
    int32_t* ids = ids_or_null ? ids_or_null : at<int32_t>(ws, L.ids);
    float* vals = vals_or_null ? vals_or_null : at<float>(ws, L.vals);
    float* scores = scores_or_null ? scores_or_null : at<float>(ws, L.scores);
    std::unique_lock<std::mutex> lock(h->mu, std::defer_lock);
    if (h->timing) lock.lock();
    Seq q{h, static_cast<hipStream_t>(stream)};
    const GemmJob hj = hproj_job(h, L, n, hidden, hrs, hss, ws);
    enqueue_topk(q, h, L, n, logits, lrs, lss, ids, vals, ws, &hj);
    enqueue_score(q, h, L, n, ids, vals, hidden, hrs, hss, scores, ws, tokens, choice_or_null, true);
    return q.finish();
}

}  // namespace

extern "C" {

size_t corrector_table_bytes(const corrector* h) {
    if (!live(h)) return 0;
    return sizeof(float) * static_cast<size_t>(h->d.vocab) * h->d.r;
}

int corrector_fold_table(const corrector* h, float* table, void* stream) {
    if (!live(h)) return CORR_E_HANDLE;
    if (!table) return CORR_E_NULL;
    if (!aligned(table, 16)) return CORR_E_ALIGN;
    const corrector_desc& d = h->d;
    GemmA a{};
    a.mode = GEMM_A_DENSE;
    a.base = static_cast<const uint16_t*>(h->w.embed);
    a.lda = d.d_embed;
    GemmW w{};
    w.nb = d.r;
    w.base[0] = static_cast<const uint16_t*>(h->w.w_cand);
    w.ld[0] = d.d_embed;
    const hipError_t e = launch_gemm(a, w, d.vocab, d.r, d.d_embed, 1, table, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CORR_OK : CORR_E_HIP;
}

int corrector_use_table(corrector* h, const float* table) {
    if (!live(h)) return CORR_E_HANDLE;
    if (table && !aligned(table, 16)) return CORR_E_ALIGN;
    h->table = table;
    return CORR_OK;
}

int corrector_intermediates(const corrector* h, int32_t n, const void* ws, size_t ws_bytes,
                            float* z, float* g, float* s, void* stream) {
    int rc = check_n(h, n);
    if (rc || n == 0) return rc;
    if ((rc = check_ws(h, n, ws, ws_bytes))) return rc;
    const Layout L = layout(h->d, n);
    const corrector_desc& d = h->d;
    const int64_t rows = static_cast<int64_t>(n) * d.slots;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* w = const_cast<void*>(ws);
    hipError_t e = hipSuccess;
    if (z) e = launch_zhl_to_f32(at<uint16_t>(w, L.z), z, rows * d.k, d.r, st);
    if (e == hipSuccess && g) e = launch_copy_f32(at<float>(w, L.g), g, rows * d.r, st);
    if (e == hipSuccess && s && d.variant == CORR_VARIANT_MLP && d.slots > 1)
        e = launch_copy_f32(at<float>(w, L.s), s, static_cast<int64_t>(n) * (d.slots - 1) * d.r, st);
    return e == hipSuccess ? CORR_OK : CORR_E_HIP;
}

int corrector_set_timing(corrector* h, int enabled) {
    if (!live(h)) return CORR_E_HANDLE;
    if (enabled && !h->events_ready) {
        for (int i = 0; i < 2 * kMaxKernels; ++i) {
            if (hipEventCreate(&h->ev[i]) != hipSuccess) {
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(h->ev[j]);
                return CORR_E_HIP;
            }
        }
        h->events_ready = true;
    }
    h->timing = enabled != 0;
    h->nk = 0;
    return CORR_OK;
}

int corrector_kernel_times(corrector* h, float* ms, const char** names, int cap) {
    if (!live(h)) return -CORR_E_HANDLE;
    if (!h->timing || !h->events_ready) return 0;
    const int nk = h->nk;
    if (nk > 0 && hipEventSynchronize(h->ev[2 * nk - 1]) != hipSuccess) return -CORR_E_HIP;
    for (int k = 0; k < nk && k < cap; ++k) {
        float t = 0.f;
        if (hipEventElapsedTime(&t, h->ev[2 * k], h->ev[2 * k + 1]) != hipSuccess) return -CORR_E_HIP;
        if (ms) ms[k] = t;
        if (names) names[k] = h->names[k];
    }
    return nk;
}

const char* corrector_status_string(int status) {
    switch (status) {
        case CORR_OK: return "ok";
        case CORR_E_NULL: return "null pointer";
        case CORR_E_SHAPE: return "size out of range";
        case CORR_E_UNSUPPORTED: return "unsupported value";
        case CORR_E_ALIGN: return "misaligned pointer or stride";
        case CORR_E_WORKSPACE: return "workspace too small";
        case CORR_E_HIP: return "HIP launch or runtime error";
        case CORR_E_HANDLE: return "invalid handle";
        default: return "unknown status";
    }
}

}  // extern "C"
