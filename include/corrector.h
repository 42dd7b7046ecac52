/*
 * corrector.h - C-ABI of the MI355X (gfx950) draft-correction library.
 *
 * One pass corrects a batch of draft blocks produced by a block-diffusion
 * drafter (DFlash-style).  The operations follow the DCOCO page ("Contextual
 * Correction of Parallel Drafts for Speculative Decoding", method details,
 * steps (1)-(5)) and, for the cosine variant, LiLiCorr section 3.2, Eq. 1 and
 * section 3.5, Eq. 8:
 *
 *   corrector_topk   step (1): top-K candidate ids and drafter logits per slot.
 *   corrector_topk_softmax  step (1) fused with the vocabulary-wide
 *                    normalisation of each slot row (LiLiCorr appendix A):
 *                    log Z per row and the candidates' confidence scalars.
 *   corrector_score  steps (2)-(4): candidate representations
 *                    b = LN(W_cand E[c]), g = LN(W_ctx h), z = LN_{gamma,beta}
 *                    (W_fuse [b; g]); pair state s_p = W_pair [h_p; h_{p+1}];
 *                    transition scores S_p(a,b) = l_{p+1}(b) +
 *                    Delta([s_p; z_p^a; z_{p+1}^b; l_p(a); l_{p+1}(b)]) with a
 *                    two-layer GELU MLP, or the cosine variant
 *                    S_p(a,b) = l_{p+1}(b) + sigma cos(W_out z_p^a, W_in z_{p+1}^b).
 *   corrector_walk   step (5): prefix-first greedy walk; slot 1 takes the
 *                    drafter argmax, then k_{p+1} = argmax_b S_p(k_p, b); or,
 *                    by the descriptor's path rule, the Global-Sum path of
 *                    LiLiCorr appendix E (Eq. 12) by dynamic programming.
 *   corrector_run    all of the above in one call.
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates device memory, never synchronises and keeps no global
 *     device state, so a sequence of calls can be captured into a HIP graph.
 *     Its one process-wide host structure is the registry of live handles.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  All
 *     work is enqueued on it and the call returns without waiting.
 *   - Return value: CORR_OK (0) or a positive corrector_status.  It reports
 *     host-side validation and launch errors only; a device fault surfaces at
 *     the caller's next synchronisation.  Validation happens before anything
 *     is enqueued, so a call that returns an error has launched nothing.
 *   - A handle's weights are fixed after corrector_create; concurrent calls
 *     with one handle on different streams are safe when each uses its own
 *     workspace.  Every step of a call runs in order on the call's stream;
 *     the library creates no streams of its own.
 *   - n_req = 0 is a no-op that returns CORR_OK; n_req > max_requests returns
 *     CORR_E_SHAPE.
 *   - Slots are the B drafted positions of a block (the anchor is not one of
 *     them); pairs are the B-1 adjacent drafted-slot pairs p = 0..B-2, pair p
 *     coupling slot p and slot p+1 (0-based).
 *   - Top-K order is value descending, ties to the lowest token id; -0 and +0
 *     compare equal; -inf is allowed.  NaN logits violate a precondition (the
 *     output is unspecified but every kernel still terminates in bounds).
 *   - The walk breaks ties to the lowest candidate index.
 */
#ifndef DRAFT_CORRECTION_CORRECTOR_H
#define DRAFT_CORRECTION_CORRECTOR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CORR_OK = 0,
    CORR_E_NULL = 1,        /* a required pointer is NULL */
    CORR_E_SHAPE = 2,       /* a size is out of range or inconsistent */
    CORR_E_UNSUPPORTED = 3, /* a valid value this build does not implement */
    CORR_E_ALIGN = 4,       /* a pointer or stride breaks an alignment rule */
    CORR_E_WORKSPACE = 5,   /* the workspace is smaller than required */
    CORR_E_HIP = 6,         /* a HIP launch or runtime call failed */
    CORR_E_HANDLE = 7       /* the handle is not a live corrector (never created,
                               or already destroyed) */
} corrector_status;

enum { CORR_VARIANT_MLP = 0, CORR_VARIANT_COSINE = 1 };
enum { CORR_DTYPE_BF16 = 0, CORR_DTYPE_F32 = 1 };
/* How a path is chosen through the candidate lattice (slot 1 is always rank 0,
 * the drafter's argmax):
 *   CORR_PATH_GREEDY      the prefix-first walk, k_{p+1} = argmax_b S_p(k_p, b)
 *                         (DCOCO method details step (5); LiLiCorr section
 *                         3.5, Eq. 8); ties to the lowest candidate index;
 *   CORR_PATH_GLOBAL_SUM  the path with the largest summed score
 *                         sum_p S_p(k_p, k_{p+1}) (LiLiCorr appendix E,
 *                         Eq. 12), found exactly by dynamic programming; ties
 *                         to the lowest predecessor index in the forward sweep
 *                         and the lowest index in the last slot;
 *   CORR_PATH_GEOMETRIC   the path with the largest discounted score
 *                         sum_p lambda^p S_p(k_p, k_{p+1}), lambda from the
 *                         descriptor, by the same dynamic program and ties.
 *                         The DCOCO page compares a Geometric rule with
 *                         lambda = 0.75 against the walk (path-rule table) but
 *                         gives no formula; this discounted sum is the
 *                         reading implemented;
 *   CORR_PATH_BEAM        beam search of width beam_width over the summed
 *                         score (the DCOCO page's critique suggests widening
 *                         the walk into a beam of 2-4): each step keeps the
 *                         beam_width best extensions g + S_p(last, b), summed
 *                         in float32, ordered by score, then beam index,
 *                         then b; the answer is the best final path.  Width 1
 *                         is the walk. */
enum { CORR_PATH_GREEDY = 0, CORR_PATH_GLOBAL_SUM = 1, CORR_PATH_GEOMETRIC = 2, CORR_PATH_BEAM = 3 };

/* Shapes and options fixed at create time.
 *   vocab        V, 1 <= K <= V < 2^31.
 *   slots        B, drafted slots per block, 1..64 (the anchor is not counted).
 *   k            K, candidates per slot, 1..64.
 *   d_hidden     drafter hidden width d, a multiple of 32.
 *   d_embed      embedding width d_e, a multiple of 32.
 *   r            representation width: 16, 32, 64 or 128.
 *   mlp_hidden   MLP hidden width h: a multiple of 16, at most 256 (MLP only).
 *   d_vec        in/out vector width: a multiple of 16, at most 128 (cosine only).
 *   variant      CORR_VARIANT_MLP or CORR_VARIANT_COSINE.
 *   logits_dtype CORR_DTYPE_BF16 or CORR_DTYPE_F32.
 *   max_requests upper bound on n_req for every call; sizes the workspace.
 *   ln_eps       LayerNorm epsilon (> 0).
 *   sigma        cosine scale (cosine only).
 *   path_rule    CORR_PATH_GREEDY (0, the default of a zeroed struct),
 *                CORR_PATH_GLOBAL_SUM, CORR_PATH_GEOMETRIC or CORR_PATH_BEAM; used by
 *                corrector_walk and corrector_run.
 *   path_lambda  lambda of CORR_PATH_GEOMETRIC, 0 < lambda <= 1 (otherwise
 *                CORR_E_SHAPE); ignored by the other rules.
 *   beam_width   width of CORR_PATH_BEAM, 1..4 (otherwise CORR_E_SHAPE);
 *                ignored by the other rules.
 *   succ_top_m   successors scored per predecessor: 0 (or K) scores all K;
 *                1 <= m < K scores only the first m candidates of the next
 *                slot (the drafter's top-m) and writes S = -inf for the
 *                others, cutting the transition MLP to K*m evaluations per
 *                pair (the DCOCO page's critique, weakness 3).  Outside
 *                0..K: CORR_E_SHAPE. */
typedef struct {
    int64_t vocab;
    int32_t slots;
    int32_t k;
    int32_t d_hidden;
    int32_t d_embed;
    int32_t r;
    int32_t mlp_hidden;
    int32_t d_vec;
    int32_t variant;
    int32_t logits_dtype;
    int32_t max_requests;
    float ln_eps;
    float sigma;
    int32_t path_rule;
    float path_lambda;
    int32_t beam_width;
    int32_t succ_top_m;
} corrector_desc;

/* Borrowed device pointers to the weights; the caller keeps them alive and
 * unchanged until corrector_destroy.  Matrices use the [out][in] row-major
 * layout of a PyTorch Linear weight and are bfloat16; vectors are float32.
 * Every matrix must be 16-byte aligned.
 *   embed    [V][d_e]          frozen target token-embedding table E
 *   w_cand   [r][d_e]          candidate projection (no bias)
 *   w_ctx    [r][d]            slot-context projection (no bias)
 *   w_fuse   [r][2r]           fusion of [b; g] (no bias)
 *   w_pair   [r][2d]           pair-state projection of [h_p; h_{p+1}] (no bias)
 *   ln_gamma [r], ln_beta [r]  affine parameters of the fused LayerNorm
 *   w1       [h][3r+2]         MLP layer 1; input columns in the order
 *                              s_p (r), z_p^a (r), z_{p+1}^b (r), l_p(a), l_{p+1}(b)
 *   b1 [h], w2 [h], b2 [1]     MLP layer-1 bias, layer-2 weight and bias
 *   w_out, w_in [d_vec][r]     cosine out/in maps (cosine only)
 * The MLP variant needs everything but w_out/w_in; the cosine variant needs
 * embed, w_cand, w_ctx, w_fuse, ln_gamma, ln_beta, w_out and w_in. */
typedef struct {
    const void *embed;
    const void *w_cand;
    const void *w_ctx;
    const void *w_fuse;
    const void *w_pair;
    const float *ln_gamma;
    const float *ln_beta;
    const void *w1;
    const float *b1;
    const float *w2;
    const float *b2;
    const void *w_out;
    const void *w_in;
} corrector_weights;

typedef struct corrector corrector;

/* Validate the descriptor and weight pointers and build a handle.  Host only:
 * no HIP call is made.  Errors: CORR_E_NULL, CORR_E_SHAPE,
 * CORR_E_UNSUPPORTED, CORR_E_ALIGN.  On error *out is set to NULL. */
int corrector_create(const corrector_desc *desc, const corrector_weights *weights,
                     corrector **out);

/* Free the handle (host memory only).  NULL, and a handle that is not live
 * (for example one already destroyed), are ignored.  Live handles are kept in
 * a registry: every call given a destroyed handle returns CORR_E_HANDLE (0
 * for the size queries) without reading the freed handle, unless a later
 * corrector_create has returned the same address, in which case the pointer
 * names that new corrector.  Destroying a handle while a call on it is in
 * progress on another thread is a caller error. */
void corrector_destroy(corrector *h);

/* Bytes of device workspace every call on `h` needs for n_req requests
 * (0 if h is NULL or n_req is out of range).  The caller allocates it, e.g.
 * torch.empty(bytes, dtype=torch.uint8, device="cuda"); it needs no
 * initialisation and is overwritten by every call. */
size_t corrector_workspace_bytes(const corrector *h, int32_t n_req);

/* Step (1).  logits: row (i, s) of request i and drafted slot s starts at
 * logits + i*req_stride + s*slot_stride ELEMENTS (bfloat16 or float32 per
 * logits_dtype) and holds V contiguous logits.  A caller holding a block of
 * B+1 rows per request with the anchor first passes logits + V,
 * slot_stride = V and req_stride = (B+1)*V.  The pointer must be 16-byte
 * aligned and both strides must keep every row 16-byte aligned
 * (CORR_E_ALIGN).  Outputs, [n_req][B][K] contiguous: ids (int32 token ids)
 * and vals (float32, the logit widened exactly), in top-K order. */
int corrector_topk(const corrector *h, int32_t n_req, const void *logits,
                   int64_t req_stride, int64_t slot_stride, int32_t *ids, float *vals,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Step (1) fused with the vocabulary-wide normalisation of every slot row
 * (LiLiCorr appendix A: "Serving" fuses top-K extraction with the logit
 * normalisation in one kernel; "Architecture" lists the confidence scalars
 * the head reads from the drafter's distribution).  Arguments, ids and vals
 * as for corrector_topk, plus outputs
 *   logz [n_req][B] float32: log sum_v exp(l_v) over the row's V logits
 *        (-inf for a row of -inf); required;
 *   conf_or_null [n_req][B][K][5] float32, written when non-NULL; per
 *        candidate in top-K order: log-prob l - logz, probability
 *        exp(l - logz), gap (the rank-0 logit minus this one, >= 0), rank
 *        r / (K-1) in [0, 1] (0 when K = 1), and 1 for rank 0 else 0.
 * The logits are read once: every chunk's maximum and sum of exponentials
 * come from the registers its top-K pass already holds.  Logits must be
 * finite or -inf (+inf and NaN give unspecified values).  Errors as for
 * corrector_topk; logz NULL gives CORR_E_NULL. */
int corrector_topk_softmax(const corrector *h, int32_t n_req, const void *logits,
                           int64_t req_stride, int64_t slot_stride, int32_t *ids, float *vals,
                           float *logz, float *conf_or_null, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Steps (2)-(4).  ids/vals as produced by corrector_topk ([n_req][B][K]).
 * hidden: bfloat16 row (i, s) starts at hidden + i*h_req_stride +
 * s*h_slot_stride elements, d contiguous values, rows 16-byte aligned.
 * scores: [n_req][B-1][K][K] float32, index [i][p][a][b] with a the
 * predecessor candidate (slot p) and b the successor (slot p+1); fully
 * overwritten.  Ids outside [0, V) are clamped to the table when gathering
 * (the caller must pass valid ids). */
int corrector_score(const corrector *h, int32_t n_req, const int32_t *ids, const float *vals,
                    const void *hidden, int64_t h_req_stride, int64_t h_slot_stride,
                    float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* Step (5), by the handle's path rule.  scores [n_req][B-1][K][K] and ids
 * [n_req][B][K] as above.  Outputs [n_req][B]: tokens[i][s] =
 * ids[i][s][choice[i][s]] and choice[i][s], with choice[i][0] = 0.  choice may
 * be NULL. */
int corrector_walk(const corrector *h, int32_t n_req, const float *scores, const int32_t *ids,
                   int32_t *tokens, int32_t *choice, void *stream);

/* Steps (1)-(5) in one call; the benchmarked entry point.  Arguments as in the
 * calls above.  tokens [n_req][B] is required; choice_or_null [n_req][B],
 * ids_or_null / vals_or_null [n_req][B][K] and scores_or_null
 * [n_req][B-1][K][K] are written only when non-NULL (the workspace holds
 * them otherwise). */
int corrector_run(const corrector *h, int32_t n_req, const void *logits, int64_t l_req_stride,
                  int64_t l_slot_stride, const void *hidden, int64_t h_req_stride,
                  int64_t h_slot_stride, int32_t *tokens, int32_t *choice_or_null,
                  int32_t *ids_or_null, float *vals_or_null, float *scores_or_null,
                  void *workspace, size_t workspace_bytes, void *stream);

/* corrector_run for callers that cannot allocate device memory: code under
 * graph capture, serving loops that must not allocate, harnesses that forbid
 * hipMalloc.  There is no workspace argument; the workspace is a static
 * device array of the library, 64 MiB on each GPU the library runs on (held
 * until the process ends).  Arguments, outputs and errors are those of
 * corrector_run; an n_req whose corrector_workspace_bytes exceeds 64 MiB
 * returns CORR_E_WORKSPACE with nothing launched (32 requests at the DCOCO
 * Qwen3-8B shape need 28.6 MiB for the MLP variant, 34.4 MiB for the cosine
 * variant).  The current device must be the stream's device.  The first call
 * on a device looks up that device's copy of the array (CORR_E_HIP if that
 * fails), so it should not be the first call made under a graph capture.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (on other streams or threads, with any handle) race and their results
 * are undefined, so serialise them.  The array needs no initialisation and
 * keeps whatever the last call left in it. */
int corrector_run_static(const corrector *h, int32_t n_req, const void *logits, int64_t l_req_stride,
                         int64_t l_slot_stride, const void *hidden, int64_t h_req_stride,
                         int64_t h_slot_stride, int32_t *tokens, int32_t *choice_or_null,
                         int32_t *ids_or_null, float *vals_or_null, float *scores_or_null,
                         void *stream);

/* Folded candidate projection.  E and W_cand are frozen at inference, so
 * u = W_cand E[c] can be tabulated once for the whole vocabulary:
 * T = E W_cand^T, [V][r] float32 (an MFMA GEMM over every embedding row).
 * corrector_table_bytes gives the size; corrector_fold_table fills a caller
 * buffer on `stream`; corrector_use_table attaches it (NULL detaches), after
 * which corrector_score / corrector_run gather rows of T instead of running
 * the gathered-embedding GEMM each pass.  Results match the unfolded path to
 * float32 rounding.  Attaching is the one mutation of a handle: it must not
 * race with calls in flight on the handle.  Errors: CORR_E_NULL, CORR_E_ALIGN
 * (the table must be 16-byte aligned), CORR_E_HANDLE. */
size_t corrector_table_bytes(const corrector *h);
int corrector_fold_table(const corrector *h, float *table, void *stream);
int corrector_use_table(corrector *h, const float *table);

/* Copy intermediates of the most recent corrector_score / corrector_run that
 * used `workspace` (same handle, same n_req) into caller buffers (float32,
 * any pointer may be NULL): z [n_req][B][K][r] (as stored, bfloat16 widened),
 * g [n_req][B][r], s [n_req][B-1][r] (MLP only).  For parity testing. */
int corrector_intermediates(const corrector *h, int32_t n_req, const void *workspace,
                            size_t workspace_bytes, float *z, float *g, float *s, void *stream);

/* Kernel timing for measurement.  When enabled, every call records a HIP
 * event before and after each kernel it launches, on the call's stream.
 * corrector_kernel_times waits for the most recent call's events and writes
 * up to `cap` per-kernel durations in milliseconds (launch order) and their
 * names; it returns the number of kernels of that call or a negative status.
 * Enabling creates HIP events and is not meant for graph capture. */
int corrector_set_timing(corrector *h, int enabled);
int corrector_kernel_times(corrector *h, float *ms, const char **names, int cap);

/* Human-readable name of a corrector_status value. */
const char *corrector_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DRAFT_CORRECTION_CORRECTOR_H */
