// Step (1) of the DCOCO method details: the K largest drafter logits of every
// drafted slot, ordered by value descending with ties to the lowest token id.
//
// Two launches:
//   topk_partial  one wave per (row, chunk): a chunk of the row (6144 bf16 or
//                 3072 float32 logits) is streamed into registers with 16-byte
//                 coalesced loads.  bf16 path: one packed pass (v_pk_max_i16 /
//                 v_pk_min_u16 over pairs of logits) gives every lane its
//                 maximum; the target-th largest lane maximum is a threshold
//                 at or below the chunk's K-th largest value; a per-lane
//                 bitmask marks the 16-byte vectors holding an element at or
//                 above it, and those vectors are staged in LDS at slots from
//                 a prefix sum over lanes; their passing elements become 32-bit
//                 composite keys (order-preserving value key << 16 | inverted
//                 local index) and a bitwise search selects the exact top-K of
//                 the chunk.  If the staged set overflows (heavy ties) an
//                 exact search that re-reads the chunk takes over.
//   topk_merge    one wave per row: the chunks' candidates, as 64-bit
//                 composites (value key << 32 | inverted token id), go through
//                 a threshold-then-search selection and the K winners are
//                 written in order.
// Keys map float bits to an unsigned integer order with -0 == +0, so the
// selection is exact integer work: results are bit-identical to a full sort.
//
// Optionally (the fused top-K and vocabulary-wide normalisation of LiLiCorr
// appendix A) every partial wave also leaves its chunk's share of the row's
// softmax normaliser, the pair (m, s) with m the chunk maximum and
// s = sum of exp(l - m) over the chunk, from the registers the top-K already
// holds; the merge wave folds a row's pairs into log Z and writes the
// candidates' log-probs and confidence scalars.
#include "common.h"
#include "gemm.h"
#include "kernels.h"

namespace corr {

namespace {

constexpr int kNV = 12;        // 16-byte loads per lane
constexpr int kCap = 256;      // compacted candidates per wave (float32 path)
constexpr int kStage = 64;     // staged 16-byte vectors per wave (bf16 path, K <= 16)
constexpr int kStageWide = 128; // the same for K > 16
constexpr int kCand16 = 256;   // candidate keys per wave (bf16 path)

typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2, a),
                                                                  __builtin_bit_cast(i16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// Order-preserving 16-bit key of a bf16 bit pattern (-0 and +0 share 0x8000;
// -inf -> 0x007F; the NaN pattern 0xFFFF used for padding -> 0).
__device__ __forceinline__ uint32_t key16_of(uint32_t x) {
    return (x & 0x8000u) ? ((x == 0x8000u) ? 0x8000u : (0xFFFFu - x)) : (x | 0x8000u);
}
__device__ __forceinline__ uint32_t raw16_of_key16(uint32_t k) {
    return (k & 0x8000u) ? (k & 0x7FFFu) : (0xFFFFu - k);
}

// 64-bit merge composite: value key (float32 order) << 32 | inverted token id.
__device__ __forceinline__ uint64_t merge_comp(uint32_t key32, int64_t gid) {
    return (static_cast<uint64_t>(key32) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(gid));
}

// ------------------------------------------------- softmax normaliser --
constexpr float kLog2e = 1.44269504088896341f;

// Wave-wide sum and maximum over the 64 lanes, the same value in every lane
// (fixed combination order, so the results are deterministic).
__device__ __forceinline__ float wave_sum64(float v) {
    const float r = row16_sum(v);
    return (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32)) +
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48)));
}
__device__ __forceinline__ float wave_max64(float v) {
    const float r = row16_max(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 0)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 32)),
                       __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), 48))));
}

// exp(x - ref) as 2^((x - ref) log2 e); x = -inf gives 0.
__device__ __forceinline__ float exp_rel(float x, float ref) {
    return __builtin_amdgcn_exp2f((x - ref) * kLog2e);
}

// A reference point for sums of exp(x - m): m itself, or 0 when m = -inf (the
// lane or chunk holds no finite value, every term is 0, and -inf - -inf must
// not be formed).
__device__ __forceinline__ float exp_ref(float m) { return m == -INFINITY ? 0.f : m; }

// The chunk's (m, s) from every lane's maximum ml and sum sl of exp(x - ref(ml)).
__device__ __forceinline__ float2 chunk_expsum(float ml, float sl) {
    const float m = wave_max64(ml);
    const float ref = exp_ref(m);
    return make_float2(m, wave_sum64(sl * exp_rel(exp_ref(ml), ref)));
}

// --------------------------------------------------------------- bf16 path --


// One chunk of one drafted row: kNV * 512 consecutive logits (fewer at the
// end of the row).  Chunk numbers are wave-uniform, so all of this is scalar.
struct Chunk {
    const uint16_t* src;
    int nvalid;
    uint32_t row, chunk;
};

// Issues the 16-byte loads of a full chunk into registers.
__device__ __forceinline__ void load_full_chunk(u32x4 (&raw)[kNV], const uint16_t* src) {
    const int l = lane_id();
    const u32x4* p = reinterpret_cast<const u32x4*>(src);
#pragma unroll
    for (int t = 0; t < kNV; ++t) raw[t] = __builtin_nontemporal_load(p + t * kWave + l);
}

// Loads the last, shorter chunk of a row; elements past the end of the row
// read as 0xFFFF (key 0: "no element").
__device__ __forceinline__ void load_ragged_chunk(u32x4 (&raw)[kNV], const Chunk& c) {
    const int l = lane_id();
    const u32x4* src = reinterpret_cast<const u32x4*>(c.src);
#pragma unroll
    for (int t = 0; t < kNV; ++t) {
        const int e0 = (t * kWave + l) * 8;
        if (e0 + 8 <= c.nvalid) {
            raw[t] = __builtin_nontemporal_load(src + t * kWave + l);
        } else {
            u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
            for (int j = 0; j < 8; ++j) {
                if (e0 + j < c.nvalid) {
                    const uint32_t b = c.src[e0 + j];
                    const int q = j >> 1;
                    v[q] = (j & 1) ? ((v[q] & 0x0000FFFFu) | (b << 16)) : ((v[q] & 0xFFFF0000u) | b);
                }
            }
            raw[t] = v;
        }
    }
}

// key16_of without branches: flip the magnitude bits of negatives and the
// sign bit of non-negatives, then move -0 (0x7FFF after the flip) onto +0.
__device__ __forceinline__ uint32_t key16_flip(uint32_t x) {
    const uint32_t k = x ^ ((x & 0x8000u) ? 0xFFFFu : 0x8000u);
    return k == 0x7FFFu ? 0x8000u : k;
}

// Vector t of this lane's share of a chunk, loaded again (16 bytes; the
// elements past the end of a row's last chunk read as 0xFFFF, key 0).
__device__ __forceinline__ u32x4 chunk_vec(const Chunk& c, int t) {
    const int l = lane_id();
    const int e0 = (t * kWave + l) * 8;
    if (e0 + 8 <= c.nvalid) return load16(c.src + e0);
    u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    for (int j = 0; j < 8; ++j) {
        if (e0 + j < c.nvalid) {
            const uint32_t b = c.src[e0 + j];
            const int q = j >> 1;
            v[q] = (j & 1) ? ((v[q] & 0x0000FFFFu) | (b << 16)) : ((v[q] & 0xFFFF0000u) | b);
        }
    }
    return v;
}

// Exact top-`target` of a chunk without the threshold and staging (used when
// too many elements reach the lane-maximum threshold, i.e. heavy ties):
// T = the target-th largest value key by a bitwise search over every element
// (per-lane counts summed over the wave), then every element above T and, of
// those equal to T, the ones with the lowest local indices (vector-major:
// vector t*64 + lane, then its 8 elements).  Each pass loads the chunk again
// with coalesced 16-byte loads, half of it in flight at a time (the compiler
// barriers keep the loads inside the pass and bound what is live, so this
// rarely used path needs fewer registers than the usual one).  Writes the
// winners unordered to `out` and returns how many there are.
__device__ __forceinline__ int topk_bf16_reread(const Chunk& c, int64_t c0, int K, int target, uint64_t* out) {
    const int l = lane_id();
    constexpr int kHalf = kNV / 2;
    auto count_ge = [&](uint32_t cc) {
        int cnt = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            asm volatile("" ::: "memory");
            u32x4 v[kHalf];
#pragma unroll
            for (int t = 0; t < kHalf; ++t) v[t] = chunk_vec(c, h * kHalf + t);
#pragma unroll
            for (int t = 0; t < kHalf; ++t) {
#pragma unroll
                for (int j = 0; j < 8; ++j) cnt += key16_flip((v[t][j >> 1] >> (16 * (j & 1))) & 0xFFFFu) >= cc;
                asm volatile("" : "+v"(cnt));   // one vector's compares at a time
            }
        }
        return static_cast<int>(wave_sum64(static_cast<float>(cnt)));   // <= 6144: exact in float
    };
    uint32_t T = 0;
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cc = T | (1u << bit);
        if (count_ge(cc) >= target) T = cc;
    }
    T = max(T, 1u);  // key 0 is padding, never a winner
    const int ngt = T < 0xFFFFu ? count_ge(T + 1u) : 0;
    const int need = target - ngt;   // >= 1 elements equal to T
    int ogt = 0, oeq = 0;
    for (int t = 0; t < kNV; ++t) {   // one vector at a time (rolled)
        asm volatile("" ::: "memory");
        const u32x4 vt = chunk_vec(c, t);
        // elements above T, any order
        int eqn = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t k = key16_flip((vt[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
            const bool gt = k > T;
            const uint64_t m = ballot(gt);
            const int pos = ogt + prefix_count(m);
            if (gt && pos < K)
                out[pos] = merge_comp(key_of_bits(raw16_of_key16(k) << 16),
                                      c0 + (static_cast<int64_t>(t * kWave + l) * 8 + j));
            ogt += popc64(m);
            eqn += k == T;
        }
        // elements equal to T in index order: this lane's first slot is the
        // count of equal elements in lower lanes (four bit planes: <= 8 each)
        int base = 0, tot = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint64_t m = ballot((eqn >> b) & 1);
            base += prefix_count(m) << b;
            tot += popc64(m) << b;
        }
        int r = oeq + base;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t k = key16_flip((vt[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
            if (k == T) {
                if (r < need)
                    out[ngt + r] = merge_comp(key_of_bits(raw16_of_key16(k) << 16),
                                              c0 + (static_cast<int64_t>(t * kWave + l) * 8 + j));
                ++r;
            }
        }
        oeq += tot;
    }
    return ngt + min(oeq, need);
}

// Bit t set when 16-byte vector t of this lane holds an element at or above
// the threshold, tested on the packed maximum (positive threshold: signed
// max against tpos) or packed minimum (otherwise: unsigned min against
// uneg + 1) of the vector's four words.
template <bool kPos>
__device__ __forceinline__ uint32_t hit_mask(const u32x4 (&raw)[kNV], uint32_t bound2) {
    uint32_t hm = 0;
#pragma unroll
    for (int t = 0; t < kNV; ++t) {
        const u32x4& v = raw[t];
        bool hit;
        if (kPos) {
            const uint32_t m = pk_max_i16(pk_max_i16(v[0], v[1]), pk_max_i16(v[2], v[3]));
            hit = pk_max_i16(m, bound2) != bound2;
        } else {
            const uint32_t m = pk_min_u16(pk_min_u16(v[0], v[1]), pk_min_u16(v[2], v[3]));
            hit = pk_min_u16(m, bound2) != bound2;
        }
        hm |= hit ? (1u << t) : 0u;
    }
    return hm;
}

// The key16 of the lane's largest element: signed max finds the largest
// positive, unsigned min the negative closest to zero; together they give the
// largest value (key 0 when the lane holds padding only).
__device__ __forceinline__ uint32_t lane_key_bf16(const u32x4 (&raw)[kNV]) {
    uint32_t mxp = 0x80008000u, mnp = 0xFFFFFFFFu;
#pragma unroll
    for (int t = 0; t < kNV; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            mxp = pk_max_i16(mxp, raw[t][q]);
            mnp = pk_min_u16(mnp, raw[t][q]);
        }
    const int mx16 = max(static_cast<int>(static_cast<int16_t>(mxp & 0xFFFFu)),
                         static_cast<int>(static_cast<int16_t>(mxp >> 16)));
    const uint32_t mn16 = min(mnp & 0xFFFFu, mnp >> 16);
    return key16_of(mx16 >= 0 ? static_cast<uint32_t>(mx16) : mn16);
}

// Sums of exp(x - ref) over a lane's elements take one fma per element:
// exp(x - ref) = 2^(x log2e - m2) * 2^c with m2 = fl(ref log2e) and
// c = ref log2e - m2, the rounding of that product, which an fma recovers
// exactly; the lane's sum of 2^(x log2e - m2) is scaled by 2^c once.  Where
// ref log2e would overflow (|ref| >= 2^126) the lane subtracts first instead.
constexpr float kFmaRefLimit = 0x1p126f;

template <bool kPad, bool kFma>
__device__ __forceinline__ float lane_sum_bf16(const u32x4 (&raw)[kNV], float ref, float m2) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int t = 0; t < kNV; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = raw[t][q];
            float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
            if (kPad) {
                lo = (w & 0xFFFFu) == 0xFFFFu ? -INFINITY : lo;
                hi = (w >> 16) == 0xFFFFu ? -INFINITY : hi;
            }
            s0 += kFma ? __builtin_amdgcn_exp2f(fmaf(lo, kLog2e, -m2)) : exp_rel(lo, ref);
            s1 += kFma ? __builtin_amdgcn_exp2f(fmaf(hi, kLog2e, -m2)) : exp_rel(hi, ref);
        }
    return s0 + s1;
}

// The lane's (maximum, sum of exp(x - ref)) over its elements.  kPad: the
// chunk is a row's last, shorter one, whose padding (0xFFFF) counts as -inf.
template <bool kPad>
__device__ __forceinline__ float2 lane_expsum_bf16(const u32x4 (&raw)[kNV], uint32_t lane_key) {
    const float m = lane_key ? __uint_as_float(raw16_of_key16(lane_key) << 16) : -INFINITY;
    const float ref = exp_ref(m);
    float s;
    if (fabsf(ref) < kFmaRefLimit) {
        const float m2 = ref * kLog2e;
        const float c = fmaf(ref, kLog2e, -m2);
        s = lane_sum_bf16<kPad, true>(raw, ref, m2) * __builtin_amdgcn_exp2f(c);
    } else {
        s = lane_sum_bf16<kPad, false>(raw, ref, 0.f);
    }
    return make_float2(m, s);
}

// The exact top-K of one register-resident chunk, written to part[the chunk's
// K slots] as merge composites (padded with 0 = "no element").  The LDS lists
// have one trash slot per lane past their capacity, so every list write is
// issued by every lane (no branches): lanes with nothing to add write there.
template <int kSt>
__device__ __forceinline__ void select_chunk(const u32x4 (&raw)[kNV], uint32_t lane_key, const Chunk& c, int K,
                                             uint32_t chunks, u32x4* stage, uint16_t* meta, uint32_t* cand,
                                             uint64_t* outb, uint64_t* __restrict__ part) {
    constexpr int kChunk = kNV * 8 * kWave;
    const int l = lane_id();
    const int64_t c0 = static_cast<int64_t>(c.chunk) * kChunk;

    // ---- threshold: the target-th largest lane maximum (at least `target`
    // distinct elements are >= it, so the chunk's top-`target` are too)
    const int target = min(K, c.nvalid);
    uint32_t thr = 0;
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cc = thr | (1u << bit);
        if (popc64(ballot(lane_key >= cc)) >= target) thr = cc;
    }
    thr = max(thr, 1u);
    // Raw-domain form of "key16 >= thr": positives only (signed compare) when
    // thr is above zero; otherwise an unsigned bound that admits every
    // non-negative value, both zeros and negatives down to the threshold.
    const bool posmode = thr > 0x8000u;
    const uint32_t tpos = posmode ? thr - 0x8000u - 1u : 0u;                 // raw > tpos
    const uint32_t uneg = thr == 0x8000u ? 0x8000u : 0xFFFFu - thr;          // raw <= uneg
    const uint32_t hm = posmode ? hit_mask<true>(raw, tpos | (tpos << 16))
                                : hit_mask<false>(raw, (uneg + 1u) | ((uneg + 1u) << 16));

    // ---- slots of the hit vectors: exclusive prefix over lanes of the hit
    // counts (at most kNV < 32: five bit planes), and their total
    const uint32_t cnt = __popc(hm);
    uint32_t base = 0, nst = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {
        const uint64_t m = ballot((cnt >> b) & 1u);
        base += static_cast<uint32_t>(prefix_count(m)) << b;
        nst += static_cast<uint32_t>(popc64(m)) << b;
    }

    const int64_t obase = (static_cast<int64_t>(c.row) * chunks + c.chunk) * K;
    int outn = 0;
    bool fast = nst <= static_cast<uint32_t>(kSt);
    uint32_t nc = 0;
    if (fast) {
        // stage the hit vectors (and their local vector numbers)
        uint32_t k = base;
#pragma unroll
        for (int t = 0; t < kNV; ++t) {
            const uint32_t hit = (hm >> t) & 1u;
            const uint32_t slot = hit ? k : kSt + l;
            stage[slot] = raw[t];
            meta[slot] = static_cast<uint16_t>(t * kWave + l);
            k += hit;
        }
        wave_lds_sync();
        // their elements that pass, as 32-bit composites (key16 << 16 |
        // inverted local index); lanes past the staged count see padding
        u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
        uint32_t vbase = 0;
        if (static_cast<uint32_t>(l) < nst) {
            v = stage[l];
            vbase = static_cast<uint32_t>(meta[l]) * 8u;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t k16 = key16_flip((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
            const bool pass = k16 >= thr;
            const uint64_t m = ballot(pass);
            const uint32_t pos = nc + static_cast<uint32_t>(prefix_count(m));
            cand[(pass && pos < static_cast<uint32_t>(kCand16)) ? pos : kCand16 + l] =
                (k16 << 16) | (0xFFFFu - (vbase + j));
            nc += static_cast<uint32_t>(popc64(m));
        }
        fast = nc <= static_cast<uint32_t>(kCand16);
    }
    if (fast && nc <= static_cast<uint32_t>(kWave)) {
        // the usual case: at most one candidate per lane, so each step of the
        // bitwise search is one compare, one ballot and one popcount
        wave_lds_sync();
        const uint32_t e0 = static_cast<uint32_t>(l) < nc ? cand[l] : 0u;
        uint32_t tc = 0;
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t cc = tc | (1u << bit);
            if (popc64(ballot(e0 >= cc)) >= target) tc = cc;
        }
        if (popc64(ballot(e0 >= tc)) > target) {
            for (int bit = 15; bit >= 0; --bit) {
                const uint32_t cc = tc | (1u << bit);
                if (popc64(ballot(e0 >= cc)) >= target) tc = cc;
            }
        }
        const bool p = e0 >= tc && e0 != 0u;
        const uint64_t m = ballot(p);
        const int pos = prefix_count(m);
        if (p && pos < K) {
            const uint32_t raw16 = raw16_of_key16(e0 >> 16);
            outb[pos] = merge_comp(key_of_bits(raw16 << 16), c0 + (0xFFFFu - (e0 & 0xFFFFu)));
        }
        outn = popc64(m);
    } else if (fast) {
        wave_lds_sync();
        uint32_t e[kCand16 / kWave];
#pragma unroll
        for (int q = 0; q < kCand16 / kWave; ++q)
            e[q] = static_cast<uint32_t>(q * kWave + l) < nc ? cand[q * kWave + l] : 0u;
        // bitwise search for the target-th largest composite: the value-key
        // half first; the index half only when values tie at the boundary
        auto count_ge = [&](uint32_t cc) {
            int cnt2 = 0;
#pragma unroll
            for (int q = 0; q < kCand16 / kWave; ++q)
                if (static_cast<uint32_t>(q * kWave) < nc) cnt2 += popc64(ballot(e[q] >= cc));
            return cnt2;
        };
        uint32_t tc = 0;
        for (int bit = 31; bit >= 16; --bit) {
            const uint32_t cc = tc | (1u << bit);
            if (count_ge(cc) >= target) tc = cc;
        }
        if (count_ge(tc) > target) {
            for (int bit = 15; bit >= 0; --bit) {
                const uint32_t cc = tc | (1u << bit);
                if (count_ge(cc) >= target) tc = cc;
            }
        }
#pragma unroll
        for (int q = 0; q < kCand16 / kWave; ++q) {
            if (static_cast<uint32_t>(q * kWave) >= nc) break;
            const bool p = e[q] >= tc && e[q] != 0u;
            const uint64_t m = ballot(p);
            const int pos = outn + prefix_count(m);
            if (p && pos < K) {
                const uint32_t raw16 = raw16_of_key16(e[q] >> 16);
                outb[pos] = merge_comp(key_of_bits(raw16 << 16), c0 + (0xFFFFu - (e[q] & 0xFFFFu)));
            }
            outn += popc64(m);
        }
    } else {
        outn = topk_bf16_reread(c, c0, K, target, outb);
    }
    // One store instruction per chunk: lane l writes slot min(l, K-1) (lanes
    // past K-1 repeat that slot's value); chunks with fewer than K elements
    // pad with 0 ("no element").
    wave_lds_sync();
    const int slot = min(l, K - 1);
    part[obase + slot] = slot < outn ? outb[slot] : 0ull;
}

// One wave per chunk.  The rows' shorter last chunks (when V is not a multiple
// of the chunk) come first: their loads take the slower ragged path, which
// then overlaps the other chunks instead of lengthening the kernel's tail.
// The full chunks follow, numbered f = row * full + chunk.  Each chunk's
// result slot is fixed by its (row, chunk).
// kLse: also write the chunk's normaliser pair to lse_part[row * chunks + chunk].
// Workgroups hold four waves, or one with kLse: that form needs more registers
// (fewer waves per SIMD), and single-wave workgroups free their slots as soon
// as their one wave ends instead of waiting for the slowest of four.
template <bool kLse>
constexpr int partial_waves_per_block() { return kLse ? 1 : 4; }

template <bool kLse, int kSt>
__global__ __launch_bounds__(64 * partial_waves_per_block<kLse>()) void topk_partial_bf16_kernel(
    const uint16_t* __restrict__ logits, int64_t req_stride, int64_t slot_stride, int B, int64_t V,
    int K, int chunks, int64_t rows, uint64_t* __restrict__ part, float2* __restrict__ lse_part) {
    constexpr int kChunk = kNV * 8 * kWave;
    constexpr int kWPB = partial_waves_per_block<kLse>();
    __shared__ u32x4 stage_all[kWPB][kSt + kWave];
    __shared__ uint16_t meta_all[kWPB][kSt + kWave];
    __shared__ uint32_t cand_all[kWPB][kCand16 + kWave];
    __shared__ uint64_t out_all[kWPB][kWave];
    const uint32_t wave = kWPB == 1 ? 0u : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t w = blockIdx.x * static_cast<uint32_t>(kWPB) + wave;
    const uint32_t uB = static_cast<uint32_t>(B), uch = static_cast<uint32_t>(chunks);
    const uint32_t nrows = static_cast<uint32_t>(rows);
    const bool ragged = V % kChunk != 0;
    const uint32_t full = ragged ? uch - 1u : uch;  // full chunks per row
    const uint32_t nrag = ragged ? nrows : 0u;      // shorter last chunks, one per row
    if (w >= nrows * uch) return;  // whole wave; this kernel has no block barrier
    Chunk c;
    const bool isfull = w >= nrag;
    if (isfull) {
        const uint32_t f = w - nrag;
        c.row = f / full;
        c.chunk = f - c.row * full;
    } else {
        c.row = w;
        c.chunk = uch - 1u;
    }
    const uint32_t req = c.row / uB, slot = c.row - req * uB;
    const int64_t c0 = static_cast<int64_t>(c.chunk) * kChunk;
    c.src = logits + req * req_stride + slot * slot_stride + c0;
    c.nvalid = static_cast<int>(min(static_cast<int64_t>(kChunk), V - c0));
    u32x4 raw[kNV];
    if (isfull)
        load_full_chunk(raw, c.src);
    else
        load_ragged_chunk(raw, c);
    const uint32_t lane_key = lane_key_bf16(raw);
    if (kLse) {
        const float2 ls = isfull ? lane_expsum_bf16<false>(raw, lane_key) : lane_expsum_bf16<true>(raw, lane_key);
        const float2 cs = chunk_expsum(ls.x, ls.y);
        if (lane_id() == 0) lse_part[static_cast<int64_t>(c.row) * uch + c.chunk] = cs;
    }
    select_chunk<kSt>(raw, lane_key, c, K, uch, stage_all[wave], meta_all[wave], cand_all[wave], out_all[wave], part);
}

// ---------------------------------------------------------- float32 path --
// Generic version on 32-bit value keys (used for float32 logits).
template <bool kLse>
__global__ __launch_bounds__(256) void topk_partial_f32_kernel(
    const float* __restrict__ logits, int64_t req_stride, int64_t slot_stride, int B, int64_t V,
    int K, int chunks, int64_t rows, uint64_t* __restrict__ part, float2* __restrict__ lse_part) {
    constexpr int kEPV = 4;
    constexpr int kChunk = kNV * kEPV * kWave;  // 4096 logits per wave
    __shared__ uint64_t cand_all[4][kCap];
    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (w >= rows * chunks) return;
    uint64_t* cand = cand_all[wave];
    const int64_t row = w / chunks;
    const int chunk = static_cast<int>(w % chunks);
    const int64_t req = row / B, slot = row % B;
    const int64_t c0 = static_cast<int64_t>(chunk) * kChunk;
    const float* src = logits + req * req_stride + slot * slot_stride + c0;
    const int nvalid = static_cast<int>(min(static_cast<int64_t>(kChunk), V - c0));

    u32x4 raw[kNV];
#pragma unroll
    for (int t = 0; t < kNV; ++t) {
        const int e0 = (t * kWave + l) * kEPV;
        if (e0 + kEPV <= nvalid) {
            raw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + t * kWave + l);
        } else {
            u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};  // key 0
            for (int j = 0; j < kEPV; ++j)
                if (e0 + j < nvalid) v[j] = reinterpret_cast<const uint32_t*>(src)[e0 + j];
            raw[t] = v;
        }
    }
    uint32_t mx = 0;
#pragma unroll
    for (int t = 0; t < kNV; ++t)
#pragma unroll
        for (int j = 0; j < kEPV; ++j) mx = max(mx, key_of_bits(raw[t][j]));
    if (kLse) {
        // padding (0xFFFFFFFF, key 0) counts as -inf
        const float m = mx > kKeyFloor ? __uint_as_float(bits_of_key(mx)) : -INFINITY;
        const float ref = exp_ref(m);
        const bool fma_ok = fabsf(ref) < kFmaRefLimit;
        const float m2 = fma_ok ? ref * kLog2e : 0.f;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int t = 0; t < kNV; ++t)
#pragma unroll
            for (int j = 0; j < kEPV; j += 2) {
                const float x0 = raw[t][j] == 0xFFFFFFFFu ? -INFINITY : __uint_as_float(raw[t][j]);
                const float x1 = raw[t][j + 1] == 0xFFFFFFFFu ? -INFINITY : __uint_as_float(raw[t][j + 1]);
                s0 += fma_ok ? __builtin_amdgcn_exp2f(fmaf(x0, kLog2e, -m2)) : exp_rel(x0, ref);
                s1 += fma_ok ? __builtin_amdgcn_exp2f(fmaf(x1, kLog2e, -m2)) : exp_rel(x1, ref);
            }
        const float sc = fma_ok ? __builtin_amdgcn_exp2f(fmaf(ref, kLog2e, -m2)) : 1.f;
        const float2 cs = chunk_expsum(m, (s0 + s1) * sc);
        if (l == 0) lse_part[row * chunks + chunk] = cs;
    }
    const int target = min(K, nvalid);
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = thr | (1u << bit);
        if (popc64(ballot(mx >= c)) >= target) thr = c;
    }
    thr = max(thr, kKeyFloor + 1);
    int total = 0;
#pragma unroll
    for (int t = 0; t < kNV; ++t)
#pragma unroll
        for (int j = 0; j < kEPV; ++j) {
            const uint32_t k = key_of_bits(raw[t][j]);
            const bool p = k >= thr;
            const uint64_t m = ballot(p);
            if (m) {
                const int pos = total + prefix_count(m);
                const uint32_t local = static_cast<uint32_t>((t * kWave + l) * kEPV + j);
                if (p && pos < kCap) cand[pos] = (static_cast<uint64_t>(k) << 16) | (0xFFFFu - local);
                total += popc64(m);
            }
        }
    wave_lds_sync();
    const int64_t obase = (row * chunks + chunk) * K;
    int outn = 0;
    if (total <= kCap) {
        uint64_t e[kCap / kWave];
#pragma unroll
        for (int q = 0; q < kCap / kWave; ++q) e[q] = q * kWave + l < total ? cand[q * kWave + l] : 0ull;
        uint64_t tc = 0;
        for (int bit = 47; bit >= 0; --bit) {
            const uint64_t c = tc | (1ull << bit);
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < kCap / kWave; ++q) cnt += popc64(ballot(e[q] >= c));
            if (cnt >= target) tc = c;
        }
#pragma unroll
        for (int q = 0; q < kCap / kWave; ++q) {
            const bool p = e[q] >= tc && e[q] != 0ull;
            const uint64_t m = ballot(p);
            const int pos = outn + prefix_count(m);
            if (p && pos < K)
                part[obase + pos] = merge_comp(static_cast<uint32_t>(e[q] >> 16), c0 + (0xFFFFu - (e[q] & 0xFFFFu)));
            outn += popc64(m);
        }
    } else {
        uint64_t tc = 0;
        for (int bit = 47; bit >= 0; --bit) {
            const uint64_t c = tc | (1ull << bit);
            int cnt = 0;
            // the composites are formed again on every pass (hoisted out of
            // the bit loop, they and their index halves would take about a
            // hundred more registers): 0xFFFF - local = lb - (256 t + j)
            uint32_t lb = 0xFFFFu - static_cast<uint32_t>(kEPV * l);
            asm volatile("" : "+v"(lb));
#pragma unroll
            for (int t = 0; t < kNV; ++t)
#pragma unroll
                for (int j = 0; j < kEPV; ++j) {
                    uint32_t x = raw[t][j];
                    asm volatile("" : "+v"(x));
                    const uint32_t inv = lb - static_cast<uint32_t>(t * kWave * kEPV + j);
                    cnt += popc64(ballot(((static_cast<uint64_t>(key_of_bits(x)) << 16) | inv) >= c));
                }
            if (cnt >= target) tc = c;
        }
        uint32_t lb = 0xFFFFu - static_cast<uint32_t>(kEPV * l);
        asm volatile("" : "+v"(lb));
#pragma unroll
        for (int t = 0; t < kNV; ++t)
#pragma unroll
            for (int j = 0; j < kEPV; ++j) {
                const uint32_t inv = lb - static_cast<uint32_t>(t * kWave * kEPV + j);
                const uint32_t local = 0xFFFFu - inv;
                const uint32_t k = key_of_bits(raw[t][j]);
                const bool p = ((static_cast<uint64_t>(k) << 16) | inv) >= tc && k > kKeyFloor;
                const uint64_t m = ballot(p);
                const int pos = outn + prefix_count(m);
                if (p && pos < K) part[obase + pos] = merge_comp(k, c0 + local);
                outn += popc64(m);
            }
    }
    for (int pos = outn + l; pos < K; pos += kWave) part[obase + pos] = 0ull;
}

// ------------------------------------------------------------------ merge --
// One wave selects the K largest of M 64-bit composites of one row and writes
// them in order.  Lane maxima give a threshold (K-th largest lane maximum);
// the entries at or above it (usually K..2K of them) are compacted into LDS
// and searched bitwise; with more than kMergeCap of them the search runs over
// all entries.
constexpr int kMergeCap = 128;

// The K winners (fin, exactly K distinct composites) in top-K order: lane l <
// K finds its rank among them and writes id and value; with conf given, also
// the candidate's five confidence scalars from the row's log-normaliser:
// log-prob, probability, gap to the rank-0 logit, rank / (K-1), top flag.
__device__ __forceinline__ void write_ranked(const uint64_t* fin, int K, int32_t* __restrict__ ids,
                                             float* __restrict__ vals, float* __restrict__ conf, float logz) {
    const int l = lane_id();
    int rank = 0;
    float v = -INFINITY;
    if (l < K) {
        const uint64_t me = fin[l];
        for (int m2 = 0; m2 < K; ++m2) rank += fin[m2] > me ? 1 : 0;
        v = __uint_as_float(bits_of_key(static_cast<uint32_t>(me >> 32)));
        ids[rank] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(me & 0xFFFFFFFFu));
        vals[rank] = v;
    }
    if (conf) {
        const float top = wave_max64(v);   // the rank-0 value: lanes past K hold -inf
        if (l < K) {
            const float lp = v - logz;
            float* c = conf + rank * kConfFields;
            c[0] = lp;
            c[1] = expf(lp);
            c[2] = top - v;
            c[3] = K > 1 ? static_cast<float>(rank) / static_cast<float>(K - 1) : 0.f;
            c[4] = rank == 0 ? 1.f : 0.f;
        }
    }
}

// log Z of one row from its chunks' (m, s) pairs: M = max m, then
// log Z = M + ln(sum_c s_c exp(m_c - M)); -inf when no chunk has a finite value.
__device__ __forceinline__ float row_log_normaliser(const float2* __restrict__ p, int chunks) {
    const int l = lane_id();
    float mx = -INFINITY;
    for (int q = l; q < chunks; q += kWave) mx = fmaxf(mx, p[q].x);
    const float M = wave_max64(mx);
    const float ref = exp_ref(M);
    float sum = 0.f;
    for (int q = l; q < chunks; q += kWave) sum += p[q].y * exp_rel(exp_ref(p[q].x), ref);
    const float S = wave_sum64(sum);
    return M == -INFINITY ? -INFINITY : M + logf(S);
}

__device__ void merge_row_wave(const uint64_t* __restrict__ ent, int M, int K, uint64_t* sel,
                               uint64_t* fin, int32_t* __restrict__ ids, float* __restrict__ vals,
                               float* __restrict__ conf, float logz) {
    const int l = lane_id();
    uint64_t lm = 0;
    for (int q = l; q < M; q += kWave) lm = max(lm, ent[q]);
    uint64_t thr = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t c = thr | (1ull << bit);
        if (popc64(ballot(lm >= c)) >= K) thr = c;
    }
    int n = 0;
    for (int q0 = 0; q0 < M; q0 += kWave) {
        const int q = q0 + l;
        const uint64_t e = q < M ? ent[q] : 0ull;
        const bool p = q < M && e >= thr && e != 0ull;
        const uint64_t m = ballot(p);
        const int pos = n + prefix_count(m);
        if (p && pos < kMergeCap) sel[pos] = e;
        n += popc64(m);
    }
    wave_lds_sync();
    uint64_t tc = 0;
    if (n <= kMergeCap) {
        const uint64_t e0 = l < n ? sel[l] : 0ull;
        const uint64_t e1 = l + kWave < n ? sel[l + kWave] : 0ull;
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t c = tc | (1ull << bit);
            if (popc64(ballot(e0 >= c)) + popc64(ballot(e1 >= c)) >= K) tc = c;
        }
    } else {
        for (int bit = 63; bit >= 0; --bit) {
            const uint64_t c = tc | (1ull << bit);
            int cnt = 0;
            for (int q0 = 0; q0 < M; q0 += kWave) {
                const int q = q0 + l;
                cnt += popc64(ballot(q < M && ent[q] >= c));
            }
            if (cnt >= K) tc = c;
        }
    }
    // exactly K distinct composites are >= tc
    int outn = 0;
    for (int q0 = 0; q0 < M; q0 += kWave) {
        const int q = q0 + l;
        const uint64_t e = q < M ? ent[q] : 0ull;
        const bool p = q < M && e >= tc && e != 0ull;
        const uint64_t m = ballot(p);
        const int pos = outn + prefix_count(m);
        if (p && pos < K) fin[pos] = e;
        outn += popc64(m);
    }
    wave_lds_sync();
    write_ranked(fin, K, ids, vals, conf, logz);
}

// Fast path of the merge for rows of at most kMergePer * 64 candidates, held in
// registers (the merge launch's register count is set by its GEMM tiles).  Value keys are compared on their top `kbits` bits: for bf16
// logits the rest of the float32-order key is fixed by those bits, so the
// searches are exact with kbits = 16.  Steps: threshold T0 = K-th largest lane
// maximum; the entries at or above it (at least K) are compacted; T = K-th
// largest value key among them; the winners are the entries above T plus,
// among those equal to T, the ones with the largest composites (smallest
// ids).  Returns false, having written nothing, when more than kMergeCap
// entries reach T0; the general search then takes over.
constexpr int kMergePer = 16;   // up to 1024 candidates per row (64 chunks at K = 16, 32 at K = 32)

__device__ __forceinline__ bool merge_row_fast(const uint64_t* __restrict__ ent, int M, int K, int kbits,
                                               uint64_t* sel, uint64_t* fin, int32_t* __restrict__ ids,
                                               float* __restrict__ vals, float* __restrict__ conf, float logz) {
    const int l = lane_id();
    const int lowbit = 32 - kbits;
    uint64_t e[kMergePer];
    uint32_t lane_hi = 0;
#pragma unroll
    for (int q = 0; q < kMergePer; ++q) {
        const int i = q * kWave + l;
        e[q] = i < M ? ent[i] : 0ull;
        lane_hi = max(lane_hi, static_cast<uint32_t>(e[q] >> 32));
    }
    uint32_t t0 = 0;
    for (int bit = 31; bit >= lowbit; --bit) {
        const uint32_t c = t0 | (1u << bit);
        if (popc64(ballot(lane_hi >= c)) >= K) t0 = c;
    }
    int n = 0;
#pragma unroll
    for (int q = 0; q < kMergePer; ++q) {
        if (q * kWave >= M) break;
        const bool p = e[q] != 0ull && static_cast<uint32_t>(e[q] >> 32) >= t0;
        const uint64_t m = ballot(p);
        const int pos = n + prefix_count(m);
        sel[(p && pos < kMergeCap) ? pos : kMergeCap + l] = e[q];
        n += popc64(m);
    }
    if (n > kMergeCap) return false;
    wave_lds_sync();
    const uint64_t a0 = l < n ? sel[l] : 0ull;
    const uint64_t a1 = l + kWave < n ? sel[l + kWave] : 0ull;
    const uint32_t h0 = static_cast<uint32_t>(a0 >> 32), h1 = static_cast<uint32_t>(a1 >> 32);
    uint32_t T = 0;
    for (int bit = 31; bit >= lowbit; --bit) {
        const uint32_t c = T | (1u << bit);
        if (popc64(ballot(h0 >= c)) + popc64(ballot(h1 >= c)) >= K) T = c;
    }
    const uint32_t tt = T >> lowbit;
    const bool up0 = a0 != 0ull && (h0 >> lowbit) > tt, up1 = a1 != 0ull && (h1 >> lowbit) > tt;
    const bool eq0 = a0 != 0ull && (h0 >> lowbit) == tt, eq1 = a1 != 0ull && (h1 >> lowbit) == tt;
    const int need = K - popc64(ballot(up0)) - popc64(ballot(up1));
    // among the entries equal to T, the `need` largest low words (inverted ids)
    uint32_t L = 0;
    if (popc64(ballot(eq0)) + popc64(ballot(eq1)) > need) {
        const uint32_t w0 = static_cast<uint32_t>(a0), w1 = static_cast<uint32_t>(a1);
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = L | (1u << bit);
            if (popc64(ballot(eq0 && w0 >= c)) + popc64(ballot(eq1 && w1 >= c)) >= need) L = c;
        }
    }
    const bool win0 = up0 || (eq0 && static_cast<uint32_t>(a0) >= L);
    const bool win1 = up1 || (eq1 && static_cast<uint32_t>(a1) >= L);
    const uint64_t m0 = ballot(win0);
    const int p0 = prefix_count(m0), c0 = popc64(m0);
    fin[(win0 && p0 < kWave) ? p0 : kWave + l] = a0;
    const uint64_t m1 = ballot(win1);
    const int p1 = c0 + prefix_count(m1);
    fin[(win1 && p1 < kWave) ? p1 : kWave + l] = a1;
    wave_lds_sync();
    // exactly K distinct composites won; order them by rank
    write_ranked(fin, K, ids, vals, conf, logz);
    return true;
}

// The merge of one row by one wave: the K winners of the row's chunk
// candidates, in order.  `sel` and `fin` are the wave's LDS lists.  With the
// normaliser pairs given (lse_part), also the row's log Z and, when conf is
// given, the candidates' confidence scalars.
__device__ __forceinline__ void merge_row(const uint64_t* __restrict__ part, int chunks, int K, int kbits, int64_t row,
                                          uint64_t* sel, uint64_t* fin, int32_t* __restrict__ ids,
                                          float* __restrict__ vals, const float2* __restrict__ lse_part,
                                          float* __restrict__ logz, float* __restrict__ conf) {
    const int M = chunks * K;
    const uint64_t* ent = part + row * M;
    float lz = 0.f;
    if (lse_part) {
        lz = row_log_normaliser(lse_part + row * chunks, chunks);
        if (lane_id() == 0) logz[row] = lz;
    }
    float* rc = conf ? conf + row * K * kConfFields : nullptr;
    if (M <= kMergePer * kWave && merge_row_fast(ent, M, K, kbits, sel, fin, ids + row * K, vals + row * K, rc, lz))
        return;
    wave_lds_sync();
    merge_row_wave(ent, M, K, sel, fin, ids + row * K, vals + row * K, rc, lz);
}

// Workgroups [0, nmerge) merge four rows each (one per wave); with a GEMM job
// given, the workgroups after them run its tiles (the hidden-state
// projection, which does not depend on the top-K and fills the machine while
// the few merge waves run).  Both paths take their LDS from one buffer.
__global__ __launch_bounds__(256) void topk_merge_kernel(const uint64_t* __restrict__ part, int chunks,
                                                         int K, int kbits, int64_t rows,
                                                         int32_t* __restrict__ ids, float* __restrict__ vals,
                                                         const float2* __restrict__ lse_part,
                                                         float* __restrict__ logz, float* __restrict__ conf,
                                                         int64_t nmerge, GemmJob hj) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kGemmSmem];
    static_assert(4 * (kMergeCap + kWave) * 8 + 4 * 2 * kWave * 8 <= kGemmSmem, "merge lists fit the GEMM's LDS");
    if (static_cast<int64_t>(blockIdx.x) >= nmerge) {
        gemm_any_body(hj, static_cast<int64_t>(blockIdx.x) - nmerge, smem);
        return;
    }
    uint64_t (*sel_all)[kMergeCap + kWave] = reinterpret_cast<uint64_t (*)[kMergeCap + kWave]>(smem);
    uint64_t (*fin_all)[2 * kWave] =
        reinterpret_cast<uint64_t (*)[2 * kWave]>(smem + 4 * (kMergeCap + kWave) * sizeof(uint64_t));
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (row >= rows) return;
    merge_row(part, chunks, K, kbits, row, sel_all[wave], fin_all[wave], ids, vals, lse_part, logz, conf);
}

}  // namespace

int topk_chunk_elems(int dtype) { return dtype == CORR_DT_BF16 ? kNV * 8 * kWave : kNV * 4 * kWave; }

hipError_t launch_topk_partial(int dtype, const void* logits, int64_t req_stride,
                               int64_t slot_stride, int B, int64_t V, int K, int chunks,
                               int64_t rows, uint64_t* part, float2* lse_part, hipStream_t stream) {
    const int64_t waves = rows * chunks;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
    const uint16_t* lb = static_cast<const uint16_t*>(logits);
    const float* lf = static_cast<const float*>(logits);
    if (dtype == CORR_DT_BF16) {
        // the staging area holds the vectors reaching the lane-maximum
        // threshold: about K of them, so larger K gets the wider area
        constexpr int w1 = partial_waves_per_block<true>(), w4 = partial_waves_per_block<false>();
        const dim3 g1(static_cast<unsigned>((waves + w1 - 1) / w1)), g4(static_cast<unsigned>((waves + w4 - 1) / w4));
        const bool wide = K > 16;
        if (lse_part)
            return wide ? launch(topk_partial_bf16_kernel<true, kStageWide>, g1, 64 * w1, 0, stream, lb, req_stride,
                                 slot_stride, B, V, K, chunks, rows, part, lse_part)
                        : launch(topk_partial_bf16_kernel<true, kStage>, g1, 64 * w1, 0, stream, lb, req_stride,
                                 slot_stride, B, V, K, chunks, rows, part, lse_part);
        return wide ? launch(topk_partial_bf16_kernel<false, kStageWide>, g4, 64 * w4, 0, stream, lb, req_stride,
                             slot_stride, B, V, K, chunks, rows, part, lse_part)
                    : launch(topk_partial_bf16_kernel<false, kStage>, g4, 64 * w4, 0, stream, lb, req_stride,
                             slot_stride, B, V, K, chunks, rows, part, lse_part);
    }
    return lse_part ? launch(topk_partial_f32_kernel<true>, grid, 256, 0, stream, lf, req_stride, slot_stride, B, V,
                             K, chunks, rows, part, lse_part)
                    : launch(topk_partial_f32_kernel<false>, grid, 256, 0, stream, lf, req_stride, slot_stride, B,
                             V, K, chunks, rows, part, lse_part);
}

hipError_t launch_topk_merge(int dtype, const uint64_t* part, int chunks, int K, int64_t rows, int32_t* ids,
                             float* vals, const float2* lse_part, float* logz, float* conf, const GemmJob* hj,
                             hipStream_t stream) {
    const int kbits = dtype == CORR_DT_BF16 ? 16 : 32;
    const int64_t nmerge = (rows + 3) / 4;
    GemmJob none{};
    const GemmJob& j = hj ? *hj : none;
    const int64_t ng = hj ? gemm_launch_blocks(*hj) : 0;
    return launch(topk_merge_kernel, dim3(static_cast<unsigned>(nmerge + ng)), 256, 0, stream, part, chunks, K,
                  kbits, rows, ids, vals, lse_part, logz, conf, nmerge, j);
}


}  // namespace corr
