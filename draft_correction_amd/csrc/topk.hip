// Step (1) of the DCOCO method details: the K largest drafter logits of every
// drafted slot, ordered by value descending with ties to the lowest token id.
//
// Two launches:
//   topk_partial  one wave per (row, chunk): a chunk of the row (8192 bf16 or
//                 4096 float32 logits) is streamed with 16-byte coalesced loads
//                 into registers.  The wave takes the target-th largest of its
//                 64 lane maxima as a threshold (a lower bound of the chunk's
//                 K-th largest value), compacts the few elements at or above
//                 it into LDS, and selects the exact top-K of the chunk by a
//                 bitwise search on 48-bit composite keys (value key << 16 |
//                 inverted local index), so equal values order by id.  If the
//                 compacted set overflows LDS (heavy ties) the same search runs
//                 over all register-resident elements instead.
//   topk_merge    one wave per row: the chunks' candidates (value key, id)
//                 become 64-bit composites (value key << 32 | inverted id);
//                 the K largest are found by the same bitwise search and
//                 written in order.
// Keys map float bits to an unsigned integer order with -0 == +0, so the
// selection is exact integer work: results are bit-identical to a full sort.
#include "common.h"
#include "kernels.h"

namespace corr {

namespace {

constexpr int kNV = 16;     // 16-byte loads per lane
constexpr int kCap = 256;   // compacted candidates per wave

template <int DT>
struct TopkShape {
    static constexpr int kEPV = DT == CORR_DT_BF16 ? 8 : 4;   // elements per 16-byte load
    static constexpr int kEPL = kNV * kEPV;                   // elements per lane
    static constexpr int kChunk = kEPL * kWave;               // elements per wave
    static constexpr int kElem = DT == CORR_DT_BF16 ? 2 : 4;  // bytes per element
};

// Float32 bits of element j of a 16-byte vector.
template <int DT>
__device__ __forceinline__ uint32_t elem_bits(const u32x4& v, int j) {
    if constexpr (DT == CORR_DT_BF16) {
        const uint32_t w = v[j >> 1];
        return (j & 1) ? (w & 0xFFFF0000u) : (w << 16);
    } else {
        return v[j];
    }
}

template <int DT>
__device__ __forceinline__ uint32_t elem_key(const u32x4* raw, int t, int j) {
    return key_of_bits(elem_bits<DT>(raw[t], j));
}

template <int DT>
__global__ __launch_bounds__(256) void topk_partial_kernel(
    const char* __restrict__ logits, int64_t req_stride, int64_t slot_stride, int B, int64_t V,
    int K, int chunks, int64_t rows, uint32_t* __restrict__ part_key,
    int32_t* __restrict__ part_id) {
    using S = TopkShape<DT>;
    __shared__ uint64_t cand_all[4][kCap];
    const int wave = threadIdx.x >> 6;
    const int l = lane_id();
    const int64_t w = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    if (w >= rows * chunks) return;  // whole wave; this kernel has no block barrier
    uint64_t* cand = cand_all[wave];
    const int64_t row = w / chunks;
    const int chunk = static_cast<int>(w % chunks);
    const int64_t req = row / B, slot = row % B;
    const int64_t c0 = static_cast<int64_t>(chunk) * S::kChunk;
    const char* src = logits + (req * req_stride + slot * slot_stride + c0) * S::kElem;
    const int nvalid = static_cast<int>(min(static_cast<int64_t>(S::kChunk), V - c0));

    // Stream the chunk into registers.  Elements past the row end get a NaN
    // pattern whose key is <= kKeyFloor, i.e. "no element".
    u32x4 raw[kNV];
#pragma unroll
    for (int t = 0; t < kNV; ++t) {
        const int e0 = (t * kWave + l) * S::kEPV;
        if (e0 + S::kEPV <= nvalid) {
            raw[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + t * kWave + l);
        } else {
            u32x4 v = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
            for (int j = 0; j < S::kEPV; ++j) {
                if (e0 + j < nvalid) {
                    if constexpr (DT == CORR_DT_BF16) {
                        const uint32_t b = reinterpret_cast<const uint16_t*>(src)[e0 + j];
                        const int q = j >> 1;
                        v[q] = (j & 1) ? ((v[q] & 0x0000FFFFu) | (b << 16)) : ((v[q] & 0xFFFF0000u) | b);
                    } else {
                        v[j] = reinterpret_cast<const uint32_t*>(src)[e0 + j];
                    }
                }
            }
            raw[t] = v;
        }
    }

    uint32_t mx = 0;
#pragma unroll
    for (int t = 0; t < kNV; ++t)
#pragma unroll
        for (int j = 0; j < S::kEPV; ++j) mx = max(mx, elem_key<DT>(raw, t, j));

    const int target = min(K, nvalid);
    // thr = target-th largest lane maximum: at least `target` distinct
    // elements of the chunk are >= thr, so the chunk's top-`target` are too.
    uint32_t thr = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = thr | (1u << bit);
        if (popc64(ballot(mx >= c)) >= target) thr = c;
    }
    thr = max(thr, kKeyFloor + 1);

    // Compact the elements >= thr into LDS, in (load, lane, element) order.
    int total = 0;
#pragma unroll
    for (int t = 0; t < kNV; ++t) {
#pragma unroll
        for (int j = 0; j < S::kEPV; ++j) {
            const uint32_t k = elem_key<DT>(raw, t, j);
            const bool p = k >= thr;
            const uint64_t m = ballot(p);
            if (m) {
                const int pos = total + prefix_count(m);
                const uint32_t local = static_cast<uint32_t>((t * kWave + l) * S::kEPV + j);
                if (p && pos < kCap) cand[pos] = (static_cast<uint64_t>(k) << 16) | (0xFFFFu - local);
                total += popc64(m);
            }
        }
    }
    wave_lds_sync();

    const int64_t obase = (row * chunks + chunk) * K;
    int outn = 0;
    if (total <= kCap) {
        uint64_t e[kCap / kWave];
#pragma unroll
        for (int q = 0; q < kCap / kWave; ++q) {
            const int idx = q * kWave + l;
            e[q] = idx < total ? cand[idx] : 0ull;
        }
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
            if (p && pos < K) {
                part_key[obase + pos] = static_cast<uint32_t>(e[q] >> 16);
                part_id[obase + pos] = static_cast<int32_t>(c0 + (0xFFFFu - (e[q] & 0xFFFFu)));
            }
            outn += popc64(m);
        }
    } else {
        // Heavy ties at the threshold: exact search over every element.
        uint64_t tc = 0;
        for (int bit = 47; bit >= 0; --bit) {
            const uint64_t c = tc | (1ull << bit);
            int cnt = 0;
#pragma unroll
            for (int t = 0; t < kNV; ++t)
#pragma unroll
                for (int j = 0; j < S::kEPV; ++j) {
                    const uint32_t local = static_cast<uint32_t>((t * kWave + l) * S::kEPV + j);
                    const uint64_t comp = (static_cast<uint64_t>(elem_key<DT>(raw, t, j)) << 16) | (0xFFFFu - local);
                    cnt += popc64(ballot(comp >= c));
                }
            if (cnt >= target) tc = c;
        }
#pragma unroll
        for (int t = 0; t < kNV; ++t)
#pragma unroll
            for (int j = 0; j < S::kEPV; ++j) {
                const uint32_t local = static_cast<uint32_t>((t * kWave + l) * S::kEPV + j);
                const uint32_t k = elem_key<DT>(raw, t, j);
                const uint64_t comp = (static_cast<uint64_t>(k) << 16) | (0xFFFFu - local);
                const bool p = comp >= tc && k > kKeyFloor;
                const uint64_t m = ballot(p);
                const int pos = outn + prefix_count(m);
                if (p && pos < K) {
                    part_key[obase + pos] = k;
                    part_id[obase + pos] = static_cast<int32_t>(c0 + local);
                }
                outn += popc64(m);
            }
    }
    // Chunks with fewer than K elements pad with "no element".
    for (int pos = outn + l; pos < K; pos += kWave) {
        part_key[obase + pos] = 0u;
        part_id[obase + pos] = -1;
    }
}

// One wave per row; the row's chunk candidates are staged in dynamic LDS.
__global__ __launch_bounds__(64) void topk_merge_kernel(
    const uint32_t* __restrict__ part_key, const int32_t* __restrict__ part_id, int chunks, int K,
    int64_t rows, int32_t* __restrict__ ids, float* __restrict__ vals) {
    extern __shared__ uint64_t ent[];
    __shared__ uint64_t sel[64];
    const int l = lane_id();
    const int64_t row = blockIdx.x;
    if (row >= rows) return;
    const int M = chunks * K;
    const int64_t ibase = row * M;
    for (int q = l; q < M; q += kWave) {
        const uint32_t k = part_key[ibase + q];
        const int32_t id = part_id[ibase + q];
        ent[q] = (k > kKeyFloor && id >= 0)
                     ? ((static_cast<uint64_t>(k) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(id)))
                     : 0ull;
    }
    wave_lds_sync();
    uint64_t tc = 0;
    for (int bit = 63; bit >= 0; --bit) {
        const uint64_t c = tc | (1ull << bit);
        int cnt = 0;
        for (int q0 = 0; q0 < M; q0 += kWave) {
            const int q = q0 + l;
            cnt += popc64(ballot(q < M && ent[q] >= c));
        }
        if (cnt >= K) tc = c;
    }
    int outn = 0;
    for (int q0 = 0; q0 < M; q0 += kWave) {
        const int q = q0 + l;
        const bool p = q < M && ent[q] >= tc && ent[q] != 0ull;
        const uint64_t m = ballot(p);
        const int pos = outn + prefix_count(m);
        if (p && pos < 64) sel[pos] = ent[q];
        outn += popc64(m);
    }
    wave_lds_sync();
    if (l < K) {
        const uint64_t me = sel[l];
        int rank = 0;
        for (int m2 = 0; m2 < K; ++m2) rank += sel[m2] > me ? 1 : 0;
        const uint32_t key = static_cast<uint32_t>(me >> 32);
        const int32_t id = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(me & 0xFFFFFFFFu));
        ids[row * K + rank] = id;
        vals[row * K + rank] = __uint_as_float(bits_of_key(key));
    }
}

}  // namespace

int topk_chunk_elems(int dtype) {
    return dtype == CORR_DT_BF16 ? TopkShape<CORR_DT_BF16>::kChunk : TopkShape<CORR_DT_F32>::kChunk;
}

hipError_t launch_topk_partial(int dtype, const void* logits, int64_t req_stride,
                               int64_t slot_stride, int B, int64_t V, int K, int chunks,
                               int64_t rows, uint32_t* part_key, int32_t* part_id,
                               hipStream_t stream) {
    const int64_t waves = rows * chunks;
    const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
    if (dtype == CORR_DT_BF16)
        topk_partial_kernel<CORR_DT_BF16><<<grid, 256, 0, stream>>>(
            static_cast<const char*>(logits), req_stride, slot_stride, B, V, K, chunks, rows,
            part_key, part_id);
    else
        topk_partial_kernel<CORR_DT_F32><<<grid, 256, 0, stream>>>(
            static_cast<const char*>(logits), req_stride, slot_stride, B, V, K, chunks, rows,
            part_key, part_id);
    return hipGetLastError();
}

hipError_t launch_topk_merge(const uint32_t* part_key, const int32_t* part_id, int chunks, int K,
                             int64_t rows, int32_t* ids, float* vals, hipStream_t stream) {
    const size_t lds = static_cast<size_t>(chunks) * K * sizeof(uint64_t);
    topk_merge_kernel<<<dim3(static_cast<unsigned>(rows)), 64, lds, stream>>>(
        part_key, part_id, chunks, K, rows, ids, vals);
    return hipGetLastError();
}

}  // namespace corr
