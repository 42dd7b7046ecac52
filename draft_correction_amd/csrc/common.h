// Shared device helpers for the gfx950 corrector kernels: bfloat16 bit
// handling, order-preserving float keys, wave64 primitives and the
// v_mfma_f32_16x16x32_bf16 operand layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace corr {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ---------------------------------------------------------------- bfloat16 --

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// ----------------------------------------------------- order-preserving key --
// Maps float32 bits to an unsigned key whose integer order is the numeric
// order of the values, with -0 and +0 mapped to the same key.  Every finite
// value and -inf maps above kKeyFloor, so keys <= kKeyFloor mark "no element".

constexpr uint32_t kKeyFloor = 0x007FFFFEu;

__device__ __forceinline__ uint32_t key_of_bits(uint32_t b) {
    b = (b == 0x80000000u) ? 0u : b;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t bits_of_key(uint32_t k) {
    return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}

// ----------------------------------------------------------- wave helpers --

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ int prefix_count(uint64_t m) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

__device__ __forceinline__ float wave_sum16(float v) {
    // Sum over the 16 lanes that share lane / 16 (fixed butterfly order).
    v += __shfl_xor(v, 8, kWave);
    v += __shfl_xor(v, 4, kWave);
    v += __shfl_xor(v, 2, kWave);
    v += __shfl_xor(v, 1, kWave);
    return v;
}

// ------------------------------------------------------------ DPP rows --
// Cross-lane moves inside 16-lane rows without LDS (quad_perm, row mirrors).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each row

// Sum over the 16 lanes of each row, returned to all of them (every lane
// computes the same additions in the same order, so the results agree bitwise).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    return v;
}

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    return v;
}

// Lowest lane l < n (n <= 64) holding the largest v (wave-uniform result).
__device__ __forceinline__ int wave_argmax_lowest(float v, int n) {
    const int l = threadIdx.x & 63;
    const float x = l < n ? v : -INFINITY;
    const float m = row16_max(x);
    float best = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 0));
    if (n > 16) {
        best = fmaxf(best, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 16)));
        best = fmaxf(best, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 32)));
        best = fmaxf(best, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), 48)));
    }
    const uint64_t mask = __ballot(l < n && x == best);
    return mask ? __ffsll(static_cast<unsigned long long>(mask)) - 1 : 0;
}

// Make this wave's LDS writes visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sum of n (1 <= n <= NMAX) values v[0], v[stride], ... in index order.  The
// loads are unconditional (terms past n re-read term n-1, always in bounds)
// and the unwanted ones are dropped with selects, so the code is straight-line
// and every load is issued before the first add.
template <int NMAX>
__device__ __forceinline__ float sum_strided(const float* v, int64_t stride, int n) {
    float t[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) t[i] = v[static_cast<int64_t>(i < n ? i : n - 1) * stride];
    float s = t[0];
#pragma unroll
    for (int i = 1; i < NMAX; ++i) s = i < n ? s + t[i] : s;
    return s;
}

// ------------------------------------------------------------------- MFMA --
// v_mfma_f32_16x16x32_bf16, D = A (16x32) * B (32x16) + C, one wave:
//   lane l supplies A[l % 16][8*(l/16) .. 8*(l/16)+7]
//   lane l supplies B[8*(l/16) .. 8*(l/16)+7][l % 16]
//   lane l holds    D[4*(l/16) + i][l % 16], i = 0..3
// With both operands stored K-contiguous (row-major [M][K] and [N][K]), each
// lane's fragment is 16 contiguous bytes.

__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
    bf16x8 av = __builtin_bit_cast(bf16x8, a);
    bf16x8 bv = __builtin_bit_cast(bf16x8, b);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace corr
