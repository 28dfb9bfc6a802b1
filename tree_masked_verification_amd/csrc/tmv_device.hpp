// tmv_device.hpp -- small device helpers shared by the gfx950 kernels of libtmv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tmv.h"

namespace tmv {

// a compile-time integer passed as a value (to generic lambdas)
template <int N>
struct Const {
    static constexpr int value = N;
};

constexpr int kWave = 64;       // CDNA wavefront width
constexpr int kXcds = 8;        // MI355X: workgroups are dealt round-robin to 8 XCDs

// ---------------------------------------------------------------- bf16 as raw bits
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// two floats to a packed bf16 pair (low half first), round to nearest even, by the hardware
// conversion (v_cvt_pk_bf16_f32): equal to f32_to_bf16 for every non-NaN value
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, kWave);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint64_t w = shfl_xor_u64(v, o);
        v = w > v ? w : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += shfl_xor_u64(v, o);
    return v;
}

typedef unsigned __int128 u128;

__device__ __forceinline__ u128 shfl_xor_u128(u128 v, int o) {
    uint64_t lo = shfl_xor_u64(static_cast<uint64_t>(v), o);
    uint64_t hi = shfl_xor_u64(static_cast<uint64_t>(v >> 64), o);
    return (static_cast<u128>(hi) << 64) | lo;
}

__device__ __forceinline__ u128 wave_sum_u128(u128 v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += shfl_xor_u128(v, o);
    return v;
}

// ---------------------------------------------------------------- Philox4x64-10
// Counter-based generator of Salmon, Moraes, Dror and Shaw (SC'11): ten rounds of two
// 64x64->128-bit products with the published multipliers, keys bumped by the published
// Weyl constants.  word(n) is 64-bit lane n%4 of the block at counter {n/4 + 1, 0, 0, 0}.
__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t k0, uint64_t k1, uint64_t out[4]) {
    uint64_t x0 = c0, x1 = 0, x2 = 0, x3 = 0;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
        uint64_t hi0 = __umul64hi(m0, x0), lo0 = m0 * x0;
        uint64_t hi1 = __umul64hi(m1, x2), lo1 = m1 * x2;
        uint64_t y0 = hi1 ^ x1 ^ k0, y2 = hi0 ^ x3 ^ k1;
        x0 = y0; x1 = lo1; x2 = y2; x3 = lo0;
        k0 += 0x9E3779B97F4A7C15ull;
        k1 += 0xBB67AE8584CAA73Bull;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

__device__ __forceinline__ uint64_t philox_word(uint64_t seed, uint64_t stream, uint64_t n) {
    uint64_t o[4];
    philox4x64_10(n / 4 + 1, seed, stream, o);
    const int lane = static_cast<int>(n & 3);
    return lane == 0 ? o[0] : lane == 1 ? o[1] : lane == 2 ? o[2] : o[3];
}

__device__ __forceinline__ int bitlen_u128(u128 x) {
    uint64_t hi = static_cast<uint64_t>(x >> 64), lo = static_cast<uint64_t>(x);
    if (hi) return 128 - __clzll(static_cast<long long>(hi));
    if (lo) return 64 - __clzll(static_cast<long long>(lo));
    return 0;
}

}  // namespace tmv

// host-side helpers shared by the entry points
namespace tmv_host {
inline int launch_status(hipError_t e) { return e == hipSuccess ? TMV_OK : TMV_ERR_DEVICE; }
}
