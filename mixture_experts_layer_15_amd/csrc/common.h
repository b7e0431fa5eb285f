// common.h -- device types and helpers shared by the gfx950 kernels of the
// MoE FFN forward.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// 16-byte vector used for every coalesced global/LDS copy.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// MFMA operand and accumulator fragments.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 is the upper half of an IEEE binary32, so widening is
// exact; narrowing rounds to nearest, ties to even, a NaN stays a NaN.  The
// narrowing is gfx950's v_cvt_pk_bf16_f32 (what a conversion to __bf16
// compiles to), two values per instruction; an exhaustive check over all 2^32
// inputs found it equal to the integer rounding (add 0x7fff plus the kept
// lsb, truncate) on every non-NaN input, denormals included.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// Two fp32 -> packed pair of bf16 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// GELU in its erf form, v * Phi(v), in fp32 with the device library's erff.
__device__ __forceinline__ float gelu_erf(float v) {
    return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

// The same GELU for results rounded to bf16: Phi through the complementary
// error function of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (erfc z = t P(t) exp(-z^2), t = 1 / (1 + p z), z >= 0, with
// |error| <= 1.5e-7), on the hardware reciprocal and exp2.  The error it adds
// to v * Phi(v) is below 1e-7 |v|, four orders under bf16's rounding step.
__device__ __forceinline__ float gelu_erf_bf16(float v) {
    const float z = fabsf(v) * 0.70710678118654752440f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
    float p = fmaf(t, 1.061405429f, -1.453152027f);
    p = fmaf(t, p, 1.421413741f);
    p = fmaf(t, p, -0.284496736f);
    p = fmaf(t, p, 0.254829592f);
    const float half_erfc = 0.5f * t * p * __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);
    return v * (v >= 0.0f ? 1.0f - half_erfc : half_erfc);
}

// Element type traits: raw storage type and 16-byte vector width.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPerVec = 4;
    __device__ __forceinline__ static float to_f32(const u32x4& v, int i) {
        return __uint_as_float(v[i]);
    }
};
template <> struct Elem<uint16_t> {
    static constexpr int kPerVec = 8;
    __device__ __forceinline__ static float to_f32(const u32x4& v, int i) {
        uint32_t w = v[i >> 1];
        return bf16_bits_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
    }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
