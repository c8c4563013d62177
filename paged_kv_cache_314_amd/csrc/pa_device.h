// Device-side helpers for the gfx950 kernels: raw 16-bit storage, conversions,
// MFMA wrappers, wave shuffles.  CDNA4 only (wave64, v_mfma_*_16x16x32 / 32x32x16).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- conversions
// 16-bit storage -> f32 (exact for both formats).
template <bool BF16>
__device__ __forceinline__ float half_to_f32(uint32_t bits16) {
    if constexpr (BF16) {
        return __uint_as_float(bits16 << 16);
    } else {
        _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16));
        return static_cast<float>(h);
    }
}

// f32 -> 16-bit storage, round to nearest even.
template <bool BF16>
__device__ __forceinline__ uint32_t f32_to_half(float x) {
    if constexpr (BF16) {
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)));
    } else {
        return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
    }
}

// Two f32 -> one dword holding two 16-bit values (lo = a).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return f32_to_half<BF16>(a) | (f32_to_half<BF16>(b) << 16);
}

// Four int8 (one dword) -> four exact f16 values in two dwords.  Offset-binary trick:
// byte u = x + 128 placed under exponent byte 0x64 is the f16 number 1024 + u, and
// subtracting 1152 leaves x exactly (every integer below 2048 is an f16).
__device__ __forceinline__ u32x2 i8x4_to_f16x4(uint32_t w) {
    const uint32_t u = w ^ 0x80808080u;
    const uint32_t lo = (u & 0xffu) | ((u & 0xff00u) << 8) | 0x64006400u;
    const uint32_t hi = ((u >> 16) & 0xffu) | ((u >> 8) & 0xff0000u) | 0x64006400u;
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
    const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
    u32x2 r;
    r.x = __builtin_bit_cast(uint32_t, a);
    r.y = __builtin_bit_cast(uint32_t, b);
    return r;
}

// ----------------------------------------------------------------------- MFMA
// D(16x16 f32) += A(16x32) * B(32x16); lane l holds A row l%16 / B column l%16 with
// k = 8*(l/16) .. 8*(l/16)+7, and D column l%16, rows 4*(l/16) .. 4*(l/16)+3.
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// D(32x32 f32) += A(32x16) * B(16x32); lane l holds A row l%32 / B column l%32 with
// k = 8*(l/32) .. +7, and D column l%32, rows 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

// --------------------------------------------------------------------- misc
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// Select the lo (even element) or hi (odd element) 16-bit halves of two dwords.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

}  // namespace pa
