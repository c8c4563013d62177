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

// Two f32 -> one dword holding two 16-bit values (lo = a), round to nearest even; one
// v_cvt_pk_{f16,bf16}_f32 on gfx950.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2_t v = {a, b};
    if constexpr (BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}

// max over the two 32-lane halves of the wave (lane l and l ^ 32), one v_permlane32_swap
__device__ __forceinline__ float max_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // elements go through scalars: a bit_cast of a vector element reads element 0 here
    const uint32_t lo = r[0], hi = r[1];
    return fmaxf(__builtin_bit_cast(float, lo), __builtin_bit_cast(float, hi));
}

// sum over the two 32-lane halves of the wave (lane l and l ^ 32)
__device__ __forceinline__ float sum_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t lo = r[0], hi = r[1];
    return __builtin_bit_cast(float, lo) + __builtin_bit_cast(float, hi);
}

// Four int8 (one dword) -> four exact f16 values in two dwords.  Offset-binary trick:
// byte u = x + 128 placed under exponent byte 0x64 is the f16 number 1024 + u, and
// subtracting 1152 leaves x exactly (every integer below 2048 is an f16).
// v_perm_b32 (perm(s0, s1, sel)): result byte i = byte sel.byte[i] of the 8-byte value
// whose bytes 0-3 are s1 and 4-7 are s0.  With s0 = 0x64646464 the selectors below put
// byte values under the f16 exponent byte 0x64.
constexpr uint32_t kF16Exp = 0x64646464u;
constexpr uint32_t kSelLoPair = 0x04010400u;   // [s1.b0, 64, s1.b1, 64]
constexpr uint32_t kSelHiPair = 0x04030402u;   // [s1.b2, 64, s1.b3, 64]

__device__ __forceinline__ uint32_t f16_unbias(uint32_t biased_pair) {
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, biased_pair) - bias);
}

__device__ __forceinline__ u32x2 i8x4_to_f16x4(uint32_t w) {
    const uint32_t u = w ^ 0x80808080u;
    u32x2 r;
    r.x = f16_unbias(__builtin_amdgcn_perm(kF16Exp, u, kSelLoPair));
    r.y = f16_unbias(__builtin_amdgcn_perm(kF16Exp, u, kSelHiPair));
    return r;
}

// Transpose-and-convert for the PV operands of an int8 V tile, one half at a time.
// rows[r] holds 8 int8 of token row r (columns c = 0..7, little-endian in .x then .y).
// Half w returns, for column n = 4w + j, the 8 f16 values rows[0..7][n] packed as the
// 4 dwords (rows 2i, 2i+1) of an MFMA operand: out[j][i].  Offset-binary bytes
// (x ^ 0x80) are paired across two rows by one perm, then each pair is placed under
// the f16 exponent and unbiased.
__device__ __forceinline__ void i8_rows_to_f16_cols_half(const u32x2 (&rows)[8], int w,
                                                         u32x4 (&out)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = rows[2 * i][w] ^ 0x80808080u;       // row 2i
        const uint32_t b = rows[2 * i + 1][w] ^ 0x80808080u;   // row 2i+1
        // [a.b0, b.b0, a.b1, b.b1] and [a.b2, b.b2, a.b3, b.b3]
        const uint32_t t01 = __builtin_amdgcn_perm(b, a, 0x05010400u);
        const uint32_t t23 = __builtin_amdgcn_perm(b, a, 0x07030602u);
        out[0][i] = f16_unbias(__builtin_amdgcn_perm(kF16Exp, t01, kSelLoPair));
        out[1][i] = f16_unbias(__builtin_amdgcn_perm(kF16Exp, t01, kSelHiPair));
        out[2][i] = f16_unbias(__builtin_amdgcn_perm(kF16Exp, t23, kSelLoPair));
        out[3][i] = f16_unbias(__builtin_amdgcn_perm(kF16Exp, t23, kSelHiPair));
    }
}

// FLOAT8_E4M3FN codes -> f16, exactly (every E4M3 value is an f16 value): the gfx950
// conversion takes the two codes of one 16-bit word of its source.
template <bool HI>
__device__ __forceinline__ uint32_t f8x2_to_f16x2(uint32_t w) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(uint32_t, r);
}

// 8 codes (a = codes 0..3, b = 4..7) -> 8 f16 in order
__device__ __forceinline__ u32x4 f8x8_to_f16x8(uint32_t a, uint32_t b) {
    return u32x4{f8x2_to_f16x2<false>(a), f8x2_to_f16x2<true>(a),
                 f8x2_to_f16x2<false>(b), f8x2_to_f16x2<true>(b)};
}

// The fp8 counterpart of i8_rows_to_f16_cols_half: 8 rows of 8 codes (dword w = columns
// 4w .. 4w+3) -> 4 PV operands, out[j][i] = f16 pair (row 2i, row 2i+1) of column 4w + j.
// One perm pairs the two rows' codes per column, one conversion expands a pair.
__device__ __forceinline__ void f8_rows_to_f16_cols_half(const u32x2 (&rows)[8], int w,
                                                         u32x4 (&out)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = rows[2 * i][w];        // row 2i
        const uint32_t b = rows[2 * i + 1][w];    // row 2i+1
        // [a.b0, b.b0, a.b1, b.b1] and [a.b2, b.b2, a.b3, b.b3]
        const uint32_t t01 = __builtin_amdgcn_perm(b, a, 0x05010400u);
        const uint32_t t23 = __builtin_amdgcn_perm(b, a, 0x07030602u);
        out[0][i] = f8x2_to_f16x2<false>(t01);
        out[1][i] = f8x2_to_f16x2<true>(t01);
        out[2][i] = f8x2_to_f16x2<false>(t23);
        out[3][i] = f8x2_to_f16x2<true>(t23);
    }
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

// D(16x16 i32) += A(16x64 i8) * B(64x16 i8); lane l holds A row l%16 / B column l%16,
// 16 bytes of k each (lane group l/16 takes its own quarter of k); exact in i32.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 mfma16x16x64_i8(u32x4 a, u32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                 __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// D(32x32 f32) += A(32x8) * B(8x32); lane l holds A row l%32 / B column l%32 with
// k = 4*(l/32) .. +3 (two 16-bit values per dword).
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x8(u32x2 a, u32x2 b, f32x16 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
    if constexpr (BF16) {
        return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(
            __builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_32x32x8f16(
            __builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
}

// c + the two 16-bit values of dword a, in f32 (v_dot2 against (1, 1): the products
// are exact, the sums are f32).
template <bool BF16>
__device__ __forceinline__ float dot2_ones(uint32_t a, float c) {
    if constexpr (BF16) {
        const bf16x2_t one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), one, c, false);
    } else {
        const f16x2_t one = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), one, c, false);
    }
}

// c + the sum of squares of the two 16-bit values of dword a, in f32 (the squares are
// exact, the sums are f32).
template <bool BF16>
__device__ __forceinline__ float dot2_self(uint32_t a, float c) {
    if constexpr (BF16) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, a), c, false);
    } else {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                      __builtin_bit_cast(f16x2_t, a), c, false);
    }
}

// --------------------------------------------------------------------- misc
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// v from the lane that DPP control `ctrl` names (quad_perm / row_ror / mirrors: every
// lane has a source inside its row, so bound_ctrl, which zeroes lanes without one,
// changes nothing; it lets the compiler fold the move into the instruction that uses it)
template <int ctrl>
__device__ __forceinline__ float dpp_f(float v) {
    const int x = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, ctrl, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;    // row_ror:4
constexpr int kDppRor8 = 0x128;    // row_ror:8

// sum over the 4 lanes of each quad (every lane of the quad gets it)
__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<kDppXor1>(v);
    return v + dpp_f<kDppXor2>(v);
}

constexpr int kDppHalfMirror = 0x141;   // row_half_mirror: lane i <- lane 7 - i of its 8
constexpr int kDppMirror = 0x140;       // row_mirror: lane i <- lane 15 - i of its 16

// sum over each aligned group of N lanes (N = 4, 8 or 16; every lane of the group gets
// it): the quad sums, then the mirrored half, then the mirrored row
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
    v = quad_sum(v);
    if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_f<kDppMirror>(v);
    return v;
}

// max / min over the 64 lanes of the wave (wave-uniform result): DPP within each row of
// 16 lanes, then the four rows' values through v_readlane
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppRor4>(v));
    v = fmaxf(v, dpp_f<kDppRor8>(v));
    const int x = __builtin_bit_cast(int, v);
    return fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48))));
}
__device__ __forceinline__ float wave_min(float v) {
    v = fminf(v, dpp_f<kDppXor1>(v));
    v = fminf(v, dpp_f<kDppXor2>(v));
    v = fminf(v, dpp_f<kDppRor4>(v));
    v = fminf(v, dpp_f<kDppRor8>(v));
    const int x = __builtin_bit_cast(int, v);
    return fminf(fminf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 16))),
                 fminf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 48))));
}

// Select the lo (even element) or hi (odd element) 16-bit halves of two dwords.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
    return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
    return (a >> 16) | (b & 0xffff0000u);
}

}  // namespace pa
