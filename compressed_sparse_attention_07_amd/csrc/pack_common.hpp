// Exact format conversions shared by the pack kernels and by the attention kernel's window
// write: FP4 (E2M1 elements + one E4M3 scale per 16 channels), MXFP4 (E2M1 + one E8M0 scale per
// 32 channels) and E4M3 values.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token",
// section XI (main KV in FP4 with E4M3 scales per 16 channels and no second-level scale; the
// indexer key in MXFP4; the recent window at FP8) and section VII (the formats' byte budget).
//
// Rounding is round-to-nearest-even everywhere.  Nothing divides: every decision compares the
// input with an exactly representable product (6 times an E4M3 midpoint, an E2M1 midpoint
// times a scale), so exact ties are seen as ties.
#pragma once

#include "csa2_device.hpp"

namespace csa2 {

// Exact value of a non-negative E4M3 ("fn") code 0..126.
__device__ __forceinline__ float e4m3_pos_value(int c) {
    int e = c >> 3, m = c & 7;
    if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
    return __uint_as_float((uint32_t)((e + 120) << 23) | (uint32_t)(m << 20));
}

__device__ __forceinline__ int e4m3_round_amax_over_6(float amax) {
    // largest code c with 6 * v(c) <= amax, then round half to even against the midpoint
    int lo = 0;
#pragma unroll
    for (int step = 64; step > 0; step >>= 1) {
        int c = lo + step;
        if (c <= 126 && 6.0f * e4m3_pos_value(c) <= amax) lo = c;
    }
    if (lo < 126) {
        float t = 3.0f * (e4m3_pos_value(lo) + e4m3_pos_value(lo + 1));  // 6 * midpoint, exact
        if (amax > t || (amax == t && (lo & 1))) lo += 1;
    }
    return lo;
}

// E2M1 code (sign bit 3) of a bf16 value for scale s: the magnitude code counts the midpoints
// between consecutive E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 that |x| passes (a tie goes to
// the even code: > at midpoints below an odd code, >= below an even one).
__device__ __forceinline__ uint32_t e2m1_code(uint32_t bits16, float s) {
    float a = __uint_as_float((bits16 & 0x7fffu) << 16);
    uint32_t mag = 0;
    if (s != 0.0f) {
        const float t0 = 0.25f * s, t1 = 0.75f * s, t2 = 1.25f * s, t3 = 1.75f * s;
        const float t4 = 2.5f * s, t5 = 3.5f * s, t6 = 5.0f * s;
        mag = (a > t0) + (a >= t1) + (a > t2) + (a >= t3) + (a > t4) + (a >= t5) + (a > t6);
    }
    return mag | ((bits16 >> 12) & 0x8u);
}

// Two 16-bit lanes compared at once: all ones in each half of the result where the half of a is
// below the half of b.  Exact as long as the two halves differ by less than 2^15 (the FP4
// packer's operands are 15-bit bf16 magnitude patterns and thresholds).  Non-negative bf16
// values order like their 15-bit patterns, so the packer decides E2M1 codes two channels per
// instruction with these.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lt16_mask(uint32_t a, uint32_t b) {
    const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, a) - __builtin_bit_cast(u16x2_t, b));
    uint32_t m;
    // the sign of each 16-bit difference spread over its half (one packed shift; written out
    // because the compiler otherwise compares and selects each half on its own).  The shift
    // amount is a register holding 15 in both halves: a packed instruction's high half reads
    // bits 31..16 of each operand, which an inline constant 15 leaves zero.
    asm("v_pk_ashrrev_i16 %0, %1, %2" : "=v"(m) : "s"(0x000f000fu), "v"(d));
    return m;
}

// One 32-channel MXFP4 block (microscaling conversion): scale X = 2^(floor(log2 amax) - 2), its
// E8M0 code = (bf16 exponent field of amax) - 2 clamped to [1, 254]; elements nearest to x / X,
// ties to even, saturating at 6, decided by the threshold compares above (X is a power of two,
// so every threshold times X is exact).  w: 16 dwords of bf16 pairs -> 4 code dwords.
__device__ __forceinline__ uint32_t mx_pack_block(const uint32_t (&w)[16], uint32_t (&out)[4]) {
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        am = max(am, w[k] & 0x7fffu);
        am = max(am, (w[k] >> 16) & 0x7fffu);
    }
    const int code = min(254, max(1, (int)(am >> 7) - 2));
    const float X = __uint_as_float((uint32_t)code << 23);  // 2^(code - 127), a normal float
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t o = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t v = w[4 * k + j];
            o |= (e2m1_code(v & 0xffffu, X) | (e2m1_code(v >> 16, X) << 4)) << (8 * j);
        }
        out[k] = o;
    }
    return (uint32_t)code;
}

// Nearest E4M3 ("fn") code of a bf16 value, ties to even, saturating at 448 (the format has no
// infinity), with the value's sign bit.  Exact integer rounding of the bf16 fields: normal E4M3
// targets round the 7-bit mantissa to 3 bits (a carry moves into the exponent by plain
// addition: codes are ordered like values); below 2^-6 the code is the subnormal count
// RNE(|x| * 2^9), exact in fp32.
__device__ __forceinline__ uint32_t e4m3_code_of_bf16(uint32_t b) {
    const uint32_t a = b & 0x7fffu;
    uint32_t c;
    if (a >= 0x43E0u) {  // |x| >= 448 (and inf): saturate
        c = 0x7Eu;
    } else if (a >= 0x3C80u) {  // |x| >= 2^-6: normal target, biased exponent (a >> 7) - 120
        const uint32_t m3 = (a >> 4) & 7u, r = a & 0xFu;
        const uint32_t up = (r > 8u || (r == 8u && (m3 & 1u))) ? 1u : 0u;
        c = ((((a >> 7) - 120u) << 3) | m3) + up;  // < 0x7F: a < 0x43E0 leaves m3 + up <= 6 at exponent 15
    } else {
        c = (uint32_t)__builtin_rintf(__uint_as_float(a << 16) * 512.0f);  // 0..8, 8 = 2^-6 = code 0x08
    }
    return c | ((b >> 8) & 0x80u);
}

// Four E4M3 bytes of the two bf16 pairs w0, w1 (channel order kept).
__device__ __forceinline__ uint32_t e4m3_pack4(uint32_t w0, uint32_t w1) {
    return e4m3_code_of_bf16(w0 & 0xffffu) | (e4m3_code_of_bf16(w0 >> 16) << 8) |
           (e4m3_code_of_bf16(w1 & 0xffffu) << 16) | (e4m3_code_of_bf16(w1 >> 16) << 24);
}

}  // namespace csa2
