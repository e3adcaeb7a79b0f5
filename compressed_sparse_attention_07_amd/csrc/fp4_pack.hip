// FP4 pack-on-write: post-RoPE bf16 vectors -> E2M1 codes + one E4M3 scale per 16 channels.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token",
// section XI, and the visualisation page's FP4 caption: E2M1 elements, one E4M3 scale
// shared by 16 channels, no second-level global scale, applied after RoPE.
//
// Rounding is round-to-nearest-even for both the scale (of amax/6, 6 being the largest
// E2M1 magnitude) and the elements (of x/scale, saturating at 6).  Nothing divides:
// every decision compares the input with an exactly representable product (6 times an
// E4M3 midpoint, or an E2M1 midpoint times the scale), so exact ties are seen as ties.
//
// One thread packs one 16-channel group: it reads 32 B of bf16, writes 8 B of codes and
// 1 B of scale.  Consecutive threads own consecutive groups, so a wave reads 2 KiB and
// writes 512 B + 64 B contiguously.  The kernel is a pure HBM stream.
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

__device__ __forceinline__ uint32_t e2m1_code(uint32_t bits16, float s) {
    float a = __uint_as_float((bits16 & 0x7fffu) << 16);
    uint32_t mag = 0;
    if (s != 0.0f) {
        // midpoints between consecutive E2M1 magnitudes 0,.5,1,1.5,2,3,4,6 (exact times s)
        const float t0 = 0.25f * s, t1 = 0.75f * s, t2 = 1.25f * s, t3 = 1.75f * s;
        const float t4 = 2.5f * s, t5 = 3.5f * s, t6 = 5.0f * s;
        mag = (a > t0) + (a >= t1) + (a > t2) + (a >= t3) + (a > t4) + (a >= t5) + (a > t6);
    }
    return mag | ((bits16 >> 12) & 0x8u);
}

__global__ __launch_bounds__(256) void k_fp4_pack(const uint16_t* __restrict__ x, int64_t n_tok, int dim,
                                                  const int64_t* __restrict__ dst_rows, int64_t row0,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  int64_t cap_rows) {
    const int groups = dim >> 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_tok * groups) return;
    const int64_t t = gid / groups;
    const int g = (int)(gid - t * groups);
    const int64_t row = dst_rows ? dst_rows[t] : row0 + t;
    if (row < 0 || row >= cap_rows) return;

    const uint4* src = reinterpret_cast<const uint4*>(x + t * dim + g * 16);
    uint4 v0 = src[0], v1 = src[1];
    uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};

    // amax: bf16 magnitudes order like their 15-bit patterns
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        am = max(am, w[k] & 0x7fffu);
        am = max(am, (w[k] >> 16) & 0x7fffu);
    }
    const float amax = __uint_as_float(am << 16);
    const int sc = e4m3_round_amax_over_6(amax);
    const float s = e4m3_pos_value(sc);

    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t c0 = e2m1_code(w[k] & 0xffffu, s);
        uint32_t c1 = e2m1_code(w[k] >> 16, s);
        lo |= (c0 | (c1 << 4)) << (8 * k);
        uint32_t c2 = e2m1_code(w[k + 4] & 0xffffu, s);
        uint32_t c3 = e2m1_code(w[k + 4] >> 16, s);
        hi |= (c2 | (c3 << 4)) << (8 * k);
    }
    *reinterpret_cast<uint2*>(codes + row * (dim >> 1) + g * 8) = make_uint2(lo, hi);
    scales[row * groups + g] = (uint8_t)sc;
}

hipError_t launch_fp4_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream) {
    const int64_t total = n_tok * (dim >> 4);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_fp4_pack, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dim, dst_rows, row0,
                       codes, scales, cap_rows);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// MXFP4 indexer keys ([Article] sections VII and XI: indexer K in MXFP4, E2M1 elements with
// one E8M0 scale per 32 channels).  Microscaling conversion: the block's scale is
// X = 2^(floor(log2 amax) - 2), i.e. E8M0 code = (bf16 exponent field of amax) - 2, clamped to
// [1, 254]; each element is the E2M1 value nearest to x / X, ties to even, saturating at 6,
// decided by the same exact threshold compares as the KV packer (X is a power of two, so
// every threshold times X is exact).  One thread packs one 32-channel block: 64 B in,
// 16 B of codes and 1 scale byte out.
// ----------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_mx_pack(const uint16_t* __restrict__ x, int64_t n_tok, int dim,
                                                 const int64_t* __restrict__ dst_rows, int64_t row0,
                                                 uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                 int64_t cap_rows) {
    const int blocks = dim >> 5;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_tok * blocks) return;
    const int64_t t = gid / blocks;
    const int b = (int)(gid - t * blocks);
    const int64_t row = dst_rows ? dst_rows[t] : row0 + t;
    if (row < 0 || row >= cap_rows) return;

    const uint4* src = reinterpret_cast<const uint4*>(x + t * dim + b * 32);
    uint32_t w[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint4 v = src[k];
        w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
    }
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        am = max(am, w[k] & 0x7fffu);
        am = max(am, (w[k] >> 16) & 0x7fffu);
    }
    const int code = min(254, max(1, (int)(am >> 7) - 2));
    const float X = __uint_as_float((uint32_t)code << 23);  // 2^(code - 127), a normal float
    uint32_t out[4];
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
    *reinterpret_cast<uint4*>(codes + row * (dim >> 1) + b * 16) = make_uint4(out[0], out[1], out[2], out[3]);
    scales[row * blocks + b] = (uint8_t)code;
}

hipError_t launch_mx_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                          uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream) {
    const int64_t total = n_tok * (dim >> 5);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_mx_pack, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dim, dst_rows, row0, codes,
                       scales, cap_rows);
    return hipGetLastError();
}

// ----------------------------------------------------------------------------------------
// FP8 window store ([Article] section XI: the recent-window cache stays at FP8): each bf16
// value becomes the nearest E4M3 ("fn") value, ties to even, saturating at 448 (the format
// has no infinity), keeping the value's sign bit.  Exact integer rounding of the bf16
// fields: normal E4M3 targets round the 7-bit mantissa to 3 bits (a carry moves into the
// exponent by plain addition: codes are ordered like values); below 2^-6 the code is the
// subnormal count RNE(|x| * 2^9), exact in fp32.  One thread converts 8 channels.
// ----------------------------------------------------------------------------------------
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

__global__ __launch_bounds__(256) void k_fp8_pack(const uint16_t* __restrict__ x, int64_t n_tok, int dim,
                                                  const int64_t* __restrict__ dst_rows, int64_t row0,
                                                  uint8_t* __restrict__ out, int64_t cap_rows) {
    const int octs = dim >> 3;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_tok * octs) return;
    const int64_t t = gid / octs;
    const int k = (int)(gid - t * octs);
    const int64_t row = dst_rows ? dst_rows[t] : row0 + t;
    if (row < 0 || row >= cap_rows) return;
    const uint4 v = *reinterpret_cast<const uint4*>(x + t * dim + k * 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        lo |= (e4m3_code_of_bf16(w[j] & 0xffffu) | (e4m3_code_of_bf16(w[j] >> 16) << 8)) << (16 * j);
        hi |= (e4m3_code_of_bf16(w[j + 2] & 0xffffu) | (e4m3_code_of_bf16(w[j + 2] >> 16) << 8)) << (16 * j);
    }
    *reinterpret_cast<uint2*>(out + row * dim + k * 8) = make_uint2(lo, hi);
}

hipError_t launch_fp8_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint8_t* out, int64_t cap_rows, hipStream_t stream) {
    const int64_t total = n_tok * (dim >> 3);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_fp8_pack, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dim, dst_rows, row0, out,
                       cap_rows);
    return hipGetLastError();
}

}  // namespace csa2
