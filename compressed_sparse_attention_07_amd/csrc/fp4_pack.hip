// Pack-on-write kernels: post-RoPE bf16 KV vectors -> FP4 (E2M1 codes + one E4M3 scale per 16
// channels), indexer keys -> MXFP4 (E2M1 + one E8M0 scale per 32 channels), window vectors ->
// E4M3 bytes, and the decode step's own token (FP4 row + indexer key row) in one launch.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token",
// section XI, and the visualisation page's FP4 caption: E2M1 elements, one E4M3 scale shared by
// 16 channels, no second-level global scale, applied after RoPE; the indexer key in MXFP4 and
// the recent window at FP8.  The conversions themselves (exact, division-free, ties to even)
// are in pack_common.hpp.
#include "pack_common.hpp"

namespace csa2 {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// The E4M3 scale code of every possible group amax: index = the 15-bit pattern of amax (bf16
// magnitudes order like their patterns), value = e4m3_round_amax_over_6 of that amax.  Built by
// the compiler from the same search, so a group's scale is one byte load (from L2 after the
// first groups) instead of a seven-step search of ~80 instructions per group.
struct ScaleLut {
    uint8_t c[32768];
};

constexpr float e4m3_pos_value_cx(int c) {
    const int e = c >> 3, m = c & 7;
    return e == 0 ? (float)m * 0.001953125f
                  : __builtin_bit_cast(float, (uint32_t)((e + 120) << 23) | (uint32_t)(m << 20));
}

constexpr ScaleLut make_scale_lut() {
    ScaleLut t{};
    for (int a = 0; a < 32768; ++a) {
        const float amax = __builtin_bit_cast(float, (uint32_t)a << 16);
        int lo = 0;  // largest code c with 6 v(c) <= amax, then round half to even at the midpoint
        for (int step = 64; step > 0; step >>= 1) {
            const int c = lo + step;
            if (c <= 126 && 6.0f * e4m3_pos_value_cx(c) <= amax) lo = c;
        }
        if (lo < 126) {
            const float th = 3.0f * (e4m3_pos_value_cx(lo) + e4m3_pos_value_cx(lo + 1));
            if (amax > th || (amax == th && (lo & 1))) lo += 1;
        }
        t.c[a] = (uint8_t)lo;
    }
    return t;
}

__device__ constexpr ScaleLut kScaleLut = make_scale_lut();

// (m & a) | (~m & b) as one instruction: written out, because the compiler otherwise re-forms
// these selects and the code-bit merges into two or three instructions each
__device__ __forceinline__ uint32_t bfi32(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t d;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "v"(m), "v"(a), "v"(b));
    return d;
}

__device__ __forceinline__ uint32_t bf16_both_halves(float x) {  // x's bf16 pattern (exact) in both halves
    return __builtin_amdgcn_perm(__float_as_uint(x), __float_as_uint(x), 0x03020302u);
}

// One 16-channel FP4 group: w = 8 dwords of bf16 pairs (channel 2k in the low half) ->
// codes (lo: channels 0..7, hi: 8..15; low nibble = even channel) and the E4M3 scale code.
// The seven E2M1 midpoint thresholds m * s (m = 1/4, 3/4, 5/4, 7/4, 5/2, 7/2, 5) are s, 3s, 5s
// and 7s times powers of two: four exact bf16 patterns (s has at most 4 significant bits, 7s at
// most 7) and exponent-field subtractions give all seven.  Each pair of channels then replaces
// e2m1_code's seven compares by a three-level tree on 16-bit lanes (|x| >= t3; >= t5 or t1; >
// one of t6, t4, t2, t0: e2m1_code's tie rules), with ">= t" written as "> t - 1" so that every
// level's mask is a code bit.
__device__ __forceinline__ uint32_t fp4_pack_group(const uint32_t (&w)[8], uint32_t& lo, uint32_t& hi) {
    // magnitudes (bf16 magnitudes order like their 15-bit patterns) and their maximum
    uint32_t A[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) A[k] = w[k] & 0x7fff7fffu;
    u16x2_t mx = __builtin_bit_cast(u16x2_t, A[0]);
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2_t, A[k]));
    const uint32_t am = max((uint32_t)mx[0], (uint32_t)mx[1]);
    const int sc = kScaleLut.c[am];
    const float s = e4m3_pos_value(sc);
    const uint32_t Q1 = bf16_both_halves(s), Q3 = bf16_both_halves(3.0f * s), Q5 = bf16_both_halves(5.0f * s),
                   Q7 = bf16_both_halves(7.0f * s);
    // (s >= 2^-9 when sc > 0: no field borrows across the halves; sc == 0 is handled below)
    constexpr uint32_t kE2 = 0x01000100u, kE1 = 0x00800080u, kOne = 0x00010001u;
    const uint32_t T0 = Q1 - kE2, T1m = Q3 - kE2 - kOne, T2 = Q5 - kE2, T3m = Q7 - kE2 - kOne;
    const uint32_t T4 = Q5 - kE1, T5m = Q7 - kE1 - kOne, T6 = Q5;
    uint32_t c[8];  // code of channel 2k in bits 0..3, of channel 2k + 1 in bits 16..19
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t a = A[k];
        const uint32_t g4 = lt16_mask(T3m, a);                       // |x| >= t3
        const uint32_t pa = bfi32(g4, T6, T2), pb = bfi32(g4, T4, T0);
        const uint32_t g2 = lt16_mask(bfi32(g4, T5m, T1m), a);       // |x| >= t5 (or t1)
        const uint32_t g1 = lt16_mask(bfi32(g2, pa, pb), a);         // |x| > t6, t4, t2 (or t0)
        const uint32_t sg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, w[k]) >> (unsigned short)12);
        c[k] = bfi32(0x00040004u, g4, bfi32(0x00020002u, g2, bfi32(0x00010001u, g1, sg)));  // sign: bit 3
    }
    // bytes: channel pairs (2k, 2k + 1) as one byte each, even channel in the low nibble
    auto four = [&](int k0) {
        const uint32_t x0 = __builtin_amdgcn_perm(c[k0 + 1], c[k0], 0x06040200u);
        const uint32_t x1 = __builtin_amdgcn_perm(c[k0 + 3], c[k0 + 2], 0x06040200u);
        return __builtin_amdgcn_perm(x1 | (x1 >> 4), x0 | (x0 >> 4), 0x06040200u);
    };
    const uint32_t keep = sc == 0 ? 0x88888888u : 0xffffffffu;  // a zero scale codes every magnitude 0
    lo = four(0) & keep;
    hi = four(4) & keep;
    return (uint32_t)sc;
}


// Generic FP4 pack (any dim % 16 == 0): one thread per 16-channel group, 32 B in, 8 B of codes
// and 1 B of scale out.
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
    const uint4 v0 = src[0], v1 = src[1];
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint32_t lo, hi;
    const uint32_t sc = fp4_pack_group(w, lo, hi);
    *reinterpret_cast<uint2*>(codes + row * (dim >> 1) + g * 8) = make_uint2(lo, hi);
    scales[row * groups + g] = (uint8_t)sc;
}

// 128-channel vectors (the KV latent): a wave packs 64 * U consecutive groups (8 U tokens), U
// groups per lane, all of the lane's loads issued first (streaming, read once); 8 lanes own one
// token, so its 64 code bytes are one contiguous 512-byte wave store per step and its 8 scale
// bytes are gathered across the 8 lanes into one 8-byte store.
constexpr int kPackU = 2;  // groups per lane (4 measured 82 us per 2^20 tokens against 79, 1 took 87)

__global__ __launch_bounds__(256) void k_fp4_pack128(const uint16_t* __restrict__ x, int64_t n_tok,
                                                     const int64_t* __restrict__ dst_rows, int64_t row0,
                                                     uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                     int64_t cap_rows) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane & 7;
    const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t n_groups = n_tok * 8;
    const int64_t gbase = wave * (kWave * kPackU);
    u32x4_t v[kPackU][2];
    int64_t row[kPackU];
#pragma unroll
    for (int k = 0; k < kPackU; ++k) {
        const int64_t gid = gbase + kWave * k + lane;
        v[k][0] = v[k][1] = u32x4_t{0u, 0u, 0u, 0u};
        row[k] = -1;
        if (gid < n_groups) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + gid * 16);
            v[k][0] = __builtin_nontemporal_load(src);
            v[k][1] = __builtin_nontemporal_load(src + 1);
            row[k] = dst_rows ? dst_rows[gid >> 3] : row0 + (gid >> 3);
        }
    }
#pragma unroll
    for (int k = 0; k < kPackU; ++k) {
        const uint32_t w[8] = {v[k][0][0], v[k][0][1], v[k][0][2], v[k][0][3],
                               v[k][1][0], v[k][1][1], v[k][1][2], v[k][1][3]};
        uint32_t lo, hi;
        const uint32_t sc = fp4_pack_group(w, lo, hi);
        // the token's 8 scale bytes: each quad of lanes ORs its four (quad_perm exchanges), and
        // the token's first lane takes the second quad's word from 4 lanes up (row_shl:4)
        uint32_t sq = sc << (8 * (g & 3));
        sq |= (uint32_t)__builtin_amdgcn_mov_dpp((int)sq, 0xB1, 0xF, 0xF, true);  // quad_perm [1,0,3,2]
        sq |= (uint32_t)__builtin_amdgcn_mov_dpp((int)sq, 0x4E, 0xF, 0xF, true);  // quad_perm [2,3,0,1]
        const uint32_t sh4 = (uint32_t)__builtin_amdgcn_mov_dpp((int)sq, 0x104, 0xF, 0xF, true);
        const int64_t r = row[k];
        if (r >= 0 && r < cap_rows) {
            *reinterpret_cast<uint2*>(codes + r * 64 + g * 8) = make_uint2(lo, hi);
            if (g == 0) *reinterpret_cast<uint2*>(scales + r * 8) = make_uint2(sq, sh4);
        }
    }
}

hipError_t launch_fp4_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream) {
    if (dim == 128 && (reinterpret_cast<uintptr_t>(scales) & 7u) == 0) {
        const int64_t waves = (n_tok * 8 + kWave * kPackU - 1) / (kWave * kPackU);
        const int64_t blocks = (waves + 3) / 4;
        hipLaunchKernelGGL(k_fp4_pack128, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dst_rows, row0,
                           codes, scales, cap_rows);
        return hipGetLastError();
    }
    const int64_t total = n_tok * (dim >> 4);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_fp4_pack, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dim, dst_rows, row0,
                       codes, scales, cap_rows);
    return hipGetLastError();
}

// MXFP4 indexer keys: one thread packs one 32-channel block: 64 B in, 16 B of codes and 1 scale
// byte out.
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
    uint32_t out[4];
    const uint32_t code = mx_pack_block(w, out);
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

// FP8 window store: one thread converts 8 channels.
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
    *reinterpret_cast<uint2*>(out + row * dim + k * 8) = make_uint2(e4m3_pack4(v.x, v.y), e4m3_pack4(v.z, v.w));
}

hipError_t launch_fp8_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint8_t* out, int64_t cap_rows, hipStream_t stream) {
    const int64_t total = n_tok * (dim >> 3);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_fp8_pack, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dim, dst_rows, row0, out,
                       cap_rows);
    return hipGetLastError();
}

// The decode step's own token of a Full layer ([Article] section VIII: a Full layer computes its
// main KV and its indexer key fresh; section XI: the main KV is cached in FP4, the indexer key in
// bf16 or MXFP4): 16 threads per token, threads 0..7 pack the 128-channel KV vector's groups,
// threads 8..15 write the 64-channel key row (bf16: 16 B each; MXFP4: threads 8 and 9 pack one
// 32-channel block each).
__global__ __launch_bounds__(256) void k_token_append(const uint16_t* __restrict__ x, const uint16_t* __restrict__ k_new,
                                                      int64_t n_tok, const int64_t* __restrict__ dst_rows,
                                                      uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                      void* __restrict__ k_idx, uint8_t* __restrict__ k_scales,
                                                      int64_t cap_rows) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t t = gid >> 4;
    const int j = (int)(gid & 15);
    if (t >= n_tok) return;
    const int64_t row = dst_rows[t];
    if (row < 0 || row >= cap_rows) return;
    if (j < 8) {
        const uint4* src = reinterpret_cast<const uint4*>(x + t * 128 + j * 16);
        const uint4 v0 = src[0], v1 = src[1];
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint32_t lo, hi;
        const uint32_t sc = fp4_pack_group(w, lo, hi);
        *reinterpret_cast<uint2*>(codes + row * 64 + j * 8) = make_uint2(lo, hi);
        scales[row * 8 + j] = (uint8_t)sc;
    } else if (k_new != nullptr) {
        const int kk = j - 8;
        if (k_scales == nullptr) {  // bf16 key row: a copy
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(k_idx) + row * 64 + kk * 8) =
                *reinterpret_cast<const uint4*>(k_new + t * 64 + kk * 8);
        } else if (kk < 2) {        // MXFP4 key row
            const uint4* src = reinterpret_cast<const uint4*>(k_new + t * 64 + kk * 32);
            uint32_t w[16];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 v = src[k];
                w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
            }
            uint32_t out[4];
            const uint32_t code = mx_pack_block(w, out);
            *reinterpret_cast<uint4*>(static_cast<uint8_t*>(k_idx) + row * 32 + kk * 16) =
                make_uint4(out[0], out[1], out[2], out[3]);
            k_scales[row * 2 + kk] = (uint8_t)code;
        }
    }
}

hipError_t launch_token_append(const uint16_t* x, const uint16_t* k_new, int64_t n_tok, const int64_t* dst_rows,
                               uint8_t* codes, uint8_t* scales, void* k_idx, uint8_t* k_scales, int64_t cap_rows,
                               hipStream_t stream) {
    const int64_t blocks = (n_tok * 16 + 255) / 256;
    hipLaunchKernelGGL(k_token_append, dim3((unsigned)blocks), dim3(256), 0, stream, x, k_new, n_tok, dst_rows, codes,
                       scales, k_idx, k_scales, cap_rows);
    return hipGetLastError();
}

// bf16 window rows (a copy into the store's rows): one thread moves 16 bytes.
__global__ __launch_bounds__(256) void k_row_copy(const uint16_t* __restrict__ x, int64_t n_tok, int dim,
                                                  const int64_t* __restrict__ dst_rows, int64_t row0,
                                                  uint16_t* __restrict__ out, int64_t cap_rows) {
    const int octs = dim >> 3;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= n_tok * octs) return;
    const int64_t t = gid / octs;
    const int k = (int)(gid - t * octs);
    const int64_t row = dst_rows ? dst_rows[t] : row0 + t;
    if (row < 0 || row >= cap_rows) return;
    *reinterpret_cast<uint4*>(out + row * dim + k * 8) = *reinterpret_cast<const uint4*>(x + t * dim + k * 8);
}

hipError_t launch_row_copy(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint16_t* out, int64_t cap_rows, hipStream_t stream) {
    const int64_t total = n_tok * (dim >> 3);
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(k_row_copy, dim3((unsigned)blocks), dim3(256), 0, stream, x, n_tok, dim, dst_rows, row0, out,
                       cap_rows);
    return hipGetLastError();
}

}  // namespace csa2
