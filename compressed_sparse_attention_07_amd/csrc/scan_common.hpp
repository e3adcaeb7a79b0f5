// Shared pieces of the indexer kernels: scan shape constants, raw buffer loads, the MFMA
// query fragments and score, MXFP4 key fragments and the 8-lane block maximum.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token", section
// IX (indexer scores) and section XI (MXFP4 indexer keys).
#pragma once

#include "csa2_device.hpp"

namespace csa2 {
constexpr int kScoreNT = 256;
// Scan-kernel shape (compile-time; the defaults are the tuned ones):
//   CSA2_SCAN_TILE  positions per tile of the tile map,
//   CSA2_SCAN_U     64-position steps per load batch (each lane has 2U 16-byte loads in flight),
//   CSA2_SCAN_WGS_PER_CU  resident workgroups of the persistent scan per compute unit.
#ifndef CSA2_SCAN_TILE
#define CSA2_SCAN_TILE 4096
#endif
#ifndef CSA2_SCAN_U
#define CSA2_SCAN_U 8
#endif
#ifndef CSA2_SCAN_WGS_PER_CU
#define CSA2_SCAN_WGS_PER_CU 4
#endif
//   CSA2_SCAN_U_LP  256-position steps per load batch in the lane-per-position layout.
#ifndef CSA2_SCAN_U_LP
#define CSA2_SCAN_U_LP 4
#endif
constexpr int kFullTile = CSA2_SCAN_TILE;       // positions per Full-scan workgroup
constexpr int kReindexTile = 512;               // pool positions (64 blocks) per Reindex workgroup
constexpr int kFilterTile = 8192;               // positions per filter workgroup (2 scan tiles)


typedef __amdgpu_buffer_rsrc_t BufRsrc;
constexpr int kBufWord3 = 0x00020000;  // gfx9 buffer resource word 3: raw 32-bit-format access

// Raw buffer view of `bytes` bytes at p (offsets at or past `bytes` read as zero).  Both
// arguments must be the same in every lane; they are passed through readfirstlane so the
// descriptor is built in scalar registers (a descriptor the compiler thinks may vary across
// lanes costs a waterfall loop per load).
__device__ __forceinline__ BufRsrc tile_rsrc(const void* p, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufWord3);
}

__device__ __forceinline__ uint4 buf_ld16(BufRsrc rs, int voff, int soff) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0);
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// 16-byte load marked non-temporal (streamed past the caches)
__device__ __forceinline__ uint4 buf_ld16_nt(BufRsrc rs, int voff, int soff) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 2);
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// Whole-row loads for the MFMA key fragments (bf16 keys, 128-byte rows).  The two loads of a
// 16-position step each read 8 whole rows: in 16-lane group x, lane i < 8 reads 16-byte chunk x
// of row i and lane i >= 8 chunk x + 4 of row i - 8 (rows 8..15 in the second load).  One
// exchange of half groups then gives the layout mfma_score takes (lane (x, i): chunk x, then
// chunk x + 4, of row i): lanes i >= 8 of the first fragment take the second load's lanes
// i - 8, lanes i < 8 of the second fragment the first load's lanes i + 8.
__device__ __forceinline__ int rowline_voff(int lane) {
    const int i = lane & 15, x = lane >> 4;
    return (i & 7) * 128 + (x + 4 * (i >> 3)) * 16;
}

__device__ __forceinline__ void rowline_to_frags(uint4& a, uint4& b, int lane) {
    const bool hi = (lane & 8) != 0;
    uint32_t* pa = &a.x;
    uint32_t* pb = &b.x;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t from_b = (uint32_t)__builtin_amdgcn_mov_dpp((int)pb[d], 0x118, 0xF, 0xF, true);  // row_shr:8
        const uint32_t from_a = (uint32_t)__builtin_amdgcn_mov_dpp((int)pa[d], 0x108, 0xF, 0xF, true);  // row_shl:8
        const uint32_t na = hi ? from_b : pa[d];
        const uint32_t nb = hi ? pb[d] : from_a;
        pa[d] = na;
        pb[d] = nb;
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8_t, u32x4_t{v.x, v.y, v.z, v.w});
}

// Decode and Reindex scoring on MFMA: for 16 positions at a time,
//   D[head][pos] = Q . K^T  on v_mfma_f32_16x16x32_bf16 (two k-steps cover the 64 channels),
// with the query's heads on the M rows (zero-padded to 16) and the 16 positions on N.  Lane
// (g, r) = (lane / 16, lane % 16) supplies head r of Q and position r of K^T with channels
// 32s + 8g .. 32s + 8g + 7 (one 16-byte load per k-step), and its accumulator holds heads
// 4g .. 4g + 3 at position r, so lanes 0..15 hold all four heads of their position and the
// ReLU-weighted head sum needs no cross-lane reduction (heads 4..7 sit in lanes 16..31).
struct QFrag {
    bf16x8_t a[2];  // head r, channels 32s + 8g .. + 7
    float w[4];     // weights of heads 4g .. 4g + 3 (0 past n_heads)
};

__device__ __forceinline__ void load_qfrag(QFrag& qf, const uint16_t* q, const float* w, int n_heads, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const bool hv = r < n_heads;
    const uint16_t* qp = q + (hv ? r : 0) * 64 + 8 * g;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
        qf.a[s2] = as_bf16x8(hv ? *reinterpret_cast<const uint4*>(qp + 32 * s2) : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) qf.w[i] = (4 * g + i < n_heads) ? w[4 * g + i] : 0.f;
}

// Lane-per-position layout (at most 4 indexer heads): 64 positions per wave step, lane l
// holding position l.  Eight k-steps of 8 channels each cover the 64 channels; in k-step s,
// lane (g, r) supplies channels 8s .. 8s + 7 of its own position as column r, K slots
// 8g .. 8g + 7 of B, and A is block-diagonal: row 4g + h holds head h's channels 8s .. 8s + 7
// in K slots 8g .. 8g + 7 and zeros elsewhere.  Then D[4g + h][r] sums only lane group g's
// slots, i.e. head h times the position of lane 16g + r, and the accumulator of lane l ends
// up with all four heads of ITS position: every lane carries a score (the M rows and K slots
// spent on zeros are the price, the same MFMA count as the layout above).
struct QFragLP {
    bf16x8_t a[8];  // k-step s: head (r & 3)'s channels 8s .. 8s + 7 when r / 4 == g, else zeros
    float w[4];     // weights of heads 0 .. 3 (0 past n_heads)
};

__device__ __forceinline__ void load_qfrag_lp(QFragLP& qf, const uint16_t* q, const float* w, int n_heads,
                                              int lane) {
    const int g = lane >> 4, r = lane & 15, h = r & 3;
    const bool on = (r >> 2) == g && h < n_heads;
    const uint16_t* qp = q + (on ? h : 0) * 64;
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
        qf.a[s2] = as_bf16x8(on ? *reinterpret_cast<const uint4*>(qp + 8 * s2) : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) qf.w[i] = i < n_heads ? w[i] : 0.f;
}

__device__ __forceinline__ float relu(float x) {
    return __builtin_elementwise_maximum(x, 0.f);  // one v_maximum3_f32 (fmaxf adds a canonicalize)
}

// Score of position r in lanes 0..15 (kb: the lane's two 16-byte slices of that position).
template <int HI>
__device__ __forceinline__ float mfma_score(const QFrag& qf, const uint4& k0, const uint4& k1) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf.a[0], as_bf16x8(k0), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf.a[1], as_bf16x8(k1), acc, 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(qf.w[i], fmaxf(acc[i], 0.f), s);
    if (HI > 4) s += __shfl_down(s, 16, kWave);  // heads 4..7 from lanes 16..31
    return s;
}

// MXFP4 keys (E2M1 + one E8M0 scale per 32 channels): k-step s of the contraction covers
// exactly scale block s, so lane (g, r)'s 8 channels of k-step s are the 4 code bytes
// 16s + 4g .. 16s + 4g + 3 of position r.  The hardware conversion applies the power-of-two
// scale exactly (its scale operand carries only an exponent): E2M1 x 2^(code - 127) -> bf16.
__device__ __forceinline__ uint4 mx_frag(uint32_t dw, uint32_t code) {
    const float sc = __uint_as_float(code << 23);  // 2^(code - 127); written codes are >= 1
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 0)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 1)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 2)),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, sc, 3)));
}

__device__ __forceinline__ uint32_t buf_ld4(BufRsrc rs, int voff, int soff) {
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
}

__device__ __forceinline__ uint32_t buf_ld2(BufRsrc rs, int voff, int soff) {
    return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0);
}

// Largest key of each aligned group of 8 lanes within lanes 0..15, in lanes 4 and 12
// (quad butterflies, then row_ror:4 brings the quad just below).
__device__ __forceinline__ uint32_t max_over_8_lanes(uint32_t k) {
    k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0xB1, 0xF, 0xF, true));
    k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x4E, 0xF, 0xF, true));
    k = max(k, (uint32_t)__builtin_amdgcn_mov_dpp((int)k, 0x124, 0xF, 0xF, true));
    return k;
}

}  // namespace csa2
