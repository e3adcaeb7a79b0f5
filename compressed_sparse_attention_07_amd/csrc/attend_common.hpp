// Pieces shared by the attention kernels: operand types, the FP4 -> f16 dequantisation, the
// transposed LDS read, per-query vector loads and the P.V tile geometry.
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token", section XI:
// cached FP4 values are dequantised before attention.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "csa2_device.hpp"

namespace csa2 {

constexpr int kD = 128;                      // latent / head dim
constexpr int kNH = 16;                      // heads (padded)
constexpr int kRowB = 288;                   // bytes per tile row: 128 x 16-bit + 32 B skew
constexpr int kTileB = 32 * kRowB;           // one wave's tile: 32 entries
constexpr int kOStride = 132;                // floats per head row of the merge buffer

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

// Element i of a small per-query array through the vector memory path (a raw buffer load):
// vector loads are counted in order, so a wait for these leaves later loads in flight, while
// a wait for a scalar load waits for every scalar load, kernel arguments included.
__device__ __forceinline__ int64_t vload_i64(const int64_t* p, int i) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int64_t*>(p), (short)0, 0x7fffffff, 0x00020000);
    typedef int i32x2_t __attribute__((ext_vector_type(2)));
    const i32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rs, 0, i * 8, 0);
    return (int64_t)(((uint64_t)(uint32_t)v[1] << 32) | (uint32_t)v[0]);
}

__device__ __forceinline__ int32_t vload_i32(const int32_t* p, int i) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(p), (short)0, 0x7fffffff, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b32(rs, 0, i * 4, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {
    uint32_t b = __float_as_uint(v);
    return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t f16pair(float a, float b) {
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Byte Q of w (low nibble = even channel, high nibble = odd channel) as two f16 values times
// the group scale.  The conversion is given scale 1.0 (its scale operand only carries a power
// of two); E2M1 x E4M3 needs at most 6 significant bits, so the f16 product is exact.
template <int Q>
__device__ __forceinline__ uint32_t fp4_pair_f16(uint32_t w, f16x2 sc) {
    const f16x2 v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, Q);
    return __builtin_bit_cast(uint32_t, v * sc);
}

// One lane's 32 FP4 codes (channels [32g, 32g+32)) and its two E4M3 scale bytes (low 16 bits
// of sb) -> four f16x8 A fragments (fragment s = channels 32g + 8s .. 32g + 8s + 7).  The
// hardware E4M3 -> f16 conversion is exact for every finite E4M3 value (the packer never
// writes the NaN codes 0x7f / 0xff).
__device__ __forceinline__ void dequant_f16(const uint4 cb, uint32_t sb, u32x4 (&f)[4]) {
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb, 1.0f, false);
    const f16x2 sc0 = {sc[0], sc[0]}, sc1 = {sc[1], sc[1]};
    const uint32_t w[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const f16x2 sc = s < 2 ? sc0 : sc1;
        f[s][0] = fp4_pair_f16<0>(w[s], sc);
        f[s][1] = fp4_pair_f16<1>(w[s], sc);
        f[s][2] = fp4_pair_f16<2>(w[s], sc);
        f[s][3] = fp4_pair_f16<3>(w[s], sc);
    }
}

__device__ __forceinline__ s16x4 lds_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

}  // namespace csa2
