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

// kFp4: top_k > 0 (the FP4 cache is read); kWin: window > 0 and the window store has rows.
// Both are fixed per launch so that every gather below is unconditional (clamped addresses,
// masked results): loads under branches make the compiler wait on some of them early.
// kW8: the window store holds E4M3 bytes ([Article] section XI keeps the recent-window cache
// in FP8); they are converted to f16 exactly and take the FP4 entries' f16 path.
// replay (may be NULL): per-query replay start s; the window then holds only positions >= s
// ([Article] section XII, SWA Bounded Replay).
// win_new (may be NULL): the step's own window vector per query (bf16 [n_q, 128]): every layer
// computes its own window entry for the new token ([Article] section VI).  The kernel attends it
// as position N - 1 of the window straight from win_new (the store's row for that position is
// never read) and writes it to that row (converted to E4M3 for an FP8 store) once everything
// else is done.
struct AttendArgs {
    const uint16_t* q;
    const uint8_t* codes;
    const uint8_t* scales;
    const int64_t* kv_row0;
    const int32_t* kv_len;
    int32_t max_len;
    int64_t cache_rows;
    const int32_t* idx;  // [n_q, top_k]
    int top_k;
    const void* swa;
    const int64_t* swa_row0;
    int swa_cap;
    int64_t swa_rows;
    int window;
    const int64_t* replay;
    int n_heads;
    float scale_log2;
    float* out;
    const uint16_t* win_new;
};

// The first level of loads of query i's attention: everything that needs only the query number
// (the length and rows, the new window vector, the query), so the kernel pays one memory latency
// before the gathers rather than one per dependent load.  The per-query values go first, as
// vector loads (counted in order: waiting for them leaves the later loads in flight); absent
// arrays are replaced by a valid one whose value is unused.
struct AttendPre {
    int32_t len_raw;
    int64_t row0_raw, wrow0_raw, replay_raw;
    uint32_t nwv;     // channels 2l, 2l + 1 of the query's new window vector
    u32x4 qb[4];      // Q^T fragment of head r, channels 32g + 8s .. + 7 (bf16 as given)
};

template <bool kWin>
__device__ __forceinline__ AttendPre attend_pre(int i, const AttendArgs& a) {
    AttendPre p;
    const int l = threadIdx.x & 63;
    const int g = l >> 4, r = l & 15;
    p.len_raw = vload_i32(a.kv_len, i);
    p.row0_raw = vload_i64(a.kv_row0, i);
    p.wrow0_raw = vload_i64(kWin ? a.swa_row0 : a.kv_row0, i);
    p.replay_raw = vload_i64(a.replay != nullptr ? a.replay : a.kv_row0, i);  // replay[i] when given
    const bool has_new = kWin && a.win_new != nullptr;
    p.nwv = has_new ? *reinterpret_cast<const uint32_t*>(a.win_new + (int64_t)i * kD + 2 * l) : 0u;
    // rows r >= n_heads repeat head 0: every head's softmax is its own and only heads < n_heads
    // are written
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + ((int64_t)i * a.n_heads + (r < a.n_heads ? r : 0)) * kD +
                                                     32 * g);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint4 v = qp[s];
        p.qb[s] = u32x4{v.x, v.y, v.z, v.w};
    }
    return p;
}

}  // namespace csa2
