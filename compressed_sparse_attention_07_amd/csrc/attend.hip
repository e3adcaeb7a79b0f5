// Gather-dequant sparse attention: each query attends its selected FP4 entries plus its
// bf16 sliding window, with one softmax over both.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token":
//   section VI, "What one layer looks like" - a layer's own query attends the 512 selected
//               entries of the shared cache plus its own recent window;
//   section XI  - cached FP4 values are dequantised before attention (no FP4 matmul).
// The cached latent is both key and value; 16 query heads share it.
//
// One workgroup (8 waves) per query, no cross-workgroup merge.  The entry list (top_k
// selected slots, then min(W, N) window positions) is cut into pairs of 16-entry blocks;
// waves take pairs round-robin and keep their own online-softmax state.  Both small
// contractions run on bf16 MFMA (v_mfma_f32_16x16x32_bf16, 16 heads = the MFMA N size):
//   S^T[entry][head] = K . Q^T   A = 16 entries x 32 channels, dequantised FP4 -> bf16
//                                (exact: E2M1 x E4M3 needs at most 6 significant bits),
//                                B = Q^T from registers;
//   O^T[dim][head]  += V^T . P^T A = 16 channels x 32 entries read from a wave-private LDS
//                                copy of the entries, B = P^T, which is exactly the S^T
//                                accumulator layout, so P never leaves registers.  P is
//                                split into bf16 hi + lo parts (two MFMAs) so the product
//                                keeps ~16 mantissa bits; accumulation is fp32.
// MFMA 16x16x32 lane layout (checked on gfx950): lane l supplies row/column l%16 of A/B and
// eight K elements chosen by the lane group l/16 (the same K set for A and B); the
// accumulator of lane l holds rows 4*(l/16)+i, column l%16.  Channel slice of lane group g:
// channels [32g, 32g+32), k-step s covers channels 32g+8s .. 32g+8s+7.
#include "csa2_device.hpp"

namespace csa2 {

constexpr int kAttWaves = 8;
constexpr int kAttNT = kAttWaves * 64;
constexpr int kD = 128;                 // latent / head dim
constexpr int kNH = 16;                 // heads (padded)
constexpr int kMaxEntries = 4096 + 4096;  // top_k + window at their limits
constexpr int kVtStride = 40;           // bf16 per LDS row of V^T (32 entries + 8 pad)
constexpr int kVtSize = kD * kVtStride + 64;  // + skew: rows of channel quarter c>>5 shift by 16 bf16

// V^T tile address of (channel c, entry e): the 16-bf16 skew per 32-channel quarter puts the four
// lane groups (which write different quarters) on different LDS banks.
__device__ __forceinline__ int vt_at(int c, int e) { return c * kVtStride + (c >> 5) * 16 + e; }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e4m3_val(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -v : v;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

__device__ __forceinline__ uint32_t bf16_rne(float v) {
    uint32_t b = __float_as_uint(v);
    return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}

// One entry's 32-channel slice (channels [32g, 32g+32)) as four bf16x8 MFMA fragments.
struct KSlice {
    u32x4 f[4];
};

// Dequantise one lane's 32 FP4 codes (16 B, channels [32g, 32g+32)) with their two E4M3 scales.
// The hardware conversion gives the raw E2M1 values exactly (its scale operand only carries a
// power of two, so it is given 1.0); the E4M3 scale is applied with one exact fp32 multiply and
// v_perm keeps the upper halves, which are the exact bf16 values.
template <int Q>  // byte Q of w: (low nibble, high nibble) -> packed bf16 pair of value * sc
__device__ __forceinline__ uint32_t fp4_pair_bf16(uint32_t w, float sc) {
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, Q);
    return __builtin_amdgcn_perm(__float_as_uint(v[1] * sc), __float_as_uint(v[0] * sc), 0x07060302u);
}

__device__ __forceinline__ void dequant_fp4_slice(const uint4 cb, uint32_t sb, KSlice& ks) {
    const float s0 = e4m3_val(sb & 0xffu), s1 = e4m3_val((sb >> 8) & 0xffu);
    const uint32_t w[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const float sc = s < 2 ? s0 : s1;
        ks.f[s][0] = fp4_pair_bf16<0>(w[s], sc);
        ks.f[s][1] = fp4_pair_bf16<1>(w[s], sc);
        ks.f[s][2] = fp4_pair_bf16<2>(w[s], sc);
        ks.f[s][3] = fp4_pair_bf16<3>(w[s], sc);
    }
}

// One lane's raw data for one entry: FP4 codes (16 B) + 2 scale bytes, or 64 B of bf16 window.
struct RawEntry {
    uint4 a[4];
    uint32_t sb;
    int kind;  // 0: nothing to attend, 1: FP4 cache entry, 2: window entry
};

__device__ __forceinline__ RawEntry load_entry(int32_t row, int e, int top_k, const uint8_t* codes,
                                               const uint8_t* scales, const uint16_t* swa, int64_t row0, int g) {
    RawEntry x;
    x.kind = 0;
    x.sb = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) x.a[s] = make_uint4(0, 0, 0, 0);
    if (row >= 0 && e < top_k) {
        const int64_t cr = row0 + row;
        x.a[0] = *reinterpret_cast<const uint4*>(codes + cr * 64 + 16 * g);
        x.sb = *reinterpret_cast<const uint16_t*>(scales + cr * 8 + 2 * g);
        x.kind = 1;
    } else if (row >= 0) {
        const uint4* src = reinterpret_cast<const uint4*>(swa + (int64_t)row * kD + 32 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) x.a[s] = src[s];
        x.kind = 2;
    }
    return x;
}

__device__ __forceinline__ void entry_slice(const RawEntry& x, KSlice& ks) {
    if (x.kind == 1) {
        dequant_fp4_slice(x.a[0], x.sb, ks);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) ks.f[s] = u32x4{x.a[s].x, x.a[s].y, x.a[s].z, x.a[s].w};
    }
}

__global__ __launch_bounds__(kAttNT) void k_attend(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int64_t* __restrict__ kv_row0, const int32_t* __restrict__ kv_len, int32_t max_len, int64_t cache_rows,
    const int32_t* __restrict__ idx, int top_k, const uint16_t* __restrict__ swa, const int64_t* __restrict__ swa_row0,
    int swa_cap, int64_t swa_rows, int window, int n_heads, float scale_log2, float* __restrict__ out) {
    // LDS: per-wave V^T tile [128 channels][32 entries] (bf16); reused for the cross-wave merge
    __shared__ __align__(16) uint16_t s_vt[kAttWaves][kVtSize];
    __shared__ int32_t s_row[kMaxEntries];  // cache row (FP4) or window row (>= 0), -1 = skip
    __shared__ float s_m[kAttWaves][kNH], s_l[kAttWaves][kNH];

    const int i = blockIdx.x;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int l = t & 63;
    const int g = l >> 4;   // lane group
    const int r = l & 15;   // row / column within the 16
    const int n = eff_len(kv_len, kv_row0, i, max_len, cache_rows);
    const int wc = min(window, n);
    const int n_ent = top_k + wc;
    const int n_pairs = (n_ent + 31) >> 5;
    const int64_t row0 = kv_row0[i];
    const int64_t wrow0 = wc > 0 ? swa_row0[i] : 0;

    // entry list -> rows
    for (int e = t; e < n_pairs * 32; e += kAttNT) {
        int32_t row = -1;
        if (e < top_k) {
            const int pos = idx[(int64_t)i * top_k + e];
            if (pos >= 0 && pos < n) row = pos;  // relative to row0
        } else if (e < n_ent) {
            const int p = n - wc + (e - top_k);
            const int64_t sr = wrow0 + (p % swa_cap);
            if (sr >= 0 && sr < swa_rows) row = (int32_t)sr;
        }
        s_row[e] = row;
    }

    // Q^T as B fragments: lane (g, r) holds Q[head r][32g + 8s + j], pre-scaled later (logits)
    u32x4 qf[4];
    {
        const bool hv = r < n_heads;
        const uint4* qp = reinterpret_cast<const uint4*>(q + ((int64_t)i * n_heads + (hv ? r : 0)) * kD + 32 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint4 v = hv ? qp[s] : make_uint4(0, 0, 0, 0);
            qf[s] = u32x4{v.x, v.y, v.z, v.w};
        }
    }
    __syncthreads();

    float m_run = -INFINITY;  // running max (log2 units) of head r
    float l_run = 0.f;        // this lane's share of the running sum
    f32x4 o[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint16_t* vt = s_vt[wave];

    // raw entry data of the current and the next pair (software pipeline: the next pair's
    // gathers are in flight while the current pair is computed)
    RawEntry cur[2], nxt[2];
    if (wave < n_pairs) {
#pragma unroll
        for (int b = 0; b < 2; ++b) cur[b] = load_entry(s_row[wave * 32 + 16 * b + r], wave * 32 + 16 * b + r, top_k,
                                                        codes, scales, swa, row0, g);
    }
    for (int pr = wave; pr < n_pairs; pr += kAttWaves) {
        if (pr + kAttWaves < n_pairs) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int e = (pr + kAttWaves) * 32 + 16 * b + r;
                nxt[b] = load_entry(s_row[e], e, top_k, codes, scales, swa, row0, g);
            }
        }
        f32x4 sacc[2];
        uint64_t vmask[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            KSlice ks;
            entry_slice(cur[b], ks);
            vmask[b] = __ballot(cur[b].kind != 0);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ks.f[s]),
                                                              __builtin_bit_cast(bf16x8, qf[s]), acc, 0, 0, 0);
            sacc[b] = acc;
            // V^T tile: channel 32g + 8s + j, entry 16b + r
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) {
                    const int c0 = 32 * g + 8 * s + 2 * q2;
                    vt[vt_at(c0, 16 * b + r)] = (uint16_t)(ks.f[s][q2] & 0xffffu);
                    vt[vt_at(c0 + 1, 16 * b + r)] = (uint16_t)(ks.f[s][q2] >> 16);
                }
            }
        }
        // the V^T tile is read by other lanes of this wave below: order LDS writes before reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // logits of head r for entries 16b + 4g + i (valid bits come from the loading lanes 0..15)
        float x[8];
        float mx = -INFINITY;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const bool ok = (vmask[b] >> (4 * g + ii)) & 1ull;
                x[4 * b + ii] = ok ? sacc[b][ii] * scale_log2 : -INFINITY;
                mx = fmaxf(mx, x[4 * b + ii]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
        uint32_t ph[4], pl[4];
        float psum = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            float p0 = (m_new == -INFINITY || x[2 * k2] == -INFINITY) ? 0.f : exp2f(x[2 * k2] - m_new);
            float p1 = (m_new == -INFINITY || x[2 * k2 + 1] == -INFINITY) ? 0.f : exp2f(x[2 * k2 + 1] - m_new);
            psum += p0 + p1;
            const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
            const float r0 = p0 - __uint_as_float(h0 << 16), r1 = p1 - __uint_as_float(h1 << 16);
            ph[k2] = pack2(h0, h1);
            pl[k2] = pack2(bf16_rne(r0), bf16_rne(r1));
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        const u32x4 phv = {ph[0], ph[1], ph[2], ph[3]};
        const u32x4 plv = {pl[0], pl[1], pl[2], pl[3]};
        // P^T fragment's K set for lane group g: entries {4g..4g+3} of block 0, then of block 1
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const uint16_t* vr = vt + vt_at(16 * db + r, 0);
            const uint2 a0 = *reinterpret_cast<const uint2*>(vr + 4 * g);
            const uint2 a1 = *reinterpret_cast<const uint2*>(vr + 16 + 4 * g);
            const u32x4 af = {a0.x, a0.y, a1.x, a1.y};
            f32x4 acc = o[db] * alpha;
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                          __builtin_bit_cast(bf16x8, phv), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af),
                                                          __builtin_bit_cast(bf16x8, plv), acc, 0, 0, 0);
            o[db] = acc;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        cur[0] = nxt[0];
        cur[1] = nxt[1];
    }
    // per-head sums of this wave (the 4 lane groups hold different entries of head r)
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (g == 0) {
        s_m[wave][r] = m_run;
        s_l[wave][r] = l_run;
    }
    __syncthreads();  // all waves done with their V^T tiles
    // merge: each wave's O^T goes to LDS as [head][128] fp32 (reusing the V^T space)
    float* ob = reinterpret_cast<float*>(&s_vt[0][0]) + wave * (kNH * kD);
    {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, s_m[w][r]);
        const float f = (m_run == -INFINITY) ? 0.f : exp2f(m_run - M);
#pragma unroll
        for (int db = 0; db < 8; ++db)
            *reinterpret_cast<float4*>(&ob[r * kD + 16 * db + 4 * g]) =
                make_float4(o[db][0] * f, o[db][1] * f, o[db][2] * f, o[db][3] * f);
    }
    __syncthreads();
    const float* all = reinterpret_cast<const float*>(&s_vt[0][0]);
    for (int x = t; x < kNH * kD; x += kAttNT) {
        const int h = x / kD;
        if (h >= n_heads) break;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int w = 0; w < kAttWaves; ++w) {
            const float f = (s_m[w][h] == -INFINITY) ? 0.f : exp2f(s_m[w][h] - M);
            L = fmaf(s_l[w][h], f, L);
            O += all[w * kNH * kD + x];
        }
        out[(int64_t)i * n_heads * kD + x] = L > 0.f ? O / L : 0.f;
    }
}

hipError_t launch_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* kv_row0,
                         const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, const int32_t* idx,
                         int top_k, const uint16_t* swa, const int64_t* swa_row0, int swa_cap, int64_t swa_rows,
                         int window, int n_heads, float softmax_scale, float* out, hipStream_t stream) {
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(k_attend, dim3(n_q), dim3(kAttNT), 0, stream, q, codes, scales, kv_row0, kv_len, max_len,
                       cache_rows, idx, top_k, swa, swa_row0, swa_cap, swa_rows, window, n_heads, scale_log2, out);
    return hipGetLastError();
}

// zero-fill used to initialise a workspace (a kernel rather than a memset, so it can be captured)
__global__ void k_zero(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
    size_t k = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; k < n16; k += (size_t)gridDim.x * blockDim.x) p[k] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_zero(void* ws, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t ntail = bytes - n16 * 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<uint4*>(ws), n16,
                       reinterpret_cast<uint8_t*>(ws) + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace csa2
