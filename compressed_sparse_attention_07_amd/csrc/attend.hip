// Gather-dequant sparse attention: each query attends its selected FP4 entries plus its
// bf16 sliding window, with one softmax over both.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token":
//   section VI, "What one layer looks like" - a layer's own query attends the 512 selected
//               entries of the shared cache plus its own recent window;
//   section XI  - cached FP4 values are dequantised before attention (no FP4 matmul).
// The cached latent is both key and value.
//
// Kernel shape: the entry list of query i (top_k selected slots, then min(W, N) window
// positions) is cut into splits of 64 entries, one workgroup each.  A workgroup
//   1. gathers its 64 entries (FP4: 64 B of codes + 8 B of scales per entry; window:
//      256 B of bf16) and dequantises them into LDS as fp32 (exact: E2M1 x E4M3 has at
//      most 6 significant bits);
//   2. computes the 16 x 64 logits, the per-head max m and sum l of exp, and the
//      16 x 128 partial output o, all in fp32;
//   3. writes (m, l, o) to the workspace and takes a ticket; the last workgroup of the
//      query merges all splits in split order (so the result does not depend on which
//      workgroup finishes last) and writes the output.
#include "csa2_device.hpp"

namespace csa2 {

constexpr int kAttNT = 256;
constexpr int kAttSplit = 64;     // entries per workgroup
constexpr int kD = 128;           // latent / head dim
constexpr int kNH = 16;           // heads per workgroup (padded)
constexpr int kKvStride = kD + 4; // LDS row stride (floats) of the dequantised entries
constexpr int kQStride = 36;      // LDS stride of one 32-channel quarter of a query row
constexpr int kPartStride = kD + 4;  // o[128], m, l, pad

__device__ __forceinline__ float e2m1_val(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float v = e == 0 ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
    return (c & 8u) ? -v : v;
}

__device__ __forceinline__ float e4m3_val(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float v = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -v : v;
}

__global__ __launch_bounds__(kAttNT) void k_attend(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int64_t* __restrict__ kv_row0, const int32_t* __restrict__ kv_len, int32_t max_len, int64_t cache_rows,
    const int32_t* __restrict__ idx, int top_k, const uint16_t* __restrict__ swa, const int64_t* __restrict__ swa_row0,
    int swa_cap, int64_t swa_rows, int window, int n_heads, float scale_log2, float* __restrict__ out,
    uint32_t* __restrict__ ctrl, float* __restrict__ part, int n_split) {
    __shared__ float sq[kNH * 4 * kQStride];
    __shared__ float skv[kAttSplit * kKvStride];
    __shared__ float sp[kNH * kAttSplit];
    __shared__ float sm[kNH], sl[kNH];
    __shared__ int svalid[kAttSplit];
    __shared__ int sh_last;

    const int i = blockIdx.y;
    const int split = blockIdx.x;
    const int t = threadIdx.x;
    const int n = eff_len(kv_len, kv_row0, i, max_len, cache_rows);
    const int wc = min(window, n);
    const int n_ent = top_k + wc;
    const int64_t row0 = kv_row0[i];

    // 1a. query, pre-scaled by softmax_scale * log2(e): sq[h][quarter][32 (+4 pad)]
    for (int x = t; x < kNH * kD / 2; x += kAttNT) {
        const int h = x / (kD / 2), d2 = x % (kD / 2);
        float a = 0.f, b = 0.f;
        if (h < n_heads) {
            const uint32_t v = reinterpret_cast<const uint32_t*>(q + ((int64_t)i * n_heads + h) * kD)[d2];
            a = bf16lo(v) * scale_log2;
            b = bf16hi(v) * scale_log2;
        }
        const int d = 2 * d2;
        sq[h * 4 * kQStride + (d >> 5) * kQStride + (d & 31)] = a;
        sq[h * 4 * kQStride + (d >> 5) * kQStride + (d & 31) + 1] = b;
    }

    // 1b. gather + dequantise: thread -> (entry le, channel quarter c)
    const int le = t >> 2, c = t & 3;
    const int e = split * kAttSplit + le;
    float kv[32];
    bool ok = false;
    if (e < top_k) {
        const int pos = idx[(int64_t)i * top_k + e];
        if (pos >= 0 && pos < n) {
            ok = true;
            const int64_t row = row0 + pos;
            const uint4 cb = *reinterpret_cast<const uint4*>(codes + row * 64 + c * 16);
            const uint32_t sb = *reinterpret_cast<const uint16_t*>(scales + row * 8 + c * 2);
            const float s0 = e4m3_val(sb & 0xffu), s1 = e4m3_val(sb >> 8);
            const uint32_t wds[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float s = k < 2 ? s0 : s1;
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) kv[8 * k + nb] = e2m1_val((wds[k] >> (4 * nb)) & 0xfu) * s;
            }
        }
    } else if (e < n_ent) {
        const int p = n - wc + (e - top_k);
        const int64_t srow = swa_row0[i] + (p % swa_cap);
        if (srow >= 0 && srow < swa_rows) {
            ok = true;
            const uint4* src = reinterpret_cast<const uint4*>(swa + srow * kD + c * 32);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint4 v = src[k];
                const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int m2 = 0; m2 < 4; ++m2) {
                    kv[8 * k + 2 * m2] = bf16lo(wds[m2]);
                    kv[8 * k + 2 * m2 + 1] = bf16hi(wds[m2]);
                }
            }
        }
    }
    if (!ok) {
#pragma unroll
        for (int k = 0; k < 32; ++k) kv[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 32; k += 4)
        *reinterpret_cast<float4*>(&skv[le * kKvStride + c * 32 + k]) = make_float4(kv[k], kv[k + 1], kv[k + 2], kv[k + 3]);
    if (c == 0) svalid[le] = ok;
    __syncthreads();

    // 2a. logits: each lane dots its 32 channels with every head, the quad finishes the sum
    float lg[kNH];
#pragma unroll
    for (int h = 0; h < kNH; ++h) {
        const float* qq = &sq[h * 4 * kQStride + c * kQStride];
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < 32; k += 4) {
            const float4 qv = *reinterpret_cast<const float4*>(qq + k);
            acc = fmaf(qv.x, kv[k], acc);
            acc = fmaf(qv.y, kv[k + 1], acc);
            acc = fmaf(qv.z, kv[k + 2], acc);
            acc = fmaf(qv.w, kv[k + 3], acc);
        }
        acc += __shfl_xor(acc, 1, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        lg[h] = acc;
    }
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
        const int h = 4 * c + hh;
        sp[h * kAttSplit + le] = ok ? lg[h] : -INFINITY;
    }
    __syncthreads();

    // 2b. per-head max and exp-sum over the 64 entries: 16 lanes per head, 4 entries per lane
    {
        const int h = t >> 4, l16 = t & 15;
        float v[4];
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = sp[h * kAttSplit + 4 * l16 + k];
            m = fmaxf(m, v[k]);
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float p = m == -INFINITY ? 0.f : exp2f(v[k] - m);
            sp[h * kAttSplit + 4 * l16 + k] = p;
            s += p;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, kWave);
        if (l16 == 0) {
            sm[h] = m;
            sl[h] = s;
        }
    }
    __syncthreads();

    // 2c. partial output: thread -> 4 channels x 2 heads
    {
        const int d4 = t & 31, hp = t >> 5;
        const int h0 = 2 * hp, h1 = h0 + 1;
        float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
        for (int e4 = 0; e4 < kAttSplit; e4 += 4) {
            const float4 p0 = *reinterpret_cast<const float4*>(&sp[h0 * kAttSplit + e4]);
            const float4 p1 = *reinterpret_cast<const float4*>(&sp[h1 * kAttSplit + e4]);
            const float pa[4] = {p0.x, p0.y, p0.z, p0.w};
            const float pb[4] = {p1.x, p1.y, p1.z, p1.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float4 vv = *reinterpret_cast<const float4*>(&skv[(e4 + k) * kKvStride + 4 * d4]);
                o0.x = fmaf(pa[k], vv.x, o0.x); o0.y = fmaf(pa[k], vv.y, o0.y);
                o0.z = fmaf(pa[k], vv.z, o0.z); o0.w = fmaf(pa[k], vv.w, o0.w);
                o1.x = fmaf(pb[k], vv.x, o1.x); o1.y = fmaf(pb[k], vv.y, o1.y);
                o1.z = fmaf(pb[k], vv.z, o1.z); o1.w = fmaf(pb[k], vv.w, o1.w);
            }
        }
        float* P = part + ((int64_t)i * n_split + split) * kNH * kPartStride;
        *reinterpret_cast<float4*>(&P[h0 * kPartStride + 4 * d4]) = o0;
        *reinterpret_cast<float4*>(&P[h1 * kPartStride + 4 * d4]) = o1;
        if (t < kNH) {
            P[t * kPartStride + kD] = sm[t];
            P[t * kPartStride + kD + 1] = sl[t];
        }
    }
    __threadfence();
    __syncthreads();
    if (t == 0) sh_last = (atomicAdd(&ctrl[(int64_t)i * kCtlSlots + kCtlAttendDone], 1u) == (uint32_t)(n_split - 1));
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    // 3. merge the splits in order
    {
        const int d = t & (kD - 1), hh = t >> 7;
        const float* P = part + (int64_t)i * n_split * kNH * kPartStride;
        for (int h = hh * 8; h < hh * 8 + 8; ++h) {
            float M = -INFINITY;
            for (int s = 0; s < n_split; ++s) M = fmaxf(M, P[(s * kNH + h) * kPartStride + kD]);
            float L = 0.f, O = 0.f;
            if (M != -INFINITY) {
                for (int s = 0; s < n_split; ++s) {
                    const float* ps = P + (s * kNH + h) * kPartStride;
                    const float ms = ps[kD];
                    const float f = ms == -INFINITY ? 0.f : exp2f(ms - M);
                    L = fmaf(ps[kD + 1], f, L);
                    O = fmaf(ps[d], f, O);
                }
            }
            if (h < n_heads) out[((int64_t)i * n_heads + h) * kD + d] = L > 0.f ? O / L : 0.f;
        }
    }
    if (t == 0) ctrl[(int64_t)i * kCtlSlots + kCtlAttendDone] = 0u;
}

hipError_t launch_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* kv_row0,
                         const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, const int32_t* idx,
                         int top_k, const uint16_t* swa, const int64_t* swa_row0, int swa_cap, int64_t swa_rows,
                         int window, int n_heads, float softmax_scale, float* out, uint32_t* ctrl, float* part,
                         int n_split, hipStream_t stream) {
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    hipLaunchKernelGGL(k_attend, dim3(n_split, n_q), dim3(kAttNT), 0, stream, q, codes, scales, kv_row0, kv_len, max_len,
                       cache_rows, idx, top_k, swa, swa_row0, swa_cap, swa_rows, window, n_heads, scale_log2, out, ctrl,
                       part, n_split);
    return hipGetLastError();
}

int attend_split_count(int top_k, int window) { return (top_k + window + kAttSplit - 1) / kAttSplit; }
size_t attend_part_floats(int n_q, int n_split) { return (size_t)n_q * n_split * kNH * kPartStride; }

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
