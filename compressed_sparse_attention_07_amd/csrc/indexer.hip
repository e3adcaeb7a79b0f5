// Lightning-style indexer on gfx950: Full-mode scan with block pool, Reindex over the pool,
// and exact Top-K selection.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token":
//   section IX  - the Full layer scores every causally visible position, scores each
//                 8-position block by the maximum index score among its positions, and
//                 keeps the winning blocks as a shared candidate pool (up to 2,048 blocks);
//                 Reindex layers take their own Top-512 from that pool;
//   section VIII - Reindex reuses the Full layer's main KV and indexer keys.
// Summary page "DeepSeek Cuts KV Cache Footprint Fourfold", Technical Approach: Full mode
// computes Top-K fresh; Reindex recomputes selection over reused keys.
//
// Score of position p for one query: sum_h w_h * max(0, q_h . k_p)  (fp32; exact for
// integer-valued inputs below 2^24).
//
// Decode scan (VALU; 4 bytes of arithmetic per byte moved is far below the fp32 ridge,
// so the scan is HBM-bound and stays off the matrix cores):
//   * 4 lanes share one 128-byte key row: lane j loads bytes [16j,16j+16) and
//     [64+16j, 64+16j+16), so one wave instruction moves 16 rows (2 KiB over two loads)
//     and each 128-byte line is consumed whole by one wave;
//   * each lane does 8 v_dot2_f32_bf16 per head, two DPP adds finish the row's dot;
//   * the row's key (order-preserving u32 of the score) is stored; the 8-row block
//     maximum and the top-11-bit histogram of both are fused in (LDS histograms,
//     flushed with integer atomics).
// The last workgroup of a query (ticket counter) turns the histograms into the
// threshold bucket, so the filter pass only reads 4 B per position.
#include "csa2_device.hpp"

namespace csa2 {

constexpr int kScoreNT = 256;
constexpr int kFullTile = 2048;                 // positions per Full-scan workgroup
constexpr int kFullTileBlocks = kFullTile / 8;  // 256 blocks
constexpr int kReindexTile = 512;               // pool positions (64 blocks) per Reindex workgroup

struct IndexWs {
    uint32_t* ctrl;      // [n_q][kCtlSlots]          self-cleaning counters
    uint32_t* hist;      // [n_q][2][2048]            self-cleaning histograms
    Thresh* meta;        // [n_q][2]
    uint32_t* keys;      // [grid_tiles * 2048]       per-position keys (Full) / per-candidate keys (Reindex)
    uint32_t* bkeys;     // [grid_tiles * 256]        per-block max keys
    int32_t* sure_idx;   // [n_q][top_k]
    int32_t* sure_pool;  // [n_q][pool_blocks]
    int32_t* cand_idx;   // [grid_tiles * 2048]
    int32_t* cand_pool;  // [grid_tiles * 256]
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                          false);
}

__device__ __forceinline__ float quad_sum(float v) {
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    return v;
}

// This lane's share of the query: heads h < HI, dims [8j, 8j+8) and [32+8j, 32+8j+8).
template <int HI>
struct QSlice {
    uint32_t a[HI][4];
    uint32_t b[HI][4];
    float w[HI];
};

template <int HI>
__device__ __forceinline__ void load_qslice(QSlice<HI>& qs, const uint16_t* q, const float* w, int n_heads,
                                            int j) {
#pragma unroll
    for (int h = 0; h < HI; ++h) {
        if (h < n_heads) {
            const uint4 va = *reinterpret_cast<const uint4*>(q + h * 64 + 8 * j);
            const uint4 vb = *reinterpret_cast<const uint4*>(q + h * 64 + 32 + 8 * j);
            qs.a[h][0] = va.x; qs.a[h][1] = va.y; qs.a[h][2] = va.z; qs.a[h][3] = va.w;
            qs.b[h][0] = vb.x; qs.b[h][1] = vb.y; qs.b[h][2] = vb.z; qs.b[h][3] = vb.w;
            qs.w[h] = w[h];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) { qs.a[h][k] = 0u; qs.b[h][k] = 0u; }
            qs.w[h] = 0.0f;
        }
    }
}

// Score of the row whose two 16-byte slices this lane holds (all 4 lanes of the quad return it).
template <int HI>
__device__ __forceinline__ float row_score(const uint4& A, const uint4& B, const QSlice<HI>& qs) {
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < HI; ++h) {
        float d = 0.0f;
        d = dot2(A.x, qs.a[h][0], d);
        d = dot2(A.y, qs.a[h][1], d);
        d = dot2(A.z, qs.a[h][2], d);
        d = dot2(A.w, qs.a[h][3], d);
        d = dot2(B.x, qs.b[h][0], d);
        d = dot2(B.y, qs.b[h][1], d);
        d = dot2(B.z, qs.b[h][2], d);
        d = dot2(B.w, qs.b[h][3], d);
        d = quad_sum(d);
        s = fmaf(qs.w[h], fmaxf(d, 0.0f), s);
    }
    return s;
}

__device__ __forceinline__ uint32_t max_over_8_quads(uint32_t k) {
    k = max(k, (uint32_t)__shfl_xor((int)k, 4, kWave));
    k = max(k, (uint32_t)__shfl_xor((int)k, 8, kWave));
    k = max(k, (uint32_t)__shfl_xor((int)k, 16, kWave));
    return k;
}

// Append `val` at the next free slot of list[] (counter *ctr) for every lane with pred set.
__device__ __forceinline__ void wave_append(bool pred, int32_t val, int32_t* list, uint32_t* ctr) {
    const uint64_t m = __ballot(pred);
    if (m == 0) return;
    const int lane = __lane_id();
    const int leader = __ffsll((unsigned long long)m) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
    base = (uint32_t)__shfl((int)base, leader, kWave);
    if (pred) {
        const uint64_t below = m & ((1ull << lane) - 1ull);
        list[base + __popcll(below)] = val;
    }
}

// ----------------------------------------------------------------------------------------
// Full mode, pass 1: scores -> keys, block-max keys, histograms; last workgroup -> thresholds
// ----------------------------------------------------------------------------------------
template <int HI>
__global__ __launch_bounds__(kScoreNT) void k_idx_score_full(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    const int64_t* __restrict__ kv_row0, const int32_t* __restrict__ kv_len, int n_q, int32_t max_len,
    int64_t cache_rows, int n_heads, int grid_tiles, int top_k, int pool_blocks, IndexWs ws) {
    __shared__ uint32_t sh_hist[kHistBins];
    __shared__ uint32_t sh_bhist[kHistBins];
    __shared__ int sh_scan[8];
    __shared__ TileInfo sh_ti;
    __shared__ Thresh sh_th;
    __shared__ int sh_last;

    const TileInfo ti =
        tile_lookup<kScoreNT>(kv_len, kv_row0, n_q, max_len, cache_rows, kFullTile, grid_tiles, blockIdx.x, sh_scan,
                              &sh_ti);
    if (ti.q < 0) return;
    const int i = ti.q;
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int wid = t / kWave;
    const int j = lane & 3;
    const bool want_pool = pool_blocks > 0;

    for (int b = t; b < kHistBins; b += kScoreNT) {
        sh_hist[b] = 0u;
        sh_bhist[b] = 0u;
    }
    QSlice<HI> qs;
    load_qslice<HI>(qs, q_idx + (int64_t)i * n_heads * 64, w + (int64_t)i * n_heads, n_heads, j);
    __syncthreads();

    const int n = ti.n;
    const int64_t row0 = kv_row0[i];
    const int64_t key_base = (int64_t)ti.start * kFullTile;
    const int p_tile = ti.chunk * kFullTile;
    const int p_wave = p_tile + wid * (kFullTile / 4);

    for (int b = 0; b < kFullTile / 4; b += 64) {
        const int base = p_wave + b;
        if (base >= n) break;
        uint4 A[4], B[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int p = base + 16 * u + (lane >> 2);
            int pc = p < n ? p : n - 1;
            const uint16_t* row = k_idx + (row0 + pc) * 64;
            A[u] = *reinterpret_cast<const uint4*>(row + 8 * j);
            B[u] = *reinterpret_cast<const uint4*>(row + 32 + 8 * j);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = base + 16 * u + (lane >> 2);
            const float s = row_score<HI>(A[u], B[u], qs);
            const uint32_t key = p < n ? score_key(s) : 0u;
            if (j == 0 && p < n) {
                ws.keys[key_base + p] = key;
                atomicAdd(&sh_hist[key >> 21], 1u);
            }
            if (want_pool) {
                const uint32_t bk = max_over_8_quads(key);
                if ((lane & 31) == 0 && p < n) {
                    ws.bkeys[key_base / 8 + (p >> 3)] = bk;
                    atomicAdd(&sh_bhist[bk >> 21], 1u);
                }
            }
        }
    }
    __syncthreads();
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins;
    for (int b = t; b < kHistBins; b += kScoreNT) {
        const uint32_t h = sh_hist[b];
        if (h) atomicAdd(&gh[b], h);
        if (want_pool) {
            const uint32_t hb = sh_bhist[b];
            if (hb) atomicAdd(&gh[kHistBins + b], hb);
        }
    }
    __threadfence();
    __syncthreads();
    if (t == 0) sh_last = (atomicAdd(&ws.ctrl[(int64_t)i * kCtlSlots + kCtlScoreDone], 1u) == (uint32_t)(ti.ntiles - 1));
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    find_threshold_256(gh, top_k, sh_scan, &sh_th);
    if (t == 0) ws.meta[(int64_t)i * 2] = sh_th;
    __syncthreads();
    if (want_pool) {
        find_threshold_256(gh + kHistBins, pool_blocks, sh_scan, &sh_th);
        if (t == 0) ws.meta[(int64_t)i * 2 + 1] = sh_th;
    }
    __syncthreads();
    for (int b = t; b < 2 * kHistBins; b += kScoreNT) gh[b] = 0u;
    if (t == 0) ws.ctrl[(int64_t)i * kCtlSlots + kCtlScoreDone] = 0u;
}

// ----------------------------------------------------------------------------------------
// Full mode, pass 2: compact the threshold bucket, last workgroup selects and writes
// ----------------------------------------------------------------------------------------
struct FullElem {
    const int32_t* cand;
    const uint32_t* keys;
    __device__ __forceinline__ void operator()(int e, uint32_t& key, uint32_t& pos) const {
        pos = (uint32_t)cand[e];
        key = keys[pos];
    }
};

__global__ __launch_bounds__(kScoreNT) void k_idx_filter_full(const int64_t* __restrict__ kv_row0,
                                                              const int32_t* __restrict__ kv_len, int n_q,
                                                              int32_t max_len, int64_t cache_rows, int grid_tiles,
                                                              int top_k, int pool_blocks, IndexWs ws,
                                                              int32_t* __restrict__ idx_out,
                                                              int32_t* __restrict__ pool_out) {
    __shared__ SelectShared S;
    __shared__ TileInfo sh_ti;
    __shared__ int sh_last;

    const TileInfo ti = tile_lookup<kScoreNT>(kv_len, kv_row0, n_q, max_len, cache_rows, kFullTile, grid_tiles,
                                              blockIdx.x, S.scan, &sh_ti);
    if (ti.q < 0) return;
    const int i = ti.q;
    const int t = threadIdx.x;
    const int n = ti.n;
    const int64_t key_base = (int64_t)ti.start * kFullTile;
    const int p_tile = ti.chunk * kFullTile;
    uint32_t* ctrl = ws.ctrl + (int64_t)i * kCtlSlots;
    const Thresh th = ws.meta[(int64_t)i * 2];
    const bool want_pool = pool_blocks > 0;

    for (int r = t; r < kFullTile; r += kScoreNT) {
        const int p = p_tile + r;
        const uint32_t key = p < n ? ws.keys[key_base + p] : 0u;
        const int dg = (int)(key >> 21);
        wave_append(p < n && dg > th.digit, p, ws.sure_idx + (int64_t)i * top_k, ctrl + kCtlSureIdx);
        wave_append(p < n && dg == th.digit, p, ws.cand_idx + key_base, ctrl + kCtlCandIdx);
    }
    if (want_pool) {
        const Thresh tp = ws.meta[(int64_t)i * 2 + 1];
        const int nb = (n + 7) >> 3;
        const int b_tile = ti.chunk * kFullTileBlocks;
        for (int r = t; r < kFullTileBlocks; r += kScoreNT) {
            const int bl = b_tile + r;
            const uint32_t key = bl < nb ? ws.bkeys[key_base / 8 + bl] : 0u;
            const int dg = (int)(key >> 21);
            wave_append(bl < nb && dg > tp.digit, bl, ws.sure_pool + (int64_t)i * pool_blocks, ctrl + kCtlSurePool);
            wave_append(bl < nb && dg == tp.digit, bl, ws.cand_pool + key_base / 8, ctrl + kCtlCandPool);
        }
    }
    __threadfence();
    __syncthreads();
    if (t == 0) sh_last = (atomicAdd(ctrl + kCtlFilterDone, 1u) == (uint32_t)(ti.ntiles - 1));
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    {
        FullElem el{ws.cand_idx + key_base, ws.keys + key_base};
        wg_select_write(el, th.in_bucket, top_k - th.above, th.digit, ws.sure_idx + (int64_t)i * top_k,
                        min(th.above, top_k), top_k, idx_out + (int64_t)i * top_k, S);
    }
    if (want_pool) {
        const Thresh tp = ws.meta[(int64_t)i * 2 + 1];
        FullElem el{ws.cand_pool + key_base / 8, ws.bkeys + key_base / 8};
        wg_select_write(el, tp.in_bucket, pool_blocks - tp.above, tp.digit, ws.sure_pool + (int64_t)i * pool_blocks,
                        min(tp.above, pool_blocks), pool_blocks, pool_out + (int64_t)i * pool_blocks, S);
    }
    if (t < kCtlSlots && t != kCtlScoreDone && t != kCtlAttendDone) ctrl[t] = 0u;
}

// ----------------------------------------------------------------------------------------
// Reindex: score the pool's positions with this layer's query, select Top-K among them
// ----------------------------------------------------------------------------------------
struct ReindexElem {
    const int32_t* cand;  // candidate element ids e (slot * 8 + r)
    const uint32_t* keys;
    const int32_t* pool;
    __device__ __forceinline__ void operator()(int e, uint32_t& key, uint32_t& pos) const {
        const int c = cand[e];
        key = keys[c];
        pos = (uint32_t)(pool[c >> 3] * 8 + (c & 7));
    }
};

template <int HI>
__global__ __launch_bounds__(kScoreNT) void k_idx_reindex(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    const int64_t* __restrict__ kv_row0, const int32_t* __restrict__ kv_len, int32_t max_len, int64_t cache_rows,
    int n_heads, const int32_t* __restrict__ pool, int pool_blocks, int top_k, IndexWs ws,
    int32_t* __restrict__ idx_out) {
    __shared__ SelectShared S;
    __shared__ Thresh sh_th;
    __shared__ int sh_last;

    const int i = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int wid = t / kWave;
    const int j = lane & 3;
    const int n = eff_len(kv_len, kv_row0, i, max_len, cache_rows);
    const int64_t row0 = kv_row0[i];
    const int n_elem = pool_blocks * 8;
    const int32_t* qpool = pool + (int64_t)i * pool_blocks;
    uint32_t* keys = ws.keys + (int64_t)i * n_elem;
    uint32_t* ctrl = ws.ctrl + (int64_t)i * kCtlSlots;
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins;

    for (int b = t; b < kHistBins; b += kScoreNT) S.hist[b] = 0u;
    QSlice<HI> qs;
    load_qslice<HI>(qs, q_idx + (int64_t)i * n_heads * 64, w + (int64_t)i * n_heads, n_heads, j);
    __syncthreads();

    const int e_wave = blockIdx.x * kReindexTile + wid * (kReindexTile / 4);
    for (int b = 0; b < kReindexTile / 4; b += 64) {
        uint4 A[4], B[4];
        bool valid[4];
        int e_of[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e_wave + b + 16 * u + (lane >> 2);
            const int slot = e >> 3;
            const int blk = slot < pool_blocks ? qpool[slot] : -1;
            const int64_t p = (int64_t)blk * 8 + (e & 7);
            valid[u] = blk >= 0 && p < n;
            e_of[u] = e;
            if (valid[u]) {
                const uint16_t* row = k_idx + (row0 + p) * 64;
                A[u] = *reinterpret_cast<const uint4*>(row + 8 * j);
                B[u] = *reinterpret_cast<const uint4*>(row + 32 + 8 * j);
            } else {
                A[u] = make_uint4(0, 0, 0, 0);
                B[u] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float s = row_score<HI>(A[u], B[u], qs);
            const uint32_t key = valid[u] ? score_key(s) : 0u;
            if (j == 0 && e_of[u] < n_elem) {
                keys[e_of[u]] = key;
                if (key) atomicAdd(&S.hist[key >> 21], 1u);
            }
        }
    }
    __syncthreads();
    for (int b = t; b < kHistBins; b += kScoreNT) {
        const uint32_t h = S.hist[b];
        if (h) atomicAdd(&gh[b], h);
    }
    __threadfence();
    __syncthreads();
    if (t == 0) sh_last = (atomicAdd(ctrl + kCtlScoreDone, 1u) == (uint32_t)(gridDim.x - 1));
    __syncthreads();
    if (!sh_last) return;
    __threadfence();

    find_threshold_256(gh, top_k, S.scan, &sh_th);
    const Thresh th = sh_th;
    for (int b = t; b < kHistBins; b += kScoreNT) gh[b] = 0u;
    // compact: above-threshold positions to the sure list, threshold bucket to the candidate list
    int32_t* sure = ws.sure_idx + (int64_t)i * top_k;
    int32_t* cand = ws.cand_idx + (int64_t)i * n_elem;
    for (int e0 = 0; e0 < n_elem; e0 += kScoreNT) {  // uniform trip count: wave_append needs whole waves
        const int e = e0 + t;
        const uint32_t key = e < n_elem ? keys[e] : 0u;
        const int dg = (int)(key >> 21);
        const bool ok = key != 0u;
        const int pos = ok ? qpool[e >> 3] * 8 + (e & 7) : 0;
        wave_append(ok && dg > th.digit, pos, sure, ctrl + kCtlSureIdx);
        wave_append(ok && dg == th.digit, e, cand, ctrl + kCtlCandIdx);
    }
    __threadfence();
    __syncthreads();
    ReindexElem el{cand, keys, qpool};
    wg_select_write(el, th.in_bucket, top_k - th.above, th.digit, sure, min(th.above, top_k), top_k,
                    idx_out + (int64_t)i * top_k, S);
    if (t == kCtlScoreDone || t == kCtlSureIdx || t == kCtlCandIdx) ctrl[t] = 0u;
}

// ----------------------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------------------
hipError_t launch_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, const int64_t* kv_row0,
                             const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, int n_heads,
                             int grid_tiles, int top_k, int pool_blocks, const IndexWs& ws, int32_t* idx_out,
                             int32_t* pool_out, hipStream_t stream) {
    if (n_heads <= 4) {
        hipLaunchKernelGGL(k_idx_score_full<4>, dim3(grid_tiles), dim3(kScoreNT), 0, stream, q_idx, w, k_idx, kv_row0,
                           kv_len, n_q, max_len, cache_rows, n_heads, grid_tiles, top_k, pool_blocks, ws);
    } else {
        hipLaunchKernelGGL(k_idx_score_full<8>, dim3(grid_tiles), dim3(kScoreNT), 0, stream, q_idx, w, k_idx, kv_row0,
                           kv_len, n_q, max_len, cache_rows, n_heads, grid_tiles, top_k, pool_blocks, ws);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_idx_filter_full, dim3(grid_tiles), dim3(kScoreNT), 0, stream, kv_row0, kv_len, n_q, max_len,
                       cache_rows, grid_tiles, top_k, pool_blocks, ws, idx_out, pool_out);
    return hipGetLastError();
}

hipError_t launch_index_reindex(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, const int64_t* kv_row0,
                                const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, int n_heads,
                                const int32_t* pool, int pool_blocks, int top_k, const IndexWs& ws, int32_t* idx_out,
                                hipStream_t stream) {
    const int chunks = (pool_blocks * 8 + kReindexTile - 1) / kReindexTile;
    dim3 grid(chunks, n_q);
    if (n_heads <= 4) {
        hipLaunchKernelGGL(k_idx_reindex<4>, grid, dim3(kScoreNT), 0, stream, q_idx, w, k_idx, kv_row0, kv_len,
                           max_len, cache_rows, n_heads, pool, pool_blocks, top_k, ws, idx_out);
    } else {
        hipLaunchKernelGGL(k_idx_reindex<8>, grid, dim3(kScoreNT), 0, stream, q_idx, w, k_idx, kv_row0, kv_len,
                           max_len, cache_rows, n_heads, pool, pool_blocks, top_k, ws, idx_out);
    }
    return hipGetLastError();
}

}  // namespace csa2
