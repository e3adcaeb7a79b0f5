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
// Decode scan (HBM-bound: 4 flop per key byte for bf16 keys): the dot products run on MFMA
// (v_mfma_f32_16x16x32_bf16), which leaves the vector ALUs to the per-position epilogue:
//   * bf16 keys: 4 lanes share one 128-byte key row (lane group g loads bytes [16g, 16g+16)
//     and [64+16g, 64+16g+16)), so one wave instruction moves 16 whole rows; heads sit on the
//     MFMA's M rows and 16 positions on N, so lanes 0..15 end with one score each;
//   * MXFP4 keys (34 bytes per position, so the epilogue rather than HBM sets the pace): the
//     lane-per-position layout, 64 positions per wave step with a score in every lane, each
//     lane converting its own row with the hardware E2M1 -> bf16 conversion;
//   * the row's key (order-preserving u32 of the score) is stored; the 8-row block maximum
//     and the top-11-bit histogram of both are fused in (LDS histograms, flushed with
//     integer atomics).
// Kernels hand data to each other only across kernel boundaries (no device-scope fences
// inside a kernel: on a multi-XCD part such a fence writes back the L2).
//   Full:    scan (keys, block-max keys, histograms)
//            -> filter (each workgroup derives the threshold buckets from the histograms and
//               compacts its share of the keys: above-threshold positions to a "sure" list,
//               threshold-bucket candidates to a candidate list, one global atomic per list)
//            -> select (one workgroup per query and list: exact order inside the bucket).
//   Reindex: score (pool positions) -> select (one workgroup per query).
#include <type_traits>

#include <hip/hip_ext.h>

#include "csa2_device.hpp"
#include "reindex_select.hpp"
#include "reindex_score.hpp"
#include "scan_common.hpp"
#include "scan_full.hpp"

namespace csa2 {

// ----------------------------------------------------------------------------------------
// Full mode, kernel 0: per-query metadata.  Query i owns max(1, ceil(n_i / tile)) consecutive
// scan tiles (kFullTile positions) and filter tiles (kFilterTile), clamped so the map fits the grids the
// host sized from its bounds (every query keeps at least one tile of each).  One workgroup.
// maps: which tile -> query maps the following kernels read (kMapScan: the decode scan's,
// kMapFilter: the filter pass's); the per-query metadata is always written.
// ----------------------------------------------------------------------------------------
constexpr int kPrepNT = 1024;
constexpr int kMapScan = 1, kMapFilter = 2;

// Tile -> query map of one chunk of cnt queries (first tiles s[0..cnt), end s[cnt]).  Few
// queries with long runs: every thread fills tiles and finds each one's query by binary
// search, so the work is spread evenly; many queries (short runs): each thread writes its own
// query's run, no search.
__device__ __forceinline__ void fill_tile_map(int32_t* __restrict__ map, const int* s, int cnt, int base) {
    const int t = threadIdx.x;
    if (cnt > kPrepNT / 4) {
        if (t < cnt)
            for (int k = s[t]; k < s[t + 1]; ++k) map[k] = base + t;
        return;
    }
    for (int k = s[0] + t; k < s[cnt]; k += kPrepNT) {
        int lo = 0, hi = cnt - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s[mid] <= k) lo = mid; else hi = mid - 1;
        }
        map[k] = base + lo;
    }
}

__global__ __launch_bounds__(kPrepNT) void k_idx_prep(const int64_t* __restrict__ kv_row0,
                                                      const int32_t* __restrict__ kv_len, int n_q, int32_t max_len,
                                                      int64_t cache_rows, int grid_tiles, int grid_ftiles, int maps,
                                                      IndexWs ws) {
    __shared__ int sh_scan[kPrepNT / kWave];
    __shared__ int s_ts[kPrepNT + 1];  // first scan tile of each query of the chunk, then the end
    __shared__ int s_fs[kPrepNT + 1];  // same for filter tiles
    const int t = threadIdx.x;
    const int cap_s = grid_tiles - n_q, cap_f = grid_ftiles - n_q;
    int run_s = 0, run_f = 0;
    for (int base = 0; base < n_q; base += kPrepNT) {
        const int i = base + t;
        const int cnt = min(kPrepNT, n_q - base);
        int n = 0, xs = 0, xf = 0;
        if (i < n_q) {
            n = eff_len(kv_len, kv_row0, i, max_len, cache_rows);
            const int ts = (int)(((int64_t)n + kFullTile - 1) / kFullTile);
            const int tf = (int)(((int64_t)n + kFilterTile - 1) / kFilterTile);
            xs = ts > 1 ? ts - 1 : 0;
            xf = tf > 1 ? tf - 1 : 0;
        }
        int tot_s, tot_f;
        const int ex_s = block_exclusive_scan<kPrepNT>(xs, sh_scan, tot_s);
        const int ex_f = block_exclusive_scan<kPrepNT>(xf, sh_scan, tot_f);
        if (i < n_q) {
            const int p0 = min(cap_s, run_s + ex_s), p1 = min(cap_s, run_s + ex_s + xs);
            const int f0 = min(cap_f, run_f + ex_f), f1 = min(cap_f, run_f + ex_f + xf);
            QMeta m;
            m.start = i + p0;
            m.ntiles = 1 + (p1 - p0);
            m.fstart = i + f0;
            m.fntiles = 1 + (f1 - f0);
            m.n = (int)min((int64_t)n, min((int64_t)m.ntiles * kFullTile, (int64_t)m.fntiles * kFilterTile));
            ws.qmeta[i] = m;
            // consecutive queries own consecutive tile runs (every query has at least one)
            s_ts[t] = m.start;
            s_fs[t] = m.fstart;
            if (t == cnt - 1) {
                s_ts[cnt] = m.start + m.ntiles;
                s_fs[cnt] = m.fstart + m.fntiles;
            }
        }
        __syncthreads();
        // tile -> query maps (tile k belongs to the largest q with s[q] <= k)
        if (maps & kMapScan) fill_tile_map(ws.tmap, s_ts, cnt, base);
        if (maps & kMapFilter) fill_tile_map(ws.fmap, s_fs, cnt, base);
        __syncthreads();  // s_ts / s_fs are rewritten by the next chunk
        run_s = min(run_s + tot_s, cap_s + 1);
        run_f = min(run_f + tot_f, cap_f + 1);
    }
    const int used_s = n_q + min(cap_s, run_s), used_f = n_q + min(cap_f, run_f);
    if (maps & kMapScan)
        for (int k = used_s + t; k < grid_tiles; k += kPrepNT) ws.tmap[k] = -1;
    if (maps & kMapFilter)
        for (int k = used_f + t; k < grid_ftiles; k += kPrepNT) ws.fmap[k] = -1;
}

// ----------------------------------------------------------------------------------------
// Full mode, prefill chunk (every query reads the same sequence).  Scores are formed 16 queries
// x 16 positions per MFMA tile: for indexer head h, D_h = Q_h . K^T on v_mfma_f32_16x16x32_bf16
// (two k-steps cover the 64 channels); lane (g, r) supplies query r of Q_h and position r of
// K^T with channels 32s + 8g .. 32s + 8g + 7, so its key loads are the scan's 16-byte slices.
// The accumulator of lane (g, r) holds queries 4g+i at position r; the lane folds its four
// heads (ReLU, weights) into the score and its order-preserving key.
// The chunk's selection takes two passes over the scores:
//   sample     - k_idx_prefill_sample scores one 16-position tile in kPfStride and counts the
//                keys' first digits per query (LDS histogram: the 1,024 digits of
//                non-negative scores as two 16-bit counters per word, and one word that counts
//                every negative score as digit 0, the lowest: a threshold that falls among
//                negative scores then keeps every position, never too few);
//                k_idx_prefill_thresh turns the counts into the query's sampled threshold
//                digit: the digit holding the K-th largest key of the sample;
//   candidates - k_idx_prefill_cand scores every position and keeps those whose first digit is
//                at least the sampled one.  The sample is a subset of the visible positions,
//                so at least K visible positions reach that digit and the exact Top-K lies
//                among the candidates, where k_idx_select_cands takes it.  A sample of 1 in
//                kPfStride keeps about kPfStride x K candidates per query.
// Scores are recomputed rather than stored: a chunk has 4,096 x ~133K (query, position)
// pairs, and a 4-byte key for each (2.2 GB out and back in) costs several times the MFMA work.
// ----------------------------------------------------------------------------------------
constexpr int kPfQ = 16;           // queries per sample workgroup
constexpr int kPfPos = 32768;      // positions per sample workgroup (8,192 per wave)
constexpr int kPfStride = 8;       // the sample takes one 16-position tile in kPfStride

// Work items (position chunk x, query group y) are numbered chunk-major and split into kXcds
// contiguous slices, one per XCD: workgroups are handed to the XCDs in turn (workgroup b to
// XCD b mod kXcds), so workgroup b takes item (b mod kXcds) * per_xcd + b / kXcds.  The
// workgroups resident on one XCD then read the same few key chunks (512 KB each), which stay
// in that XCD's 4 MB L2 across all query groups instead of being fetched again for every
// group from the last-level cache.  (Only the speed depends on the hand-out order.)

__host__ __device__ __forceinline__ int pf_items_per_xcd(int n_px, int n_qg) {
    return (n_px * n_qg + kXcds - 1) / kXcds;
}

__global__ __launch_bounds__(kScoreNT) void k_idx_prefill_sample(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    const int64_t* __restrict__ kv_row0, int n_q, int64_t cache_rows, int n_heads, int n_px, int n_qg,
    IndexWs ws) {
    constexpr int kSw = kHistBins / 4;  // words of the non-negative digits; word kSw counts the rest
    __shared__ __align__(16) uint32_t sh_hist[kPfQ][kSw + 4];
    __shared__ int sh_n[kPfQ];
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int wid = t / kWave;
    const int g = lane >> 4, r = lane & 15;
    const int item = (int)(blockIdx.x % kXcds) * pf_items_per_xcd(n_px, n_qg) + (int)(blockIdx.x / kXcds);
    if (item >= n_px * n_qg) return;  // uniform: the grid is rounded up to a multiple of kXcds
    const int q0 = (item % n_qg) * kPfQ;
    const int p_wg = (item / n_qg) * kPfPos;
    const int64_t row0 = kv_row0[0];
    const int64_t row_room = (row0 >= 0 && row0 <= cache_rows) ? cache_rows - row0 : 0;
    if (t < kPfQ) {
        const int q = q0 + t;
        sh_n[t] = q < n_q ? (int)min((int64_t)ws.qmeta[q].n, row_room) : 0;
    }
    __syncthreads();
    int n_max = 0;
#pragma unroll
    for (int k = 0; k < kPfQ; ++k) n_max = max(n_max, sh_n[k]);
    if (p_wg >= n_max) return;  // uniform: nothing visible in this position chunk
    for (int k = t; k < kPfQ * (kSw + 4) / 4; k += kScoreNT)
        reinterpret_cast<uint4*>(&sh_hist[0][0])[k] = make_uint4(0, 0, 0, 0);
    // A fragments: query q0 + r, head h, channels 32s + 8g .. +8 ; weights of queries q0 + 4g + i
    bf16x8_t qa[4][2];
    float wq[4][4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int q = q0 + r;
        const bool ok = q < n_q && h < n_heads;
        const uint16_t* qp = q_idx + ((int64_t)(ok ? q : 0) * n_heads + (ok ? h : 0)) * 64 + 8 * g;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            qa[h][s2] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qp + 32 * s2) : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = q0 + 4 * g + i;
            wq[i][h] = (qi < n_q && h < n_heads) ? w[(int64_t)qi * n_heads + h] : 0.f;
        }
    }
    int nq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) nq[i] = sh_n[4 * g + i];
    __syncthreads();

    // positions below n_min are visible to every query of the workgroup (0 when the workgroup
    // holds fewer than kPfQ queries: the missing ones must never count as visible)
    int n_min = INT32_MAX;
#pragma unroll
    for (int k = 0; k < kPfQ; ++k) n_min = min(n_min, q0 + k < n_q ? sh_n[k] : 0);

    const int p_wave = p_wg + wid * (kPfPos / 4);
    constexpr int TB = 4;                   // sampled tiles per load batch
    constexpr int kTs = 16 * kPfStride;     // position step between a batch's tiles
    constexpr int kBatch = TB * kTs;        // positions a batch spans
    // key rows of one batch (rows past the longest visible length read as zero)
    auto load_batch = [&](uint4 (&kb)[TB][2], int base) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int p = base + kTs * u + r;
            if (p < n_max) {
                const uint16_t* row = k_idx + (row0 + p) * 64 + 8 * g;
                kb[u][0] = *reinterpret_cast<const uint4*>(row);
                kb[u][1] = *reinterpret_cast<const uint4*>(row + 32);
            } else {
                kb[u][0] = make_uint4(0, 0, 0, 0);
                kb[u][1] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    // ALL: every position of the batch is visible to all 16 queries, so no per-query length
    // test (and no branch around the histogram update) is needed
    auto score_batch = [&](const uint4 (&kb)[TB][2], int base, auto all_tag) {
        constexpr bool ALL = decltype(all_tag)::value;
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            f32x4_t acc[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                f32x4_t a = {0.f, 0.f, 0.f, 0.f};
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[h][0], as_bf16x8(kb[u][0]), a, 0, 0, 0);
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[h][1], as_bf16x8(kb[u][1]), a, 0, 0, 0);
                acc[h] = a;
            }
            const int p = base + kTs * u + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sc = 0.f;
#pragma unroll
                for (int h = 0; h < 4; ++h) sc = fmaf(wq[i][h], relu(acc[h][i]), sc);
                if (ALL || p < nq[i]) {
                    // the sum starts from +0, so it is never -0: flip every bit of a negative
                    // score, only the sign bit of the others.  First digit = key >> 21; for a
                    // non-negative score, digits 1024 + j and 1536 + j share word j (the
                    // increment is 1 or 1 << 16), so neighbouring digits, which nearby scores
                    // often take, update different words; a negative score counts in word kSw
                    const uint32_t sb = __float_as_uint(sc);
                    const uint32_t key = sb ^ ((uint32_t)((int32_t)sb >> 31) | 0x80000000u);
                    const bool pos = (key >> 31) != 0u;
                    const uint32_t dd = (key >> 21) & 0x3ffu;  // digit - 1024 (non-negative scores)
                    const uint32_t word = pos ? (dd & (kSw - 1)) : (uint32_t)kSw;
                    atomicAdd(&sh_hist[4 * g + i][word], pos ? 1u + (dd / kSw) * 0xffffu : 1u);
                }
            }
        }
    };
    for (int b = 0; b < kPfPos / 4; b += kBatch) {
        const int base = p_wave + b;
        if (base >= n_max) break;
        uint4 kb[TB][2];
        load_batch(kb, base);
        if (base + kBatch - kTs + 16 <= n_min)
            score_batch(kb, base, std::true_type{});
        else
            score_batch(kb, base, std::false_type{});
    }
    __syncthreads();
    // counts -> the queries' global histograms: word j's halves are digits 1024 + j and
    // 1536 + j, word kSw is digit 0
    for (int k = t; k < kPfQ * (kSw + 1); k += kScoreNT) {
        const int ql = k / (kSw + 1), j = k % (kSw + 1);
        const uint32_t c = sh_hist[ql][j];
        if (c == 0u || q0 + ql >= n_q) continue;
        uint32_t* gh = ws.hist + (int64_t)(q0 + ql) * 2 * kHistBins;
        if (j == kSw) {
            atomicAdd(&gh[0], c);
        } else {
            if (c & 0xffffu) atomicAdd(&gh[kHistBins / 2 + j], c & 0xffffu);
            if (c >> 16) atomicAdd(&gh[kHistBins / 2 + kSw + j], c >> 16);
        }
    }
}

// ----------------------------------------------------------------------------------------
// Prefill chunk, candidate pass: every visible position of every query is scored, and those
// whose first key digit reaches the query's sampled threshold digit are kept (see the sample
// pass above for why the Top-K lies inside them).  A workgroup takes kPcQ = 64 queries (16 per
// wave, one MFMA tile's worth) and kPcPos positions; the key rows go through LDS in stages of
// kPcStage positions (the next stage's loads in flight while the current one is scored), so
// each row is fetched once per 64 queries rather than once per 16.
// Kept entries are appended to a per-wave LDS ring with one ballot per (tile, query row): no
// atomics on that path.  When the ring may not take another tile, the wave flushes it:
// per-query counts reserve room in the queries' global candidate lists (one atomic per query),
// entries are scattered there as (key, position) composites, and the per-(query, digit) counts
// are added to the query's position histogram, which then holds exactly the candidates'
// first-digit counts for the selection.  A ring entry is key << 32 | wave-row << 26 | position
// (positions below 2^26).
// POOL: every query's 8-position block maxima go to the block keys as in the sample pass's
// layout (lanes 4 and 12 of each 16-lane row).
// ----------------------------------------------------------------------------------------
constexpr int kPcQ = 64;         // queries per workgroup: 16 per wave
constexpr int kPcPos = 4096;     // positions per workgroup
constexpr int kPcStage = 64;     // positions per LDS key stage (4 MFMA tiles; 128 measured slower: 2 workgroups per CU)
constexpr int kPcRowB = 144;     // bytes per staged key row: 128 + 16, which spreads rows over the banks
constexpr int kPcRing = 512;     // ring entries per wave (a tile adds at most 256)
constexpr int kPcDW = 16;        // digits at and above the sampled one counted in LDS
constexpr int kPcMaxPos = 1 << 26;

__host__ __device__ __forceinline__ int pc_items_per_xcd(int n_px, int n_qg) {
    return (n_px * n_qg + kXcds - 1) / kXcds;
}

template <bool POOL>
__global__ __launch_bounds__(kScoreNT) __attribute__((amdgpu_waves_per_eu(4))) void k_idx_prefill_cand(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const uint16_t* __restrict__ k_idx,
    const int64_t* __restrict__ kv_row0, int n_q, int64_t cache_rows, int n_heads, int n_px, int n_qg,
    IndexWs ws) {
    __shared__ __align__(16) uint8_t sh_keys[2][kPcStage * kPcRowB];
    __shared__ uint32_t sh_ring[kScoreNT / kWave][2 * kPcRing];  // per wave: keys, then low words
    __shared__ uint32_t sh_dcnt[kScoreNT / kWave][16 * kPcDW];   // [wave][row * kPcDW + digit offset]
    __shared__ uint32_t sh_qcur[kScoreNT / kWave][16];
    __shared__ int sh_n[kPcQ];
    __shared__ int sh_thr[kPcQ];
    __shared__ int64_t sh_base[kPcQ];
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int wid = t / kWave;
    const int g = lane >> 4, r = lane & 15;
    const int item = (int)(blockIdx.x % kXcds) * pc_items_per_xcd(n_px, n_qg) + (int)(blockIdx.x / kXcds);
    if (item >= n_px * n_qg) return;  // uniform: the grid is rounded up to a multiple of kXcds
    const int q0 = (item % n_qg) * kPcQ;
    const int p_wg = (item / n_qg) * kPcPos;
    const int64_t row0 = kv_row0[0];
    const int64_t row_room = (row0 >= 0 && row0 <= cache_rows) ? cache_rows - row0 : 0;
    if (t < kPcQ) {
        const int q = q0 + t;
        int n = 0, thr = -1;
        int64_t base = 0;
        if (q < n_q) {
            const QMeta m = ws.qmeta[q];
            n = (int)min((int64_t)m.n, row_room);
            base = (int64_t)m.start * kFullTile;
            thr = ws.meta[2 * q].digit;
        }
        sh_n[t] = n;
        sh_base[t] = base;
        sh_thr[t] = thr;
    }
    for (int k = t; k < (kScoreNT / kWave) * 16 * kPcDW; k += kScoreNT) (&sh_dcnt[0][0])[k] = 0u;
    __syncthreads();
    int n_max = 0;
    for (int k = 0; k < kPcQ; ++k) n_max = max(n_max, sh_n[k]);
    if (p_wg >= n_max) return;  // uniform: nothing visible in this position chunk
    const int p_end = min(n_max, p_wg + kPcPos);
    const int wq0 = wid * 16;  // this wave's first query (within the workgroup)
    int n_min = INT32_MAX;     // positions below it are visible to all 16 queries of the wave
    for (int k = 0; k < 16; ++k) n_min = min(n_min, q0 + wq0 + k < n_q ? sh_n[wq0 + k] : 0);

    // A fragments: query q0 + wq0 + r, head h, channels 32s + 8g .. +8; weights, lengths and
    // threshold keys of the lane's four queries q0 + wq0 + 4g + i
    bf16x8_t qa[4][2];
    float wq[4][4];
    int nq[4];
    uint32_t tk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const int q = q0 + wq0 + r;
        const bool ok = q < n_q && h < n_heads;
        const uint16_t* qp = q_idx + ((int64_t)(ok ? q : 0) * n_heads + (ok ? h : 0)) * 64 + 8 * g;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            qa[h][s2] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qp + 32 * s2) : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = q0 + wq0 + 4 * g + i;
            wq[i][h] = (qi < n_q && h < n_heads) ? w[(int64_t)qi * n_heads + h] : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        nq[i] = sh_n[wq0 + 4 * g + i];
        const int d = sh_thr[wq0 + 4 * g + i];
        tk[i] = d < 0 ? 0u : (uint32_t)d << 21;
    }

    // ---- the wave's candidate ring: entry e = key ring[e], low word ring[kPcRing + e] (two
    // 4-byte stores at one address and an offset, no register pair to assemble) ----
    uint32_t* ring = sh_ring[wid];
    uint32_t* dcnt = sh_dcnt[wid];
    uint32_t* qcur = sh_qcur[wid];
    int ring_n = 0;  // wave-uniform
    auto flush = [&]() {
        if (lane < 16) qcur[lane] = 0u;
        wave_lds_sync();
        for (int e = lane; e < ring_n; e += kWave) {
            const uint32_t lo = ring[kPcRing + e];
            const int row = (int)(lo >> 26) & 15;
            const int d = (int)(ring[e] >> 21);
            const int d0 = sh_thr[wq0 + row];
            atomicAdd(&qcur[row], 1u);
            if (d0 >= 0 && d - d0 < kPcDW)
                atomicAdd(&dcnt[row * kPcDW + (d - d0)], 1u);
            else  // (a digit far above the sampled one, or every position kept)
                atomicAdd(ws.hist + (int64_t)(q0 + wq0 + row) * 2 * kHistBins + d, 1u);
        }
        wave_lds_sync();
        if (lane < 16) {
            const uint32_t c = qcur[lane];
            uint32_t* ctrl = ws.ctrl + (int64_t)(q0 + wq0 + lane) * kCtlSlots;
            qcur[lane] = c ? atomicAdd(ctrl + kCtlCandIdx, c) : 0u;
        }
        for (int k = lane; k < 16 * kPcDW; k += kWave) {
            const uint32_t c = dcnt[k];
            if (c) {
                const int row = k / kPcDW;
                atomicAdd(ws.hist + (int64_t)(q0 + wq0 + row) * 2 * kHistBins + sh_thr[wq0 + row] + k % kPcDW, c);
                dcnt[k] = 0u;
            }
        }
        wave_lds_sync();
        for (int e = lane; e < ring_n; e += kWave) {
            const uint32_t lo = ring[kPcRing + e];
            const int row = (int)(lo >> 26) & 15;
            const uint32_t slot = atomicAdd(&qcur[row], 1u);
            ws.cand_idx[sh_base[wq0 + row] + slot] = composite(ring[e], lo & (kPcMaxPos - 1));
        }
        wave_lds_sync();
        ring_n = 0;
    };

    // ---- key stages: thread t moves kLdB bytes (part t % kLdParts of row t / kLdParts) ----
    constexpr int kLdB = kPcStage * 128 / kScoreNT;  // bytes per thread per stage
    constexpr int kLdParts = 128 / kLdB;             // threads per row
    static_assert(kLdB % 16 == 0 && 128 % kLdB == 0 && kPcPos % kPcStage == 0, "stage shape");
    const int ld_row = t / kLdParts, ld_part = t % kLdParts;
    uint4 stg[kLdB / 16];
    auto load_stage = [&](int ps) {
        const int p = ps + ld_row;
        const uint16_t* src = k_idx + (row0 + p) * 64 + (kLdB / 2) * ld_part;
#pragma unroll
        for (int j = 0; j < kLdB / 16; ++j)
            stg[j] = p < p_end ? *reinterpret_cast<const uint4*>(src + 8 * j) : make_uint4(0, 0, 0, 0);
    };
    auto store_stage = [&](int buf) {
        uint8_t* dst = sh_keys[buf] + ld_row * kPcRowB + kLdB * ld_part;
#pragma unroll
        for (int j = 0; j < kLdB / 16; ++j) *reinterpret_cast<uint4*>(dst + 16 * j) = stg[j];
    };
    // scores of one stage; ALL: every position of the stage is visible to the wave's queries.
    // The ring append is branch-free (a store under the kept lanes' mask).  One tile at a time
    // keeps the kernel within 128 VGPRs, four waves per SIMD: tiles in pairs (the second tile's
    // MFMAs issued before the first one's epilogue) needed 146 and measured 9 % slower.
    auto tile_mfma = [&](const uint8_t* kb, int u, f32x4_t (&acc)[4]) {
        const uint8_t* kr = kb + (16 * u + r) * kPcRowB + 16 * g;
        const bf16x8_t b0 = as_bf16x8(*reinterpret_cast<const uint4*>(kr));
        const bf16x8_t b1 = as_bf16x8(*reinterpret_cast<const uint4*>(kr + 64));
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            f32x4_t a = {0.f, 0.f, 0.f, 0.f};
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[h][0], b0, a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[h][1], b1, a, 0, 0, 0);
            acc[h] = a;
        }
    };
    auto tile_epilogue = [&](const f32x4_t (&acc)[4], int ps, int u, auto all_tag) {
        constexpr bool ALL = decltype(all_tag)::value;
        if (ring_n > kPcRing - 256) flush();  // wave-uniform
        // (kept in a scalar register, so the count and the slot base cost no vector instruction)
        int rn = __builtin_amdgcn_readfirstlane(ring_n);
        const int p = ps + 16 * u + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float sc = 0.f;
#pragma unroll
            for (int h = 0; h < 4; ++h) sc = fmaf(wq[i][h], relu(acc[h][i]), sc);
            const bool ok = ALL || p < nq[i];
            // the sum starts from +0, so it is never -0: flip every bit of a negative
            // score, only the sign bit of the others
            const uint32_t sb = __float_as_uint(sc);
            const uint32_t key = ok ? sb ^ ((uint32_t)((int32_t)sb >> 31) | 0x80000000u) : 0u;
            const bool kept = ok && key >= tk[i];
            const uint64_t m = __ballot(kept);
            // slot = entries so far + kept lanes below this one
            const int e = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)rn));
            if (kept) {
                ring[e] = key;
                ring[kPcRing + e] = ((uint32_t)(4 * g + i) << 26) | (uint32_t)p;
            }
            rn += __popcll(m);
            if constexpr (POOL) {
                const uint32_t bk = max_over_8_lanes(key);  // lanes 4 / 12 of the row
                const int pblk = ps + 16 * u + (r & 8);
                if ((r & 7) == 4 && pblk < nq[i])
                    ws.bkeys[sh_base[wq0 + 4 * g + i] / 8 + (pblk >> 3)] = bk;
            }
        }
        ring_n = rn;
    };
    auto score_stage = [&](int buf, int ps, auto all_tag) {
        const uint8_t* kb = sh_keys[buf];
        for (int u = 0; u < kPcStage / 16; ++u) {
            f32x4_t acc[4];
            tile_mfma(kb, u, acc);
            tile_epilogue(acc, ps, u, all_tag);
        }
    };

    load_stage(p_wg);
    store_stage(0);
    __syncthreads();
    int buf = 0;
    for (int ps = p_wg; ps < p_end; ps += kPcStage) {
        const bool more = ps + kPcStage < p_end;  // uniform
        if (more) load_stage(ps + kPcStage);
        if (ps + kPcStage <= n_min)
            score_stage(buf, ps, std::true_type{});
        else
            score_stage(buf, ps, std::false_type{});
        if (more) store_stage(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
    if (ring_n > 0) flush();
}

// Prefill chunk: every query's sampled threshold digit (the digit holding the K-th largest key
// of its sample; -1 when the sample holds at most K keys: then every visible position is a
// candidate), one workgroup per query.  Clears the sample histogram for the next call.
__global__ __launch_bounds__(kScoreNT) void k_idx_prefill_thresh(int top_k, IndexWs ws) {
    __shared__ int sh_scan[kScoreNT / kWave];
    __shared__ Thresh sh_th;
    const int i = blockIdx.x;
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins;
    find_threshold_256(gh, top_k, sh_scan, &sh_th);  // (ends with a barrier: every bin is read)
    if (threadIdx.x == 0) ws.meta[2 * i] = sh_th;
    for (int b = threadIdx.x; b < kHistBins; b += kScoreNT) gh[b] = 0u;
}

// First-digit histogram of each query's block-max keys (prefill chunk with pools): workgroup
// (x, i) counts blocks [x * kBhChunk, (x + 1) * kBhChunk) of query i in LDS and adds them to
// the query's block histogram.
constexpr int kBhChunk = 8192;

__global__ __launch_bounds__(kScoreNT) void k_idx_block_hist(const int64_t* __restrict__ kv_row0, int64_t cache_rows,
                                                             IndexWs ws) {
    __shared__ uint32_t sh[kHistBins];
    const int t = threadIdx.x;
    const int i = blockIdx.y;
    const int64_t row0 = kv_row0[0];
    const int64_t row_room = (row0 >= 0 && row0 <= cache_rows) ? cache_rows - row0 : 0;
    const QMeta qm = ws.qmeta[i];
    const int n = (int)min((int64_t)qm.n, row_room);  // the positions the scoring kernel wrote
    const int nb = (n + 7) >> 3;
    const int b0 = blockIdx.x * kBhChunk;
    if (b0 >= nb) return;  // uniform
    for (int b = t; b < kHistBins; b += kScoreNT) sh[b] = 0u;
    __syncthreads();
    const uint32_t* bk = ws.bkeys + (int64_t)qm.start * kFullTile / 8;
    const int b1 = min(nb, b0 + kBhChunk);
    // every block key of the thread requested before the first is counted (clamped indices, no
    // branch around the loads): one memory latency rather than one per kScoreNT keys
    constexpr int kPer = kBhChunk / kScoreNT;
    uint32_t v[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) v[k] = bk[min(b0 + k * kScoreNT + t, b1 - 1)];
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        if (b0 + k * kScoreNT + t < b1) atomicAdd(&sh[v[k] >> 21], 1u);
    __syncthreads();
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins + kHistBins;
    for (int b = t; b < kHistBins; b += kScoreNT)
        if (sh[b]) atomicAdd(&gh[b], sh[b]);
}

// ----------------------------------------------------------------------------------------
// Splitting a query's keys by the threshold bucket (the filter kernel, and the selection
// kernel for short contexts).  A workgroup of NT threads holds U quads of keys per thread,
// element e = e0 + 4 (u NT + t) + c; a zero key is padding.
// ----------------------------------------------------------------------------------------

// Loads keys[e0, e_end) (e0 a multiple of 4; the array is readable up to e_end rounded up to 4).
// Quads at or past e_end read as zero through the buffer bound; the rest of a partial last quad
// is cleared by mask_quads once the loads are waited for.
template <int NT, int U>
__device__ __forceinline__ void load_quads(uint4 (&q)[U], const uint32_t* keys, int e0, int e_end) {
    const int n = e_end > e0 ? e_end - e0 : 0;
    const BufRsrc rs = tile_rsrc(keys + e0, ((n + 3) & ~3) * 4);
#pragma unroll
    for (int u = 0; u < U; ++u) q[u] = buf_ld16_nt(rs, 16 * (u * NT + (int)threadIdx.x), 0);  // (read once)
}

template <int NT, int U>
__device__ __forceinline__ void mask_quads(uint4 (&q)[U], int e0, int e_end) {
    if ((e_end - e0) & 3) {  // uniform
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int rem = e_end - (e0 + 4 * (u * NT + (int)threadIdx.x));
            q[u].y = rem > 1 ? q[u].y : 0u;
            q[u].z = rem > 2 ? q[u].z : 0u;
            q[u].w = rem > 3 ? q[u].w : 0u;
        }
    }
}

// Key bounds of a threshold bucket: above it key > gt, in it lo <= key <= gt (digit -1: every
// nonzero key is above).
struct KeySplit {
    uint32_t gt, lo;
};
__device__ __forceinline__ KeySplit key_split(const Thresh& th) {
    return KeySplit{th.digit >= 0 ? ((uint32_t)th.digit << 21) | 0x1fffffu : 0u,
                    th.digit > 0 ? (uint32_t)th.digit << 21 : 1u};
}

// (above, in bucket) counts of this thread's keys packed as above << 16 | in bucket
template <int U>
__device__ __forceinline__ int count_quads(const uint4 (&q)[U], KeySplit ks) {
    int ns = 0, nc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t v4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            ns += v4[c] > ks.gt ? 1 : 0;
            nc += v4[c] >= ks.lo && v4[c] <= ks.gt ? 1 : 0;
        }
    }
    return (ns << 16) | nc;
}

// Writes this thread's above-bucket elements to sure[os..] and in-bucket composites to
// cand[oc..] (entries at or past cap_s / cap_c are dropped: the histogram the offsets come
// from counted the same keys, so none is).  Sure entries go out as 32-bit element indices.
template <int NT, int U, typename SureT>
__device__ __forceinline__ void write_quads(uint4 (&q)[U], KeySplit ks, int e0, int os, int oc, SureT* sure,
                                            int cap_s, uint64_t* cand, int cap_c) {
    // (the tests are recomputed here rather than 2 x 4U lane masks kept alive from the count)
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" : "+v"(q[u].x), "+v"(q[u].y), "+v"(q[u].z), "+v"(q[u].w));
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t v4[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t e = (uint32_t)(e0 + 4 * (u * NT + (int)threadIdx.x) + c);
            if (v4[c] > ks.gt) {
                if ((unsigned)os < (unsigned)cap_s) sure[os] = (SureT)e;
                ++os;
            } else if (v4[c] >= ks.lo) {
                if ((unsigned)oc < (unsigned)cap_c) cand[oc] = composite(v4[c], e);
                ++oc;
            }
        }
    }
}

// Two block-wide exclusive scans at once (one barrier).  `sh` holds 2 NT/64 ints.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(int a, int b, int* sh, int& ea, int& eb, int& ta, int& tb) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int xa = wave_inclusive_scan(a), xb = wave_inclusive_scan(b);
    if (lane == kWave - 1) {
        sh[wid] = xa;
        sh[NW + wid] = xb;
    }
    __syncthreads();
    int wa = 0, wb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int va = sh[w], vb = sh[NW + w];
        if (w < wid) {
            wa += va;
            wb += vb;
        }
        sa += va;
        sb += vb;
    }
    __syncthreads();
    ea = wa + xa - a;
    eb = wb + xb - b;
    ta = sa;
    tb = sb;
}

// ----------------------------------------------------------------------------------------
// Full mode, kernel 2: thresholds from the histograms, compaction of the keys.  One workgroup
// per filter tile (kFilterTile positions and their blocks) of a query.  Both histograms and
// all keys of the tile are requested before the first wait; both lists are split in one pass,
// with one global counter atomic per list and workgroup.
// ----------------------------------------------------------------------------------------
constexpr int kFiltU = kFilterTile / (4 * kScoreNT);       // position quads per thread
constexpr int kFiltUB = (kFilterTile / 8 + 4 * kScoreNT - 1) / (4 * kScoreNT);  // block quads per thread
// POOL_ONLY (a prefill chunk with pools: its compacting scoring pass wrote the position lists
// already): only the block list is split, and the first workgroup of every kPoolGroup filter
// tiles of a query takes all their blocks (the others return at once), so a query's ~17 tiles
// need 3 workgroups, each loading the block histogram once for 8,192 blocks.
constexpr int kPoolGroup = 8;

template <bool POOL_ONLY>
// The workspace areas of the first loads (tile map, query metadata, histograms, keys) come as
// leading arguments of their own, preloaded into SGPRs at launch; ws supplies the rest.
__global__ __launch_bounds__(kScoreNT) void k_idx_filter_full(int32_t* fmap, QMeta* qmeta, uint32_t* hist,
                                                              uint32_t* keys, uint32_t* bkeys, int top_k,
                                                              int pool_blocks, IndexWs ws) {
    ws.fmap = fmap;
    ws.qmeta = qmeta;
    ws.hist = hist;
    ws.keys = keys;
    ws.bkeys = bkeys;
    constexpr int UP = POOL_ONLY ? 1 : kFiltU;                      // position quads per thread
    constexpr int UB = POOL_ONLY ? kPoolGroup * kFiltUB : kFiltUB;  // block quads per thread
    __shared__ int sh_scan[2 * kScoreNT / kWave];
    __shared__ int sh_base[4];
    __shared__ Thresh sh_th[2];

    const int i = ws.fmap[blockIdx.x];
    if (i < 0) return;
    const int t = threadIdx.x;
    const QMeta qm = ws.qmeta[i];
    const int n = qm.n;
    const int nb = (n + 7) >> 3;
    const int fchunk = (int)blockIdx.x - qm.fstart;
    if (POOL_ONLY && fchunk % kPoolGroup != 0) return;  // uniform: the group's first workgroup takes its blocks
    const int64_t key_base = (int64_t)qm.start * kFullTile;
    uint32_t* ctrl = ws.ctrl + (int64_t)i * kCtlSlots;
    const uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins;
    const bool do_pos = !POOL_ONLY, do_pool = pool_blocks > 0;
    const int p0 = fchunk * kFilterTile, p1 = do_pos ? min(n, p0 + kFilterTile) : p0;
    const int b0 = fchunk * (kFilterTile / 8);
    const int b1 = do_pool ? min(nb, b0 + (POOL_ONLY ? kPoolGroup : 1) * (kFilterTile / 8)) : b0;

    uint32_t h0[kHistBins / kScoreNT], h1[kHistBins / kScoreNT];
    if (do_pos) hist_load<kScoreNT>(gh, h0);
    else
        for (auto& x : h0) x = 0u;
    if (do_pool) hist_load<kScoreNT>(gh + kHistBins, h1);
    else
        for (auto& x : h1) x = 0u;
    uint4 kq[UP], bq[UB];
    if constexpr (!POOL_ONLY) load_quads<kScoreNT>(kq, ws.keys + key_base, p0, p1);
    load_quads<kScoreNT>(bq, ws.bkeys + key_base / 8, b0, b1);
    if constexpr (!POOL_ONLY) find_threshold_regs<kScoreNT>(h0, top_k, sh_scan, &sh_th[0]);
    find_threshold_regs<kScoreNT>(h1, max(pool_blocks, 1), sh_scan, &sh_th[1]);
    const KeySplit s0 = POOL_ONLY ? KeySplit{0xffffffffu, 0xffffffffu} : key_split(sh_th[0]);
    const KeySplit s1 = key_split(sh_th[1]);
    if constexpr (POOL_ONLY) kq[0] = make_uint4(0, 0, 0, 0);  // no positions (keys 0 fall in no list)
    else mask_quads<kScoreNT>(kq, p0, p1);
    mask_quads<kScoreNT>(bq, b0, b1);
    int e0, e1, t0, t1;  // packed above << 16 | in bucket (a tile has at most kFilterTile of each)
    block_exclusive_scan2<kScoreNT>(count_quads(kq, s0), count_quads(bq, s1), sh_scan, e0, e1, t0, t1);
    if (t < 4) {
        const int cnt = t == 0 ? t0 >> 16 : t == 1 ? t0 & 0xffff : t == 2 ? t1 >> 16 : t1 & 0xffff;
        const int slot = t == 0 ? kCtlSureIdx : t == 1 ? kCtlCandIdx : t == 2 ? kCtlSurePool : kCtlCandPool;
        sh_base[t] = cnt ? (int)atomicAdd(ctrl + slot, (uint32_t)cnt) : 0;
    }
    __syncthreads();
    if (do_pos)
        write_quads<kScoreNT>(kq, s0, p0, sh_base[0] + (e0 >> 16), sh_base[1] + (e0 & 0xffff),
                              ws.sure_idx + (int64_t)i * top_k, top_k, ws.cand_idx + key_base, n);
    if (do_pool)
        write_quads<kScoreNT>(bq, s1, b0, sh_base[2] + (e1 >> 16), sh_base[3] + (e1 & 0xffff),
                              ws.sure_pool + (int64_t)i * pool_blocks, pool_blocks, ws.cand_pool + key_base / 8,
                              nb);
}

struct CompositeList {
    const uint64_t* c;
    __device__ __forceinline__ uint64_t operator()(int e) const { return c[e]; }
};

constexpr int kSelNT = 1024;  // threads of the per-query selection workgroups
constexpr int kSelNTMany = 512, kSortCapMany = 2048;  // the same for a prefill chunk's many queries
// A prefill chunk's selections of at most kSelMaxMany entries (top_k, and the pool list's size
// when there is one) size their output buffers for that: 48 KB of LDS, three workgroups per
// compute unit instead of two (kMaxSelect: 73 KB).
constexpr int kSelMaxMany = 1024;

// MS: the largest selection (top_k or pool blocks) the LDS output buffers hold
template <int CAP, int MS = kMaxSelect>
struct SmallSel {
    uint64_t cand[CAP];
    uint32_t sel[MS + 4];
    RadixShared R;
    int cnt;
    int nt;
};
template <int CAP, int MS = kMaxSelect>
union SelLds {
    SelectSharedT<CAP> big;
    SmallSel<CAP, MS> small;
};

constexpr int kTieCap = 1024;  // equal keys at the threshold ordered by direct counting

// Decode contexts up to this length skip the filter kernel: the selection workgroup reads the
// query's keys itself (kSelScanU four-key loads per thread, issued before the threshold search).
constexpr int kSelScanMax = 16384;
template <int NT>
constexpr int sel_scan_u() { return kSelScanMax / (4 * NT); }  // four-key loads per thread

// Ascending output of up to MS selected positions (sel[] in LDS).
template <int NT, int MS = kMaxSelect>
struct AscLds {
    uint32_t scratch[2 * kAscB + MS];
    int scan[NT / kWave];
    uint32_t mm[2];
};

template <int NT, int MS>
__device__ __forceinline__ void sort_out(const uint32_t* sel, int total, int k, int32_t* out, AscLds<NT, MS>& A) {
    bucket_write_ascending<NT>(sel, total, k, out, A.scratch, A.scan, A.mm);
}

// The LDS part of a selection: W.cand[0, m) holds the threshold bucket's composites (first
// digit d1) and W.sel[0, W.cnt) the positions already selected (those above the bucket); adds
// the `need` best of the bucket to W.sel and returns how many W.sel holds.  The threshold KEY
// comes first (at most two radix passes); equal keys at it are ranked by position.
template <int NT, int CAP, int MS>
__device__ int select_bucket_lds(SmallSel<CAP, MS>& W, AscLds<NT, MS>& A, int m, int need, int d1) {
    const int t = threadIdx.x;
    const bool any = need > 0 && m > 0;
    const KeyThr kt = any ? lds_key_threshold<NT>(W.cand, m, need, d1, W.R) : KeyThr{0u, -1, 0};
    const bool ranked = any && kt.take_eq >= 0;  // only take_eq of the n_tie equal keys go
    int total;
    if (ranked && kt.n_tie > kTieCap) {
        // many equal keys at the threshold: radix passes over the composites' position bits
        const uint64_t thr = lds_radix_threshold<NT>(W.cand, m, need, d1, W.R);
        for (int e = t; e < m; e += NT)
            if (W.cand[e] >= thr) W.sel[atomicAdd(&W.cnt, 1)] = composite_pos(W.cand[e]);
        __syncthreads();
        total = W.cnt;
    } else {
        uint32_t* ties = A.scratch;  // free until the ascending output
        for (int e = t; e < m; e += NT) {
            const uint64_t c = W.cand[e];
            const uint32_t key = (uint32_t)(c >> 32);
            if (any && (ranked ? key > kt.t : key >= kt.t))
                W.sel[atomicAdd(&W.cnt, 1)] = composite_pos(c);
            else if (ranked && key == kt.t)
                ties[atomicAdd(&W.nt, 1)] = composite_pos(c);
        }
        __syncthreads();
        total = W.cnt;
        if (ranked) {
            // each tie's place among the ties by position (distinct positions): the take_eq
            // lowest follow the keys above the threshold
            const int nt = W.nt;
            for (int j = t; j < nt; j += NT) {
                const uint32_t p = ties[j];
                int rank = 0;
                for (int e = 0; e < nt; ++e) rank += ties[e] < p ? 1 : 0;
                if (rank < kt.take_eq) W.sel[total + rank] = p;
            }
            total += kt.take_eq;
            __syncthreads();
        }
    }
    return total;
}

// ----------------------------------------------------------------------------------------
// Full mode, kernel 3: exact selection inside the threshold bucket; one workgroup per
// (query, list), list = list0 + blockIdx.y (0: positions, 1: pool blocks).  The bucket's
// candidates normally fit in LDS: radix passes there find the threshold, and each selected
// position's output slot is its rank among the selected.
// scan_keys != 0 (decode, every context <= kSelScanMax): the filter kernel did not run and this
// workgroup splits the query's keys into the above-bucket and in-bucket lists itself.
// Leaves the histograms and counters of the query zero for the next call.
// NT threads; CAP: largest threshold bucket selected in LDS (larger ones take the global-list
// radix path).  Decode: 1,024 threads, 8,192; a prefill chunk's thousands of queries: 512 and
// 2,048, which halves the LDS so that two workgroups share a compute unit.
// ----------------------------------------------------------------------------------------
template <int NT, int CAP, int MS>
// (as in the filter pass: the first loads' workspace areas lead the arguments, preloaded)
__global__ __launch_bounds__(NT) void k_idx_select_full(QMeta* qmeta, uint32_t* hist, uint32_t* keys, uint32_t* bkeys,
                                                        int top_k, int pool_blocks, int scan_keys, int list0, IndexWs ws,
                                                        int32_t* __restrict__ idx_out,
                                                        int32_t* __restrict__ pool_out) {
    ws.qmeta = qmeta;
    ws.hist = hist;
    ws.keys = keys;
    ws.bkeys = bkeys;
    __shared__ SelLds<CAP, MS> U;
    __shared__ AscLds<NT, MS> A;
    __shared__ Thresh sh_th;
    const int i = blockIdx.x;
    const int which = list0 + (int)blockIdx.y;  // 0: positions, 1: pool blocks
    const int t = threadIdx.x;
    const QMeta qm = ws.qmeta[i];
    const int64_t key_base = (int64_t)qm.start * kFullTile;
    uint32_t* ctrl = ws.ctrl + (int64_t)i * kCtlSlots;
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins + which * kHistBins;
    const int k = which ? pool_blocks : top_k;
    uint64_t* cand = which ? ws.cand_pool + key_base / 8 : ws.cand_idx + key_base;
    int32_t* sure = which ? ws.sure_pool + (int64_t)i * pool_blocks : ws.sure_idx + (int64_t)i * top_k;
    int32_t* out = which ? pool_out + (int64_t)i * pool_blocks : idx_out + (int64_t)i * top_k;
    uint32_t h[kHistBins / NT];
    hist_load<NT>(gh, h);
    // the keys, requested behind the histogram so that waiting for it leaves them in flight
    // (the key-splitting path exists in the decode variant only; the prefill one never takes it)
    constexpr bool kSplit = NT == kSelNT;
    if constexpr (!kSplit) scan_keys = 0;
    uint4 kq[kSplit ? sel_scan_u<NT>() : 1];
    const int n_elem = scan_keys ? (which ? (qm.n + 7) >> 3 : qm.n) : 0;
    if (scan_keys) load_quads<NT>(kq, which ? ws.bkeys + key_base / 8 : ws.keys + key_base, 0, n_elem);
    find_threshold_regs<NT>(h, k, U.small.R.scan, &sh_th);
    const Thresh th = sh_th;
    const int need = k - th.above;
    const int n_sure = min(th.above, k);
    const bool small = th.in_bucket <= CAP;
    if (scan_keys) {
        // above the bucket -> sure list, in the bucket -> candidate composites; in LDS when the
        // bucket fits there, else in the query's global lists for the large-bucket path
        const KeySplit ks = key_split(th);
        mask_quads<NT>(kq, 0, n_elem);
        int tot;  // sure and candidates <= kSelScanMax each: 16 + 16 bits
        const int pk = block_exclusive_scan<NT>(count_quads(kq, ks), U.small.R.scan, tot);
        if (small)
            write_quads<NT>(kq, ks, 0, pk >> 16, pk & 0xffff, U.small.sel, k, U.small.cand, CAP);
        else
            write_quads<NT>(kq, ks, 0, pk >> 16, pk & 0xffff, sure, k, cand, n_elem);
        __syncthreads();
    }
    if (small) {
        SmallSel<CAP, MS>& W = U.small;
        if (!scan_keys) {
            // both lists requested before either is stored (clamped indices): one memory
            // latency, not one per NT elements of each
            constexpr int kPc = CAP / NT, kPs = (MS + NT - 1) / NT;
            const int inb = th.in_bucket;
            uint64_t cv[kPc];
            int32_t sv[kPs];
#pragma unroll
            for (int k = 0; k < kPc; ++k)  // (k * NT < inb is uniform: no load past the list's last slot group)
                cv[k] = k * NT < inb ? cand[min(k * NT + t, inb - 1)] : 0ull;
#pragma unroll
            for (int k = 0; k < kPs; ++k) sv[k] = k * NT < n_sure ? sure[min(k * NT + t, n_sure - 1)] : 0;
#pragma unroll
            for (int k = 0; k < kPc; ++k)
                if (k * NT + t < inb) W.cand[k * NT + t] = cv[k];
#pragma unroll
            for (int k = 0; k < kPs; ++k)
                if (k * NT + t < n_sure) W.sel[k * NT + t] = (uint32_t)sv[k];
        }
        if (t == 0) {
            W.cnt = n_sure;
            W.nt = 0;
        }
        __syncthreads();
        const int total = select_bucket_lds<NT, CAP, MS>(W, A, th.in_bucket, need, th.digit);
        sort_out(W.sel, total, k, out, A);
    } else {
        SelectSharedT<CAP>& S = U.big;
        const uint64_t thr = wg_threshold<NT>(CompositeList{cand}, th.in_bucket, need, th.digit, S);
        uint32_t* sel = reinterpret_cast<uint32_t*>(S.buf);
        if (t == 0) S.cnt = 0;
        __syncthreads();
        for (int j = t; j < n_sure; j += NT) sel[atomicAdd(&S.cnt, 1)] = (uint32_t)sure[j];
        for (int e = t; e < th.in_bucket; e += NT)
            if (cand[e] >= thr) sel[atomicAdd(&S.cnt, 1)] = composite_pos(cand[e]);
        __syncthreads();
        sort_out(sel, S.cnt, k, out, A);
    }
    for (int b = t; b < kHistBins; b += NT) gh[b] = 0u;
    if (t == 0) {
        ctrl[which ? kCtlSurePool : kCtlSureIdx] = 0u;
        ctrl[which ? kCtlCandPool : kCtlCandIdx] = 0u;
    }
}

// ----------------------------------------------------------------------------------------
// Prefill chunk, positions: the exact Top-K of each query among the candidates of the
// candidate pass (composites at or above its sampled threshold digit; unique composites, so
// the K largest are the Top-K in (score desc, position asc) order), one workgroup per query.
// The query's position histogram holds the candidates' first-digit counts (added by the
// candidate pass), which give the exact threshold bucket; the candidates above it are
// selected, and those in it go to LDS for select_bucket_lds, or, when more than CAP share the
// bucket (heavy ties), to the radix passes over the global list.
// Leaves the query's histogram and candidate counter zero for the next call.
// ----------------------------------------------------------------------------------------
template <int NT, int CAP, int MS>
__global__ __launch_bounds__(NT) void k_idx_select_cands(QMeta* qmeta, uint32_t* ctrl_all, uint32_t* hist_all,
                                                         uint64_t* cand_all, int top_k, int32_t* __restrict__ idx_out) {
    __shared__ SelLds<CAP, MS> U;
    __shared__ AscLds<NT, MS> A;
    __shared__ Thresh sh_th;
    const int i = blockIdx.x;
    const int t = threadIdx.x;
    uint32_t* gh = hist_all + (int64_t)i * 2 * kHistBins;
    uint32_t h[kHistBins / NT];
    hist_load<NT>(gh, h);
    const QMeta qm = qmeta[i];
    uint32_t* ctrl = ctrl_all + (int64_t)i * kCtlSlots;
    const uint64_t* cand = cand_all + (int64_t)qm.start * kFullTile;
    int32_t* out = idx_out + (int64_t)i * top_k;
    // the candidates are distinct visible positions: at most n of them
    const int m = (int)min((int64_t)ctrl[kCtlCandIdx], (int64_t)max(qm.n, 0));
    SmallSel<CAP, MS>& W = U.small;
    find_threshold_regs<NT>(h, top_k, W.R.scan, &sh_th);
    const Thresh th = sh_th;
    if (th.digit < 0) {
        // at most K candidates: every one is selected
        const int mk = min(m, top_k);
        uint32_t* sel = W.sel;
        for (int e = t; e < mk; e += NT) sel[e] = composite_pos(cand[e]);
        __syncthreads();
        sort_out(sel, mk, top_k, out, A);
    } else if (th.in_bucket <= CAP) {
        if (t == 0) {
            W.cnt = 0;
            W.nt = 0;
            W.R.inb = 0;  // (counts the bucket's fill until the radix passes)
        }
        __syncthreads();
        // kPre candidates per thread are requested before any is examined (clamped indices, no
        // branch around the loads): one memory latency per kPre * NT candidates, not per NT
        constexpr int kPre = 16;
        for (int e0 = 0; e0 < m; e0 += kPre * NT) {
            uint64_t cv[kPre];
#pragma unroll
            for (int k = 0; k < kPre; ++k) cv[k] = cand[min(e0 + k * NT + t, m - 1)];
#pragma unroll
            for (int k = 0; k < kPre; ++k) {
                if (e0 + k * NT + t >= m) continue;
                const uint64_t c = cv[k];
                const int d = (int)(c >> 53);
                // (the histogram counts exactly these candidates: the slots stay below above / in_bucket)
                if (d > th.digit) {
                    const int j = atomicAdd(&W.cnt, 1);
                    if (j < top_k) W.sel[j] = composite_pos(c);
                } else if (d == th.digit) {
                    const int j = atomicAdd(&W.R.inb, 1);
                    if (j < CAP) W.cand[j] = c;
                }
            }
        }
        __syncthreads();
        const int total = select_bucket_lds<NT, CAP, MS>(W, A, th.in_bucket, top_k - th.above, th.digit);
        sort_out(W.sel, total, top_k, out, A);
    } else {
        SelectSharedT<CAP>& S = U.big;
        // the need-th largest of the bucket; every candidate above the bucket exceeds it
        const uint64_t thr = wg_threshold<NT>(CompositeList{cand}, m, top_k - th.above, th.digit, S);
        uint32_t* sel = reinterpret_cast<uint32_t*>(S.buf);
        if (t == 0) S.cnt = 0;
        __syncthreads();
        for (int e = t; e < m; e += NT)
            if (cand[e] >= thr) sel[atomicAdd(&S.cnt, 1)] = composite_pos(cand[e]);
        __syncthreads();
        sort_out(sel, S.cnt, top_k, out, A);
    }
    for (int b = t; b < kHistBins; b += NT) gh[b] = 0u;
    if (t == 0) ctrl[kCtlCandIdx] = 0u;
}

// ----------------------------------------------------------------------------------------
// Reindex, kernel 1: score the pool's positions with this layer's query
// ----------------------------------------------------------------------------------------
// Workgroup b scores chunk group `grp` (cpw chunks of kReindexTile pool slots) of query i; the
// items are sliced per XCD as reindex_item describes.
// cpw: chunks per workgroup (a divisor of the chunk count).  Many queries (a prefill chunk's
// tokens): each workgroup scores cpw consecutive chunks of its query and adds its first-digit
// counts to the query's histogram once, which divides the global atomics by cpw.
constexpr int kReindexWholePool = 32;  // chunks per workgroup when it scores a whole pool

template <int HI, bool MX, bool LP>
__global__ __launch_bounds__(kScoreNT) void k_idx_reindex_score(
    const int32_t* __restrict__ pool, const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    const int64_t* __restrict__ kv_row0, const int32_t* __restrict__ kv_len, int pool_blocks, int n_heads, int cpw,
    int32_t max_len, const void* __restrict__ k_idx, const uint8_t* __restrict__ k_sc, int64_t cache_rows,
    IndexWs ws) {
    // (the leading arguments, everything the first loads need, are preloaded into SGPRs)
    __shared__ uint32_t sh_hist[kHistBins];

    const int chunks = (pool_blocks * 8 + kReindexTile - 1) / kReindexTile;
    int i, grp;
    reindex_item((int)blockIdx.x, chunks / cpw, i, grp);
    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int n = eff_len(kv_len, kv_row0, i, max_len, cache_rows);
    const int64_t row0 = n > 0 ? kv_row0[i] : 0;
    const int n_elem = pool_blocks * 8;

    for (int b = t; b < kHistBins; b += kScoreNT) sh_hist[b] = 0u;
    if constexpr (LP) {  // at most 4 heads: one position per lane
        static_assert(HI == 4, "the lane-per-position form takes at most 4 heads");
        // a workgroup with many chunks (a prefill chunk's tokens: a whole pool each) stages their
        // block ids in LDS first
        __shared__ int32_t sh_pool[kReindexWholePool * (kReindexTile / 8)];
        const bool staged = cpw > 1;  // (uniform; cpw is 1 or kReindexWholePool)
        const int32_t* qpool = pool + (int64_t)i * pool_blocks;
        if (staged) {
            const int s0 = grp * cpw * (kReindexTile / 8), cnt = min(cpw * (kReindexTile / 8), pool_blocks - s0);
            for (int k = t; k < cnt; k += kScoreNT) sh_pool[k] = qpool[s0 + k];
        }
        QFragLP qf;
        load_qfrag_lp(qf, q_idx + (int64_t)i * n_heads * 64, w + (int64_t)i * n_heads, n_heads, lane);
        __syncthreads();
        if (staged)
            reindex_score_chunks_lp<MX, kScoreNT / kWave, true>(grp * cpw, (grp + 1) * cpw, n, row0, qpool, pool_blocks,
                                                                qf, k_idx, k_sc, ws.keys + (int64_t)i * n_elem, sh_hist,
                                                                sh_pool);
        else
            reindex_score_chunks_lp<MX, kScoreNT / kWave, false>(grp * cpw, (grp + 1) * cpw, n, row0, qpool,
                                                                 pool_blocks, qf, k_idx, k_sc,
                                                                 ws.keys + (int64_t)i * n_elem, sh_hist, nullptr);
    } else {
        QFrag qf;
        load_qfrag(qf, q_idx + (int64_t)i * n_heads * 64, w + (int64_t)i * n_heads, n_heads, lane);
        __syncthreads();
        reindex_score_chunks<HI, MX, kScoreNT / kWave>(grp * cpw, (grp + 1) * cpw, n, row0,
                                                       pool + (int64_t)i * pool_blocks, pool_blocks, qf, k_idx,
                                                       k_sc, ws.keys + (int64_t)i * n_elem, sh_hist);
    }
    __syncthreads();
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins;
    for (int b = t; b < kHistBins; b += kScoreNT) {
        const uint32_t h = sh_hist[b];
        if (h) atomicAdd(&gh[b], h);
    }
}

// ----------------------------------------------------------------------------------------
// Reindex, kernel 2: one workgroup per query selects Top-K among the pool's positions.
// The pool is ascending, so element order is position order: the ranking (score desc,
// position asc) is "every key above the K-th largest key T, then the keys equal to T in
// element order".  T is found by radix passes over the keys alone (the first digit's
// histogram comes from the score kernel; at most two more passes over the keys held in
// registers), and ties at T are ranked by one block scan, so no composite sort is needed.
// Each thread holds whole pool blocks (a multiple of 8 consecutive elements).
// ----------------------------------------------------------------------------------------
constexpr int kReMaxEPT = 32;  // elements per thread at pool_blocks = 4096

// EPT: elements per thread (8, 16 or 32; a multiple of 8, so threads hold whole pool blocks).
// NT threads: 1,024 (decode), or 256 with EPT = 64 for a prefill chunk's many queries (more,
// smaller workgroups per compute unit).
// The workspace's key and histogram areas come as arguments of their own, ahead of the rest, so
// that they are preloaded into SGPRs with the pool: the first loads need nothing else.
template <int NT, int EPT>
__global__ __launch_bounds__(NT) void k_idx_reindex_select(uint32_t* __restrict__ keys, uint32_t* __restrict__ hist,
                                                           const int32_t* __restrict__ pool, int pool_blocks,
                                                           int top_k, int32_t* __restrict__ idx_out) {
    __shared__ uint32_t s_hist[2][kHistBins];
    __shared__ int s_scan[NT / kWave];
    __shared__ uint32_t s_or[2];
    __shared__ Thresh sh_th;
    IndexWs ws{};
    ws.keys = keys;
    ws.hist = hist;
    reindex_select_query<NT, EPT>(blockIdx.x, pool, pool_blocks, top_k, ws, idx_out, s_hist, s_scan, s_or, &sh_th);
}

// ----------------------------------------------------------------------------------------
// host launchers
// ----------------------------------------------------------------------------------------
// Workgroups of the persistent scan: a fixed number per compute unit of the current device
// (looked up once per device).
static int scan_workgroups() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus * CSA2_SCAN_WGS_PER_CU;
    }
    return cached[dev];
}

// ----------------------------------------------------------------------------------------
// (launchers)
// ----------------------------------------------------------------------------------------
// phase bits: 1 = prep kernel (per-query metadata and tile maps), 2 = scan kernel,
// 4 = filter + select kernels; 7 = all.
// prefill != 0: every query reads the same sequence (kv_row0[0]), so the scores come from the
// MFMA kernel that tiles 16 queries x 16 positions (with per-query block pools when asked).
// mx != 0: k_idx holds MXFP4 code bytes and k_sc their E8M0 scales (never with prefill).
hipError_t launch_index_full(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                             const int64_t* kv_row0, const int32_t* kv_len, int n_q, int32_t max_len,
                             int64_t cache_rows, int n_heads, int grid_tiles, int grid_ftiles, int top_k,
                             int pool_blocks, int prefill, const IndexWs& ws, int32_t* idx_out, int32_t* pool_out,
                             int phase, hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
    // short decode contexts: the selection workgroups read the keys themselves (no filter pass)
    const int scan_keys = !prefill && max_len <= kSelScanMax ? 1 : 0;
    const bool filter = (!prefill || pool_blocks > 0) && !scan_keys;  // a prefill chunk's position lists
                                                                      // are written by its scan
    // decode calls of at most one wave of queries: the scan derives the metadata itself and
    // writes what the filter and selection read, so the metadata kernel is not launched
    const bool self_meta = !prefill && n_q <= kWave;
    if ((phase & 1) && !self_meta) {
        const int maps = (prefill ? 0 : kMapScan) | (filter ? kMapFilter : 0);
        hipLaunchKernelGGL(k_idx_prep, dim3(1), dim3(kPrepNT), 0, stream, kv_row0, kv_len, n_q, max_len, cache_rows,
                           grid_tiles, grid_ftiles, maps, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 2) {
        // ev_start / ev_stop (may be null): the decode scan kernel's own start and end are recorded
        // into them by its launch; a prefill chunk's scoring kernels are bracketed by records
        if (prefill && ev_start != nullptr) {
            hipError_t e = hipEventRecord(ev_start, stream);
            if (e != hipSuccess) return e;
        }
        if (prefill && max_len > 0) {  // (no visible position anywhere: nothing to score)
            const uint16_t* kb = static_cast<const uint16_t*>(k_idx);
            // the sample, its threshold digits, then every position against them
            const int s_px = (max_len + kPfPos - 1) / kPfPos, s_qg = (n_q + kPfQ - 1) / kPfQ;
            hipLaunchKernelGGL(k_idx_prefill_sample, dim3((unsigned)(kXcds * pf_items_per_xcd(s_px, s_qg))),
                               dim3(kScoreNT), 0, stream, q_idx, w, kb, kv_row0, n_q, cache_rows, n_heads, s_px, s_qg,
                               ws);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(k_idx_prefill_thresh, dim3(n_q), dim3(kScoreNT), 0, stream, top_k, ws);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int c_px = (max_len + kPcPos - 1) / kPcPos, c_qg = (n_q + kPcQ - 1) / kPcQ;
            auto k_cand = pool_blocks > 0 ? k_idx_prefill_cand<true> : k_idx_prefill_cand<false>;
            hipLaunchKernelGGL(k_cand, dim3((unsigned)(kXcds * pc_items_per_xcd(c_px, c_qg))), dim3(kScoreNT), 0,
                               stream, q_idx, w, kb, kv_row0, n_q, cache_rows, n_heads, c_px, c_qg, ws);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
            if (pool_blocks > 0) {
                const dim3 bgrid((unsigned)(((max_len + 7) / 8 + kBhChunk - 1) / kBhChunk), (unsigned)n_q);
                hipLaunchKernelGGL(k_idx_block_hist, bgrid, dim3(kScoreNT), 0, stream, kv_row0, cache_rows, ws);
            }
        } else if (!prefill) {
            // tiles split into 2 or 4 units while the host's tile bound leaves the grid half empty
            int sub_log2 = 0;
            while (sub_log2 < 2 && ((int64_t)grid_tiles << (sub_log2 + 1)) <= scan_workgroups()) ++sub_log2;
            const int wgs = (int)std::min<int64_t>((int64_t)grid_tiles << sub_log2, scan_workgroups());
            // (kernel variants: key format, head count, lane-per-position layout, split tiles)
            if (self_meta) {
                auto pick = [&](auto split) {
                    constexpr bool S = decltype(split)::value;
                    return mx ? (n_heads <= 4 ? k_idx_score_full_self<4, true, true, S>
                                              : k_idx_score_full_self<8, true, false, S>)
                              : (n_heads <= 4 ? k_idx_score_full_self<4, false, false, S>
                                              : k_idx_score_full_self<8, false, false, S>);
                };
                auto kern = sub_log2 == 0 ? pick(std::false_type{}) : pick(std::true_type{});
                const int fmap_out = filter ? 1 : 0;
                if (ev_start != nullptr || ev_stop != nullptr)
                    hipExtLaunchKernelGGL(kern, dim3(wgs), dim3(kScoreNT), 0, stream, ev_start, ev_stop, 0, kv_len,
                                               kv_row0, n_q, max_len, q_idx, w, k_idx, grid_tiles, sub_log2, cache_rows,
                                               n_heads, k_sc, pool_blocks, grid_ftiles, fmap_out, ws);
                else
                    hipLaunchKernelGGL(kern, dim3(wgs), dim3(kScoreNT), 0, stream, kv_len, kv_row0, n_q, max_len,
                                       q_idx, w, k_idx, grid_tiles, sub_log2, cache_rows, n_heads, k_sc, pool_blocks,
                                       grid_ftiles, fmap_out, ws);
            } else {
                auto pick = [&](auto split) {
                    constexpr bool S = decltype(split)::value;
                    return mx ? (n_heads <= 4 ? k_idx_score_full<4, true, true, S> : k_idx_score_full<8, true, false, S>)
                              : (n_heads <= 4 ? k_idx_score_full<4, false, false, S>
                                              : k_idx_score_full<8, false, false, S>);
                };
                auto kern = sub_log2 == 0 ? pick(std::false_type{}) : pick(std::true_type{});
                if (ev_start != nullptr || ev_stop != nullptr)
                    hipExtLaunchKernelGGL(kern, dim3(wgs), dim3(kScoreNT), 0, stream, ev_start, ev_stop, 0,
                                               ws.tmap, ws.qmeta, kv_row0, q_idx, w, k_idx, grid_tiles, sub_log2, n_heads,
                                               k_sc, pool_blocks, ws);
                else
                    hipLaunchKernelGGL(kern, dim3(wgs), dim3(kScoreNT), 0, stream, ws.tmap, ws.qmeta, kv_row0, q_idx, w,
                                       k_idx, grid_tiles, sub_log2, n_heads, k_sc, pool_blocks, ws);
            }
        }
        if (prefill && ev_stop != nullptr) {
            hipError_t e = hipEventRecord(ev_stop, stream);
            if (e != hipSuccess) return e;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 4) {
        if (filter) {
            // (a prefill chunk's compacting pass wrote the position lists: only the block list is left)
            hipLaunchKernelGGL(prefill ? k_idx_filter_full<true> : k_idx_filter_full<false>, dim3(grid_ftiles),
                               dim3(kScoreNT), 0, stream, ws.fmap, ws.qmeta, ws.hist, ws.keys, ws.bkeys, top_k,
                               pool_blocks, ws);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        const bool many = prefill && n_q >= 512;
        const bool many_small = many && top_k <= kSelMaxMany;  // (the position list)
        if (prefill) {
            // positions: the exact Top-K among each query's candidates; pool blocks (when asked
            // for): the threshold-bucket selection over the filtered block lists
            auto candk = many_small ? k_idx_select_cands<kSelNTMany, kSortCapMany, kSelMaxMany>
                         : many     ? k_idx_select_cands<kSelNTMany, kSortCapMany, kMaxSelect>
                                    : k_idx_select_cands<kSelNT, kSortCap, kMaxSelect>;
            hipLaunchKernelGGL(candk, dim3(n_q), dim3(many ? kSelNTMany : kSelNT), 0, stream, ws.qmeta, ws.ctrl,
                               ws.hist, ws.cand_idx, top_k, idx_out);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || pool_blocks <= 0) return e;
        }
        // (a prefill chunk selects only its pool list here; decode selects both lists)
        const int list0 = prefill ? 1 : 0;
        const bool sel_small = many && (prefill ? pool_blocks : max(top_k, pool_blocks)) <= kSelMaxMany;
        auto selk = sel_small ? k_idx_select_full<kSelNTMany, kSortCapMany, kSelMaxMany>
                    : many    ? k_idx_select_full<kSelNTMany, kSortCapMany, kMaxSelect>
                              : k_idx_select_full<kSelNT, kSortCap, kMaxSelect>;
        hipLaunchKernelGGL(selk, dim3(n_q, pool_blocks > 0 && !prefill ? 2 : 1), dim3(many ? kSelNTMany : kSelNT), 0,
                           stream, ws.qmeta, ws.hist, ws.keys, ws.bkeys, top_k, pool_blocks, scan_keys, list0, ws,
                           idx_out, pool_out);
        return hipGetLastError();
    }
    return hipSuccess;
}

// select == 0: the scoring kernel only.
hipError_t launch_index_reindex(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                                const int64_t* kv_row0, const int32_t* kv_len, int n_q, int32_t max_len,
                                int64_t cache_rows, int n_heads, const int32_t* pool, int pool_blocks, int top_k,
                                const IndexWs& ws, int32_t* idx_out, int select, hipStream_t stream,
                                hipEvent_t ev_start, hipEvent_t ev_stop, hipEvent_t ev_sel_start,
                                hipEvent_t ev_sel_stop) {
    const int chunks = (pool_blocks * 8 + kReindexTile - 1) / kReindexTile;
    // many queries (>= 512: a prefill chunk): a whole pool of 32 chunks per workgroup, one histogram
    // flush per query instead of one per chunk
    const int cpw = (n_q >= 512 && chunks % kReindexWholePool == 0) ? kReindexWholePool : 1;
    const dim3 grid((unsigned)(chunks / cpw * n_q));  // (query, chunk group) items, see reindex_item
    // at most 4 heads, and a prefill chunk's whole pools or a small decode batch: the
    // lane-per-position form (a lane's rows need one block id per 64 positions, where the 16-position
    // form waits on 8: at 8 queries 5.6 -> 5.0 us; at 32, where the loads set the time, 14.4 -> 14.7)
    const bool lp = n_heads <= 4 && (cpw == 32 || n_q <= 16);
    auto kern = mx ? (lp ? k_idx_reindex_score<4, true, true>
                         : (n_heads <= 4 ? k_idx_reindex_score<4, true, false> : k_idx_reindex_score<8, true, false>))
                   : lp ? k_idx_reindex_score<4, false, true>
                        : (n_heads <= 4 ? k_idx_reindex_score<4, false, false> : k_idx_reindex_score<8, false, false>);
    // ev_start / ev_stop, ev_sel_start / ev_sel_stop (may be null): the scoring kernel's and the
    // selection kernel's own start and end, recorded by their launches
    if (ev_start != nullptr || ev_stop != nullptr)
        hipExtLaunchKernelGGL(kern, grid, dim3(kScoreNT), 0, stream, ev_start, ev_stop, 0, pool, q_idx, w, kv_row0,
                              kv_len, pool_blocks, n_heads, cpw, max_len, k_idx, k_sc, cache_rows, ws);
    else
        hipLaunchKernelGGL(kern, grid, dim3(kScoreNT), 0, stream, pool, q_idx, w, kv_row0, kv_len, pool_blocks,
                           n_heads, cpw, max_len, k_idx, k_sc, cache_rows, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !select) return e;
    auto launch_sel = [&](auto kernel, int nt) {
        if (ev_sel_start != nullptr || ev_sel_stop != nullptr)
            hipExtLaunchKernelGGL(kernel, dim3(n_q), dim3(nt), 0, stream, ev_sel_start, ev_sel_stop, 0, ws.keys, ws.hist,
                                  pool, pool_blocks, top_k, idx_out);
        else
            hipLaunchKernelGGL(kernel, dim3(n_q), dim3(nt), 0, stream, ws.keys, ws.hist, pool, pool_blocks, top_k,
                               idx_out);
        return hipGetLastError();
    };
    if (n_q >= 512 && pool_blocks * 8 <= 256 * 64) return launch_sel(k_idx_reindex_select<256, 64>, 256);
    const int ept = (pool_blocks * 8 + kSelNT - 1) / kSelNT;
    auto sel = ept <= 8    ? k_idx_reindex_select<kSelNT, 8>
               : ept <= 16 ? k_idx_reindex_select<kSelNT, 16>
                           : k_idx_reindex_select<kSelNT, 32>;
    return launch_sel(sel, kSelNT);
}

}  // namespace csa2
