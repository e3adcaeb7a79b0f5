// Full-mode decode scan kernel (k_idx_score_full): every visible position's indexer score,
// its order-preserving key, the 8-position block-max key and both first-digit histograms.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token", section
// IX: the Full layer scores all causally visible positions and ranks 8-position blocks by
// their maximum score.
#pragma once

#include "scan_common.hpp"

namespace csa2 {
// ----------------------------------------------------------------------------------------
// Full mode, kernel 1: scores -> keys, block-max keys, first-digit histograms
// ----------------------------------------------------------------------------------------
// Persistent: the grid holds a few workgroups per CU and workgroup g streams the contiguous
// range [g * U / G, (g + 1) * U / G) of U work units, so the per-tile set-up (tile map, query
// slice) is paid once per query rather than once per tile, and the first-digit histograms go
// to the workspace only when the query changes.  A unit is one of the T tiles of the map, or,
// when the host's tile bound is small next to the grid, one of S = 2 or 4 equal position
// ranges of a tile (U = T * S, S = 1 << sub_log2), so a short context is not streamed by a
// single workgroup.
// MX: keys are MXFP4 (k_idx = code bytes [rows, 32], k_sc = E8M0 bytes [rows, 2]) instead of
// bf16 (k_idx = [rows, 64] bf16, k_sc unused).
// LP: the lane-per-position layout (QFragLP; MXFP4 keys, at most 4 heads): a wave step covers 64
// positions with one score per lane, so the per-position epilogue (ReLU-weighted head sum,
// key, stores, histogram atomics, block maximum) costs a quarter of the instructions of the
// 16-position layout; the lane reads its own row (16-byte loads, 32 B per MXFP4 row).
// SPLIT: sub_log2 is honoured (false: one unit per tile, the loop bounds fold to constants).
// SELF: no metadata kernel ran before (decode calls of at most 64 queries).  Every wave
// derives the per-query tile runs itself, lane i holding query i's, with the same rule as
// k_idx_prep (max(1, ceil(n_i / tile)) consecutive tiles per query, clamped to the host's
// grid bound), finds a tile's query by a ballot over the run starts, and the workgroups write
// the per-query metadata and the filter pass's tile map for the kernels that follow.  One
// dependent load (length and rows) then precedes the first key loads, instead of two (tile
// map, then metadata), and the metadata kernel's launch is saved.
template <int HI, bool MX, bool LP, bool SPLIT, bool SELF>
__device__ __forceinline__ void score_full_body(
    const int32_t* __restrict__ tmap, QMeta* __restrict__ qmeta, const int64_t* __restrict__ kv_row0,
    const int32_t* __restrict__ kv_len,
    int n_q, int32_t max_len, int64_t cache_rows, int grid_ftiles, int fmap_out, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, const void* __restrict__ k_idx, int grid_tiles, int sub_log2, int n_heads,
    const uint8_t* __restrict__ k_sc, int pool_blocks, const IndexWs& ws) {
    __shared__ uint32_t sh_hist[kHistBins];
    __shared__ uint32_t sh_bhist[kHistBins];
    // per wave: the keys and block keys of its batches of the current unit (16-position layout)
    __shared__ __align__(16) uint32_t sh_key[kScoreNT / kWave][LP ? 4 : kFullTile / 4];
    __shared__ __align__(16) uint32_t sh_bk[kScoreNT / kWave][LP ? 4 : kFullTile / 32];

    const int t = threadIdx.x;
    const int lane = __lane_id();
    const int wid = __builtin_amdgcn_readfirstlane(t / kWave);  // (uniform: scalar registers)
    const int g = lane >> 4, r = lane & 15;
    const bool want_pool = pool_blocks > 0;
    if constexpr (!SPLIT) sub_log2 = 0;
    const int64_t units = (int64_t)grid_tiles << sub_log2;
    const int ub = (int)((int64_t)blockIdx.x * units / gridDim.x);
    const int ue = (int)((int64_t)(blockIdx.x + 1) * units / gridDim.x);
    const int unit_len = kFullTile >> sub_log2;  // positions per unit

    // SELF: lane i's copy of query i's metadata (lanes past n_q: a start no tile reaches)
    int lm_n = 0, lm_start = INT32_MAX, lm_ntiles = 0, lm_fstart = INT32_MAX, lm_fntiles = 0;
    int64_t lrow0 = 0;
    int used_s = 0, used_f = 0;  // scan / filter tiles owned by some query; the rest of each bound is unused
    if constexpr (SELF) {
        // one vector load per lane (query) for the lengths and rows: a single round trip for
        // all queries (eight rounds of scalar loads at 64 queries measured 2.5 us slower at 32)
        int n = 0;
        if (lane < n_q) {
            lrow0 = kv_row0[lane];
            n = eff_len_of(kv_len[lane], lrow0, max_len, cache_rows);
        }
        const int ts = (int)(((int64_t)n + kFullTile - 1) / kFullTile);
        const int tf = (int)(((int64_t)n + kFilterTile - 1) / kFilterTile);
        const int xs = ts > 1 ? ts - 1 : 0, xf = tf > 1 ? tf - 1 : 0;  // tiles beyond each query's first
        const int in_s = wave_inclusive_scan(xs), in_f = wave_inclusive_scan(xf);
        const int cap_s = grid_tiles - n_q, cap_f = grid_ftiles - n_q;
        const int p0 = min(cap_s, in_s - xs), p1 = min(cap_s, in_s);
        const int f0 = min(cap_f, in_f - xf), f1 = min(cap_f, in_f);
        lm_start = lane < n_q ? lane + p0 : INT32_MAX;
        lm_ntiles = 1 + (p1 - p0);
        lm_fstart = lane < n_q ? lane + f0 : INT32_MAX;
        lm_fntiles = 1 + (f1 - f0);
        lm_n = (int)min((int64_t)n, min((int64_t)lm_ntiles * kFullTile, (int64_t)lm_fntiles * kFilterTile));
        used_s = n_q + min(cap_s, __builtin_amdgcn_readlane(in_s, 63));
        used_f = n_q + min(cap_f, __builtin_amdgcn_readlane(in_f, 63));
    }

    for (int b = t; b < kHistBins; b += kScoreNT) {
        sh_hist[b] = 0u;
        sh_bhist[b] = 0u;
    }
    static_assert(!LP || (HI == 4 && MX), "the lane-per-position layout: MXFP4 keys, 4 heads");
    int cur = -1;  // query whose counts the LDS histograms hold
    QMeta qm{};
    int64_t row0 = 0;
    std::conditional_t<LP, QFragLP, QFrag> qf;
    // add the LDS histograms of query `cur` to the workspace and clear them (after a barrier)
    auto flush = [&]() {
        uint32_t* gh = ws.hist + (int64_t)cur * 2 * kHistBins;
        for (int b = t; b < kHistBins; b += kScoreNT) {
            const uint32_t h = sh_hist[b];
            if (h) {
                atomicAdd(&gh[b], h);
                sh_hist[b] = 0u;
            }
            if (want_pool) {
                const uint32_t hb = sh_bhist[b];
                if (hb) {
                    atomicAdd(&gh[kHistBins + b], hb);
                    sh_bhist[b] = 0u;
                }
            }
        }
    };

    // one step = 64 consecutive positions of the workgroup (16 per wave); U steps per batch
    constexpr int U = CSA2_SCAN_U;
    // the 16-position layout's staged keys (see below): the wave's first key of the unit they
    // belong to, and how many batches of it
    constexpr int WR = 16 * U;  // positions per wave per batch
    uint32_t* s_key = sh_key[wid];
    uint32_t* s_bk = sh_bk[wid];
    uint32_t* pend_k = nullptr;
    uint32_t* pend_b = nullptr;
    int pend_j = 0;
    // (the key runs are stored non-temporally, streamed past the caches: 1M x 8 queries 186 ->
    // 178 us; the block keys, an eighth as many, stay cached)
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    auto write_run = [&]() {
        if (pend_j > 0) {  // (uniform) batch q's 16U keys go to pend_k + q 64U, from lanes 32 (q & 1) ..
            for (int q0 = 0; q0 < pend_j; q0 += 2) {
                const int q = q0 + (lane >> 5);
                if (q < pend_j)
                    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_nt*>(s_key + q * WR + 4 * (lane & 31)),
                                                reinterpret_cast<u32x4_nt*>(pend_k + q * 64 * U + 4 * (lane & 31)));
            }
            if (want_pool && lane < pend_j * (WR / 32)) {  // batch q's 2U block keys, 4 per lane
                const int q = lane / (WR / 32), c = lane % (WR / 32);
                *reinterpret_cast<uint4*>(pend_b + q * 8 * U + 4 * c) =
                    *reinterpret_cast<const uint4*>(s_bk + q * (WR / 8) + 4 * c);
            }
            pend_j = 0;
        }
    };
    static_assert((kFullTile / 4) % (64 * U) == 0 && (kFullTile / 4) % (256 * CSA2_SCAN_U_LP) == 0,
                  "a quarter tile holds whole load batches");
    for (int unit = ub; unit < ue; ++unit) {
        const int tile = unit >> sub_log2;
        const int b_lo = (unit & ((1 << sub_log2) - 1)) * unit_len, b_hi = b_lo + unit_len;
        int i;
        if constexpr (SELF) {
            if (tile >= used_s) break;  // unused tiles sit at the end of the grid bound
            // the owner is the last query whose run starts at or before the tile (starts ascend)
            i = 63 - __builtin_clzll(__ballot(lm_start <= tile));
        } else {
            i = tmap[tile];
            if (i < 0) break;  // unused tiles sit at the end of the map
        }
        if (i != cur) {
            __syncthreads();  // every wave's counts of `cur` are in LDS (and the clearing above)
            if (cur >= 0) {
                flush();
                __syncthreads();
            }
            cur = i;
            if constexpr (SELF) {
                qm.n = __builtin_amdgcn_readlane(lm_n, i);
                qm.start = __builtin_amdgcn_readlane(lm_start, i);
                row0 = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(lrow0 >> 32), i) << 32) |
                                 (uint32_t)__builtin_amdgcn_readlane((int)lrow0, i));
            } else {
                qm = qmeta[i];
                row0 = kv_row0[i];
            }
            if constexpr (LP)
                load_qfrag_lp(qf, q_idx + (int64_t)i * n_heads * 64, w + (int64_t)i * n_heads, n_heads, lane);
            else
                load_qfrag(qf, q_idx + (int64_t)i * n_heads * 64, w + (int64_t)i * n_heads, n_heads, lane);
            // the query's fragments complete here (once per query), so the batch loop's waits
            // count only its own key loads: vmcnt(0)
            __builtin_amdgcn_s_waitcnt(0x0f70);
        }
        const int n = qm.n;
        const int64_t key_base = (int64_t)qm.start * kFullTile;
        const int p_tile = (tile - qm.start) * kFullTile;
        if (p_tile >= n) continue;
        // buffer view of this tile's rows: one 32-bit lane offset for every load (the step goes
        // in the scalar offset) and rows past the sequence read as zeros
        const int rows_here = min(n - p_tile, kFullTile);
        constexpr int kRowB = MX ? 32 : 128;  // key bytes per position (codes only for MXFP4)
        const BufRsrc rs = tile_rsrc(static_cast<const uint8_t*>(k_idx) + (row0 + p_tile) * kRowB, rows_here * kRowB);
        const BufRsrc rss = tile_rsrc(MX ? k_sc + (row0 + p_tile) * 2 : nullptr, MX ? rows_here * 2 : 0);
        if constexpr (LP) {
            // one step = 256 consecutive positions of the workgroup (64 per wave, one per lane)
            constexpr int UL = CSA2_SCAN_U_LP;
            constexpr int kLd = kRowB / 16;  // 16-byte loads per row
            const int voff = (64 * wid + lane) * kRowB;
            const int voff_s = (64 * wid + lane) * 2;
            // loads pipelined across batches as in the 16-position layout below
            constexpr int kNoRow = 1 << 30;
            uint4 kr[UL][kLd];
            uint32_t ks[UL];
            auto issue = [&](int u, int bb, bool real) {
#pragma unroll
                for (int j = 0; j < kLd; ++j)
                    kr[u][j] = buf_ld16(rs, (real ? voff : kNoRow) + 16 * j, (bb + 256 * u) * kRowB);
                if constexpr (MX) ks[u] = buf_ld2(rss, real ? voff_s : kNoRow, (bb + 256 * u) * 2);
            };
            for (int b = b_lo; b < b_hi; b += 256 * UL) {
                const int pb = p_tile + b;
                if (pb >= n) break;
                if (b == b_lo) {
#pragma unroll
                    for (int u = 0; u < UL; ++u) issue(u, b, true);
                    __builtin_amdgcn_sched_barrier(0);  // every load of the batch goes out first
                }
                const int bn = b + 256 * UL;
                const bool next = bn < b_hi && p_tile + bn < n;  // (uniform) the unit has another batch
#pragma unroll
                for (int u = 0; u < UL; ++u) {
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < 8; ++s2) {
                        uint4 kf;
                        if constexpr (MX) {  // k-step s2 lies in scale block s2 / 4
                            const uint4& c = kr[u][s2 >> 2];
                            const uint32_t dw = (s2 & 3) == 0 ? c.x : (s2 & 3) == 1 ? c.y : (s2 & 3) == 2 ? c.z : c.w;
                            kf = mx_frag(dw, s2 < 4 ? (ks[u] & 0xffu) : (ks[u] >> 8));
                        } else {
                            kf = kr[u][s2];
                        }
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf.a[s2], as_bf16x8(kf), acc, 0, 0, 0);
                    }
                    float sc = 0.f;
#pragma unroll
                    for (int h = 0; h < 4; ++h) sc = fmaf(qf.w[h], relu(acc[h]), sc);
                    const int p = pb + 256 * u + 64 * wid + lane;
                    const bool mine = p < n;
                    const uint32_t key = mine ? score_key(sc) : 0u;
                    // (non-temporal stores here: with 34-byte MXFP4 rows the key writes are an eighth
                    // of the traffic, and streaming them past the caches measured 11 % faster.  The
                    // whole-line loads and staged key runs of the layout below measured slower here:
                    // 52 -> 57 us at 1M x 8 queries, each of the two alone 61-63 us)
                    if (mine) {
                        __builtin_nontemporal_store(key, &ws.keys[key_base + p]);
                        atomicAdd(&sh_hist[key >> 21], 1u);
                    }
                    if (want_pool) {
                        const uint32_t bk = max_over_8_lanes(key);  // lanes 8k + 4: block of lanes 8k .. 8k + 7
                        if ((lane & 7) == 4 && p - 4 < n) {
                            __builtin_nontemporal_store(bk, &ws.bkeys[key_base / 8 + ((p - 4) >> 3)]);
                            atomicAdd(&sh_bhist[bk >> 21], 1u);
                        }
                    }
                    issue(u, bn, next);  // this step's registers: step u of the next batch
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            // A batch of U steps covers 16U consecutive positions of each wave (64U of the
            // workgroup), so a wave's keys of one batch form one aligned run of 16U keys and 2U
            // block keys.  The runs of all the unit's batches are staged in LDS and written with
            // 16-byte stores once the next unit's first key loads are out (a store ahead of them
            // would hold them up: memory operations of a wave complete in order), so the unit's
            // keys reach memory together.  Keys of positions at or past n in a run are written as
            // 0 inside the query's own tile; every reader bounds its keys by n.
            // bf16 keys: whole-row loads, non-temporal (rowline_voff; on 128-byte rows these
            // measured faster than loads of half rows in the fragment layout)
            const int voff = MX ? (WR * wid + r) * kRowB + 4 * g : WR * wid * kRowB + rowline_voff(lane);
            const int voff_s = (WR * wid + r) * 2;
            // Loads are pipelined across the unit's batches: once step u of a batch is scored,
            // its registers take step u of the next batch, so a wave always has U steps of loads
            // in flight (no gap of a memory latency between batches).  A step of a batch that
            // does not exist is loaded through a lane offset past the view: zeros, no access.
            constexpr int kNoRow = 1 << 30;
            uint4 kb[U][2];
            uint32_t kc[U][2], ks[U];
            auto issue = [&](int u, int bb, bool real) {
                const int vo = real ? voff : kNoRow;
                if constexpr (MX) {
                    kc[u][0] = buf_ld4(rs, vo, (bb + 16 * u) * kRowB);
                    kc[u][1] = buf_ld4(rs, vo + 16, (bb + 16 * u) * kRowB);
                    ks[u] = buf_ld2(rss, real ? voff_s : kNoRow, (bb + 16 * u) * 2);
                } else {
                    kb[u][0] = buf_ld16_nt(rs, vo, (bb + 16 * u) * kRowB);
                    kb[u][1] = buf_ld16_nt(rs, vo + 8 * kRowB, (bb + 16 * u) * kRowB);
                }
            };
            int jd = 0;  // batches of this unit done
            for (int b = b_lo; b < b_hi; b += 64 * U) {
                const int pb = p_tile + b;
                if (pb >= n) break;
                if (b == b_lo) {
                    write_run();  // the previous unit's runs
                    wave_lds_sync();
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        issue(u, b, true);
                        __builtin_amdgcn_sched_barrier(0);  // in step order: step 0 waits for its own loads only
                    }
                }
                const int bn = b + 64 * U;
                const bool next = bn < b_hi && p_tile + bn < n;  // (uniform) the unit has another batch
                const int j = (b - b_lo) / (64 * U);  // batch of the unit
                const int pw = pb + WR * wid;         // first position of this wave's run
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int p0 = pw + 16 * u;  // first of this step's 16 positions
                    const int p = p0 + r;
                    if constexpr (MX) {
                        kb[u][0] = mx_frag(kc[u][0], ks[u] & 0xffu);
                        kb[u][1] = mx_frag(kc[u][1], ks[u] >> 8);
                    } else {
                        rowline_to_frags(kb[u][0], kb[u][1], lane);
                    }
                    const float sc = mfma_score<HI>(qf, kb[u][0], kb[u][1]);
                    const bool mine = g == 0 && p < n;
                    const uint32_t key = mine ? score_key(sc) : 0u;
                    if (g == 0) s_key[j * WR + 16 * u + r] = key;
                    if (mine) atomicAdd(&sh_hist[key >> 21], 1u);
                    if (want_pool) {
                        const uint32_t bk = max_over_8_lanes(key);
                        const int pblk = p0 + (r & 8);  // the 8-position pool block of lanes 4 / 12
                        if (g == 0 && (r & 7) == 4) {
                            s_bk[j * (WR / 8) + 2 * u + (r >> 3)] = pblk < n ? bk : 0u;
                            if (pblk < n) atomicAdd(&sh_bhist[bk >> 21], 1u);
                        }
                    }
                    issue(u, bn, next);  // this step's registers: step u of the next batch
                    __builtin_amdgcn_sched_barrier(0);
                }
                jd = j + 1;
            }
            if (jd > 0) {  // (uniform)
                wave_lds_sync();
                pend_k = ws.keys + key_base + p_tile + b_lo + WR * wid;
                pend_b = ws.bkeys + (key_base + p_tile + b_lo + WR * wid) / 8;
                pend_j = jd;
            }
        }
    }
    if constexpr (!LP) write_run();
    if (cur >= 0) {
        __syncthreads();
        flush();
    }
    if constexpr (SELF) {
        // what k_idx_prep would have written for the kernels that follow: the per-query
        // metadata (first workgroup) and the filter pass's tile -> query map (one entry per
        // thread, from the first workgroups on)
        if (blockIdx.x == 0 && t < n_q) {
            int4* m = reinterpret_cast<int4*>(qmeta + t);  // QMeta: n, start, ntiles, fstart, fntiles, pad
            m[0] = make_int4(lm_n, lm_start, lm_ntiles, lm_fstart);
            m[1] = make_int4(lm_fntiles, 0, 0, 0);
        }
        if (fmap_out) {
            for (int k0 = blockIdx.x * kScoreNT; k0 < grid_ftiles; k0 += gridDim.x * kScoreNT) {  // (uniform)
                const int k = k0 + t;
                // last query whose filter run starts at or before k (binary lifting over the lanes'
                // ascending starts; lanes past n_q hold INT32_MAX; every lane takes part)
                int lo = 0;
                for (int step = 32; step > 0; step >>= 1) {
                    const int fs = __shfl(lm_fstart, lo + step);
                    if (fs <= k) lo += step;
                }
                if (k < grid_ftiles) ws.fmap[k] = k < used_f ? lo : -1;
            }
        }
    }
}

// Tile map and metadata from k_idx_prep.  The tile map and everything the first loads of a
// tile need lead the arguments (preloaded into SGPRs at launch); ws supplies the output areas.
template <int HI, bool MX, bool LP, bool SPLIT>
__global__ __launch_bounds__(kScoreNT) __attribute__((amdgpu_waves_per_eu(CSA2_SCAN_WGS_PER_CU))) void k_idx_score_full(
    const int32_t* tmap, QMeta* qmeta, const int64_t* __restrict__ kv_row0, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, const void* __restrict__ k_idx, int grid_tiles, int sub_log2, int n_heads,
    const uint8_t* __restrict__ k_sc, int pool_blocks, IndexWs ws) {
    score_full_body<HI, MX, LP, SPLIT, false>(tmap, qmeta, kv_row0, nullptr, 0, 0, 0, 0, 0, q_idx, w, k_idx,
                                              grid_tiles, sub_log2, n_heads, k_sc, pool_blocks, ws);
}

// Metadata derived in the kernel (at most 64 queries, no metadata kernel before it): the
// lengths, rows and query count lead the arguments, so the first loads wait on nothing else.
// fmap_out != 0: the filter pass runs next and reads its tile map from ws.fmap.
template <int HI, bool MX, bool LP, bool SPLIT>
__global__ __launch_bounds__(kScoreNT) __attribute__((amdgpu_waves_per_eu(CSA2_SCAN_WGS_PER_CU))) void k_idx_score_full_self(
    const int32_t* __restrict__ kv_len, const int64_t* __restrict__ kv_row0, int n_q, int32_t max_len,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, const void* __restrict__ k_idx, int grid_tiles,
    int sub_log2, int64_t cache_rows, int n_heads, const uint8_t* __restrict__ k_sc, int pool_blocks,
    int grid_ftiles, int fmap_out, IndexWs ws) {
    score_full_body<HI, MX, LP, SPLIT, true>(nullptr, ws.qmeta, kv_row0, kv_len, n_q, max_len, cache_rows,
                                             grid_ftiles, fmap_out, q_idx, w, k_idx, grid_tiles, sub_log2, n_heads,
                                             k_sc, pool_blocks, ws);
}

}  // namespace csa2
