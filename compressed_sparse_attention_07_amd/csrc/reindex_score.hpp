// Reindex-mode scoring of pool positions, shared by the standalone scoring kernel and the
// one-kernel Reindex layer.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token", sections
// VIII-IX: a Reindex layer scores its own indexer query against the Full layer's keys, over the
// positions of the shared pool's blocks only.
#pragma once

#include "scan_common.hpp"

namespace csa2 {

constexpr int kXcds = 8;  // workgroup b runs on XCD b mod 8

// Workgroup b scores chunk group `chunk` of query i.  When the group count is a multiple of
// kXcds, XCD x takes the x-th eighth of every query's pool: a pool is ascending, so that eighth
// covers about one eighth of the query's positions, and where queries read the same sequence
// (the tokens of a prefill chunk) one XCD's workgroups read one eighth of its keys, a share
// that stays in the XCD's L2.
__device__ __forceinline__ void reindex_item(int b, int chunks, int& i, int& chunk) {
    if (chunks % kXcds == 0) {
        const int per = chunks / kXcds, j = b / kXcds;
        i = j / per;
        chunk = (b % kXcds) * per + j % per;
    } else {
        i = b / chunks;
        chunk = b % chunks;
    }
}

// Scores the pool slots of chunks [c0, c1) (kReindexTile positions each) of one query with NW
// waves: one MFMA unit = two pool slots (16 positions, 1 KiB of contiguous bf16 keys each),
// lanes r < 8 taking slot 2m and r >= 8 slot 2m + 1; wave wid takes units m0 + NW u.  Writes
// each position's order-preserving key (0 for positions outside [0, n) or -1 slots) to keys
// [slot * 8 + p % 8] and counts the first digit of every nonzero key in sh_hist (LDS).
template <int HI, bool MX, int NW>
__device__ __forceinline__ void reindex_score_chunks(int c0, int c1, int n, int64_t row0,
                                                     const int32_t* __restrict__ qpool, int pool_blocks,
                                                     const QFrag& qf, const void* __restrict__ k_idx,
                                                     const uint8_t* __restrict__ k_sc, uint32_t* __restrict__ keys,
                                                     uint32_t* sh_hist) {
    const int lane = __lane_id();
    const int wid = threadIdx.x / kWave;
    const int g = lane >> 4, r = lane & 15;
    constexpr int kUnits = kReindexTile / 16 / NW;  // units per wave per chunk
    for (int chunk = c0; chunk < c1; ++chunk) {
        const int m0 = chunk * (kReindexTile / 16) + wid;
        int blk[kUnits];
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int slot = 2 * (m0 + NW * u) + (r >> 3);
            blk[u] = slot < pool_blocks ? qpool[slot] : -1;
        }
        uint4 kb[kUnits][2];
        uint32_t kc[kUnits][2], ks[kUnits];
        if (n > 0) {
            // absent rows read the sequence's first row (n > 0) and are masked below
#pragma unroll
            for (int u = 0; u < kUnits; ++u) {
                const int64_t p = (int64_t)blk[u] * 8 + (r & 7);
                const bool ok = blk[u] >= 0 && p < n;
                const int64_t kr = row0 + (ok ? p : 0);
                if constexpr (MX) {
                    const uint8_t* row = static_cast<const uint8_t*>(k_idx) + kr * 32 + 4 * g;
                    kc[u][0] = *reinterpret_cast<const uint32_t*>(row);
                    kc[u][1] = *reinterpret_cast<const uint32_t*>(row + 16);
                    ks[u] = *reinterpret_cast<const uint16_t*>(k_sc + kr * 2);
                } else {
                    const uint16_t* row = static_cast<const uint16_t*>(k_idx) + kr * 64 + 8 * g;
                    kb[u][0] = *reinterpret_cast<const uint4*>(row);
                    kb[u][1] = *reinterpret_cast<const uint4*>(row + 32);
                }
            }
            if constexpr (MX) {
#pragma unroll
                for (int u = 0; u < kUnits; ++u) {
                    kb[u][0] = mx_frag(kc[u][0], ks[u] & 0xffu);
                    kb[u][1] = mx_frag(kc[u][1], ks[u] >> 8);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnits; ++u) {
            const int slot = 2 * (m0 + NW * u) + (r >> 3);
            const int64_t p = (int64_t)blk[u] * 8 + (r & 7);
            const bool ok = n > 0 && blk[u] >= 0 && p < n;
            const float sc = n > 0 ? mfma_score<HI>(qf, kb[u][0], kb[u][1]) : 0.f;
            const uint32_t key = ok ? score_key(sc) : 0u;
            if (g == 0 && slot < pool_blocks) {
                keys[slot * 8 + (r & 7)] = key;
                if (key) atomicAdd(&sh_hist[key >> 21], 1u);
            }
        }
    }
}

// The lane-per-position form (at most 4 heads; QFragLP, as the decode scan's MXFP4 layout): a
// wave step covers 8 pool slots = 64 positions, lane l taking row l % 8 of slot l / 8; the lane
// reads its own row (128 bytes of bf16 in 8 loads, or 32 MXFP4 code bytes in 2 and their 2
// scale bytes) and eight block-diagonal MFMAs leave the four head dot products of its position
// in its accumulator, so the per-position epilogue (ReLU-weighted sum, key, store, histogram)
// runs once per position instead of in one lane of four.  Wave wid takes steps 2 wid, 2 wid + 1
// of each chunk (both steps' loads in flight).
// STAGED: the block ids of chunks c0 .. c1 - 1 are already in LDS (lpool[k] = block id of pool
// slot c0 * kReindexTile / 8 + k), so that each chunk's rows wait on one memory latency instead
// of two (a workgroup that scores many chunks stages them once); otherwise they come from qpool.
template <bool MX, int NW, bool STAGED>
__device__ __forceinline__ void reindex_score_chunks_lp(int c0, int c1, int n, int64_t row0,
                                                        const int32_t* __restrict__ qpool, int pool_blocks,
                                                        const QFragLP& qf, const void* __restrict__ k_idx,
                                                        const uint8_t* __restrict__ k_sc, uint32_t* __restrict__ keys,
                                                        uint32_t* sh_hist, const int32_t* lpool) {
    const int lane = __lane_id();
    const int wid = threadIdx.x / kWave;
    constexpr int kSteps = kReindexTile / 64 / NW;  // 64-position steps per wave per chunk
    static_assert(kSteps * 64 * NW == kReindexTile, "whole steps per chunk");
    for (int chunk = c0; chunk < c1; ++chunk) {
        constexpr int kLd = MX ? 2 : 8;  // 16-byte loads per row
        int slot[kSteps], blk[kSteps];
        uint4 kr[kSteps][kLd];
        uint32_t ks[kSteps];
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            slot[j] = chunk * (kReindexTile / 8) + 8 * (kSteps * wid + j) + (lane >> 3);
            if constexpr (STAGED)
                blk[j] = slot[j] < pool_blocks ? lpool[slot[j] - c0 * (kReindexTile / 8)] : -1;
            else
                blk[j] = slot[j] < pool_blocks ? qpool[slot[j]] : -1;
        }
        if (n > 0) {
            // absent rows read the sequence's first row (n > 0) and are masked below
#pragma unroll
            for (int j = 0; j < kSteps; ++j) {
                const int64_t p = (int64_t)blk[j] * 8 + (lane & 7);
                const bool ok = blk[j] >= 0 && p < n;
                const int64_t kr_row = row0 + (ok ? p : 0);
                const uint4* row = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(k_idx) + kr_row * 16 * kLd);
#pragma unroll
                for (int s2 = 0; s2 < kLd; ++s2) kr[j][s2] = row[s2];
                if constexpr (MX) ks[j] = *reinterpret_cast<const uint16_t*>(k_sc + kr_row * 2);
            }
        }
#pragma unroll
        for (int j = 0; j < kSteps; ++j) {
            const int64_t p = (int64_t)blk[j] * 8 + (lane & 7);
            const bool ok = n > 0 && blk[j] >= 0 && p < n;
            float sc = 0.f;
            if (n > 0) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < 8; ++s2) {
                    uint4 kf;
                    if constexpr (MX) {  // k-step s2 lies in scale block s2 / 4
                        const uint4& c = kr[j][s2 >> 2];
                        const uint32_t dw = (s2 & 3) == 0 ? c.x : (s2 & 3) == 1 ? c.y : (s2 & 3) == 2 ? c.z : c.w;
                        kf = mx_frag(dw, s2 < 4 ? (ks[j] & 0xffu) : (ks[j] >> 8));
                    } else {
                        kf = kr[j][s2];
                    }
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf.a[s2], as_bf16x8(kf), acc, 0, 0, 0);
                }
#pragma unroll
                for (int h = 0; h < 4; ++h) sc = fmaf(qf.w[h], relu(acc[h]), sc);
            }
            const uint32_t key = ok ? score_key(sc) : 0u;
            if (slot[j] < pool_blocks) {
                keys[slot[j] * 8 + (lane & 7)] = key;
                if (key) atomicAdd(&sh_hist[key >> 21], 1u);
            }
        }
    }
}

}  // namespace csa2
