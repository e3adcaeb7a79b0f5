// Decode attention split over entries: the entries of one query (its selected FP4 entries and
// its sliding window) are shared out over several workgroups, each wave taking 32 of them, and
// the workgroups' softmax partials are merged by the last of them to finish.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token":
//   section VI, "What one layer looks like" - the layer's own query attends the 512 selected
//               entries of the shared cache plus its own recent window, under one softmax;
//   section XI  - cached FP4 values are dequantised before attention (no FP4 matmul).
// The cached latent is both key and value; the 16 query heads share it.
//
// A decode call has few queries (8 to 64), so a launch is latency-bound: the time goes to the
// chain index load -> gathers -> logits -> softmax -> P.V -> merge.  Splitting a query's 640
// entries over 20 waves in 5 workgroups (one wave per SIMD) puts every entry's dequantisation
// and logits on a different SIMD, where one workgroup per query would run them all on one CU.
//   * unit = 32 entries = two 16-entry blocks: FP4 units first (entries 32u .. 32u + 31 of the
//     query's idx row), then window units (window entries 32(u - U4) .. + 31, oldest first).
//     Wave w of workgroup part s takes unit 4s + w.
//   * FP4 entries: hardware E2M1 -> f16 and one packed f16 multiply by the E4M3 group scale
//     (exact), logits on v_mfma_f32_16x16x32_f16 against the query scaled per head by a power
//     of two into f16 range; bf16 window entries on v_mfma_f32_16x16x32_bf16 against the bf16
//     query; E4M3 window entries converted to f16 (exact) and taken as FP4 entries are.
//   * P.V: O^T[dim][head] += V^T . P^T with the 32 entries as K: V^T from a wave-private LDS
//     tile (row-major store, ds_read_b64_tr_b16 transposed reads), P^T straight from the logits'
//     accumulator layout; P in f16 (bf16 hi + lo for bf16 window entries).
//   * merge: the four waves of a workgroup through LDS, then across workgroups: each writes its
//     (max, sum, O) per head with agent-scope stores, waits for them, and takes a ticket from the
//     query's counter; the workgroup with the last ticket reads all the partials (agent-scope
//     loads) and combines all of them in part order, so the result does not depend on which
//     workgroup finished last.  No workgroup waits for another.
// MFMA 16x16x32 lane layout (checked on gfx950): lane l supplies row/column l%16 of A/B and eight
// K elements chosen by l/16 (the same K set for A and B); the accumulator of lane l holds rows
// 4*(l/16)+i, column l%16.  ds_read_b64_tr_b16: within each 16-lane group, lane i's element j is
// element i%4 of the four 16-bit values addressed by lane 4j + i/4.
#include <hip/hip_ext.h>

#include "attend_common.hpp"
#include "csa2_device.hpp"
#include "pack_common.hpp"

namespace csa2 {

constexpr int kDecWaves = 4;                       // waves per workgroup (one per SIMD)
constexpr int kDecNT = kDecWaves * kWave;
constexpr int kUnitE = 32;                         // entries per wave
constexpr int kPartFloats = kNH * kD + 2 * kNH;    // a workgroup's partial: O [16][128], max [16], sum [16]
constexpr int kMergeBatch = 8;                     // partials the merging workgroup loads per batch
static_assert(kNH * kOStride * 4 <= kTileB, "a wave's merge rows fit in its tile");

// workgroups per query with nw waves each (one unit of 32 entries per wave)
inline int dec_parts(int top_k, int window, int nw) {
    const int units = (top_k + kUnitE - 1) / kUnitE + (window + kUnitE - 1) / kUnitE;
    return (units + nw - 1) / nw;
}

int attend_dec_parts(int top_k, int window) { return dec_parts(top_k, window, kDecWaves); }

size_t attend_dec_part_bytes() { return (size_t)kPartFloats * 4; }

int attend_split_max_queries() { return kAttSplitMaxQ; }

// Agent-scope (sc1) 16-byte store and 4-byte store / load through a raw buffer descriptor: they
// are coherent across the XCDs, so partials written by one workgroup are read correctly by the
// merging workgroup wherever the two run.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(float* p) {
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, 0x7fffffff, 0x00020000);
}
constexpr int kSc1 = 16;  // cache-policy operand: sc1 (agent scope)

// kFp4: top_k > 0 (the FP4 cache is read); kWin: window > 0 and the store has rows; kW8: the
// window store holds E4M3 bytes ([Article] section XI: FP8 recent-window cache).
// replay (may be NULL): per-query replay start s; the window then holds positions >= s only
// ([Article] section XII, SWA Bounded Replay).
// win_new (may be NULL): the step's own window vector per query, attended as position N - 1 and
// written to that store row ([Article] section VI: every layer writes its own window entry).
// The attention of query i by workgroup part s of `parts` (NW waves, wave w takes unit
// s * NW + w); idx_row = the query's top_k selected positions (global memory or LDS); pre = the
// first level of loads (issued by the caller, possibly before other work).
template <bool kFp4, bool kWin, bool kW8, int NW>
__device__ __forceinline__ void attend_dec_body(int i, int s, int parts, int u4, const AttendArgs& a,
                                                const int32_t* idx_row, AttendPre pre, uint8_t* s_tile,
                                                float (*s_m)[kNH], float (*s_l)[kNH], uint32_t& s_ticket, float* part,
                                                uint32_t* ctrl) {
    constexpr int TPH = NW * kWave / kNH;  // merging threads per head
    constexpr int DPT = kD / TPH;          // dimensions per merging thread
    static_assert(DPT == 8 || DPT == 2, "merge vector width");
    const uint8_t* __restrict__ codes = a.codes;
    const uint8_t* __restrict__ scales = a.scales;
    int32_t max_len = a.max_len;
    int64_t cache_rows = a.cache_rows;
    const int top_k = a.top_k;
    const void* __restrict__ swa = a.swa;
    const int swa_cap = a.swa_cap;
    const int64_t swa_rows = a.swa_rows;
    const int window = a.window;
    const int64_t* __restrict__ replay = a.replay;
    const int n_heads = a.n_heads;
    const float scale_log2 = a.scale_log2;
    float* __restrict__ out = a.out;
    const uint16_t* __restrict__ win_new = a.win_new;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int l = t & 63;
    const int g = l >> 4;   // lane group
    const int r = l & 15;   // row / column within the 16
    const int u = s * NW + wave;
    const bool is_fp4 = kFp4 && u < u4;  // wave-uniform
    const int uw = u - u4;               // window unit of a non-FP4 wave

    int32_t len_raw = pre.len_raw;
    int64_t row0_raw = pre.row0_raw, wrow0_raw = pre.wrow0_raw, replay_raw = pre.replay_raw;
    uint32_t nwv = pre.nwv;
    const bool has_new = kWin && win_new != nullptr;
    int pos[2];  // selected positions of this lane's entry in the unit's two blocks (-1: none)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = kUnitE * u + 16 * j + r;
        const bool in = is_fp4 && e < top_k;
        const int v = kFp4 ? idx_row[in ? e : 0] : -1;
        pos[j] = in ? v : -1;
    }
    u32x4 qb[4], qh[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) qb[c] = pre.qb[c];
    __builtin_amdgcn_sched_barrier(0);
    // every use of the per-query values comes after this empty statement, so their wait is not
    // placed in front of the index and query loads
    asm volatile("" : "+v"(len_raw), "+v"(row0_raw), "+v"(wrow0_raw), "+v"(replay_raw), "+v"(nwv));
    asm volatile("" : "+s"(max_len), "+s"(cache_rows));

    const int n = eff_len_of(len_raw, row0_raw, max_len, cache_rows);
    // window = the last wc positions of [0, n), none before the replay start
    const int64_t s0 = (replay != nullptr && replay_raw > 0) ? replay_raw : 0;
    const int wc = (int)max((int64_t)0, min((int64_t)min(window, n), (int64_t)n - s0));
    const int64_t row0 = n > 0 ? row0_raw : 0;
    const int64_t wrow0 = (kWin && wc > 0) ? wrow0_raw : 0;

    // The new window entry goes to its store row at once: this call never reads that row
    // (position n - 1 comes from win_new, and the row's previous position n - 1 - swa_cap lies
    // before the window since window <= swa_cap), and other queries use other rings.
    if (has_new && s == 0 && wave == 0 && n > 0) {
        const int64_t wr = wrow0_raw + ((n - 1) % swa_cap);
        if (wr >= 0 && wr < swa_rows) {
            if constexpr (kW8)
                *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(const_cast<void*>(swa)) + wr * kD + 2 * l) =
                    (uint16_t)(e4m3_code_of_bf16(nwv & 0xffffu) | (e4m3_code_of_bf16(nwv >> 16) << 8));
            else
                *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(const_cast<void*>(swa)) + wr * kD + 2 * l) = nwv;
        }
    }

    float cf4 = 0.f;  // logit multiplier of the f16 contraction: scale_log2 * 2^-qe
    auto convert_q = [&]() {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                amax = fmaxf(amax, fmaxf(fabsf(bf16lo(qb[c][k])), fabsf(bf16hi(qb[c][k]))));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        int ex = 0;
        if (amax > 0.f) (void)frexpf(amax, &ex);      // amax < 2^ex
        const int qe = min(120, max(-120, 15 - ex));  // scaled |q| < 2^15 < f16 max
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int k = 0; k < 4; ++k)
                qh[c][k] = f16pair(ldexpf(bf16lo(qb[c][k]), qe), ldexpf(bf16hi(qb[c][k]), qe));
        cf4 = scale_log2 * ldexpf(1.f, -qe);
    };

    float m_w = -INFINITY;  // this wave's max (log2 units) for head r
    float l_w = 0.f;        // this lane's share of the wave's sum
    f32x4 o[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint8_t* tile = s_tile + wave * kTileB;
    // tile addresses: row-major store of this lane's entry r; transposed read of rows 4g + r/4
    const int st_off = r * kRowB + 64 * g;
    const int tr_off = (4 * g + (r >> 2)) * kRowB + 8 * (r & 3);

    // The softmax of the wave's two blocks: x[j][ii] = masked logits (log2 units) of entries
    // 4g + ii of block j for head r.  Returns false when no entry of the wave is valid.
    auto softmax2 = [&](float (&x)[2][4], float (&p)[2][4]) -> bool {
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) mx = fmaxf(mx, x[j][ii]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (mx == -INFINITY) return false;  // (the same for every head: masks are per entry)
        m_w = mx;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                p[j][ii] = __builtin_amdgcn_exp2f(x[j][ii] - mx);  // masked: exp2(-inf) = 0
                l_w += p[j][ii];
            }
        return true;
    };
    // O^T += V^T . P^T over the two blocks held in the tile (rows 0-15 and 16-31)
    auto pv_f16 = [&](const u32x4& pf) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const u32x2 u0 = __builtin_bit_cast(u32x2, lds_tr16(tile + tr_off + 32 * db));
            const u32x2 u1 = __builtin_bit_cast(u32x2, lds_tr16(tile + 16 * kRowB + tr_off + 32 * db));
            const u32x4 af = {u0[0], u0[1], u1[0], u1[1]};
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af), __builtin_bit_cast(f16x8, pf),
                                                           o[db], 0, 0, 0);
        }
    };
    auto store_tile = [&](const u32x4 (&b0)[4], const u32x4 (&b1)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            *reinterpret_cast<u32x4*>(tile + st_off + 16 * c) = b0[c];
            *reinterpret_cast<u32x4*>(tile + 16 * kRowB + st_off + 16 * c) = b1[c];
        }
        wave_lds_sync();
    };

    if (is_fp4) {
        if (n > 0) {  // uniform; row0 is then a cache row, which absent entries read (masked)
            uint4 cw[2];
            uint32_t sw[2], vb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bool ok = pos[j] >= 0 && pos[j] < n;
                const int64_t cr = row0 + (ok ? pos[j] : 0);
                cw[j] = *reinterpret_cast<const uint4*>(codes + cr * 64 + 16 * g);
                sw[j] = (uint32_t)*reinterpret_cast<const uint16_t*>(scales + cr * 8 + 2 * g);
                vb[j] = (uint32_t)__ballot(ok) & 0xffffu;
            }
            __builtin_amdgcn_sched_barrier(0);  // every gather above the first wait
            convert_q();
            __builtin_amdgcn_sched_barrier(0);
            u32x4 kf[2][4];
            float x[2][4];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                dequant_f16(cw[j], sw[j], kf[j]);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kf[j][c]),
                                                                 __builtin_bit_cast(f16x8, qh[c]), acc, 0, 0, 0);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) x[j][ii] = ((vb[j] >> (4 * g + ii)) & 1u) ? acc[ii] * cf4 : -INFINITY;
            }
            float p[2][4];
            if (softmax2(x, p)) {
                store_tile(kf[0], kf[1]);
                const u32x4 pf = {f16pair(p[0][0], p[0][1]), f16pair(p[0][2], p[0][3]), f16pair(p[1][0], p[1][1]),
                                  f16pair(p[1][2], p[1][3])};
                pv_f16(pf);
            }
        }
    } else if (kWin && uw * kUnitE < wc) {  // uniform: the unit holds window entries
        u32x4 wf[2][4];
        bool wvalid[2], wnew[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ew = kUnitE * uw + 16 * j + r;
            int64_t sr = -1;
            if (ew < wc) {
                const int p = n - wc + ew;
                sr = wrow0 + (p % swa_cap);
                if (sr >= swa_rows) sr = -1;
            }
            wvalid[j] = sr >= 0;
            wnew[j] = has_new && wvalid[j] && ew == wc - 1;
            const int64_t wr = wvalid[j] ? sr : 0;  // (the store has rows: kWin)
            if constexpr (kW8) {
                const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(swa) + wr * kD + 32 * g);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const uint4 v = src[c];
                    wf[j][c] = u32x4{v.x, v.y, v.z, v.w};
                }
                wf[j][2] = wf[j][3] = u32x4{0u, 0u, 0u, 0u};
            } else {
                // the new entry comes from win_new (same layout as a store row)
                const uint16_t* row =
                    wnew[j] ? win_new + (int64_t)i * kD : static_cast<const uint16_t*>(swa) + wr * kD;
                const uint4* src = reinterpret_cast<const uint4*>(row + 32 * g);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint4 v = src[c];
                    wf[j][c] = u32x4{v.x, v.y, v.z, v.w};
                }
            }
        }
        const uint32_t vbw[2] = {(uint32_t)__ballot(wvalid[0]) & 0xffffu, (uint32_t)__ballot(wvalid[1]) & 0xffffu};
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kW8) convert_q();
        __builtin_amdgcn_sched_barrier(0);
        float x[2][4];
        if constexpr (kW8) {
            // the new entry (E4M3 store): this wave converts the vector (two channels per lane)
            // through its tile, and the entry's lanes take their 32 channels from there
            if (has_new && (wc - 1) / kUnitE == uw) {
                *reinterpret_cast<uint16_t*>(tile + 2 * l) =
                    (uint16_t)(e4m3_code_of_bf16(nwv & 0xffffu) | (e4m3_code_of_bf16(nwv >> 16) << 8));
                wave_lds_sync();
                const uint4 v0 = *reinterpret_cast<const uint4*>(tile + 32 * g);
                const uint4 v1 = *reinterpret_cast<const uint4*>(tile + 32 * g + 16);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    if (wnew[j]) {
                        wf[j][0] = u32x4{v0.x, v0.y, v0.z, v0.w};
                        wf[j][1] = u32x4{v1.x, v1.y, v1.z, v1.w};
                    }
                wave_lds_sync();
            }
            // E4M3 -> f16 (exact): fragment c = channels 32g + 8c .. + 7 = bytes 8c .. 8c + 7
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                u32x4 wh[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t d0 = wf[j][c >> 1][2 * (c & 1)], d1 = wf[j][c >> 1][2 * (c & 1) + 1];
                    wh[c] = u32x4{
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true))};
                }
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    wf[j][c] = wh[c];
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wf[j][c]),
                                                                 __builtin_bit_cast(f16x8, qh[c]), acc, 0, 0, 0);
                }
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) x[j][ii] = ((vbw[j] >> (4 * g + ii)) & 1u) ? acc[ii] * cf4 : -INFINITY;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[j][c]),
                                                                  __builtin_bit_cast(bf16x8, qb[c]), acc, 0, 0, 0);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    x[j][ii] = ((vbw[j] >> (4 * g + ii)) & 1u) ? acc[ii] * scale_log2 : -INFINITY;
            }
        }
        float p[2][4];
        if (softmax2(x, p)) {
            store_tile(wf[0], wf[1]);
            if constexpr (kW8) {
                const u32x4 pf = {f16pair(p[0][0], p[0][1]), f16pair(p[0][2], p[0][3]), f16pair(p[1][0], p[1][1]),
                                  f16pair(p[1][2], p[1][3])};
                pv_f16(pf);
            } else {
                // P as bf16 hi + lo (~16 significant bits) against the bf16 values
                uint32_t h[2][4], lo[2][4];
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        h[j][ii] = bf16_rne(p[j][ii]);
                        lo[j][ii] = bf16_rne(p[j][ii] - __uint_as_float(h[j][ii] << 16));
                    }
                const u32x4 ph = {pack2(h[0][0], h[0][1]), pack2(h[0][2], h[0][3]), pack2(h[1][0], h[1][1]),
                                  pack2(h[1][2], h[1][3])};
                const u32x4 pl = {pack2(lo[0][0], lo[0][1]), pack2(lo[0][2], lo[0][3]), pack2(lo[1][0], lo[1][1]),
                                  pack2(lo[1][2], lo[1][3])};
#pragma unroll
                for (int db = 0; db < 8; ++db) {
                    const u32x2 u0 = __builtin_bit_cast(u32x2, lds_tr16(tile + tr_off + 32 * db));
                    const u32x2 u1 = __builtin_bit_cast(u32x2, lds_tr16(tile + 16 * kRowB + tr_off + 32 * db));
                    const bf16x8 af = __builtin_bit_cast(bf16x8, u32x4{u0[0], u0[1], u1[0], u1[1]});
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, ph), o[db], 0, 0, 0);
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8, pl), o[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- merge the NW waves ----
    l_w += __shfl_xor(l_w, 16, 64);
    l_w += __shfl_xor(l_w, 32, 64);
    if (g == 0) {
        s_m[wave][r] = m_w;
        s_l[wave][r] = l_w;
    }
    {
        // this wave's O^T (dims 16 db + 4g + ii of head r) -> rows [head][dim] of its tile (after
        // its own transposed reads, which the wave's LDS waits have completed)
        float* ob = reinterpret_cast<float*>(tile);
#pragma unroll
        for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4*>(&ob[r * kOStride + 16 * db + 4 * g]) = o[db];
    }
    __syncthreads();
    // thread t: head h, dimensions d0 .. d0 + DPT - 1
    const int h = t / TPH;
    const int d0 = DPT * (t % TPH);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f;
    float O[DPT];
#pragma unroll
    for (int k = 0; k < DPT; ++k) O[k] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float f = (s_m[w][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
        L = fmaf(s_l[w][h], f, L);
        const float* ob = reinterpret_cast<const float*>(s_tile + w * kTileB) + h * kOStride + d0;
#pragma unroll
        for (int k = 0; k < DPT; ++k) O[k] = fmaf(f, ob[k], O[k]);
    }
    float* op = out + ((int64_t)i * n_heads + h) * kD + d0;
    auto store_out = [&](const float (&v)[DPT], float lsum) {
        if (h < n_heads) {
            const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
            for (int k = 0; k < DPT; k += 2) *reinterpret_cast<float2*>(op + k) = make_float2(v[k] * inv, v[k + 1] * inv);
        }
    };
    if (parts == 1) {
        store_out(O, L);
        return;
    }

    // ---- merge across the query's workgroups ----
    float* qpart = part + (int64_t)i * parts * kPartFloats;
    const __amdgpu_buffer_rsrc_t rs = part_rsrc(qpart);
    {
        const int base = s * kPartFloats;
#pragma unroll
        for (int k = 0; k < DPT; k += 2)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(O[k]), __float_as_uint(O[k + 1])}, rs,
                                                  4 * (base + h * kD + d0 + k), 0, kSc1);
        if (t % TPH == 0) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), rs, 4 * (base + kNH * kD + h), 0, kSc1);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(L), rs, 4 * (base + kNH * kD + kNH + h), 0, kSc1);
        }
    }
    // every partial store of this thread has completed (stores are counted in vmcnt); the barrier
    // then covers the workgroup before the ticket
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t* ctr = ctrl + (int64_t)i * kCtlSlots + kCtlAttendDone;
    if (t == 0) s_ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_ticket != (uint32_t)(parts - 1)) return;  // uniform: another workgroup merges
    asm volatile("" ::: "memory");  // nothing below moves above the ticket

    // combine every part in order 0 .. parts - 1.  The loads of a batch are unconditional (parts
    // past the last re-read the last one and are masked), so a batch costs one memory round trip;
    // this workgroup's own part is read back too (its stores have completed).
    float Mg = -INFINITY, Lg = 0.f;
    float G[DPT];
#pragma unroll
    for (int k = 0; k < DPT; ++k) G[k] = 0.f;
    for (int b0 = 0; b0 < parts; b0 += kMergeBatch) {
        float pm[kMergeBatch], pl[kMergeBatch], pv[kMergeBatch][DPT];
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            const int base = min(b0 + k, parts - 1) * kPartFloats;
#pragma unroll
            for (int c = 0; c < DPT; c += 2) {
                const u32x2 v = __builtin_bit_cast(u32x2,
                    __builtin_amdgcn_raw_buffer_load_b64(rs, 4 * (base + h * kD + d0 + c), 0, kSc1));
                pv[k][c] = __uint_as_float(v[0]);
                pv[k][c + 1] = __uint_as_float(v[1]);
            }
            pm[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (base + kNH * kD + h), 0, kSc1));
            pl[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (base + kNH * kD + kNH + h), 0, kSc1));
        }
#pragma unroll
        for (int k = 0; k < kMergeBatch; ++k) {
            // an empty part (max -inf) or one past the last adds nothing
            const bool use = b0 + k < parts && pm[k] != -INFINITY;
            const float pmk = use ? pm[k] : -INFINITY;
            const float mn = fmaxf(Mg, pmk);
            const float fa = (Mg == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(Mg - mn);
            const float fb = use ? __builtin_amdgcn_exp2f(pmk - mn) : 0.f;
            Lg = Lg * fa + pl[k] * fb;
#pragma unroll
            for (int c = 0; c < DPT; ++c) G[c] = G[c] * fa + pv[k][c] * fb;
            Mg = mn;
        }
    }
    store_out(G, Lg);
    // the counter back to zero for the next call, only now: vector memory operations complete
    // in order, so a store issued before the partial loads would hold up every one of them
    if (t == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Standalone decode attention: 4 waves per workgroup, parts = gridDim.x / n_q workgroups per
// query.  The arguments of the first level of loads lead (preloaded into SGPRs at launch).
template <bool kFp4, bool kWin, bool kW8>
__global__ __launch_bounds__(kDecNT) void k_attend_dec(
    const int32_t* kv_len, const int64_t* kv_row0, const int64_t* swa_row0, const int64_t* replay,
    const int32_t* idx, const uint16_t* q, const uint16_t* win_new, int top_k, int n_heads, int n_q, int u4,
    int32_t max_len, int64_t cache_rows, const uint8_t* codes, const uint8_t* scales, const void* swa, int swa_cap,
    int64_t swa_rows, int window, float scale_log2, float* out, float* part, uint32_t* ctrl) {
    __shared__ __align__(16) uint8_t s_tile[kDecWaves * kTileB];
    __shared__ float s_m[kDecWaves][kNH], s_l[kDecWaves][kNH];
    __shared__ uint32_t s_ticket;
    const AttendArgs a{q,        codes,   scales,   kv_row0, kv_len, max_len, cache_rows, idx,        top_k,
                       swa,      swa_row0, swa_cap, swa_rows, window, replay, n_heads,   scale_log2, out,
                       win_new};
    // workgroups i + n_q * s serve query i (with n_q a multiple of 8 they share one XCD)
    const int i = (int)blockIdx.x % n_q, s = (int)blockIdx.x / n_q;
    const AttendPre pre = attend_pre<kWin>(i, a);
    attend_dec_body<kFp4, kWin, kW8, kDecWaves>(i, s, (int)gridDim.x / n_q, u4, a, idx + (int64_t)i * top_k, pre,
                                                s_tile, s_m, s_l, s_ticket, part, ctrl);
}

// Decode attention of n_q queries (their entries split over workgroups).  part: n_q * parts
// partials of kPartFloats floats; ctrl: the per-query counters (zero between calls; the merging
// workgroup resets its query's).  Both unused when one workgroup covers a query (parts == 1).
hipError_t launch_attend_dec(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* kv_row0,
                             const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, const int32_t* idx,
                             int top_k, const void* swa, int window_fp8, const int64_t* swa_row0, int swa_cap,
                             int64_t swa_rows, int window, const int64_t* replay, int n_heads, float softmax_scale,
                             float* out, const uint16_t* win_new, float* part, uint32_t* ctrl, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop) {
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    const bool fp4 = top_k > 0, win = window > 0 && swa_rows > 0;
    const int u4 = fp4 ? (top_k + kUnitE - 1) / kUnitE : 0;
    const int parts = attend_dec_parts(fp4 ? top_k : 0, win ? window : 0);
    using K = decltype(&k_attend_dec<true, true, false>);
    K kern;
    if (window_fp8)
        kern = fp4 ? (win ? k_attend_dec<true, true, true> : k_attend_dec<true, false, true>)
                   : (win ? k_attend_dec<false, true, true> : k_attend_dec<false, false, true>);
    else
        kern = fp4 ? (win ? k_attend_dec<true, true, false> : k_attend_dec<true, false, false>)
                   : (win ? k_attend_dec<false, true, false> : k_attend_dec<false, false, false>);
    const dim3 grid((unsigned)(n_q * parts));
    // ev_start / ev_stop (may be null): the kernel's own start and end, recorded by its launch
    if (ev_start != nullptr || ev_stop != nullptr)
        hipExtLaunchKernelGGL(kern, grid, dim3(kDecNT), 0, stream, ev_start, ev_stop, 0, kv_len, kv_row0, swa_row0,
                              replay, idx, q, win_new, top_k, n_heads, n_q, u4, max_len, cache_rows, codes, scales, swa,
                              swa_cap, swa_rows, window, scale_log2, out, part, ctrl);
    else
        hipLaunchKernelGGL(kern, grid, dim3(kDecNT), 0, stream, kv_len, kv_row0, swa_row0, replay, idx, q, win_new,
                           top_k, n_heads, n_q, u4, max_len, cache_rows, codes, scales, swa, swa_cap, swa_rows, window,
                           scale_log2, out, part, ctrl);
    return hipGetLastError();
}

}  // namespace csa2
