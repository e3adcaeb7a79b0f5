// Gather-dequant sparse attention: each query attends its selected FP4 entries plus its
// bf16 sliding window, with one softmax over both.
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token":
//   section VI, "What one layer looks like" - a layer's own query attends the 512 selected
//               entries of the shared cache plus its own recent window;
//   section XI  - cached FP4 values are dequantised before attention (no FP4 matmul).
// The cached latent is both key and value; 16 query heads share it.
//
// One workgroup (W waves) per query; used for calls with more queries than a decode batch (a
// prefill chunk's tokens), where the queries fill the chip by themselves.  It puts every
// memory access of a round in flight at once and keeps the per-entry instruction count low:
//   * work goes in rounds; in one round wave w owns FP4 blocks (16 entries each)
//     4WR + 4w .. 4WR + 4w + 3 and window block WR + w.  All gathers of a round are issued
//     before anything waits on them.
//   * FP4 entries are dequantised to f16 (hardware E2M1 -> f16, then one packed f16 multiply
//     by the E4M3 group scale: both factors and the product are exact in f16) and contracted
//     on v_mfma_f32_16x16x32_f16; window entries stay bf16 (v_mfma_f32_16x16x32_bf16).
//     The query is given to the f16 contraction scaled per head by a power of two that
//     keeps it inside f16 range; the logit is scaled back exactly.
//   * every logit of the round is formed before any probability, so each wave exponentiates
//     against its own round maximum and rescales its accumulator at most once per round.
//   * P.V: V^T operands come from a wave-private LDS tile written row-major (one 16-byte
//     store per 8 channels) and read with ds_read_b64_tr_b16, which returns the transposed
//     4 x 16 sub-block the MFMA A operand needs.  P is f16 for FP4 entries (one MFMA) and a
//     bf16 hi + lo pair for window entries (two MFMAs, ~16 mantissa bits).
//   * waves merge once at the end: (max, sum, O) of each wave go through LDS and each
//     thread finishes the outputs of one head's 128 / (4 W) dimensions.
// MFMA 16x16x32 lane layout (checked on gfx950): lane l supplies row/column l%16 of A/B and
// eight K elements chosen by the lane group l/16 (the same K set for A and B); the
// accumulator of lane l holds rows 4*(l/16)+i, column l%16.  16x16x16: four K elements.
// ds_read_b64_tr_b16 (checked on gfx950): within each 16-lane group, lane i's element j is
// element i%4 of the four 16-bit values addressed by lane 4j + i/4.
// Logits use S^T[entry][head] = K . Q^T (A = 16 entries x 32 channels from registers,
// B = Q^T); the S^T accumulator is already the B operand layout P^T needs for
// O^T[dim][head] += V^T . P^T, so P never leaves registers.
#include <hip/hip_ext.h>

#include <type_traits>

#include "attend_common.hpp"
#include "csa2_device.hpp"
#include "pack_common.hpp"

namespace csa2 {

// waves per workgroup: 4, at most 256 VGPRs each (two waves per SIMD), so two queries share a
// compute unit (8 waves with every VGPR they ask for kept one query per unit: 123 -> 92 us for a
// 4,096-token prefill chunk)
constexpr int kAttWaves = 4;
constexpr int kAttWavesPerEu = 2;
constexpr int kRB = 4;                       // FP4 blocks per wave per round
static_assert(kNH * kOStride * 4 <= kTileB, "a wave's merge rows fit in its tile");


// LDS of one attention workgroup: per-wave tiles (P.V operands, then the merge rows) and the
// per-wave softmax statistics.
struct AttendLds {
    uint8_t* tile;            // [kAttWaves][kTileB], 16-byte aligned
    float (*m)[kNH];          // [kAttWaves][kNH]
    float (*l)[kNH];
};

// The attention of query i (one workgroup of WAVES waves; wave w takes RB FP4 blocks and one
// window block of a round); idx_row = the query's top_k selected positions (global memory or
// LDS); pre = its first level of loads.
template <bool kFp4, bool kWin, bool kW8, int WAVES = kAttWaves, int RB = kRB>
__device__ __forceinline__ void attend_query(int i, const AttendArgs& a, const int32_t* idx_row, const AttendLds& lds,
                                             AttendPre pre) {
    constexpr int NDB = 8;  // 16-dimension output blocks
    constexpr int kRoundFp4 = WAVES * RB;  // FP4 blocks per round
    constexpr int kRoundWin = WAVES;       // window blocks per round
    static_assert(RB % 2 == 0, "FP4 blocks go to P.V in pairs");
    const uint8_t* __restrict__ codes = a.codes;
    const uint8_t* __restrict__ scales = a.scales;
    int32_t max_len = a.max_len;     // (made opaque below, after the first level of loads)
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
    float (*s_m)[kNH] = lds.m;
    float (*s_l)[kNH] = lds.l;

    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int l = t & 63;
    const int g = l >> 4;   // lane group
    const int r = l & 15;   // row / column within the 16
    int32_t len_raw = pre.len_raw;
    int64_t row0_raw = pre.row0_raw, wrow0_raw = pre.wrow0_raw, replay_raw = pre.replay_raw;
    uint32_t nwv = pre.nwv;
    const uint16_t* __restrict__ win_new = a.win_new;
    const bool has_new = kWin && win_new != nullptr;
    int pos[RB];     // selected positions of this lane's entry in each FP4 block (-1: none)
    // indices of one round (lanes past top_k read entry 0 and are masked; a length of 0 masks
    // every position later)
    auto issue_idx = [&](int R) {
        const int b0 = R * kRoundFp4 + wave * RB;
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            const int e = 16 * (b0 + j) + r;
            const int v = kFp4 ? idx_row[e < top_k ? e : 0] : -1;
            pos[j] = e < top_k ? v : -1;
        }
    };
    issue_idx(0);
    // Q^T fragments: bf16 as given (pre), and f16 scaled by 2^qe (converted while round 0's
    // gathers are in flight)
    u32x4 qb[4], qh[4];
    float cf4 = 0.f;  // logit multiplier of the f16 contraction: scale_log2 * 2^-qe
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = pre.qb[s];
    __builtin_amdgcn_sched_barrier(0);
    // an empty statement that takes and returns the four per-query values: every use of them
    // comes after it, so no wait for them is placed in front of the index and query loads
    asm volatile("" : "+v"(len_raw), "+v"(row0_raw), "+v"(wrow0_raw), "+v"(replay_raw), "+v"(nwv));
    // the same for the bounds (kernel arguments not preloaded into SGPRs): their loads are not
    // waited for in front of the first level
    asm volatile("" : "+s"(max_len), "+s"(cache_rows));

    const int n = eff_len_of(len_raw, row0_raw, max_len, cache_rows);
    // window = the last wc positions of [0, n), none before the replay start (branch-free, so
    // the replay load stays with the first level)
    const int64_t s0 = (replay != nullptr && replay_raw > 0) ? replay_raw : 0;
    const int wc = (int)max((int64_t)0, min((int64_t)min(window, n), (int64_t)n - s0));
    const int64_t row0 = n > 0 ? row0_raw : 0;
    const bool win_ok = kWin && wc > 0;
    const int64_t wrow0 = win_ok ? wrow0_raw : 0;
    const int nb4 = (kFp4 && n > 0) ? (top_k + 15) >> 4 : 0;  // FP4 blocks (none when nothing is visible)
    const int nbw = win_ok ? (wc + 15) >> 4 : 0;              // window blocks
    const int rounds = max((nb4 + kRoundFp4 - 1) / kRoundFp4, (nbw + kRoundWin - 1) / kRoundWin);

    // ---- the round's window gathers (second level: they need the length) ----
    u32x4 wf[4];      // window entry: channels [32g, 32g+32) as bf16 (E4M3: wf[0..1] hold them)
    bool wvalid = false;
    bool wnew = false;       // this lane's window entry is position n - 1, taken from win_new
    bool wnew_wave = false;  // this wave's window block of the round holds that entry
    auto issue_win = [&](int R) {
        const int wb = R * kRoundWin + wave;
        int64_t sr = -1;
        const int ew = 16 * wb + r;
        if (wb < nbw && ew < wc) {
            const int p = n - wc + ew;
            sr = wrow0 + (p % swa_cap);
            if (sr >= swa_rows) sr = -1;
        }
        wvalid = sr >= 0;
        wnew = has_new && wvalid && ew == wc - 1;
        wnew_wave = has_new && wb < nbw && (wc - 1) >> 4 == wb;
        // rows of absent entries are clamped to row 0 (kWin: the store has rows) and masked
        const int64_t wr = wvalid ? sr : 0;
        if constexpr (kW8) {
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(swa) + wr * kD + 32 * g);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const uint4 v = kWin ? src[s] : make_uint4(0, 0, 0, 0);
                wf[s] = u32x4{v.x, v.y, v.z, v.w};
            }
            wf[2] = wf[3] = u32x4{0u, 0u, 0u, 0u};
        } else {
            // the new entry comes from win_new (same layout as a store row)
            const uint16_t* row = wnew ? win_new + (int64_t)i * kD : static_cast<const uint16_t*>(swa) + wr * kD;
            const uint4* src = reinterpret_cast<const uint4*>(row + 32 * g);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint4 v = kWin ? src[s] : make_uint4(0, 0, 0, 0);
                wf[s] = u32x4{v.x, v.y, v.z, v.w};
            }
        }
    };
    issue_win(0);

    auto convert_q = [&]() {
        float amax = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                amax = fmaxf(amax, fmaxf(fabsf(bf16lo(qb[s][c])), fabsf(bf16hi(qb[s][c]))));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        int ex = 0;
        if (amax > 0.f) (void)frexpf(amax, &ex);    // amax < 2^ex
        const int qe = min(120, max(-120, 15 - ex));  // scaled |q| < 2^15 < f16 max
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                qh[s][c] = f16pair(ldexpf(bf16lo(qb[s][c]), qe), ldexpf(bf16hi(qb[s][c]), qe));
        cf4 = scale_log2 * ldexpf(1.f, -qe);
    };

    float m_run = -INFINITY;  // running max (log2 units) of head r over this wave's entries
    float l_run = 0.f;        // this lane's share of the running sum
    f32x4 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint8_t* tile = lds.tile + wave * kTileB;
    // tile addresses: row-major store of this lane's entry r; transposed read of rows 4g + r/4
    const int st_off = r * kRowB + 64 * g;
    const int tr_off = (4 * g + (r >> 2)) * kRowB + 8 * (r & 3);

    for (int R = 0; R < rounds; ++R) {
        if (R > 0) {
            issue_idx(R);
            issue_win(R);
        }
        const int b0 = R * kRoundFp4 + wave * RB;
        const int wb = R * kRoundWin + wave;
        const bool wblk = wb < nbw;
        uint4 cw[RB];
        uint32_t sw[RB];
        uint32_t vb[RB];  // validity of the 16 entries of each block (bit e)
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            // inside the loop n > 0, so row0 is a cache row: absent entries read it and are masked
            const bool ok = pos[j] >= 0 && pos[j] < n;
            const int64_t cr = row0 + (ok ? pos[j] : 0);
            cw[j] = kFp4 ? *reinterpret_cast<const uint4*>(codes + cr * 64 + 16 * g) : make_uint4(0, 0, 0, 0);
            sw[j] = kFp4 ? (uint32_t)*reinterpret_cast<const uint16_t*>(scales + cr * 8 + 2 * g) : 0u;
            vb[j] = (uint32_t)__ballot(ok) & 0xffffu;
        }
        const uint32_t vbw = (uint32_t)__ballot(wvalid) & 0xffffu;
        // keep every gather above this point: the scheduler would otherwise sink some of them
        // below the first wait and pay a second memory latency
        __builtin_amdgcn_sched_barrier(0);
        if (R == 0) convert_q();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kW8) {
            // E4M3 store: the wave holding the new entry converts its vector (two channels per
            // lane, from the first-level load) through its tile; the entry's lanes take their 32
            // channels from there in place of the store row
            if (wnew_wave) {
                const uint32_t e = e4m3_code_of_bf16(nwv & 0xffffu) | (e4m3_code_of_bf16(nwv >> 16) << 8);
                *reinterpret_cast<uint16_t*>(tile + 2 * l) = (uint16_t)e;
                wave_lds_sync();
                const uint4 v0 = *reinterpret_cast<const uint4*>(tile + 32 * g);
                const uint4 v1 = *reinterpret_cast<const uint4*>(tile + 32 * g + 16);
                if (wnew) {
                    wf[0] = u32x4{v0.x, v0.y, v0.z, v0.w};
                    wf[1] = u32x4{v1.x, v1.y, v1.z, v1.w};
                }
                wave_lds_sync();
            }
        }

        // ---- logits of the whole round ----
        u32x4 kf[RB][4];
        f32x4 sa[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            dequant_f16(cw[j], sw[j], kf[j]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, kf[j][s]),
                                                             __builtin_bit_cast(f16x8, qh[s]), acc, 0, 0, 0);
            sa[j] = acc;
        }
        f32x4 swc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kW8) {
            // E4M3 -> f16 (exact): fragment s = channels 32g + 8s .. + 7 = bytes 8s .. 8s + 7
            u32x4 wh[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t d0 = wf[s >> 1][2 * (s & 1)], d1 = wf[s >> 1][2 * (s & 1) + 1];
                wh[s] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, false)),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, 1.0f, true)),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, false)),
                              __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, 1.0f, true))};
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                wf[s] = wh[s];
                swc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, wf[s]),
                                                             __builtin_bit_cast(f16x8, qh[s]), swc, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                swc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[s]),
                                                              __builtin_bit_cast(bf16x8, qb[s]), swc, 0, 0, 0);
        }
        // logits of head r for entries 4g + ii of each block (log2 units), masked
        float x[RB + 1][4];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j <= RB; ++j) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const uint32_t bits = j < RB ? vb[j] : vbw;
                const bool ok = (bits >> (4 * g + ii)) & 1u;
                const float v = j < RB ? sa[j][ii] * cf4 : swc[ii] * (kW8 ? cf4 : scale_log2);
                x[j][ii] = ok ? v : -INFINITY;
                mx = fmaxf(mx, x[j][ii]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx);
        if (m_new == -INFINITY) continue;  // nothing valid yet (the same for every head)
        if (m_run != -INFINITY) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;
        }
        m_run = m_new;
        // probabilities: f16 for FP4 (and E4M3 window) entries, bf16 hi + lo for bf16 window entries
        uint32_t ph[RB][2], pwh[2], pwl[2];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j <= RB; ++j) {
            float p[4];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                p[ii] = __builtin_amdgcn_exp2f(x[j][ii] - m_new);  // masked: exp2(-inf) = 0
                psum += p[ii];
            }
            if (j < RB) {
                ph[j][0] = f16pair(p[0], p[1]);
                ph[j][1] = f16pair(p[2], p[3]);
            } else if (kW8) {
                pwh[0] = f16pair(p[0], p[1]);
                pwh[1] = f16pair(p[2], p[3]);
                pwl[0] = pwl[1] = 0u;
            } else {
                uint32_t h[4], lo[4];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    h[ii] = bf16_rne(p[ii]);
                    lo[ii] = bf16_rne(p[ii] - __uint_as_float(h[ii] << 16));
                }
                pwh[0] = pack2(h[0], h[1]);
                pwh[1] = pack2(h[2], h[3]);
                pwl[0] = pack2(lo[0], lo[1]);
                pwl[1] = pack2(lo[2], lo[3]);
            }
        }
        l_run += psum;

        // ---- P.V over FP4 block pairs (K = 32 entries: 16 of each block) ----
#pragma unroll
        for (int pp = 0; pp < RB / 2; ++pp) {
            if (b0 + 2 * pp >= nb4) break;  // wave-uniform
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                *reinterpret_cast<u32x4*>(tile + st_off + 16 * s) = kf[2 * pp][s];
                *reinterpret_cast<u32x4*>(tile + 16 * kRowB + st_off + 16 * s) = kf[2 * pp + 1][s];
            }
            wave_lds_sync();
            const u32x4 pf = {ph[2 * pp][0], ph[2 * pp][1], ph[2 * pp + 1][0], ph[2 * pp + 1][1]};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const s16x4 a0 = lds_tr16(tile + tr_off + 32 * db);
                const s16x4 a1 = lds_tr16(tile + 16 * kRowB + tr_off + 32 * db);
                const u32x2 u0 = __builtin_bit_cast(u32x2, a0), u1 = __builtin_bit_cast(u32x2, a1);
                const u32x4 af = {u0[0], u0[1], u1[0], u1[1]};
                o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af),
                                                               __builtin_bit_cast(f16x8, pf), o[db], 0, 0, 0);
            }
            wave_lds_sync();
        }
        // ---- P.V over the window block (K = 16 entries) ----
        if (wblk) {
#pragma unroll
            for (int s = 0; s < 4; ++s) *reinterpret_cast<u32x4*>(tile + st_off + 16 * s) = wf[s];
            wave_lds_sync();
            const u32x2 hv2 = {pwh[0], pwh[1]}, lv2 = {pwl[0], pwl[1]};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const s16x4 a = lds_tr16(tile + tr_off + 32 * db);
                if constexpr (kW8) {
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                                  __builtin_bit_cast(f16x4, hv2), o[db], 0, 0, 0);
                } else {
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4, hv2), o[db], 0, 0, 0);
                    o[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4, lv2), o[db], 0, 0, 0);
                }
            }
            wave_lds_sync();
        }
    }

    // ---- merge the eight waves ----
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (g == 0) {
        s_m[wave][r] = m_run;
        s_l[wave][r] = l_run;
    }
    {
        // this wave's O^T (dims 16 db + 4g + ii of head r) -> rows [head][dim] of its tile
        float* ob = reinterpret_cast<float*>(tile);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<f32x4*>(&ob[r * kOStride + 16 * db + 4 * g]) = o[db];
    }
    __syncthreads();
    constexpr int kTpH = WAVES * kWave / kNH;  // threads per head
    constexpr int kDv = kD / kTpH / 4;         // four-dimension vectors per thread
    static_assert(kTpH * kNH == WAVES * kWave && kDv >= 1, "merge thread layout");
    const int h = t / kTpH;
    const int d0 = 4 * kDv * (t % kTpH);
    if (h < n_heads) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f;
        f32x4 O[kDv];
#pragma unroll
        for (int v = 0; v < kDv; ++v) O[v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float f = (s_m[w][h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(s_m[w][h] - M);
            L = fmaf(s_l[w][h], f, L);
            const float* ob = reinterpret_cast<const float*>(lds.tile + w * kTileB) + h * kOStride + d0;
#pragma unroll
            for (int v = 0; v < kDv; ++v) O[v] += f * *reinterpret_cast<const f32x4*>(ob + 4 * v);
        }
#pragma unroll
        for (int v = 0; v < kDv; ++v) {
            const f32x4 res = L > 0.f ? O[v] / L : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(out + ((int64_t)i * n_heads + h) * kD + d0 + 4 * v) = res;
        }
    }
    // the new window entry into its store row, after every read of the store by this query
    // (wave 0, two channels per lane); whether or not the replay bound lets it be attended
    if (has_new && wave == 0 && n > 0) {
        const int64_t wr = wrow0_raw + ((n - 1) % swa_cap);
        if (wr >= 0 && wr < swa_rows) {
            if constexpr (kW8)
                *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(const_cast<void*>(swa)) + wr * kD + 2 * l) =
                    (uint16_t)(e4m3_code_of_bf16(nwv & 0xffffu) | (e4m3_code_of_bf16(nwv >> 16) << 8));
            else
                *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(const_cast<void*>(swa)) + wr * kD + 2 * l) = nwv;
        }
    }
}

// The arguments one by one (not the AttendArgs block), those of the first level of loads first:
// the leading ones are preloaded into SGPRs at launch, so those loads need no scalar load of
// the argument block before them.
template <bool kFp4, bool kWin, bool kW8, int W>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(kAttWavesPerEu))) void k_attend(
    const int32_t* kv_len, const int64_t* kv_row0,
                                                   const int64_t* swa_row0, const int64_t* replay, const int32_t* idx,
                                                   const uint16_t* q, int top_k, int n_heads, int32_t max_len,
                                                   int64_t cache_rows, const uint8_t* codes, const uint8_t* scales,
                                                   const void* swa, int swa_cap, int64_t swa_rows, int window,
                                                   float scale_log2, float* out, const uint16_t* win_new) {
    __shared__ __align__(16) uint8_t s_tile[W * kTileB];
    __shared__ float s_m[W][kNH], s_l[W][kNH];
    const AttendArgs a{q,        codes,   scales,   kv_row0, kv_len, max_len, cache_rows, idx,   top_k,
                       swa,      swa_row0, swa_cap, swa_rows, window, replay, n_heads,   scale_log2, out,
                       win_new};
    const int i = (int)blockIdx.x;
    attend_query<kFp4, kWin, kW8, W>(i, a, idx + (int64_t)i * top_k, AttendLds{s_tile, s_m, s_l},
                                     attend_pre<kWin>(i, a));
}

hipError_t launch_attend_dec(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* kv_row0,
                             const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, const int32_t* idx,
                             int top_k, const void* swa, int window_fp8, const int64_t* swa_row0, int swa_cap,
                             int64_t swa_rows, int window, const int64_t* replay, int n_heads, float softmax_scale,
                             float* out, const uint16_t* win_new, float* part, uint32_t* ctrl, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop);

// window_fp8: the window store holds E4M3 bytes; replay: per-query replay starts or NULL.
// Decode-sized calls (at most kAttSplitMaxQ queries) split each query's entries over workgroups
// (k_attend_dec, csrc/attend_decode.hip; part / ctrl: its merge workspace); larger calls (a
// prefill chunk's tokens, which fill the chip by themselves) take one workgroup per query.
hipError_t launch_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* kv_row0,
                         const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, const int32_t* idx,
                         int top_k, const void* swa, int window_fp8, const int64_t* swa_row0, int swa_cap,
                         int64_t swa_rows, int window, const int64_t* replay, int n_heads, float softmax_scale,
                         float* out, const uint16_t* win_new, float* part, uint32_t* ctrl, hipStream_t stream,
                         hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (n_q <= kAttSplitMaxQ)
        return launch_attend_dec(q, codes, scales, kv_row0, kv_len, n_q, max_len, cache_rows, idx, top_k, swa,
                                 window_fp8, swa_row0, swa_cap, swa_rows, window, replay, n_heads, softmax_scale, out,
                                 win_new, part, ctrl, stream, ev_start, ev_stop);
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    const bool fp4 = top_k > 0, win = window > 0 && swa_rows > 0;
    constexpr int W = kAttWaves;
    using K = decltype(&k_attend<true, true, false, W>);
    K kern;
    if (window_fp8)
        kern = fp4 ? (win ? k_attend<true, true, true, W> : k_attend<true, false, true, W>)
                   : (win ? k_attend<false, true, true, W> : k_attend<false, false, true, W>);
    else
        kern = fp4 ? (win ? k_attend<true, true, false, W> : k_attend<true, false, false, W>)
                   : (win ? k_attend<false, true, false, W> : k_attend<false, false, false, W>);
    const dim3 grid((unsigned)n_q);
    // ev_start / ev_stop (may be null): the kernel's own start and end, recorded by its launch
    if (ev_start != nullptr || ev_stop != nullptr)
        hipExtLaunchKernelGGL(kern, grid, dim3(W * 64), 0, stream, ev_start, ev_stop, 0, kv_len, kv_row0, swa_row0,
                              replay, idx, q, top_k, n_heads, max_len, cache_rows, codes, scales, swa, swa_cap, swa_rows,
                              window, scale_log2, out, win_new);
    else
        hipLaunchKernelGGL(kern, grid, dim3(W * 64), 0, stream, kv_len, kv_row0, swa_row0, replay, idx, q, top_k,
                           n_heads, max_len, cache_rows, codes, scales, swa, swa_cap, swa_rows, window, scale_log2, out,
                           win_new);
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
