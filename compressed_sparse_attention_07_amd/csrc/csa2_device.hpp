// Device helpers shared by the CSA2 kernels (gfx950, wave64).
//
// Selection order everywhere: (score descending, position ascending).  A score is
// mapped to an order-preserving 32-bit key; a (key, position) pair is mapped to a
// unique 64-bit composite  key << 32 | (0xffffffff - position),  so "the K largest
// composites" is exactly the ranking the indexer asks for (Article "DeepSeek-V4.1-
// Flash: Pushing KV Cache Compression to 890 Bytes per Token", section IX: Top-K
// positions, block pool by block-max score), ties going to the lower index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kWave = 64;
constexpr int kHistBits = 11;                 // first radix digit = top 11 key bits
constexpr int kHistBins = 1 << kHistBits;     // 2048
constexpr int kSortCap = 8192;                // largest candidate set selected in LDS
constexpr int kMaxSelect = 4096;
constexpr int kAttSplitMaxQ = 64;           // attention calls up to this many queries are decode-sized

// Per-query self-cleaning counters at the start of the workspace (16 x u32 = 64 B).
enum CtrlSlot {
    kCtlScoreDone = 0,
    kCtlFilterDone = 1,
    kCtlSureIdx = 2,
    kCtlCandIdx = 3,
    kCtlSurePool = 4,
    kCtlCandPool = 5,
    kCtlAttendDone = 6,
    kCtlSlots = 16,
};

// Per-query metadata of the Full-mode kernels (written by the prep kernel).
struct QMeta {
    int32_t n;        // clamped visible length
    int32_t start;    // first scan tile (keys of the query start at start * scan tile)
    int32_t ntiles;   // scan tiles
    int32_t fstart;   // first filter tile
    int32_t fntiles;  // filter tiles
    int32_t pad[3];
};

// Result of the first-digit threshold search for one query and one selection.
struct Thresh {
    int32_t digit;      // bucket holding the K-th largest key; -1: everything is selected
    int32_t above;      // elements in buckets above `digit`
    int32_t in_bucket;  // elements in bucket `digit`
    int32_t total;      // valid elements
};

// Workspace views of the Full / Reindex indexer (carved by the host from one caller buffer).
struct IndexWs {
    uint32_t* ctrl;      // [n_q][kCtlSlots]          self-cleaning counters
    uint32_t* hist;      // [n_q][2][2048]            self-cleaning histograms
    Thresh* meta;        // [n_q][2]
    uint32_t* keys;      // [grid_tiles * kFullTile]  per-position keys (Full) / per-candidate keys (Reindex)
    uint32_t* bkeys;     // [grid_tiles * kFullTile / 8] per-block max keys
    int32_t* sure_idx;   // [n_q][top_k]
    int32_t* sure_pool;  // [n_q][pool_blocks]
    uint64_t* cand_idx;  // [grid_tiles * kFullTile]  threshold-bucket composites
    uint64_t* cand_pool; // [grid_tiles * kFullTile / 8]
    QMeta* qmeta;        // [n_q]                      per-query length and tile ranges (prep kernel)
    int32_t* tmap;       // [grid_tiles]               scan tile -> query (-1: unused)
    int32_t* fmap;       // [grid_ftiles]              filter tile -> query (-1: unused)
};

__device__ __forceinline__ uint32_t score_key(float s) {
    s = s + 0.0f;  // -0 -> +0 so both zeros share one key
    uint32_t b = __float_as_uint(s);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// LDS writes of this wave visible to its own later LDS reads (a wave-private buffer).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
    return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - pos);
}

__device__ __forceinline__ uint32_t composite_pos(uint64_t c) {
    return 0xffffffffu - (uint32_t)(c & 0xffffffffu);
}

__device__ __forceinline__ int pow2_ceil(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Valid length of query i: kv_len clamped to [0, max_len] and to the rows after kv_row0.
__device__ __forceinline__ int32_t eff_len_of(int64_t n, int64_t r0, int32_t max_len, int64_t cache_rows) {
    if (n < 0) n = 0;
    if (n > max_len) n = max_len;
    if (r0 < 0 || r0 > cache_rows) return 0;
    if (n > cache_rows - r0) n = cache_rows - r0;
    return (int32_t)n;
}

__device__ __forceinline__ int32_t eff_len(const int32_t* kv_len, const int64_t* kv_row0, int i,
                                           int32_t max_len, int64_t cache_rows) {
    return eff_len_of(kv_len[i], kv_row0[i], max_len, cache_rows);
}

// Inclusive prefix sum across a wave64 with DPP moves (no LDS round trips): Hillis-Steele
// within each 16-lane row (row_shr 1, 2, 4, 8), then row 0's total into row 1 and row 2's
// into row 3 (row_bcast:15), then the total of rows 0-1 into rows 2-3 (row_bcast:31).  Lanes
// without a source add the `old` operand, 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Block-wide exclusive scan of one int per thread (blockDim.x == NT).  `sh` holds NT/64 ints.
// TAIL_SYNC = false leaves out the closing barrier: the caller must pass a barrier before
// anything writes `sh` again.
template <int NT, bool TAIL_SYNC = true>
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int x = wave_inclusive_scan(v);
    if (lane == kWave - 1) sh[wid] = x;
    __syncthreads();
    int wbase = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        int s = sh[w];
        if (w < wid) wbase += s;
        tot += s;
    }
    if (TAIL_SYNC) __syncthreads();
    total = tot;
    return wbase + x - v;
}

// Search a 2048-bin histogram (counts of the top key digit) from the top for the bucket
// holding the k-th largest element.  NT threads (a divisor of 2048).  Result in *out (shared).
// hist_load reads thread t's bins (h[j] is bin kHistBins - 1 - (kHistBins / NT * t + j)) and
// find_threshold_regs searches them, so a caller can issue other loads in between.
template <int NT>
__device__ inline void hist_load(const uint32_t* hist, uint32_t (&h)[kHistBins / NT]) {
    constexpr int BPT = kHistBins / NT;
#pragma unroll
    for (int j = 0; j < BPT; ++j) h[j] = hist[kHistBins - 1 - (BPT * (int)threadIdx.x + j)];
}

template <int NT>
__device__ inline void find_threshold_regs(const uint32_t (&h)[kHistBins / NT], int k, int* sh_scan, Thresh* out) {
    constexpr int BPT = kHistBins / NT;  // bins per thread, highest bins to thread 0
    const int t = threadIdx.x;
    int local = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) local += (int)h[j];
    int total;
    // no closing barrier: the barrier below separates these reads of sh_scan from later writes
    int above = block_exclusive_scan<NT, false>(local, sh_scan, total);
    if (total > k) {  // uniform: exactly one thread holds the crossing bin
        int a = above;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            int c = (int)h[j];
            if (a < k && a + c >= k) {
                out->digit = kHistBins - 1 - (BPT * t + j);
                out->above = a;
                out->in_bucket = c;
                out->total = total;
            }
            a += c;
        }
    } else if (t == 0) {
        out->digit = -1;
        out->above = total;
        out->in_bucket = 0;
        out->total = total;
    }
    __syncthreads();
}

template <int NT>
__device__ inline void find_threshold(const uint32_t* hist, int k, int* sh_scan, Thresh* out) {
    uint32_t h[kHistBins / NT];
    hist_load<NT>(hist, h);
    find_threshold_regs<NT>(h, k, sh_scan, out);
}

__device__ inline void find_threshold_256(const uint32_t* hist, int k, int* sh_scan, Thresh* out) {
    find_threshold<256>(hist, k, sh_scan, out);
}

// Among m <= kSortCap candidate composites in LDS (all sharing the 11-bit key prefix d1),
// find the need-th largest (1 <= need <= m) with radix passes over LDS.  NT threads.
// Returns the threshold: exactly `need` candidates are >= it.
struct RadixShared {
    uint32_t hist[kHistBins];
    int scan[16];
    int digit, above, inb;
    uint32_t low_or;  // nonzero: some key of the bucket has a bit below the current digit
};

// Key-only threshold among m composites in LDS whose keys all lie in first-digit bucket d1:
// the need-th largest KEY, by at most two more radix passes (the key's remaining 21 bits).
// take_eq < 0: every composite with key >= t is selected (exactly `need` of them).  Otherwise
// the key t itself is the threshold: keys above t are selected, and of the n_tie composites
// with key == t the take_eq lowest positions (the caller orders those few ties itself).
struct KeyThr {
    uint32_t t;
    int take_eq;
    int n_tie;
};

template <int NT>
__device__ KeyThr lds_key_threshold(const uint64_t* c, int m, int need, int d1, RadixShared& R) {
    constexpr int BPT = kHistBins / NT;
    const int t = threadIdx.x;
    uint32_t prefix = (uint32_t)d1;
    int pbits = kHistBits;
    int matching = m;
    bool low_zero = false;  // every key of the bucket has zeros below the digit just taken
    while (pbits < 32 && matching > need && !low_zero) {
        const int w = (32 - pbits) >= kHistBits ? kHistBits : (32 - pbits);
        const int shift = 32 - pbits - w;
        for (int b = t; b < kHistBins; b += NT) R.hist[b] = 0u;
        if (t == 0) R.low_or = 0u;
        __syncthreads();
        uint32_t low = 0u;
        for (int e = t; e < m; e += NT) {
            const uint32_t key = (uint32_t)(c[e] >> 32);
            if ((key >> (32 - pbits)) == prefix) {
                atomicAdd(&R.hist[(key >> shift) & ((1u << w) - 1)], 1u);
                low |= key & ((1u << shift) - 1u);
            }
        }
        if (__ballot(low != 0u) != 0ull && (t & (kWave - 1)) == 0) R.low_or = 1u;  // (one flag store per wave)
        __syncthreads();
        // when no key of the bucket has a bit below this digit, every key of the sub-bucket the
        // digit selects is the same key: a further pass could not split it (the ties at that
        // key are ordered by position, as after a pass over all 32 bits)
        low_zero = R.low_or == 0u;
        const int nb = 1 << w;
        uint32_t h[BPT];
        int local = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = nb - 1 - (BPT * t + j);
            h[j] = b >= 0 ? R.hist[b] : 0u;
            local += (int)h[j];
        }
        int tot;
        int a = block_exclusive_scan<NT>(local, R.scan, tot);
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int cnt = (int)h[j];
            if (a < need && a + cnt >= need) {
                R.digit = nb - 1 - (BPT * t + j);
                R.above = a;
                R.inb = cnt;
            }
            a += cnt;
        }
        __syncthreads();
        prefix = (prefix << w) | (uint32_t)R.digit;
        pbits += w;
        need -= R.above;
        matching = R.inb;
        __syncthreads();
    }
    KeyThr r;
    if (matching > need) {  // ties at the threshold key (all 32 bits fixed, or the bits left are 0)
        r.t = prefix << (32 - pbits);
        r.take_eq = need;
        r.n_tie = matching;
    } else {
        r.t = prefix << (32 - pbits);
        r.take_eq = -1;
        r.n_tie = 0;
    }
    return r;
}

template <int NT>
__device__ uint64_t lds_radix_threshold(const uint64_t* c, int m, int need, int d1, RadixShared& R) {
    constexpr int BPT = kHistBins / NT;
    const int t = threadIdx.x;
    uint64_t prefix = (uint64_t)(uint32_t)d1;
    int pbits = kHistBits;
    int matching = m;
    while (pbits < 64 && matching > need) {
        const int w = (64 - pbits) >= kHistBits ? kHistBits : (64 - pbits);
        const int shift = 64 - pbits - w;
        for (int b = t; b < kHistBins; b += NT) R.hist[b] = 0u;
        __syncthreads();
        for (int e = t; e < m; e += NT) {
            const uint64_t v = c[e];
            if ((v >> (64 - pbits)) == prefix) atomicAdd(&R.hist[(v >> shift) & ((1u << w) - 1)], 1u);
        }
        __syncthreads();
        const int nb = 1 << w;
        uint32_t h[BPT];
        int local = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = nb - 1 - (BPT * t + j);
            h[j] = b >= 0 ? R.hist[b] : 0u;
            local += (int)h[j];
        }
        int tot;
        int a = block_exclusive_scan<NT>(local, R.scan, tot);
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int cnt = (int)h[j];
            if (a < need && a + cnt >= need) {
                R.digit = nb - 1 - (BPT * t + j);
                R.above = a;
                R.inb = cnt;
            }
            a += cnt;
        }
        __syncthreads();
        prefix = (prefix << w) | (uint64_t)R.digit;
        pbits += w;
        need -= R.above;
        matching = R.inb;
        __syncthreads();
    }
    // every composite with this prefix (and `matching == need` of them remain) is selected
    return pbits >= 64 ? prefix : (prefix << (64 - pbits));
}

// Ascending output of `total` distinct values sel[0..total) (LDS) to out[0..k), -1 padded,
// without a sort network: one counting pass over kAscB buckets of the values' range
// [vmin, vmax] (bucket = (v - vmin) >> shift), an exclusive scan of the counts, a scatter into
// bucket order, then each value's place inside its bucket by counting the bucket's smaller
// values.  Distinct values keep a bucket of width 2^shift at <= 2^shift values, so the last
// step costs at most total * 2^shift comparisons (2^shift = 512 for a 2^20 range).
// scratch: >= 2 * kAscB + total words of LDS; sh_scan: NT / 64 ints; sh_mm: 2 words.
constexpr int kAscB = 2048;

template <int NT>
__device__ void bucket_write_ascending(const uint32_t* sel, int total, int k, int32_t* out, uint32_t* scratch,
                                       int* sh_scan, uint32_t* sh_mm) {
    static_assert(kAscB % NT == 0, "buckets per thread");
    constexpr int BPT = kAscB / NT;
    const int t = threadIdx.x;
    uint32_t* cnt = scratch;              // counts, then bucket starts
    uint32_t* fill = scratch + kAscB;     // values placed per bucket
    uint32_t* grp = scratch + 2 * kAscB;  // the values grouped by bucket
    if (t == 0) {
        sh_mm[0] = 0xffffffffu;
        sh_mm[1] = 0u;
    }
    for (int b = t; b < kAscB; b += NT) {
        cnt[b] = 0u;
        fill[b] = 0u;
    }
    __syncthreads();
    uint32_t lo = 0xffffffffu, hi = 0u;
    for (int j = t; j < total; j += NT) {
        lo = min(lo, sel[j]);
        hi = max(hi, sel[j]);
    }
    // wave reduction first: a thousand LDS atomics on one address serialise
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, kWave));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, kWave));
    }
    if ((t & (kWave - 1)) == 0 && lo != 0xffffffffu) {
        atomicMin(&sh_mm[0], lo);
        atomicMax(&sh_mm[1], hi);
    }
    __syncthreads();
    const uint32_t vmin = sh_mm[0];
    const uint32_t range = total > 0 ? sh_mm[1] - vmin : 0u;
    int shift = 0;
    while ((range >> shift) >= (uint32_t)kAscB) ++shift;
    for (int j = t; j < total; j += NT) atomicAdd(&cnt[(sel[j] - vmin) >> shift], 1u);
    __syncthreads();
    uint32_t c[BPT];
    int run = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        c[b] = cnt[BPT * t + b];
        run += (int)c[b];
    }
    int tot;
    int base = block_exclusive_scan<NT>(run, sh_scan, tot);
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
        cnt[BPT * t + b] = (uint32_t)base;
        base += (int)c[b];
    }
    __syncthreads();
    for (int j = t; j < total; j += NT) {
        const uint32_t v = sel[j];
        const uint32_t b = (v - vmin) >> shift;
        grp[cnt[b] + atomicAdd(&fill[b], 1u)] = v;
    }
    __syncthreads();
    for (int j = t; j < total; j += NT) {
        const uint32_t v = grp[j];
        const uint32_t b = (v - vmin) >> shift;
        const int s0 = (int)cnt[b], s1 = s0 + (int)fill[b];
        int rank = 0;
        for (int e = s0; e < s1; ++e) rank += grp[e] < v ? 1 : 0;
        out[s0 + rank] = (int32_t)v;
    }
    for (int j = total + t; j < k; j += NT) out[j] = -1;
}

// Bitonic sort of n (power of two, <= kSortCap) 64-bit values in LDS, descending.
template <int NT>
__device__ inline void bitonic_desc_u64(uint64_t* a, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (n >> 1); t += NT) {
                int lo = 2 * t - (t & (stride - 1));
                int hi = lo + stride;
                bool desc = ((lo & size) == 0);
                uint64_t x = a[lo], y = a[hi];
                if ((x < y) == desc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

// LDS working set of one workgroup-level selection (CAP: candidates sorted in LDS, a power of 2).
template <int CAP>
struct SelectSharedT {
    uint64_t buf[CAP];          // candidate composites, then reused for the output positions
    uint32_t hist[kHistBins];
    int scan[16];
    int cnt;
    int digit;
    int above;
    int inb;
};
using SelectShared = SelectSharedT<kSortCap>;

// The need-th largest of `count` candidate composites (src(e), e in [0, count)) whose keys all
// start with the 11-bit digit `d1`, for candidate sets of any size: 11-bit radix passes over
// the (global) list narrow the set until it fits in LDS, where it is sorted.  NT threads.
// Returns the threshold composite (exactly `need` candidates are >= it), ~0 if need <= 0.
template <int NT, class Src, int CAP>
__device__ uint64_t wg_threshold(const Src& src, int count, int need, int d1, SelectSharedT<CAP>& S) {
    const int t = threadIdx.x;
    constexpr int BPT = kHistBins / NT;
    uint64_t thr = ~0ull;
    if (need <= 0 || count <= 0) return thr;
    uint64_t prefix = (uint64_t)(uint32_t)d1;
    int pbits = kHistBits;
    int matching = count;
    while (matching > CAP && pbits < 64) {
        const int w = (64 - pbits) >= kHistBits ? kHistBits : (64 - pbits);
        const int shift = 64 - pbits - w;
        for (int b = t; b < kHistBins; b += NT) S.hist[b] = 0;
        __syncthreads();
        for (int e0 = 0; e0 < count; e0 += 4 * NT) {
            uint64_t c[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * NT + t;
                c[u] = e < count ? src(e) : 0ull;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * NT + t;
                if (e < count && (c[u] >> (64 - pbits)) == prefix)
                    atomicAdd(&S.hist[(c[u] >> shift) & ((1u << w) - 1)], 1u);
            }
        }
        __syncthreads();
        const int nb = 1 << w;
        uint32_t h[BPT];
        int local = 0;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int b = nb - 1 - (BPT * t + j);
            h[j] = b >= 0 ? S.hist[b] : 0u;
            local += (int)h[j];
        }
        int tot;
        int a = block_exclusive_scan<NT>(local, S.scan, tot);
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int cnt = (int)h[j];
            if (a < need && a + cnt >= need) {
                S.digit = nb - 1 - (BPT * t + j);
                S.above = a;
                S.inb = cnt;
            }
            a += cnt;
        }
        __syncthreads();
        prefix = (prefix << w) | (uint64_t)S.digit;
        pbits += w;
        need -= S.above;
        matching = S.inb;
        __syncthreads();
    }
    if (pbits >= 64) return prefix;  // fully resolved (composites are unique)
    if (t == 0) S.cnt = 0;
    __syncthreads();
    for (int e0 = 0; e0 < count; e0 += 4 * NT) {
        uint64_t c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * NT + t;
            c[u] = e < count ? src(e) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int e = e0 + u * NT + t;
            if (e < count && (c[u] >> (64 - pbits)) == prefix) S.buf[atomicAdd(&S.cnt, 1)] = c[u];
        }
    }
    __syncthreads();
    const int m = S.cnt;
    const int p2 = pow2_ceil(m);
    for (int j = m + t; j < p2; j += NT) S.buf[j] = 0ull;
    __syncthreads();
    bitonic_desc_u64<NT>(S.buf, p2);
    thr = S.buf[need - 1];
    __syncthreads();
    return thr;
}

}  // namespace csa2
