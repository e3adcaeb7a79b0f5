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
constexpr int kSortCap = 4096;                // largest candidate set sorted in LDS
constexpr int kMaxSelect = 4096;

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

// Result of the first-digit threshold search for one query and one selection.
struct Thresh {
    int32_t digit;      // bucket holding the K-th largest key; -1: everything is selected
    int32_t above;      // elements in buckets above `digit`
    int32_t in_bucket;  // elements in bucket `digit`
    int32_t total;      // valid elements
};

__device__ __forceinline__ uint32_t score_key(float s) {
    s = s + 0.0f;  // -0 -> +0 so both zeros share one key
    uint32_t b = __float_as_uint(s);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t pos) {
    return ((uint64_t)key << 32) | (uint64_t)(0xffffffffu - pos);
}

__device__ __forceinline__ uint32_t composite_pos(uint64_t c) {
    return 0xffffffffu - (uint32_t)(c & 0xffffffffu);
}

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Valid length of query i: kv_len clamped to [0, max_len] and to the rows after kv_row0.
__device__ __forceinline__ int32_t eff_len(const int32_t* kv_len, const int64_t* kv_row0, int i,
                                           int32_t max_len, int64_t cache_rows) {
    int64_t n = kv_len[i];
    int64_t r0 = kv_row0[i];
    if (n < 0) n = 0;
    if (n > max_len) n = max_len;
    if (r0 < 0 || r0 > cache_rows) return 0;
    if (n > cache_rows - r0) n = cache_rows - r0;
    return (int32_t)n;
}

// Block-wide exclusive scan of one int per thread (blockDim.x == NT).  `sh` holds NT/64 ints.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh, int& total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    int x = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int y = __shfl_up(x, o, kWave);
        if (lane >= o) x += y;
    }
    if (lane == kWave - 1) sh[wid] = x;
    __syncthreads();
    int wbase = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        int s = sh[w];
        if (w < wid) wbase += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return wbase + x - v;
}

// Ragged tile map: query i owns T_i = max(1, ceil(n_i / CH)) consecutive tiles of the grid,
// clamped so that the whole map fits `grid_tiles` (every query keeps at least one tile).
// Every workgroup derives the same map; this one returns the query that owns tile `tile`.
struct TileInfo {
    int32_t q;       // query index, -1 if the tile is unused
    int32_t chunk;   // tile index within the query
    int32_t start;   // first tile of the query
    int32_t ntiles;  // tiles of the query
    int32_t n;       // clamped visible length
};

template <int NT>
__device__ TileInfo tile_lookup(const int32_t* kv_len, const int64_t* kv_row0, int n_q, int32_t max_len,
                                int64_t cache_rows, int ch, int grid_tiles, int tile, int* sh_scan,
                                TileInfo* sh_out) {
    const int extra_cap = grid_tiles - n_q;  // tiles beyond one per query
    if (threadIdx.x == 0) sh_out->q = -1;
    int run = 0;  // raw prefix of extra tiles before this chunk of queries
    for (int base = 0; base < n_q; base += NT) {
        int i = base + (int)threadIdx.x;
        int n = 0, x = 0;
        if (i < n_q) {
            n = eff_len(kv_len, kv_row0, i, max_len, cache_rows);
            int t = (int)(((int64_t)n + ch - 1) / ch);
            x = t > 1 ? t - 1 : 0;
        }
        int tot;
        int ex = block_exclusive_scan<NT>(x, sh_scan, tot);
        if (i < n_q) {
            int p0 = min(extra_cap, run + ex);
            int p1 = min(extra_cap, run + ex + x);
            int start = i + p0;
            int nt = 1 + (p1 - p0);
            if (tile >= start && tile < start + nt) {
                TileInfo ti;
                ti.q = i;
                ti.chunk = tile - start;
                ti.start = start;
                ti.ntiles = nt;
                ti.n = min(n, nt * ch);
                *sh_out = ti;
            }
        }
        run += tot;
        if (run > extra_cap) run = extra_cap + 1;  // saturate (keeps ints small)
    }
    __syncthreads();
    TileInfo r = *sh_out;
    __syncthreads();
    return r;
}

// Search a 2048-bin histogram (global, counts of the top key digit) from the top for the
// bucket holding the k-th largest element.  256 threads.  Result in *out (shared).
__device__ inline void find_threshold_256(const uint32_t* hist, int k, int* sh_scan, Thresh* out) {
    const int t = threadIdx.x;
    // thread t owns bins [2048 - 8(t+1), 2048 - 8t): thread 0 holds the highest bins
    uint32_t h[8];
    int local = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        h[j] = hist[kHistBins - 1 - (8 * t + j)];
        local += (int)h[j];
    }
    int total;
    int above = block_exclusive_scan<256>(local, sh_scan, total);
    if (t == 0) {
        out->digit = -1;
        out->above = total;
        out->in_bucket = 0;
        out->total = total;
    }
    __syncthreads();
    if (total > k) {
        int a = above;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int c = (int)h[j];
            if (a < k && a + c >= k) {
                out->digit = kHistBins - 1 - (8 * t + j);
                out->above = a;
                out->in_bucket = c;
            }
            a += c;
        }
    }
    __syncthreads();
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

// Bitonic sort of n (power of two) 32-bit values in LDS, ascending.
template <int NT>
__device__ inline void bitonic_asc_u32(uint32_t* a, int n) {
    for (int size = 2; size <= n; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = threadIdx.x; t < (n >> 1); t += NT) {
                int lo = 2 * t - (t & (stride - 1));
                int hi = lo + stride;
                bool asc = ((lo & size) == 0);
                uint32_t x = a[lo], y = a[hi];
                if ((x > y) == asc) {
                    a[lo] = y;
                    a[hi] = x;
                }
            }
            __syncthreads();
        }
    }
}

__device__ __forceinline__ int pow2_ceil(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// LDS working set of one workgroup-level selection.
struct SelectShared {
    uint64_t buf[kSortCap];     // candidate composites, then reused for the output positions
    uint32_t hist[kHistBins];
    int scan[8];
    int cnt;
    int digit;
    int above;
    int inb;
};

// Select, with one 256-thread workgroup, the `need` largest composites among `count`
// candidates whose keys all start with the 11-bit digit `d1`, then write the union of
// those positions and `n_sure` positions already chosen (sure[]) to out[0..k) in
// ascending order, -1 padded.
//   elem(e) -> (key, pos) of candidate e (e in [0, count)).
template <class Elem>
__device__ void wg_select_write(const Elem& elem, int count, int need, int d1, const int32_t* sure, int n_sure,
                                int k, int32_t* out, SelectShared& S) {
    const int t = threadIdx.x;
    constexpr int NT = 256;
    uint64_t thr = ~0ull;  // composites >= thr are selected
    if (need > 0 && count > 0) {
        uint64_t prefix = (uint64_t)(uint32_t)d1;
        int pbits = kHistBits;
        int matching = count;
        // radix passes until the matching set fits in LDS
        while (matching > kSortCap && pbits < 64) {
            int w = (64 - pbits) >= kHistBits ? kHistBits : (64 - pbits);
            int shift = 64 - pbits - w;
            for (int b = t; b < kHistBins; b += NT) S.hist[b] = 0;
            __syncthreads();
            for (int e = t; e < count; e += NT) {
                uint32_t key, pos;
                elem(e, key, pos);
                uint64_t c = composite(key, pos);
                if ((c >> (64 - pbits)) == prefix) atomicAdd(&S.hist[(c >> shift) & ((1u << w) - 1)], 1u);
            }
            __syncthreads();
            // top-down search over the (up to) 2048 bins; thread t owns 8 bins
            int nb = 1 << w;
            uint32_t h[8];
            int local = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int b = nb - 1 - (8 * t + j);
                h[j] = b >= 0 ? S.hist[b] : 0u;
                local += (int)h[j];
            }
            int tot;
            int a = block_exclusive_scan<NT>(local, S.scan, tot);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                int c = (int)h[j];
                if (a < need && a + c >= need) {
                    S.digit = nb - 1 - (8 * t + j);
                    S.above = a;
                    S.inb = c;
                }
                a += c;
            }
            __syncthreads();
            prefix = (prefix << w) | (uint64_t)S.digit;
            pbits += w;
            need -= S.above;
            matching = S.inb;
            __syncthreads();
        }
        if (pbits >= 64) {
            thr = prefix;  // fully resolved (composites are unique)
        } else {
            // gather the matching composites and sort them
            if (t == 0) S.cnt = 0;
            __syncthreads();
            for (int e = t; e < count; e += NT) {
                uint32_t key, pos;
                elem(e, key, pos);
                uint64_t c = composite(key, pos);
                if ((c >> (64 - pbits)) == prefix) {
                    int slot = atomicAdd(&S.cnt, 1);
                    S.buf[slot] = c;
                }
            }
            __syncthreads();
            int m = S.cnt;
            int p2 = pow2_ceil(m);
            for (int j = m + t; j < p2; j += NT) S.buf[j] = 0ull;
            __syncthreads();
            bitonic_desc_u64<NT>(S.buf, p2);
            thr = S.buf[need - 1];
            __syncthreads();
        }
    }
    // output = sure positions + candidates with composite >= thr, sorted ascending
    uint32_t* o = reinterpret_cast<uint32_t*>(S.buf);
    if (t == 0) S.cnt = 0;
    __syncthreads();
    for (int j = t; j < n_sure; j += NT) o[atomicAdd(&S.cnt, 1)] = (uint32_t)sure[j];
    if (thr != ~0ull) {
        for (int e = t; e < count; e += NT) {
            uint32_t key, pos;
            elem(e, key, pos);
            if (composite(key, pos) >= thr) o[atomicAdd(&S.cnt, 1)] = pos;
        }
    }
    __syncthreads();
    int m = S.cnt;
    int p2 = pow2_ceil(m > 1 ? m : 1);
    for (int j = m + t; j < p2; j += NT) o[j] = 0xffffffffu;
    __syncthreads();
    bitonic_asc_u32<NT>(o, p2);
    for (int j = t; j < k; j += NT) out[j] = j < m ? (int32_t)o[j] : -1;
    __syncthreads();
}

}  // namespace csa2
