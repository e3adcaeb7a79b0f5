// Reindex-mode selection of one query (one workgroup of NT threads; EPT pool elements per
// thread).
//
// Article "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per Token", section
// IX: a Reindex layer takes its own Top-K inside the shared pool.  The pool is ascending, so
// element order is position order: the K-th largest key T comes from the first-digit
// histogram the scoring kernel built plus at most two radix passes over the bucket's keys
// (in registers), and one packed (greater-than-T, equal-to-T) block scan ranks the
// ties at T and places every selected element in ascending position order.
#pragma once

#include "csa2_device.hpp"
#include "scan_common.hpp"

namespace csa2 {

// Writes the query's selection to idx_out[i * top_k ..] (entries past the selection: -1).
// Every thread of the workgroup must call it.
template <int NT, int EPT>
__device__ __forceinline__ void reindex_select_query(int i, const int32_t* __restrict__ pool, int pool_blocks,
                                                     int top_k, const IndexWs& ws, int32_t* __restrict__ idx_out,
                                                     uint32_t (*s_hist)[kHistBins], int* s_scan,
                                                     uint32_t* s_or, Thresh* sh_th_p) {
    Thresh& sh_th = *sh_th_p;
    const int t = threadIdx.x;
    const int n_elem = pool_blocks * 8;
    const int e0 = t * EPT;
    const int32_t* qpool = pool + (int64_t)i * pool_blocks;
    const uint32_t* keys = ws.keys + (int64_t)i * n_elem;
    uint32_t* gh = ws.hist + (int64_t)i * 2 * kHistBins;

    // the first-digit histogram (accumulated by the score kernel) is requested first, so its
    // threshold search runs while the keys are still in flight
    uint32_t h[kHistBins / NT];
    hist_load<NT>(gh, h);
    uint32_t kv[EPT];
    int32_t pb[EPT / 8];  // pool blocks of this thread's elements
    // bounded views: elements past n_elem (a multiple of 8) read as key 0, padding, and are
    // never selected; the loads need no branch, so the histogram's wait leaves them in flight
    const BufRsrc rk = tile_rsrc(keys, n_elem * 4), rp = tile_rsrc(qpool, pool_blocks * 4);
#pragma unroll
    for (int j = 0; j < EPT; j += 8) {
        const uint4 a = buf_ld16(rk, (e0 + j) * 4, 0), b = buf_ld16(rk, (e0 + j) * 4 + 16, 0);
        kv[j] = a.x; kv[j + 1] = a.y; kv[j + 2] = a.z; kv[j + 3] = a.w;
        kv[j + 4] = b.x; kv[j + 5] = b.y; kv[j + 6] = b.z; kv[j + 7] = b.w;
        pb[j >> 3] = (int32_t)buf_ld4(rp, ((e0 + j) >> 3) * 4, 0);
    }
    for (int b = t; b < 2 * kHistBins; b += NT) (&s_hist[0][0])[b] = 0u;
    if (t < 2) s_or[t] = 0u;
    // first digit (the search's barriers also cover the clearing above)
    find_threshold_regs<NT>(h, top_k, s_scan, &sh_th);
    Thresh th = sh_th;
    uint32_t T = 1u;           // selected: key > T, or key == T among the first need_eq of them
    int need_eq = INT32_MAX;   // (keys are >= 1 for every valid element; 0 marks padding)
    if (th.digit >= 0) {
        int need = top_k - th.above;  // 1 <= need <= inb
        int inb = th.in_bucket;
        uint32_t prefix = (uint32_t)th.digit;
        int pbits = kHistBits;
        if (inb > need) {
            // at most two more radix passes (11 and 10 bits) over the bucket's keys, straight
            // from the registers (a pass costs EPT compares per thread; no compaction)
            int hb = 0;
            bool low_zero = false;  // every key of the bucket has zeros below the digit just taken
            while (pbits < 32 && inb > need && !low_zero) {
                const int w = min(kHistBits, 32 - pbits);
                const int shift = 32 - pbits - w;
                uint32_t low = 0u;
#pragma unroll
                for (int j = 0; j < EPT; ++j)
                    if (kv[j] != 0u && (kv[j] >> (32 - pbits)) == prefix) {
                        atomicAdd(&s_hist[hb][(kv[j] >> shift) & ((1u << w) - 1u)], 1u);
                        low |= kv[j] & ((1u << shift) - 1u);
                    }
                // only whether any key has such a bit matters: one flag store per wave (an atomic OR
                // per holding thread serialised on one LDS word)
                if (__ballot(low != 0u) != 0ull && (t & (kWave - 1)) == 0) s_or[hb] = 1u;
                __syncthreads();
                // no key of the bucket has a bit below this digit: every key of the sub-bucket
                // the digit selects equals T, so a further pass could not split it
                low_zero = s_or[hb] == 0u;
                find_threshold<NT>(s_hist[hb], need, s_scan, &sh_th);
                th = sh_th;  // inb > need, so a digit is found
                prefix = (prefix << w) | (uint32_t)th.digit;
                need -= th.above;
                inb = th.in_bucket;
                pbits += w;
                hb ^= 1;     // the other histogram is still clear
            }
        }
        T = prefix << (32 - pbits);  // lowest key with the final prefix
        need_eq = inb == need ? INT32_MAX : need;  // the whole bucket, or `need` keys equal to T
    }
    // one scan of (keys > T, keys == T) counts ranks the ties at T in element order and
    // places every selected element (keys above T number < top_k <= 4096, ties <= 32768:
    // packed 16 + 16 bits)
    int n_gt = 0, n_eq = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (kv[j] != 0u) {
            n_gt += kv[j] > T ? 1 : 0;
            n_eq += kv[j] == T ? 1 : 0;
        }
    }
    int tot_pk;
    const uint32_t pk = (uint32_t)block_exclusive_scan<NT>((int)(((uint32_t)n_gt << 16) | (uint32_t)n_eq),
                                                              s_scan, tot_pk);
    int eq_rank = (int)(pk & 0xffffu);
    int off = (int)(pk >> 16) + min(eq_rank, need_eq);
    const int total = (int)((uint32_t)tot_pk >> 16) + min((int)((uint32_t)tot_pk & 0xffffu), need_eq);
    int32_t* out = idx_out + (int64_t)i * top_k;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        if (kv[j] != 0u) {
            bool sel = kv[j] > T;
            if (kv[j] == T) sel = eq_rank++ < need_eq;
            if (sel) {
                const int32_t v = pb[j >> 3] * 8 + (j & 7);
                out[off] = v;
                ++off;
            }
        }
    }
    for (int j = total + t; j < top_k; j += NT) {
        out[j] = -1;
    }
    for (int b = t; b < kHistBins; b += NT) gh[b] = 0u;
}

}  // namespace csa2
