// Host side of the CSA2 C ABI: argument validation (all of it before any HIP call),
// workspace carving, grid sizing and launches.  Declarations and contracts: include/csa2.h.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "csa2.h"
#include "csa2_timing.h"

namespace csa2 {

// ---- mirrored from the kernels (kept in one place here) ----
#ifndef CSA2_SCAN_TILE
#define CSA2_SCAN_TILE 4096
#endif
constexpr int kFullTile = CSA2_SCAN_TILE;  // must match the scan kernel's tile
constexpr int kFilterTile = 8192;
constexpr int kHistBins = 2048;
constexpr size_t kAlign = 256;

struct Thresh {
    int32_t digit, above, in_bucket, total;
};

struct QMeta {
    int32_t n, start, ntiles, fstart, fntiles, pad[3];
};

struct IndexWs {
    uint32_t* ctrl;
    uint32_t* hist;
    Thresh* meta;
    uint32_t* keys;
    uint32_t* bkeys;
    int32_t* sure_idx;
    int32_t* sure_pool;
    uint64_t* cand_idx;
    uint64_t* cand_pool;
    QMeta* qmeta;
    int32_t* tmap;
    int32_t* fmap;
};

hipError_t launch_fp4_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream);
hipError_t launch_index_full(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                             const int64_t* kv_row0, const int32_t* kv_len, int n_q, int32_t max_len,
                             int64_t cache_rows, int n_heads, int grid_tiles, int grid_ftiles, int top_k,
                             int pool_blocks, int prefill, const IndexWs& ws, int32_t* idx_out, int32_t* pool_out,
                             int phase, hipStream_t stream, hipEvent_t ev_start = nullptr,
                             hipEvent_t ev_stop = nullptr);
hipError_t launch_index_reindex(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                                const int64_t* kv_row0, const int32_t* kv_len, int n_q, int32_t max_len,
                                int64_t cache_rows, int n_heads, const int32_t* pool, int pool_blocks, int top_k,
                                const IndexWs& ws, int32_t* idx_out, int select, hipStream_t stream,
                                hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr,
                                hipEvent_t ev_sel_start = nullptr, hipEvent_t ev_sel_stop = nullptr);
hipError_t launch_token_append(const uint16_t* x, const uint16_t* k_new, int64_t n_tok, const int64_t* dst_rows,
                               uint8_t* codes, uint8_t* scales, void* k_idx, uint8_t* k_scales, int64_t cap_rows,
                               hipStream_t stream);
hipError_t launch_row_copy(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint16_t* out, int64_t cap_rows, hipStream_t stream);
hipError_t launch_mx_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                          uint8_t* codes, uint8_t* scales, int64_t cap_rows, hipStream_t stream);
hipError_t launch_fp8_pack(const uint16_t* x, int64_t n_tok, int dim, const int64_t* dst_rows, int64_t row0,
                           uint8_t* out, int64_t cap_rows, hipStream_t stream);
hipError_t launch_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const int64_t* kv_row0,
                         const int32_t* kv_len, int n_q, int32_t max_len, int64_t cache_rows, const int32_t* idx,
                         int top_k, const void* swa, int window_fp8, const int64_t* swa_row0, int swa_cap,
                         int64_t swa_rows, int window, const int64_t* replay, int n_heads, float softmax_scale,
                         float* out, const uint16_t* win_new, float* part, uint32_t* ctrl, hipStream_t stream,
                         hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);
int attend_dec_parts(int top_k, int window);
int attend_split_max_queries();
size_t attend_dec_part_bytes();
hipError_t launch_zero(void* ws, size_t bytes, hipStream_t stream);
int stream_read_groups();
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int groups, hipStream_t stream,
                              hipEvent_t ev_start, hipEvent_t ev_stop);

namespace {

constexpr int64_t kMaxTiles = (int64_t)1 << 30;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Common prefix of every workspace: counters, then the two 2048-bin histograms per query.
size_t ctrl_bytes(int n_q) { return CSA2_CTRL_BYTES(n_q); }
size_t hist_bytes(int n_q) { return align_up((size_t)n_q * 2 * kHistBins * 4); }

int64_t full_grid_tiles(int n_q, int64_t total_len_ub, int32_t max_len_ub, int tile = kFullTile) {
    const int64_t per_q = ((int64_t)max_len_ub + tile - 1) / tile;
    int64_t a = (total_len_ub + tile - 1) / tile + n_q;
    int64_t b = (int64_t)n_q * (per_q > 1 ? per_q : 1);
    return a < b ? a : b;
}

struct Carve {
    char* base;
    size_t off = 0;
    template <class T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base ? base + off : nullptr);
        off += align_up(count * sizeof(T));
        return p;
    }
};

IndexWs carve_full(void* ws, int n_q, int64_t tiles, int64_t ftiles, int top_k, int pool_blocks, size_t* used) {
    Carve c{static_cast<char*>(ws)};
    IndexWs w{};
    w.ctrl = c.take<uint32_t>(ctrl_bytes(n_q) / 4);
    w.hist = c.take<uint32_t>(hist_bytes(n_q) / 4);
    w.meta = c.take<Thresh>((size_t)n_q * 2);
    w.keys = c.take<uint32_t>((size_t)tiles * kFullTile);
    w.bkeys = c.take<uint32_t>((size_t)tiles * (kFullTile / 8));
    w.sure_idx = c.take<int32_t>((size_t)n_q * top_k);
    w.sure_pool = c.take<int32_t>((size_t)n_q * (pool_blocks > 0 ? pool_blocks : 1));
    w.cand_idx = c.take<uint64_t>((size_t)tiles * kFullTile);
    w.cand_pool = c.take<uint64_t>((size_t)tiles * (kFullTile / 8));
    w.qmeta = c.take<QMeta>((size_t)n_q);
    w.tmap = c.take<int32_t>((size_t)tiles);
    w.fmap = c.take<int32_t>((size_t)ftiles);
    *used = c.off;
    return w;
}

IndexWs carve_reindex(void* ws, int n_q, int top_k, int pool_blocks, size_t* used) {
    Carve c{static_cast<char*>(ws)};
    IndexWs w{};
    w.ctrl = c.take<uint32_t>(ctrl_bytes(n_q) / 4);
    w.hist = c.take<uint32_t>(hist_bytes(n_q) / 4);
    w.meta = c.take<Thresh>((size_t)n_q * 2);
    w.keys = c.take<uint32_t>((size_t)n_q * pool_blocks * 8);
    (void)top_k;
    *used = c.off;
    return w;
}

// Attention workspace (decode calls whose entries are split over several workgroups): the
// common prefix (per-query counters and histograms, so the workspace may be shared with index
// calls of the same n_q), then one partial per (query, workgroup).  Sized 0 when none is needed.
struct AttendWs {
    uint32_t* ctrl;
    float* part;
};

bool attend_split(int n_q) { return n_q <= attend_split_max_queries(); }

AttendWs carve_attend(void* ws, int n_q, int top_k, int window, size_t* used) {
    AttendWs w{nullptr, nullptr};
    const int parts = attend_dec_parts(top_k, window);
    if (!attend_split(n_q) || parts <= 1) {
        *used = 0;
        return w;
    }
    Carve c{static_cast<char*>(ws)};
    w.ctrl = c.take<uint32_t>(ctrl_bytes(n_q) / 4);
    (void)c.take<uint32_t>(hist_bytes(n_q) / 4);  // the histogram prefix every workspace has (left zero)
    w.part = reinterpret_cast<float*>(c.take<uint8_t>((size_t)n_q * parts * attend_dec_part_bytes()));
    *used = c.off;
    return w;
}

int check_seqs(const csa2_seqs& s) {
    if (s.n_q < 0 || s.n_q > CSA2_MAX_QUERIES || s.max_len_ub < 0 || s.total_len_ub < 0 || s.cache_rows < 0)
        return CSA2_ERR_SHAPE;
    if (s.n_q > 0 && (s.kv_row0 == nullptr || s.kv_len == nullptr)) return CSA2_ERR_NULL;
    return CSA2_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH; }

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" {

int fp4_kv_append(const uint16_t* x, int64_t n_tok, int32_t dim, const int64_t* dst_rows, int64_t row0, uint8_t* codes,
                  uint8_t* scales, int64_t cap_rows, void* stream) {
    if (n_tok < 0 || dim <= 0 || dim % 16 != 0 || dim > 1024 || cap_rows < 0) return CSA2_ERR_SHAPE;
    if (n_tok == 0) return CSA2_OK;
    if (x == nullptr || codes == nullptr || scales == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0) return CSA2_ERR_SHAPE;
    if (n_tok > ((int64_t)1 << 40)) return CSA2_ERR_SHAPE;
    if (dst_rows == nullptr && (row0 < 0 || row0 > cap_rows || n_tok > cap_rows - row0)) return CSA2_ERR_CAPACITY;
    return launch_status(launch_fp4_pack(x, n_tok, dim, dst_rows, row0, codes, scales, cap_rows,
                                         static_cast<hipStream_t>(stream)));
}

int fp8_window_append(const uint16_t* x, int64_t n_tok, int32_t dim, const int64_t* dst_rows, int64_t row0,
                      uint8_t* out, int64_t cap_rows, void* stream) {
    if (n_tok < 0 || dim <= 0 || dim % 8 != 0 || dim > 1024 || cap_rows < 0) return CSA2_ERR_SHAPE;
    if (n_tok == 0) return CSA2_OK;
    if (x == nullptr || out == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(out) & 7u) != 0) return CSA2_ERR_SHAPE;
    if (n_tok > ((int64_t)1 << 40)) return CSA2_ERR_SHAPE;
    if (dst_rows == nullptr && (row0 < 0 || row0 > cap_rows || n_tok > cap_rows - row0)) return CSA2_ERR_CAPACITY;
    return launch_status(launch_fp8_pack(x, n_tok, dim, dst_rows, row0, out, cap_rows,
                                         static_cast<hipStream_t>(stream)));
}

size_t csa2_workspace_bytes(int32_t op, int32_t n_q, int64_t total_len_ub, int32_t max_len_ub, int32_t top_k,
                            int32_t pool_blocks) {
    const size_t bad = (size_t)-1;
    if (n_q < 0 || n_q > CSA2_MAX_QUERIES || total_len_ub < 0 || max_len_ub < 0) return bad;
    size_t used = 0;
    switch (op) {
        case CSA2_OP_INDEX_FULL: {
            if (top_k < 1 || top_k > CSA2_MAX_SELECT || pool_blocks < 0 || pool_blocks > CSA2_MAX_SELECT) return bad;
            const int64_t tiles = full_grid_tiles(n_q, total_len_ub, max_len_ub);
            const int64_t ftiles = full_grid_tiles(n_q, total_len_ub, max_len_ub, kFilterTile);
            if (tiles > kMaxTiles) return bad;
            carve_full(nullptr, n_q, tiles, ftiles, top_k, pool_blocks, &used);
            return used;
        }
        case CSA2_OP_INDEX_REINDEX:
            if (top_k < 1 || top_k > CSA2_MAX_SELECT || pool_blocks < 1 || pool_blocks > CSA2_MAX_SELECT) return bad;
            carve_reindex(nullptr, n_q, top_k, pool_blocks, &used);
            return used;
        case CSA2_OP_ATTEND:
            // top_k = selected slots, pool_blocks = window length
            if (top_k < 0 || top_k > CSA2_MAX_SELECT || pool_blocks < 0 || pool_blocks > CSA2_MAX_WINDOW) return bad;
            carve_attend(nullptr, n_q, top_k, pool_blocks, &used);
            return used;
        default:
            return bad;
    }
}

static int index_full_phase(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                            const csa2_seqs& seqs, int32_t n_heads, int32_t top_k, int32_t block,
                            int32_t pool_blocks, int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws,
                            size_t ws_bytes, void* stream, int phase, void* ev_start = nullptr,
                            void* ev_stop = nullptr) {
    int st = check_seqs(seqs);
    if (st) return st;
    if (n_heads < 1 || n_heads > CSA2_MAX_IDX_HEADS || top_k < 1 || top_k > CSA2_MAX_SELECT || pool_blocks < 0 ||
        pool_blocks > CSA2_MAX_SELECT)
        return CSA2_ERR_SHAPE;
    if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
    if (seqs.n_q == 0) return CSA2_OK;
    if (q_idx == nullptr || w == nullptr || k_idx == nullptr || idx_out == nullptr) return CSA2_ERR_NULL;
    if (mx && k_sc == nullptr) return CSA2_ERR_NULL;
    if (pool_blocks > 0 && pool_out == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || (mx && (reinterpret_cast<uintptr_t>(k_sc) & 1u)))
        return CSA2_ERR_SHAPE;
    const int64_t tiles = full_grid_tiles(seqs.n_q, seqs.total_len_ub, seqs.max_len_ub);
    const int64_t ftiles = full_grid_tiles(seqs.n_q, seqs.total_len_ub, seqs.max_len_ub, kFilterTile);
    if (tiles > kMaxTiles) return CSA2_ERR_SHAPE;
    size_t need = 0;
    carve_full(nullptr, seqs.n_q, tiles, ftiles, top_k, pool_blocks, &need);
    if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return CSA2_ERR_WORKSPACE;
    const IndexWs wsp = carve_full(ws, seqs.n_q, tiles, ftiles, top_k, pool_blocks, &need);
    // prefill chunk: the MFMA scoring kernels (shared sequence, at most 4 heads, >= 16 queries,
    // positions below 2^26, which its candidate entries pack into 26 bits)
    // (MXFP4 keys always take the per-query scan)
    const int prefill =
        (!mx && shared_kv != 0 && n_heads <= 4 && seqs.n_q >= 16 && seqs.max_len_ub < (1 << 26)) ? 1 : 0;
    return launch_status(launch_index_full(q_idx, w, k_idx, k_sc, mx, seqs.kv_row0, seqs.kv_len, seqs.n_q,
                                           seqs.max_len_ub, seqs.cache_rows, n_heads, (int)tiles, (int)ftiles, top_k,
                                           pool_blocks, prefill, wsp, idx_out, pool_out, phase,
                                           static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_start),
                                           static_cast<hipEvent_t>(ev_stop)));
}

int csa2_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs, int32_t n_heads,
                    int32_t top_k, int32_t block, int32_t pool_blocks, int32_t shared_kv, int32_t* idx_out,
                    int32_t* pool_out, void* ws, size_t ws_bytes, void* stream) {
    return index_full_phase(q_idx, w, k_idx, nullptr, 0, seqs, n_heads, top_k, block, pool_blocks, shared_kv, idx_out,
                            pool_out, ws, ws_bytes, stream, 7);
}

int csa2_index_full_prep(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                         int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks, int32_t shared_kv,
                         int32_t* idx_out, int32_t* pool_out, void* ws, size_t ws_bytes, void* stream) {
    return index_full_phase(q_idx, w, k_idx, nullptr, 0, seqs, n_heads, top_k, block, pool_blocks, shared_kv, idx_out,
                            pool_out, ws, ws_bytes, stream, 1);
}

int csa2_index_full_scan(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                         int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks, int32_t shared_kv,
                         int32_t* idx_out, int32_t* pool_out, void* ws, size_t ws_bytes, void* stream) {
    return index_full_phase(q_idx, w, k_idx, nullptr, 0, seqs, n_heads, top_k, block, pool_blocks, shared_kv, idx_out,
                            pool_out, ws, ws_bytes, stream, 2);
}

int csa2_index_full_select(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                           int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks, int32_t shared_kv,
                           int32_t* idx_out, int32_t* pool_out, void* ws, size_t ws_bytes, void* stream) {
    return index_full_phase(q_idx, w, k_idx, nullptr, 0, seqs, n_heads, top_k, block, pool_blocks, shared_kv, idx_out,
                            pool_out, ws, ws_bytes, stream, 4);
}

// Checks of a Reindex call (everything but n_q == 0, which the callers handle first).
static int check_reindex(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                         const csa2_seqs& seqs, int32_t n_heads, const int32_t* pool, int32_t pool_blocks,
                         int32_t block, int32_t top_k, int32_t* idx_out, void* ws, size_t ws_bytes) {
    int st = check_seqs(seqs);
    if (st) return st;
    if (n_heads < 1 || n_heads > CSA2_MAX_IDX_HEADS || top_k < 1 || top_k > CSA2_MAX_SELECT || pool_blocks < 1 ||
        pool_blocks > CSA2_MAX_SELECT)
        return CSA2_ERR_SHAPE;
    if (block != CSA2_BLOCK) return CSA2_ERR_UNSUPPORTED;
    if (seqs.n_q == 0) return CSA2_OK;
    if (q_idx == nullptr || w == nullptr || k_idx == nullptr || pool == nullptr || idx_out == nullptr)
        return CSA2_ERR_NULL;
    if (mx && k_sc == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(q_idx) || !aligned16(k_idx) || (mx && (reinterpret_cast<uintptr_t>(k_sc) & 1u)))
        return CSA2_ERR_SHAPE;
    size_t need = 0;
    carve_reindex(nullptr, seqs.n_q, top_k, pool_blocks, &need);
    if (ws == nullptr || ws_bytes < need || !aligned16(ws)) return CSA2_ERR_WORKSPACE;
    return CSA2_OK;
}

static int index_reindex_common(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_sc, int mx,
                                const csa2_seqs& seqs, int32_t n_heads, const int32_t* pool, int32_t pool_blocks,
                                int32_t block, int32_t top_k, int32_t* idx_out, void* ws, size_t ws_bytes,
                                void* stream, void* ev_start = nullptr, void* ev_stop = nullptr,
                                void* ev_sel_start = nullptr, void* ev_sel_stop = nullptr) {
    const int st = check_reindex(q_idx, w, k_idx, k_sc, mx, seqs, n_heads, pool, pool_blocks, block, top_k, idx_out,
                                 ws, ws_bytes);
    if (st || seqs.n_q == 0) return st;
    size_t need = 0;
    const IndexWs wsp = carve_reindex(ws, seqs.n_q, top_k, pool_blocks, &need);
    return launch_status(launch_index_reindex(q_idx, w, k_idx, k_sc, mx, seqs.kv_row0, seqs.kv_len, seqs.n_q,
                                              seqs.max_len_ub, seqs.cache_rows, n_heads, pool, pool_blocks, top_k,
                                              wsp, idx_out, 1, static_cast<hipStream_t>(stream),
                                              static_cast<hipEvent_t>(ev_start), static_cast<hipEvent_t>(ev_stop),
                                              static_cast<hipEvent_t>(ev_sel_start),
                                              static_cast<hipEvent_t>(ev_sel_stop)));
}

int csa2_index_reindex(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs, int32_t n_heads,
                       const int32_t* pool, int32_t pool_blocks, int32_t block, int32_t top_k, int32_t* idx_out,
                       void* ws, size_t ws_bytes, void* stream) {
    return index_reindex_common(q_idx, w, k_idx, nullptr, 0, seqs, n_heads, pool, pool_blocks, block, top_k, idx_out,
                                ws, ws_bytes, stream);
}

int mxfp4_key_append(const uint16_t* x, int64_t n_tok, int32_t dim, const int64_t* dst_rows, int64_t row0,
                     uint8_t* codes, uint8_t* scales, int64_t cap_rows, void* stream) {
    if (n_tok < 0 || dim <= 0 || dim % 32 != 0 || dim > 1024 || cap_rows < 0) return CSA2_ERR_SHAPE;
    if (n_tok == 0) return CSA2_OK;
    if (x == nullptr || codes == nullptr || scales == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes)) return CSA2_ERR_SHAPE;
    if (n_tok > ((int64_t)1 << 40)) return CSA2_ERR_SHAPE;
    if (dst_rows == nullptr && (row0 < 0 || row0 > cap_rows || n_tok > cap_rows - row0)) return CSA2_ERR_CAPACITY;
    return launch_status(launch_mx_pack(x, n_tok, dim, dst_rows, row0, codes, scales, cap_rows,
                                        static_cast<hipStream_t>(stream)));
}

int csa2_index_full_mx(const uint16_t* q_idx, const float* w, const uint8_t* k_codes, const uint8_t* k_scales,
                       csa2_seqs seqs, int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                       int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws, size_t ws_bytes,
                       void* stream) {
    return index_full_phase(q_idx, w, k_codes, k_scales, 1, seqs, n_heads, top_k, block, pool_blocks, shared_kv,
                            idx_out, pool_out, ws, ws_bytes, stream, 7);
}

int csa2_index_full_mx_scan(const uint16_t* q_idx, const float* w, const uint8_t* k_codes, const uint8_t* k_scales,
                            csa2_seqs seqs, int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                            int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws, size_t ws_bytes,
                            void* stream) {
    return index_full_phase(q_idx, w, k_codes, k_scales, 1, seqs, n_heads, top_k, block, pool_blocks, shared_kv,
                            idx_out, pool_out, ws, ws_bytes, stream, 2);
}

// Timed launches record into caller events; they are refused on a stream under graph capture.
static int refuse_capture(void* stream, void* ev_start, void* ev_stop) {
    if (ev_start == nullptr && ev_stop == nullptr) return CSA2_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess) return CSA2_ERR_LAUNCH;
    return cap != hipStreamCaptureStatusNone ? CSA2_ERR_UNSUPPORTED : CSA2_OK;
}

int csa2_index_full_scan_timed(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_scales,
                               csa2_seqs seqs, int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                               int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws, size_t ws_bytes,
                               void* stream, void* start_event, void* stop_event) {
    const int st = refuse_capture(stream, start_event, stop_event);
    if (st) return st;
    return index_full_phase(q_idx, w, k_idx, k_scales, k_scales != nullptr ? 1 : 0, seqs, n_heads, top_k, block,
                            pool_blocks, shared_kv, idx_out, pool_out, ws, ws_bytes, stream, 2, start_event,
                            stop_event);
}

int csa2_index_reindex_timed(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_scales,
                             csa2_seqs seqs, int32_t n_heads, const int32_t* pool, int32_t pool_blocks, int32_t block,
                             int32_t top_k, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream,
                             void* score_start, void* score_stop, void* select_start, void* select_stop) {
    int st = refuse_capture(stream, score_start, score_stop);
    if (st == CSA2_OK) st = refuse_capture(stream, select_start, select_stop);
    if (st) return st;
    return index_reindex_common(q_idx, w, k_idx, k_scales, k_scales != nullptr ? 1 : 0, seqs, n_heads, pool,
                                pool_blocks, block, top_k, idx_out, ws, ws_bytes, stream, score_start, score_stop,
                                select_start, select_stop);
}

int csa2_index_reindex_mx(const uint16_t* q_idx, const float* w, const uint8_t* k_codes, const uint8_t* k_scales,
                          csa2_seqs seqs, int32_t n_heads, const int32_t* pool, int32_t pool_blocks, int32_t block,
                          int32_t top_k, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
    return index_reindex_common(q_idx, w, k_codes, k_scales, 1, seqs, n_heads, pool, pool_blocks, block, top_k,
                                idx_out, ws, ws_bytes, stream);
}

// Checks of an attention call (everything but n_q == 0, which the callers handle first).
static int check_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const csa2_seqs& seqs,
                        const int32_t* idx, int32_t top_k, const void* swa, const int64_t* swa_row0, int32_t swa_cap,
                        int64_t swa_rows, int32_t window, int32_t n_heads, float softmax_scale, const float* out,
                        const uint16_t* win_new) {
    int st = check_seqs(seqs);
    if (st) return st;
    if (top_k < 0 || top_k > CSA2_MAX_SELECT || window < 0 || window > CSA2_MAX_WINDOW || n_heads < 1 ||
        n_heads > CSA2_MAX_Q_HEADS || swa_rows < 0 || swa_rows > INT32_MAX)
        return CSA2_ERR_SHAPE;
    if (window > 0 && (swa_cap < window)) return CSA2_ERR_SHAPE;
    if (top_k + window == 0) return CSA2_ERR_SHAPE;
    if (!(softmax_scale == softmax_scale)) return CSA2_ERR_SHAPE;
    if (seqs.n_q == 0) return CSA2_OK;
    if (q == nullptr || out == nullptr) return CSA2_ERR_NULL;
    if (top_k > 0 && (codes == nullptr || scales == nullptr || idx == nullptr)) return CSA2_ERR_NULL;
    if (window > 0 && (swa == nullptr || swa_row0 == nullptr)) return CSA2_ERR_NULL;
    if (!aligned16(q) || (codes && !aligned16(codes)) || (swa && !aligned16(swa)) ||
        (scales && (reinterpret_cast<uintptr_t>(scales) & 1u)) || (win_new && !aligned16(win_new)))
        return CSA2_ERR_SHAPE;
    return CSA2_OK;
}

static int attend_common(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, const csa2_seqs& seqs,
                         const int32_t* idx, int32_t top_k, const void* swa, int window_fp8, const int64_t* swa_row0,
                         int32_t swa_cap, int64_t swa_rows, int32_t window, const int64_t* replay, int32_t n_heads,
                         float softmax_scale, float* out, const uint16_t* win_new, void* ws, size_t ws_bytes,
                         void* stream, void* ev_start = nullptr, void* ev_stop = nullptr) {
    const int st = check_attend(q, codes, scales, seqs, idx, top_k, swa, swa_row0, swa_cap, swa_rows, window, n_heads,
                                softmax_scale, out, win_new);
    if (st || seqs.n_q == 0) return st;
    size_t need = 0;
    carve_attend(nullptr, seqs.n_q, top_k, window, &need);
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws))) return CSA2_ERR_WORKSPACE;
    const AttendWs aw = carve_attend(ws, seqs.n_q, top_k, window, &need);
    return launch_status(launch_attend(q, codes, scales, seqs.kv_row0, seqs.kv_len, seqs.n_q, seqs.max_len_ub,
                                       seqs.cache_rows, idx, top_k, swa, window_fp8, swa_row0,
                                       window > 0 ? swa_cap : 1, swa_rows, window, replay, n_heads, softmax_scale,
                                       out, window > 0 ? win_new : nullptr, aw.part, aw.ctrl,
                                       static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(ev_start),
                                       static_cast<hipEvent_t>(ev_stop)));
}

// A Reindex layer: csa2_index_reindex's scoring and selection kernels, then csa2_attend's kernel.
static int reindex_attend_common(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_scales,
                                 const csa2_seqs& seqs, int32_t idx_heads, const int32_t* pool, int32_t pool_blocks,
                                 int32_t block, int32_t top_k, int32_t* idx_out, const uint16_t* q,
                                 const uint8_t* codes, const uint8_t* scales, void* swa, int32_t window_fp8,
                                 const int64_t* swa_row0, int32_t swa_cap, int64_t swa_rows, int32_t window,
                                 const int64_t* replay_start, const uint16_t* win_new, int32_t n_heads,
                                 float softmax_scale, float* out, void* ws, size_t ws_bytes, void* att_ws,
                                 size_t att_ws_bytes, void* stream) {
    const int mx = k_scales != nullptr ? 1 : 0;
    if (window_fp8 != 0 && window_fp8 != 1) return CSA2_ERR_SHAPE;
    int st = check_reindex(q_idx, w, k_idx, k_scales, mx, seqs, idx_heads, pool, pool_blocks, block, top_k, idx_out,
                           ws, ws_bytes);
    if (st) return st;
    st = check_attend(q, codes, scales, seqs, idx_out, top_k, swa, swa_row0, swa_cap, swa_rows, window, n_heads,
                      softmax_scale, out, win_new);
    if (st || seqs.n_q == 0) return st;
    size_t need_a = 0;
    carve_attend(nullptr, seqs.n_q, top_k, window, &need_a);
    if (need_a > 0 && (att_ws == nullptr || att_ws_bytes < need_a || !aligned16(att_ws))) return CSA2_ERR_WORKSPACE;
    const AttendWs aw = carve_attend(att_ws, seqs.n_q, top_k, window, &need_a);
    size_t need = 0;
    const IndexWs wsp = carve_reindex(ws, seqs.n_q, top_k, pool_blocks, &need);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_index_reindex(q_idx, w, k_idx, k_scales, mx, seqs.kv_row0, seqs.kv_len, seqs.n_q,
                                        seqs.max_len_ub, seqs.cache_rows, idx_heads, pool, pool_blocks, top_k, wsp,
                                        idx_out, 1, s);
    if (e != hipSuccess) return CSA2_ERR_LAUNCH;
    e = launch_attend(q, codes, scales, seqs.kv_row0, seqs.kv_len, seqs.n_q, seqs.max_len_ub, seqs.cache_rows,
                      idx_out, top_k, swa, window_fp8, swa_row0, window > 0 ? swa_cap : 1, swa_rows, window,
                      replay_start, n_heads, softmax_scale, out, window > 0 ? win_new : nullptr, aw.part, aw.ctrl,
                      s);
    return launch_status(e);
}

int csa2_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, csa2_seqs seqs, const int32_t* idx,
                int32_t top_k, uint16_t* swa, const int64_t* swa_row0, int32_t swa_cap, int64_t swa_rows,
                int32_t window, const uint16_t* win_new, int32_t n_heads, float softmax_scale, float* out, void* ws,
                size_t ws_bytes, void* stream) {
    return attend_common(q, codes, scales, seqs, idx, top_k, swa, 0, swa_row0, swa_cap, swa_rows, window, nullptr,
                         n_heads, softmax_scale, out, win_new, ws, ws_bytes, stream);
}

int csa2_attend_timed(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, csa2_seqs seqs,
                      const int32_t* idx, int32_t top_k, uint16_t* swa, const int64_t* swa_row0, int32_t swa_cap,
                      int64_t swa_rows, int32_t window, const uint16_t* win_new, int32_t n_heads, float softmax_scale,
                      float* out, void* ws, size_t ws_bytes, void* stream, void* start_event, void* stop_event) {
    const int st = refuse_capture(stream, start_event, stop_event);
    if (st) return st;
    return attend_common(q, codes, scales, seqs, idx, top_k, swa, 0, swa_row0, swa_cap, swa_rows, window, nullptr,
                         n_heads, softmax_scale, out, win_new, ws, ws_bytes, stream, start_event, stop_event);
}

int csa2_attend_fp8win(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, csa2_seqs seqs,
                       const int32_t* idx, int32_t top_k, uint8_t* swa, const int64_t* swa_row0, int32_t swa_cap,
                       int64_t swa_rows, int32_t window, const int64_t* replay_start, const uint16_t* win_new,
                       int32_t n_heads, float softmax_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
    return attend_common(q, codes, scales, seqs, idx, top_k, swa, 1, swa_row0, swa_cap, swa_rows, window,
                         replay_start, n_heads, softmax_scale, out, win_new, ws, ws_bytes, stream);
}

int csa2_reindex_attend(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_scales,
                        csa2_seqs seqs, int32_t idx_heads, const int32_t* pool, int32_t pool_blocks, int32_t block,
                        int32_t top_k, int32_t* idx_out, const uint16_t* q, const uint8_t* codes,
                        const uint8_t* scales, void* swa, int32_t window_fp8, const int64_t* swa_row0,
                        int32_t swa_cap, int64_t swa_rows, int32_t window, const int64_t* replay_start,
                        const uint16_t* win_new, int32_t n_heads, float softmax_scale, float* out, void* ws,
                        size_t ws_bytes, void* att_ws, size_t att_ws_bytes, void* stream) {
    return reindex_attend_common(q_idx, w, k_idx, k_scales, seqs, idx_heads, pool, pool_blocks, block, top_k, idx_out,
                                 q, codes, scales, swa, window_fp8, swa_row0, swa_cap, swa_rows, window, replay_start,
                                 win_new, n_heads, softmax_scale, out, ws, ws_bytes, att_ws, att_ws_bytes, stream);
}

int csa2_stream_read_groups(void) { return stream_read_groups(); }

int csa2_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream,
                     void* start_event, void* stop_event) {
    const int st = refuse_capture(stream, start_event, stop_event);
    if (st) return st;
    if (src == nullptr || sink == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(src) || bytes % 16 != 0 || bytes == 0) return CSA2_ERR_SHAPE;
    const int groups = stream_read_groups();
    if (sink_words < (size_t)groups) return CSA2_ERR_SHAPE;
    return launch_status(launch_stream_read(src, bytes, sink, groups, static_cast<hipStream_t>(stream),
                                            static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)));
}

int csa2_token_append(const uint16_t* x, const uint16_t* k_new, int64_t n_tok, const int64_t* dst_rows,
                      uint8_t* codes, uint8_t* scales, void* k_idx, uint8_t* k_scales, int64_t cap_rows,
                      void* stream) {
    if (n_tok < 0 || cap_rows < 0 || n_tok > ((int64_t)1 << 40)) return CSA2_ERR_SHAPE;
    if (n_tok == 0) return CSA2_OK;
    if (x == nullptr || dst_rows == nullptr || codes == nullptr || scales == nullptr) return CSA2_ERR_NULL;
    if (k_new != nullptr && k_idx == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(codes) & 7u) != 0 || (k_new && !aligned16(k_new)) ||
        (k_new && !aligned16(k_idx)))
        return CSA2_ERR_SHAPE;
    return launch_status(launch_token_append(x, k_new, n_tok, dst_rows, codes, scales, k_new ? k_idx : nullptr,
                                             k_scales, cap_rows, static_cast<hipStream_t>(stream)));
}

int csa2_window_append(const uint16_t* x, int64_t n_tok, const int64_t* dst_rows, int64_t row0, void* out,
                       int32_t window_fp8, int64_t cap_rows, void* stream) {
    if (n_tok < 0 || cap_rows < 0 || n_tok > ((int64_t)1 << 40) || (window_fp8 != 0 && window_fp8 != 1))
        return CSA2_ERR_SHAPE;
    if (n_tok == 0) return CSA2_OK;
    if (x == nullptr || out == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(x) || !aligned16(out)) return CSA2_ERR_SHAPE;
    if (dst_rows == nullptr && (row0 < 0 || row0 > cap_rows || n_tok > cap_rows - row0)) return CSA2_ERR_CAPACITY;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (window_fp8)
        return launch_status(launch_fp8_pack(x, n_tok, CSA2_KV_DIM, dst_rows, row0, static_cast<uint8_t*>(out),
                                             cap_rows, s));
    return launch_status(launch_row_copy(x, n_tok, CSA2_KV_DIM, dst_rows, row0, static_cast<uint16_t*>(out), cap_rows,
                                         s));
}

int csa2_workspace_init(void* ws, size_t bytes, void* stream) {
    if (bytes == 0) return CSA2_OK;
    if (ws == nullptr) return CSA2_ERR_NULL;
    if (!aligned16(ws)) return CSA2_ERR_SHAPE;
    return launch_status(launch_zero(ws, bytes, static_cast<hipStream_t>(stream)));
}

const char* csa2_status_string(int status) {
    switch (status) {
        case CSA2_OK: return "ok";
        case CSA2_ERR_NULL: return "a required pointer is NULL";
        case CSA2_ERR_SHAPE: return "a size argument is out of range";
        case CSA2_ERR_UNSUPPORTED: return "size not supported by these kernels";
        case CSA2_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case CSA2_ERR_CAPACITY: return "destination range exceeds capacity";
        case CSA2_ERR_LAUNCH: return "HIP launch failed";
        case CSA2_ERR_SCRATCH: return "sizes exceed the no-allocation scratch (n_q <= 64, pool_blocks <= 2048)";
        default: return "unknown status";
    }
}

int csa2_version(void) { return 100; }

}  // extern "C"
