/*
 * csa2.h -- C ABI of the CSA2 hot path on one MI355X (gfx950): FP4 pack-on-write,
 * the Full / Reindex indexer with block pool and Top-K, and gather-dequant sparse
 * attention with a bf16 sliding window.
 *
 * Sources (the method is described on three web pages):
 *   [Viz]     "DeepSeek-V4.1-Flash: shrinking KV cache at 552B scale" visualisation
 *             page (podcast.do-not-panic.com), figure captions.
 *   [Summary] "DeepSeek Cuts KV Cache Footprint Fourfold" (sotapapers.com),
 *             section "Technical Approach".
 *   [Article] "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890 Bytes per
 *             Token" (trishampatil.com), sections VI, VIII, IX, XI.
 *
 * Conventions shared by every entry point
 *   - All array pointers are DEVICE pointers owned by the caller (for example
 *     torch tensors' data_ptr()).  The library allocates nothing, keeps no mutable
 *     global state and is re-entrant; calls on one stream run in order.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - bf16 arrays are uint16 bit patterns; fp32 arrays are IEEE binary32.
 *   - Every argument that the host can see is validated before anything is
 *     launched.  On a non-zero return nothing was launched and no output was
 *     written.  After launching, hipGetLastError() is checked (CSA2_ERR_LAUNCH).
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - Values that live on the device (kv_len, kv_row0, idx, pool, dst_rows)
 *     cannot be checked on the host.  Kernels clamp them so that no access leaves
 *     the arrays described here: a length is clamped to [0, max_len_ub] and to the
 *     cache rows that exist after kv_row0, selected indices outside [0, N) are
 *     skipped, destination rows outside [0, cap_rows) are not written.  Results are
 *     then those of the clamped problem.
 *   - Inputs are finite.  Results are deterministic run to run (no float atomics).
 *   - Workspace: index calls and decode-sized attention calls take a caller-owned device workspace of
 *     at least csa2_workspace_bytes(...) bytes.  Every workspace starts with the same
 *     prefix for a given n_q: per-query counters (CSA2_CTRL_BYTES(n_q) bytes) and
 *     per-query histograms.  That prefix must be zero when a call starts and every
 *     call leaves it zero when it completes, so zero a new workspace once with
 *     csa2_workspace_init() (a kernel, so it may be captured in a HIP graph).  Calls
 *     may share a workspace (in stream order) only if they pass the same n_q; two
 *     calls that may run concurrently must not share one.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define CSA2_OK 0
#define CSA2_ERR_NULL 1        /* a required pointer is NULL */
#define CSA2_ERR_SHAPE 2       /* a size argument is out of its valid range */
#define CSA2_ERR_UNSUPPORTED 3 /* a valid size these kernels do not implement */
#define CSA2_ERR_WORKSPACE 4   /* workspace NULL or smaller than csa2_workspace_bytes() */
#define CSA2_ERR_CAPACITY 5    /* a destination range exceeds the stated capacity */
#define CSA2_ERR_LAUNCH 6      /* the HIP runtime reported an error at launch */
#define CSA2_ERR_SCRATCH 7     /* sizes past the no-allocation entry point's built-in scratch */

/* ---- limits of this implementation ---- */
#define CSA2_KV_DIM 128         /* main-KV latent width = attention head dim */
#define CSA2_IDX_DIM 64         /* indexer key / query width */
#define CSA2_MAX_IDX_HEADS 8    /* indexer heads */
#define CSA2_MAX_Q_HEADS 16     /* attention query heads sharing one KV head */
#define CSA2_MAX_SELECT 4096    /* top_k and pool_blocks */
#define CSA2_MAX_WINDOW 4096    /* sliding-window length */
#define CSA2_MAX_QUERIES 65535  /* n_q */
#define CSA2_BLOCK 8            /* positions per pool block */
#define CSA2_NOALLOC_MAX_QUERIES 64   /* csa2_index_reindex_noalloc: n_q */
#define CSA2_NOALLOC_MAX_POOL 2048    /* csa2_index_reindex_noalloc: pool_blocks */

/* ---- operation ids for csa2_workspace_bytes ---- */
#define CSA2_OP_INDEX_FULL 1
#define CSA2_OP_INDEX_REINDEX 2
#define CSA2_OP_ATTEND 3

/* Bytes of self-cleaning counters at the start of every workspace. */
#define CSA2_CTRL_BYTES(n_q) ((((size_t)(n_q) * 64u) + 255u) & ~(size_t)255u)

/*
 * Where each query's context lives.  Query i sees positions [0, N_i) of one
 * sequence; position p of that sequence is row kv_row0[i] + p of the main-KV
 * code/scale arrays and of the indexer-key array.  Decode passes one query per
 * sequence; a prefill chunk passes one query per new token, all with the same
 * kv_row0 and lengths C + t + 1 (a query sees its own token).
 */
typedef struct csa2_seqs {
    const int64_t* kv_row0; /* device [n_q] */
    const int32_t* kv_len;  /* device [n_q]: N_i */
    int32_t n_q;            /* number of queries, >= 0 */
    int32_t max_len_ub;     /* host: upper bound on every N_i, >= 0 */
    int64_t total_len_ub;   /* host: upper bound on sum_i N_i, >= 0 */
    int64_t cache_rows;     /* host: rows in the main-KV and indexer-key arrays */
} csa2_seqs;

/*
 * fp4_kv_append -- pack-on-write of post-RoPE KV vectors into the FP4 cache.
 * [Article] section XI and the [Viz] FP4 caption: E2M1 elements with one E4M3
 * scale per 16 channels, no second-level scale, quantised after RoPE.
 *
 *   x        device bf16 [n_tok, dim], row-major.
 *   dim      channels per vector; a multiple of 16, at most 1024.
 *   dst_rows device int64 [n_tok] (token t goes to row dst_rows[t]) or NULL
 *            (token t goes to row row0 + t; then row0 + n_tok <= cap_rows).
 *   codes    device uint8 [cap_rows, dim/2]: byte j holds channel 2j in its low
 *            nibble and channel 2j+1 in its high nibble (E2M1: sign bit 3).
 *   scales   device uint8 [cap_rows, dim/16]: E4M3 (OCP "fn") byte of channels
 *            [16g, 16g+16).
 * Per group: scale = the E4M3 value nearest to amax/6, ties to even; each code is
 * the E2M1 value nearest to x/scale, ties to even, saturating at 6, carrying x's
 * sign bit; a zero scale gives zero magnitudes.  Rows outside [0, cap_rows) named
 * by dst_rows are skipped.  n_tok == 0 is a no-op.
 */
int fp4_kv_append(const uint16_t* x, int64_t n_tok, int32_t dim, const int64_t* dst_rows,
                  int64_t row0, uint8_t* codes, uint8_t* scales, int64_t cap_rows, void* stream);

/*
 * fp8_window_append -- write bf16 vectors into an FP8 window store.
 * [Article] section XI (the recent-window cache stays at FP8, E4M3).
 *
 *   x        device bf16 [n_tok, dim], 16-byte aligned; dim % 8 == 0, <= 1024.
 *   dst_rows device int64 [n_tok] or NULL (rows row0 .. row0 + n_tok - 1).
 *   out      device uint8 [cap_rows, dim], 8-byte aligned: E4M3 ("fn") bytes.
 * Each value becomes the nearest E4M3 value, ties to even, saturating at +-448 (the
 * format has no infinity), with the value's sign bit; no scale.  Rows outside
 * [0, cap_rows) named by dst_rows are skipped.  n_tok == 0 is a no-op.
 */
int fp8_window_append(const uint16_t* x, int64_t n_tok, int32_t dim, const int64_t* dst_rows,
                      int64_t row0, uint8_t* out, int64_t cap_rows, void* stream);

/*
 * csa2_index_full -- Full-mode indexer for n_q queries.
 * [Article] section IX (the Full layer scores every causally visible position,
 * scores 8-position blocks by their best position and keeps the winning blocks as
 * a shared pool) and [Summary] Technical Approach (Full mode computes Top-K fresh).
 *
 *   q_idx   device bf16 [n_q, n_heads, CSA2_IDX_DIM]: indexer queries.
 *   w       device fp32 [n_q, n_heads]: per-head weights.
 *   k_idx   device bf16 [seqs.cache_rows, CSA2_IDX_DIM]: indexer keys.
 *   n_heads 1..CSA2_MAX_IDX_HEADS.
 *   top_k   1..CSA2_MAX_SELECT; block must be CSA2_BLOCK.
 *   pool_blocks 0 (no pool) or 1..CSA2_MAX_SELECT.
 *   idx_out device int32 [n_q, top_k]: the top_k positions under (score desc,
 *           position asc), written in ascending order, -1 padded when N_i < top_k.
 *   pool_out device int32 [n_q, pool_blocks] or NULL when pool_blocks == 0: block
 *           ids under (block max desc, block asc), ascending, -1 padded.  Each query
 *           gets the pool of its own visible positions: in a decode batch that is the
 *           sequence's shared pool; in a prefill chunk every query token has its own
 *           (the Reindex layers of the chunk select inside each token's pool).
 * Score of position p: sum_h w[h] * max(0, q_h . k_p), accumulated in fp32; with
 * integer-valued inputs and |score| < 2^24 it is exact.  Scores are MFMA
 * contractions: heads x positions per query, or, for a prefill chunk (shared_kv != 0:
 * every query has the same kv_row0), queries x positions.  n_q == 0 is a no-op.
 */
int csa2_index_full(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                    int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                    int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * The three parts of csa2_index_full, for callers that time or schedule them apart:
 * _prep writes per-query metadata and the tile maps the later kernels read to the
 * workspace (one kernel; a decode call of at most 64 queries launches nothing here, its
 * scan kernel derives the metadata itself and writes what the later kernels read);
 * _scan scores every visible position (fused block maxima and first-digit histograms,
 * one kernel); _select compacts the threshold buckets and writes
 * idx_out and pool_out (two kernels: a filter over all positions, then one workgroup per
 * query and output; decode calls whose contexts are all at most 16,384 positions skip
 * the filter, the selection workgroups then read the keys themselves).  Call them in this order, on the same stream, with identical
 * arguments and workspace; together they equal one csa2_index_full call.
 */
int csa2_index_full_prep(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                         int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                         int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws,
                         size_t ws_bytes, void* stream);
int csa2_index_full_scan(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                         int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                         int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws,
                         size_t ws_bytes, void* stream);
int csa2_index_full_select(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                           int32_t n_heads, int32_t top_k, int32_t block, int32_t pool_blocks,
                           int32_t shared_kv, int32_t* idx_out, int32_t* pool_out, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * MXFP4 indexer keys.  [Article] sections VII and XI: indexer K is stored in MXFP4, E2M1
 * elements with one E8M0 scale byte per 32 channels (34 B per 64-channel key instead of
 * 128 B in bf16).
 *
 * mxfp4_key_append -- quantise bf16 keys into MXFP4 rows.
 *   x        device bf16 [n_tok, dim], finite values, 16-byte aligned; dim % 32 == 0, <= 1024.
 *   dst_rows device int64 [n_tok] or NULL (rows row0 .. row0 + n_tok - 1).
 *   codes    device uint8 [cap_rows, dim/2], 16-byte aligned: byte j holds channel 2j in its
 *            low nibble, 2j+1 in its high nibble (E2M1, sign bit 3).
 *   scales   device uint8 [cap_rows, dim/32]: E8M0 byte e of channels [32b, 32b+32),
 *            value 2^(e - 127).
 * Per block: e = (exponent of the largest |x|) - 2, clamped to [1, 254] (so the largest
 * value lands in [4, 8) before rounding); each code is the E2M1 value nearest to x / 2^(e-127),
 * ties to even, saturating at 6, with x's sign bit.  Rows outside [0, cap_rows) named by
 * dst_rows are skipped.
 *
 * csa2_index_full_mx / csa2_index_full_mx_scan / csa2_index_reindex_mx -- csa2_index_full,
 * its scan part and csa2_index_reindex with MXFP4 keys: k_codes device uint8
 * [seqs.cache_rows, 32] (16-byte aligned) and k_scales device uint8 [seqs.cache_rows, 2]
 * (2-byte aligned), written by mxfp4_key_append with dim = CSA2_IDX_DIM.  Scores are those of
 * the dequantised keys (integer keys in [-4, 4] are exact, so selections equal the bf16-key
 * ones).  csa2_index_full_prep and csa2_index_full_select read no keys and serve both key
 * formats.  A prefill chunk (shared_kv != 0) is scanned per query.  Arguments, workspace,
 * outputs and errors are otherwise those of the bf16-key calls.
 */
int mxfp4_key_append(const uint16_t* x, int64_t n_tok, int32_t dim, const int64_t* dst_rows,
                     int64_t row0, uint8_t* codes, uint8_t* scales, int64_t cap_rows, void* stream);
int csa2_index_full_mx(const uint16_t* q_idx, const float* w, const uint8_t* k_codes,
                       const uint8_t* k_scales, csa2_seqs seqs, int32_t n_heads, int32_t top_k,
                       int32_t block, int32_t pool_blocks, int32_t shared_kv, int32_t* idx_out,
                       int32_t* pool_out, void* ws, size_t ws_bytes, void* stream);
int csa2_index_full_mx_scan(const uint16_t* q_idx, const float* w, const uint8_t* k_codes,
                            const uint8_t* k_scales, csa2_seqs seqs, int32_t n_heads, int32_t top_k,
                            int32_t block, int32_t pool_blocks, int32_t shared_kv, int32_t* idx_out,
                            int32_t* pool_out, void* ws, size_t ws_bytes, void* stream);
int csa2_index_reindex_mx(const uint16_t* q_idx, const float* w, const uint8_t* k_codes,
                          const uint8_t* k_scales, csa2_seqs seqs, int32_t n_heads, const int32_t* pool,
                          int32_t pool_blocks, int32_t block, int32_t top_k, int32_t* idx_out, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * csa2_index_reindex -- Reindex-mode indexer: this layer's own query scored against
 * the Full layer's keys, over the positions of the pool's blocks only.
 * [Article] sections VIII-IX (Reindex reuses main KV and indexer K, runs its own
 * selection inside the shared pool); [Summary] Technical Approach.
 *
 *   pool    device int32 [n_q, pool_blocks]: block ids in ascending order, as
 *           csa2_index_full writes them; -1 entries (anywhere in the row) and ids whose
 *           positions fall outside [0, N_i) contribute nothing.
 *   Other arguments as in csa2_index_full.  idx_out gets the top_k candidate
 *   positions under (score desc, position asc), ascending, -1 padded.
 * The kernels take a pool row's element order for position order (ties at the threshold
 * score go to the earlier element, and idx_out lists the selection in element order), which
 * is what the ranking above needs when the row is ascending.  A row in any other order is not
 * an error: its selection is the top_k candidates under (score desc, element order asc),
 * written in element order.
 */
int csa2_index_reindex(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                       int32_t n_heads, const int32_t* pool, int32_t pool_blocks, int32_t block,
                       int32_t top_k, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_attend -- sparse attention of n_q queries over their selected FP4 entries
 * plus their bf16 sliding window.  [Article] section VI ("What one layer looks
 * like": own query, 512 selected entries plus the recent window, and every layer
 * computes its own window entries) and section XI (entries are dequantised before
 * attention).
 *
 *   q       device bf16 [n_q, n_heads, CSA2_KV_DIM], 16-byte aligned.
 *   codes, scales  the FP4 cache ([seqs.cache_rows, 64] and [seqs.cache_rows, 8]).
 *   idx     device int32 [n_q, top_k]: selected positions; entries outside [0, N_i)
 *           (e.g. -1 padding) are skipped.  A Reuse layer passes the idx of the
 *           most recent index-producing layer.
 *   swa     device bf16 [swa_rows, CSA2_KV_DIM]: the layer's window store; position
 *           p of query i is row swa_row0[i] + (p mod swa_cap).
 *   swa_row0 device int64 [n_q]; swa_cap >= window (>= 1); rows outside
 *           [0, swa_rows) are skipped.
 *   window  window length W >= 0: query i attends positions [max(0, N_i - W), N_i).
 *   win_new device bf16 [n_q, CSA2_KV_DIM] (16-byte aligned) or NULL: the new token's
 *           own window vector of this layer (decode).  Query i attends it as position
 *           N_i - 1 (that store row is not read) and the call writes it to that row,
 *           after its own reads, also when the position falls outside the attended
 *           window.  Rows written for one query must not be read by another query of
 *           the same call (decode: one ring per sequence); a prefill chunk writes its
 *           window rows with csa2_window_append first and passes NULL.
 *   n_heads 1..CSA2_MAX_Q_HEADS.  softmax_scale multiplies q.k.
 *   out     device fp32 [n_q, n_heads, CSA2_KV_DIM].
 *   swa_rows must be below 2^31.
 * Each entry's vector is both key and value.  One softmax runs over the selected
 * entries and the window entries together (no de-duplication).  A query with
 * nothing to attend gets zeros.  n_q == 0 is a no-op.
 *   ws, ws_bytes  device workspace of at least
 *           csa2_workspace_bytes(CSA2_OP_ATTEND, n_q, 0, 0, top_k, window) bytes,
 *           16-byte aligned, zeroed once (csa2_workspace_init) and left as the call
 *           leaves it.  Calls of at most 64 queries share each query's entries out
 *           over several workgroups and merge their softmax partials through it; the
 *           size is 0 otherwise, and ws may then be NULL.  A workspace smaller than
 *           required gives CSA2_ERR_WORKSPACE with nothing launched.  Calls that
 *           overlap in time need separate workspaces.
 * The result is the same whatever order the workgroups finish in (the partials are
 * combined in a fixed order).
 */
int csa2_attend(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, csa2_seqs seqs,
                const int32_t* idx, int32_t top_k, uint16_t* swa, const int64_t* swa_row0,
                int32_t swa_cap, int64_t swa_rows, int32_t window, const uint16_t* win_new,
                int32_t n_heads, float softmax_scale, float* out, void* ws, size_t ws_bytes,
                void* stream);

/*
 * csa2_attend_fp8win -- csa2_attend with the pages' window format and replay bound.
 * [Article] section XI (the recent-window cache stays at FP8) and section XII (SWA
 * Bounded Replay: for a replay starting at position s, the query at position i
 * attends window keys in [max(s, i - win + 1), i]).
 *
 *   swa           device uint8 [swa_rows, CSA2_KV_DIM]: E4M3 bytes written by
 *                 fp8_window_append (the codes 0x7f / 0xff, NaN, are never written).
 *   replay_start  device int64 [n_q] or NULL (no bound): query i's window is
 *                 positions [max(replay_start[i], N_i - window, 0), N_i).
 *   win_new       as for csa2_attend (bf16); it is converted to E4M3 as
 *                 fp8_window_append does, attended in that form and written.
 * Every other argument, the layouts, the errors and the output are those of
 * csa2_attend.  Window values and FP4 values enter the contractions exactly (f16).
 */
int csa2_attend_fp8win(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, csa2_seqs seqs,
                       const int32_t* idx, int32_t top_k, uint8_t* swa, const int64_t* swa_row0,
                       int32_t swa_cap, int64_t swa_rows, int32_t window, const int64_t* replay_start,
                       const uint16_t* win_new, int32_t n_heads, float softmax_scale, float* out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_reindex_noalloc -- csa2_index_reindex without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops and harnesses that
 * forbid allocation).  The workspace is a static device array of the library (6 MiB per GPU,
 * held until the process ends); the call allocates nothing.  Sizes: n_q <= 64 and pool_blocks
 * <= 2,048 (larger: CSA2_ERR_SCRATCH, nothing launched).  The first call on a device also clears
 * the array with a kernel on `stream`; every call leaves its counters and histograms zero again.
 * All calls on one GPU share its array: calls that may overlap on one GPU (other streams, other
 * host threads) race and must not be issued.  Arguments, outputs and other errors are those of
 * csa2_index_reindex.
 */
int csa2_index_reindex_noalloc(const uint16_t* q_idx, const float* w, const uint16_t* k_idx, csa2_seqs seqs,
                               int32_t n_heads, const int32_t* pool, int32_t pool_blocks, int32_t block,
                               int32_t top_k, int32_t* idx_out, void* stream);

/*
 * csa2_reindex_attend -- one Reindex layer: csa2_index_reindex (or _mx) followed by
 * csa2_attend (or _fp8win) over the selection it produced.  [Article] sections VIII-IX (a
 * Reindex layer selects its own Top-K inside the shared pool) and section VI (the layer then
 * attends its selection plus its window).
 *
 *   q_idx, w, pool, pool_blocks, block, top_k, idx_out, ws, ws_bytes: as for
 *           csa2_index_reindex (CSA2_OP_INDEX_REINDEX workspace); idx_heads is its n_heads.
 *   k_idx, k_scales  k_scales == NULL: bf16 keys [seqs.cache_rows, CSA2_IDX_DIM];
 *           otherwise MXFP4 keys as for csa2_index_reindex_mx (k_idx = the code bytes).
 *   q, codes, scales, swa, swa_row0, swa_cap, swa_rows, window, win_new, n_heads,
 *   softmax_scale, out: as for csa2_attend; window_fp8 = 0: swa holds bf16, 1: E4M3 bytes.
 *   replay_start  device int64 [n_q] or NULL: as for csa2_attend_fp8win (either format).
 *   att_ws, att_ws_bytes  the attention workspace, as for csa2_attend
 *           (CSA2_OP_ATTEND with the same n_q, top_k and window; may be NULL when that size
 *           is 0).
 * idx_out receives the selection (a Reuse layer that follows attends with it), equal to that
 * of csa2_index_reindex, and out the attention over it, equal to that of csa2_attend: the call
 * issues the separate calls' kernels (scoring, selection, attention) in one go.  Three fused
 * forms measured slower on MI355X and are not used: everything in one kernel (the last scoring
 * workgroup of a query selecting and attending); the selection and attention in one kernel
 * (one compute unit then forms all 512 entries' logits, where the attention kernel spreads
 * them over five); and every attention workgroup repeating the selection itself with its four
 * waves (a selection four times slower than with sixteen).  All arguments are checked before
 * anything is launched; the errors are those of the separate calls.
 */
int csa2_reindex_attend(const uint16_t* q_idx, const float* w, const void* k_idx, const uint8_t* k_scales,
                        csa2_seqs seqs, int32_t idx_heads, const int32_t* pool, int32_t pool_blocks,
                        int32_t block, int32_t top_k, int32_t* idx_out, const uint16_t* q,
                        const uint8_t* codes, const uint8_t* scales, void* swa, int32_t window_fp8,
                        const int64_t* swa_row0, int32_t swa_cap, int64_t swa_rows, int32_t window,
                        const int64_t* replay_start, const uint16_t* win_new, int32_t n_heads,
                        float softmax_scale, float* out, void* ws, size_t ws_bytes, void* att_ws,
                        size_t att_ws_bytes, void* stream);

/*
 * csa2_token_append -- the decode step's own token for a Full layer's cache set: its
 * post-RoPE KV vector packed into the FP4 cache (exactly as fp4_kv_append) and its indexer
 * key written into the key cache, in one launch.  [Article] section VIII (a Full layer
 * computes its main KV and its indexer key fresh) and section XI (main KV in FP4, indexer
 * key in MXFP4; the workloads keep bf16 keys).
 *
 *   x        device bf16 [n_tok, CSA2_KV_DIM], 16-byte aligned.
 *   k_new    device bf16 [n_tok, CSA2_IDX_DIM], 16-byte aligned, or NULL (no key written).
 *   dst_rows device int64 [n_tok]: the row of token t in every cache; rows outside
 *            [0, cap_rows) are skipped.
 *   codes, scales  FP4 cache [cap_rows, 64] (8-byte aligned) and [cap_rows, 8].
 *   k_idx, k_scales  k_scales == NULL: bf16 key cache [cap_rows, CSA2_IDX_DIM]; otherwise
 *            MXFP4 code bytes [cap_rows, 32] and E8M0 scales [cap_rows, 2] (as
 *            mxfp4_key_append); k_idx 16-byte aligned.
 * n_tok == 0 is a no-op.
 */
int csa2_token_append(const uint16_t* x, const uint16_t* k_new, int64_t n_tok, const int64_t* dst_rows,
                      uint8_t* codes, uint8_t* scales, void* k_idx, uint8_t* k_scales, int64_t cap_rows,
                      void* stream);

/*
 * csa2_window_append -- write window vectors into a layer's window store ([Article]
 * section VI: every layer computes its own window entries; section XI: the pages keep
 * them at FP8).  window_fp8 = 0: bf16 rows (a copy); 1: E4M3 bytes as fp8_window_append.
 *   x        device bf16 [n_tok, CSA2_KV_DIM], 16-byte aligned.
 *   dst_rows device int64 [n_tok] or NULL (rows row0 .. row0 + n_tok - 1).
 *   out      device store [cap_rows, CSA2_KV_DIM] of bf16 or E4M3 bytes, 16-byte aligned.
 * Rows outside [0, cap_rows) named by dst_rows are skipped.  n_tok == 0 is a no-op.
 */
int csa2_window_append(const uint16_t* x, int64_t n_tok, const int64_t* dst_rows, int64_t row0, void* out,
                       int32_t window_fp8, int64_t cap_rows, void* stream);

/*
 * Workspace bytes for one call of `op` (CSA2_OP_*) with these sizes; SIZE_MAX if the
 * sizes are out of range, 0 if the call needs no workspace.  For CSA2_OP_ATTEND pass the
 * window length in `pool_blocks` (0 for calls of more than 64 queries); for
 * CSA2_OP_INDEX_REINDEX (also csa2_reindex_attend) total_len_ub and max_len_ub are unused.
 */
size_t csa2_workspace_bytes(int32_t op, int32_t n_q, int64_t total_len_ub, int32_t max_len_ub,
                            int32_t top_k, int32_t pool_blocks);

/* Zero a workspace's first `bytes` bytes with a kernel on `stream` (call once after allocation). */
int csa2_workspace_init(void* ws, size_t bytes, void* stream);

/* Static text for a status code. */
const char* csa2_status_string(int status);

/* Library version (major * 10000 + minor * 100 + patch). */
int csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_H */
