/*
 * csa2_timing.h -- measurement entry points of the CSA2 library: three calls of csa2.h whose
 * kernels record their own start and end into caller events (hipExtLaunchKernelGGL), so a
 * caller can time those kernels alone, as a kernel trace does, without event records of its
 * own around the launch.  Everything else about each call (arguments, layouts, workspace,
 * outputs, errors) is that of the plain entry point in csa2.h.
 *
 * Common rules: start_event and stop_event are hipEvent_t created by the caller, passed as
 * void*; either may be NULL (not recorded).  With an event given, a stream under graph
 * capture is refused (CSA2_ERR_UNSUPPORTED).  On an error nothing is launched or recorded.
 */
#ifndef CSA2_TIMING_H
#define CSA2_TIMING_H

#include "csa2.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * csa2_index_full_scan_timed -- csa2_index_full_scan (k_scales == NULL: bf16 keys k_idx) or
 * csa2_index_full_mx_scan (k_scales != NULL: MXFP4 code bytes k_idx and their E8M0 scales):
 * the Full-mode scan of [Article] "DeepSeek-V4.1-Flash: Pushing KV Cache Compression to 890
 * Bytes per Token", section IX.  The decode scan records the events through its launch; a
 * prefill chunk's scoring kernels are bracketed by two event records on `stream`.
 */
int csa2_index_full_scan_timed(const uint16_t* q_idx, const float* w, const void* k_idx,
                               const uint8_t* k_scales, csa2_seqs seqs, int32_t n_heads, int32_t top_k,
                               int32_t block, int32_t pool_blocks, int32_t shared_kv, int32_t* idx_out,
                               int32_t* pool_out, void* ws, size_t ws_bytes, void* stream,
                               void* start_event, void* stop_event);

/*
 * csa2_index_reindex_timed -- csa2_index_reindex (k_scales == NULL) or csa2_index_reindex_mx
 * (MXFP4 keys): [Article] sections VIII-IX.  Two event pairs: the scoring kernel's own start and
 * end, and the selection kernel's (the kernel that follows it).
 */
int csa2_index_reindex_timed(const uint16_t* q_idx, const float* w, const void* k_idx,
                             const uint8_t* k_scales, csa2_seqs seqs, int32_t n_heads, const int32_t* pool,
                             int32_t pool_blocks, int32_t block, int32_t top_k, int32_t* idx_out, void* ws,
                             size_t ws_bytes, void* stream, void* score_start, void* score_stop,
                             void* select_start, void* select_stop);

/*
 * csa2_attend_timed -- csa2_attend (bf16 window store): [Article] sections VI and XI.  The
 * attention kernel records both events through its launch.
 */
int csa2_attend_timed(const uint16_t* q, const uint8_t* codes, const uint8_t* scales, csa2_seqs seqs,
                      const int32_t* idx, int32_t top_k, uint16_t* swa, const int64_t* swa_row0,
                      int32_t swa_cap, int64_t swa_rows, int32_t window, const uint16_t* win_new,
                      int32_t n_heads, float softmax_scale, float* out, void* ws, size_t ws_bytes,
                      void* stream, void* start_event, void* stop_event);

/*
 * csa2_stream_read_groups -- the number of workgroups (and sink words) of csa2_stream_read on the
 * current device.
 * csa2_stream_read -- not a step of the method: a plain streaming read of `bytes` bytes at src
 * (device, 16-byte aligned, bytes a multiple of 16) with 16-byte loads spread over the whole
 * chip, the reference for what this HBM delivers to a read-only kernel in the same run.  Each
 * workgroup writes one word folded from what it read to sink (device uint32 [sink_words],
 * sink_words >= csa2_stream_read_groups()).  The events (as above) record the kernel's own start
 * and end.
 */
int csa2_stream_read_groups(void);
int csa2_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream,
                     void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif
#endif /* CSA2_TIMING_H */
