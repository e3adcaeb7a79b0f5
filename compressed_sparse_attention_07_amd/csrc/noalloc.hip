// csa2_index_reindex_noalloc: csa2_index_reindex with its workspace in a static device array of
// this library instead of a caller buffer, for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid allocation).  Declared in include/csa2.h.
//
// The array `scratch` is file-scope device memory, one copy per GPU, held until the process ends.
// Host code never uses its name as an address: the first call on a device (with that device
// current) asks the runtime for that device's address with hipGetSymbolAddress, keeps it in a
// per-device table, and every later call passes that pointer to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "csa2.h"

namespace {

// Sized for the largest call it takes: 64 queries x 2,048 pool blocks (counters and first-digit
// histograms per query, then one 4-byte key per pool position): 5.05 MiB of the 6 MiB.
constexpr size_t kScratchBytes = (size_t)6 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// This device's address of `scratch` (nullptr on a runtime error).  The first call on a device
// also clears the array with the library's zero-fill kernel on the caller's stream, so the
// counters and histograms that must start at zero do; every call leaves them zero again.
void* scratch_ptr(hipStream_t stream, int* status) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = CSA2_ERR_LAUNCH;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            *status = CSA2_ERR_LAUNCH;
            return nullptr;
        }
        const int st = csa2_workspace_init(p, kScratchBytes, stream);
        if (st != CSA2_OK) {
            *status = st;
            return nullptr;
        }
        g_ptr[dev] = p;
    }
    *status = CSA2_OK;
    return g_ptr[dev];
}

}  // namespace

extern "C" int csa2_index_reindex_noalloc(const uint16_t* q_idx, const float* w, const uint16_t* k_idx,
                                          csa2_seqs seqs, int32_t n_heads, const int32_t* pool, int32_t pool_blocks,
                                          int32_t block, int32_t top_k, int32_t* idx_out, void* stream) {
    if (seqs.n_q < 0 || pool_blocks < 0) return CSA2_ERR_SHAPE;
    if (seqs.n_q > CSA2_NOALLOC_MAX_QUERIES || pool_blocks > CSA2_NOALLOC_MAX_POOL) return CSA2_ERR_SCRATCH;
    const size_t need = csa2_workspace_bytes(CSA2_OP_INDEX_REINDEX, seqs.n_q, 0, 0, top_k, pool_blocks);
    if (need == (size_t)-1) return CSA2_ERR_SHAPE;  // top_k or pool_blocks out of range
    if (need > kScratchBytes) return CSA2_ERR_SCRATCH;
    if (seqs.n_q == 0)  // nothing to do once the sizes are checked (the plain call returns before its workspace)
        return csa2_index_reindex(q_idx, w, k_idx, seqs, n_heads, pool, pool_blocks, block, top_k, idx_out, nullptr, 0,
                                  stream);
    int st = CSA2_OK;
    void* ws = scratch_ptr(static_cast<hipStream_t>(stream), &st);
    if (ws == nullptr) return st;
    return csa2_index_reindex(q_idx, w, k_idx, seqs, n_heads, pool, pool_blocks, block, top_k, idx_out, ws,
                              kScratchBytes, stream);
}
