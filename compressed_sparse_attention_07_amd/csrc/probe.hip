// Measurement kernel: a plain streaming read, the reference point for the HBM-bound kernels'
// fractions of peak (what this memory delivers to a read-only kernel, measured in the same run).
#include <hip/hip_ext.h>

#include <cstdint>

namespace csa2 {

constexpr int kProbeNT = 256;
constexpr int kProbeWgPerCu = 16;
constexpr int kProbeU = 8;  // 16-byte loads in flight per thread per iteration

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each workgroup reads one contiguous slice of the buffer, its threads 16 bytes apart, kProbeU
// non-temporal 16-byte loads at a time, and folds every word with XOR; each workgroup writes one
// word, so no load can be dropped.  (Contiguous slices with non-temporal loads measured fastest
// among grid-stride and slice orders, 2 to 8 loads in flight and 2 to 32 workgroups per CU.)
__global__ __launch_bounds__(kProbeNT) void k_stream_read(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
    __shared__ uint32_t sh[kProbeNT / 64];
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per;
    const size_t end = b0 + per < n16 ? b0 + per : n16;
    size_t k = b0 + threadIdx.x;
    uint32_t acc = 0u;
    for (; k + (kProbeU - 1) * kProbeNT < end; k += kProbeU * kProbeNT) {
        u32x4 v[kProbeU];
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) v[u] = __builtin_nontemporal_load(src + k + u * kProbeNT);
#pragma unroll
        for (int u = 0; u < kProbeU; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; k < end; k += kProbeNT) {
        const u32x4 v = src[k];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = sh[0] ^ sh[1] ^ sh[2] ^ sh[3];
}

int stream_read_groups() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return cus * kProbeWgPerCu;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int groups, hipStream_t stream,
                              hipEvent_t ev_start, hipEvent_t ev_stop) {
    const size_t n16 = bytes / 16;
    hipExtLaunchKernelGGL(k_stream_read, dim3((unsigned)groups), dim3(kProbeNT), 0, stream, ev_start, ev_stop, 0,
                          static_cast<const u32x4*>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace csa2
