// sfi_stream.hip -- a plain streaming-read kernel, the yardstick for the attention kernels.
//
// The datasheet HBM peak of MI355X (8 TB/s) is not what a kernel can reach; a sequential
// read of a large buffer shows what the memory system delivers on the same box.  Each
// workgroup reads one contiguous chunk of the buffer with 16-byte nontemporal loads, four
// loads in flight per thread, and folds the words into an XOR so that no load is dead.  The
// fold is compared with a constant and written only on a match (practically never), so the
// kernel moves no bytes to HBM beyond the reads.
#include "sfi_internal.h"

namespace sfi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const u32x4* __restrict__ p, uint64_t n16, uint64_t per_wg,
                   uint32_t* __restrict__ sink) {
    const uint64_t begin = (uint64_t)blockIdx.x * per_wg;
    const uint64_t end = begin + per_wg < n16 ? begin + per_wg : n16;
    uint32_t acc = 0;
    for (uint64_t i = begin + threadIdx.x; i < end; i += kStreamThreads * kStreamUnroll) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) {
            const uint64_t k = i + (uint64_t)u * kStreamThreads;
            v[u] = k < end ? __builtin_nontemporal_load(p + k) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x & (kStreamSinkWords - 1)] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, uint64_t bytes, int n_wg, uint32_t* sink,
                              hipStream_t s) {
    const uint64_t n16 = bytes / 16;
    const uint64_t per_wg = (n16 + n_wg - 1) / n_wg;
    hipLaunchKernelGGL(stream_read_kernel, dim3(n_wg), dim3(kStreamThreads), 0, s,
                       (const u32x4*)buf, n16, per_wg, sink);
    return hipGetLastError();
}

}  // namespace sfi
