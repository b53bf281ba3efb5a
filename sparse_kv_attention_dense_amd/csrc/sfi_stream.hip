// sfi_stream.hip -- measurement yardsticks for the attention kernels: a plain streaming read,
// and a gather read of exactly the key and value rows a fast step reads.
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

// Gather yardstick: the key and value rows of a fast step's slots, read with no arithmetic in
// one launch, in the fast step's own order.  Workgroup (split, h, b) takes slots
// [split * split_len, ...) of unit (b, h): slot s < n_idx reads the row of idx[s] when
// 0 <= idx[s] < r0, else of position len - 1 (as the fast step reads a stand-in row for a
// skipped entry), and the rest walk the recent window [r0, len).  As in the fast step, the
// workgroup first builds the row numbers of its slots in LDS (every index load of a segment
// issued together, then every block-table load), kGatherTab slots per segment; then each
// wavefront takes the segment's 32-slot tiles w, w + 4, ...; lane l loads 16 bytes of row
// l / (row_bytes / 16) of every group of rows, so each load instruction covers whole rows, and
// every key and value load of a tile is issued before any is used.
constexpr int kGatherTab = 4096;                     // row-table slots per segment (16 KB)
constexpr int kGatherFill = kGatherTab / kStreamThreads;
template <int ROWB>                                  // row bytes: 128, 256 or 512
__global__ void __launch_bounds__(kStreamThreads)
gather_read_kernel(GatherArgs a) {
    constexpr int kLpr = ROWB / 16;                  // lanes per row
    constexpr int kRpi = 64 / kLpr;                  // rows per load instruction
    constexpr int kPer = 32 / kRpi;                  // rows of a tile per lane
    __shared__ uint32_t tab[kGatherTab];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int unit = b * a.Hkv + h;
    const int s0 = split * a.split_len;
    const int32_t* irow = a.idx + (int64_t)unit * a.idx_stride;
    // the first segment's index entries depend only on the slot: loaded beside the lengths
    int pos[kGatherFill];
#pragma unroll
    for (int u = 0; u < kGatherFill; ++u) {
        const int t = u * kStreamThreads + tid, slot = s0 + t;
        pos[u] = (t < a.split_len && slot < a.idx_stride) ? irow[slot] : 0;
    }
    const int len_b = a.len[b];
    const int n_sel = min(max(a.n_idx[unit], 0), a.idx_stride);
    const int r0 = max(0, len_b - a.n_recent);
    const int n_tot = len_b > 0 ? n_sel + (len_b - r0) : 0;
    const int s1 = min(n_tot, s0 + a.split_len);
    const unsigned char* kb = (const unsigned char*)a.k;
    const unsigned char* vb = (const unsigned char*)a.v;
    const int bmask = (1 << a.block_shift) - 1;
    uint32_t acc = 0;
    for (int g0 = s0; g0 < s1; g0 += kGatherTab) {
        const int n = min(kGatherTab, s1 - g0);
        if (g0 != s0) {
#pragma unroll
            for (int u = 0; u < kGatherFill; ++u) {
                const int slot = g0 + u * kStreamThreads + tid;
                pos[u] = (u * kStreamThreads + tid < n && slot < n_sel) ? irow[slot] : 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherFill; ++u) {
            const int slot = g0 + u * kStreamThreads + tid;
            if (slot < n_sel) {
                if (pos[u] < 0 || pos[u] >= r0) pos[u] = len_b - 1;
            } else {
                pos[u] = r0 + (slot - n_sel);
            }
        }
        uint32_t row[kGatherFill];
#pragma unroll
        for (int u = 0; u < kGatherFill; ++u) {
            if (a.block_table) {
                const uint32_t blk = u * kStreamThreads + tid < n
                    ? (uint32_t)a.block_table[(int64_t)b * a.max_blocks + (pos[u] >> a.block_shift)]
                    : 0u;
                row[u] = (((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)h) << a.block_shift) |
                         (uint32_t)(pos[u] & bmask);
            } else {
                row[u] = (uint32_t)((int64_t)unit * a.n_cap + pos[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kGatherFill; ++u)
            if (u * kStreamThreads + tid < n) tab[u * kStreamThreads + tid] = row[u];
        __syncthreads();
        const int ntiles = (n + 31) / 32;
        for (int t = w; t < ntiles; t += kStreamThreads / 64) {
            u32x4 kv[kPer], vv[kPer];
#pragma unroll
            for (int k = 0; k < kPer; ++k) {             // every key and value load of the tile
                const int slot = min(t * 32 + lane / kLpr + k * kRpi, n - 1);
                const uint64_t off = (uint64_t)tab[slot] * ROWB + (uint64_t)(lane % kLpr) * 16;
                kv[k] = *(const u32x4*)(kb + off);
                vv[k] = *(const u32x4*)(vb + off);
            }
            __builtin_amdgcn_sched_barrier(0);        // all of them issued before any is used
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                acc ^= kv[k].x ^ kv[k].y ^ kv[k].z ^ kv[k].w ^ vv[k].x ^ vv[k].y ^ vv[k].z ^ vv[k].w;
        }
        __syncthreads();                              // the table is read before it is replaced
    }
    if (acc == 0x9e3779b9u) a.sink[(blockIdx.x + blockIdx.y) & (kStreamSinkWords - 1)] = acc;
}

}  // namespace

hipError_t launch_gather_read(const GatherArgs& a, int nsplit, int B, hipStream_t s) {
    const dim3 grid(nsplit, a.Hkv, B);
    if (a.row_bytes == 128) hipLaunchKernelGGL(gather_read_kernel<128>, grid, dim3(kStreamThreads), 0, s, a);
    else if (a.row_bytes == 256) hipLaunchKernelGGL(gather_read_kernel<256>, grid, dim3(kStreamThreads), 0, s, a);
    else if (a.row_bytes == 512) hipLaunchKernelGGL(gather_read_kernel<512>, grid, dim3(kStreamThreads), 0, s, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, uint64_t bytes, int n_wg, uint32_t* sink,
                              hipStream_t s) {
    const uint64_t n16 = bytes / 16;
    const uint64_t per_wg = (n16 + n_wg - 1) / n_wg;
    hipLaunchKernelGGL(stream_read_kernel, dim3(n_wg), dim3(kStreamThreads), 0, s,
                       (const u32x4*)buf, n16, per_wg, sink);
    return hipGetLastError();
}

}  // namespace sfi
