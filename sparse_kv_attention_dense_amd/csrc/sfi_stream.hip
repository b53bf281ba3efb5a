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
// one launch.  Workgroup (split, h, b) takes slots [split * split_len, ...) of unit (b, h):
// slot s < n_idx reads the row of idx[s] when 0 <= idx[s] < r0, else of position len - 1 (as
// the fast step reads a stand-in row for a skipped entry), and the rest walk the recent
// window [r0, len).  Each wavefront takes 32-slot tiles; lane l loads 16 bytes of row
// l / (row_bytes / 16) of every group of rows, so each load instruction covers whole rows.  A
// tile's index entries (and block-table entries) are loaded together, then all of its key and
// value loads are issued before any is used.
constexpr int kGatherRowsMax = 32 / 2;               // rows per lane per tile (rows of 512 B)
__global__ void __launch_bounds__(kStreamThreads)
gather_read_kernel(GatherArgs a) {
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int unit = b * a.Hkv + h;
    const int len_b = a.len[b];
    const int n_sel = min(max(a.n_idx[unit], 0), a.idx_stride);
    const int r0 = max(0, len_b - a.n_recent);
    const int n_tot = len_b > 0 ? n_sel + (len_b - r0) : 0;
    const int s0 = split * a.split_len;
    const int s1 = min(n_tot, s0 + a.split_len);
    const int lpr = a.row_bytes / 16;                  // lanes per row
    const int rpi = 64 / lpr;                          // rows per load instruction
    const int per = 32 / rpi;                          // rows of a tile per lane (<= 16)
    const int32_t* irow = a.idx + (int64_t)unit * a.idx_stride;
    const unsigned char* kb = (const unsigned char*)a.k;
    const unsigned char* vb = (const unsigned char*)a.v;
    const int bmask = (1 << a.block_shift) - 1;
    uint32_t acc = 0;
    for (int t0 = s0 + 32 * w; t0 < s1; t0 += 32 * 4) {
        int pos[kGatherRowsMax];
#pragma unroll
        for (int k = 0; k < kGatherRowsMax; ++k) {     // index entries of the tile, together
            const int slot = min(t0 + lane / lpr + k * rpi, s1 - 1);
            pos[k] = (k < per && slot < n_sel) ? irow[slot] : 0;
        }
#pragma unroll
        for (int k = 0; k < kGatherRowsMax; ++k) {
            const int slot = min(t0 + lane / lpr + k * rpi, s1 - 1);
            if (slot < n_sel) {
                if (pos[k] < 0 || pos[k] >= r0) pos[k] = len_b - 1;
            } else {
                pos[k] = r0 + (slot - n_sel);
            }
        }
        uint64_t row[kGatherRowsMax];
#pragma unroll
        for (int k = 0; k < kGatherRowsMax; ++k) {     // block-table entries, together
            if (a.block_table) {
                const uint32_t blk = k < per
                    ? (uint32_t)a.block_table[(int64_t)b * a.max_blocks + (pos[k] >> a.block_shift)]
                    : 0u;
                row[k] = (((uint64_t)blk * a.Hkv + h) << a.block_shift) + (uint64_t)(pos[k] & bmask);
            } else {
                row[k] = (uint64_t)unit * (uint64_t)a.n_cap + (uint64_t)pos[k];
            }
        }
        u32x4 kv[kGatherRowsMax], vv[kGatherRowsMax];
#pragma unroll
        for (int k = 0; k < kGatherRowsMax; ++k) {     // every key and value load of the tile
            const uint64_t off = row[k] * (uint64_t)a.row_bytes + (uint64_t)(lane % lpr) * 16;
            kv[k] = k < per ? *(const u32x4*)(kb + off) : u32x4{0u, 0u, 0u, 0u};
            vv[k] = k < per ? *(const u32x4*)(vb + off) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kGatherRowsMax; ++k)
            acc ^= kv[k].x ^ kv[k].y ^ kv[k].z ^ kv[k].w ^ vv[k].x ^ vv[k].y ^ vv[k].z ^ vv[k].w;
    }
    if (acc == 0x9e3779b9u) a.sink[(blockIdx.x + blockIdx.y) & (kStreamSinkWords - 1)] = acc;
}

}  // namespace

hipError_t launch_gather_read(const GatherArgs& a, int nsplit, int B, hipStream_t s) {
    hipLaunchKernelGGL(gather_read_kernel, dim3(nsplit, a.Hkv, B), dim3(kStreamThreads), 0, s, a);
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
