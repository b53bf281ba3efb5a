// sfi_reorg.hip -- Reorg for the two-segment fast-step layout (Slow-Fast Inference, Sec. 4.1
// and Sec. 4.2 "Coalesced reads with a two-segment KV layout"): after the Selector, the key and
// value rows of the sink and selected positions of every (sequence b, KV head h) are copied,
// in index order, into a compact segment that the fast steps of the cycle read slot by slot;
// the recent window stays in the cache and is read in place.
//
// reorg_kernel: one workgroup copies kReorgSlots slots of one (b, h).  Slot s < n (n = n_idx
// clamped to [0, idx_stride]) whose entry p = idx[s] lies in [0, len[b]) gets the rows of
// position p and cpos[s] = p; every other slot (an entry outside the sequence, or s >= n) gets
// zero rows and cpos[s] = -1, so the segment never holds stale or non-finite rows.  Each
// thread moves 16-byte pieces: the index loads of all its slots are issued first, then (paged)
// all block-table loads, then all row loads, then the stores, so a workgroup costs three or
// four memory round trips whatever its number of slots.
#include "sfi_internal.h"

namespace sfi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kReorgThreads = 256;
constexpr int kReorgSlots = 128;     // slots per workgroup

template <int RB, bool PAGED>      // RB: bytes per row (head_dim * element size)
__global__ void __launch_bounds__(kReorgThreads) reorg_kernel(ReorgArgs a) {
    constexpr int kLpr = RB / 16;                 // threads per row
    constexpr int kRpp = kReorgThreads / kLpr;    // rows per pass
    constexpr int kPass = kReorgSlots / kRpp;
    const int b = blockIdx.z, h = blockIdx.y;
    const int unit = b * a.Hkv + h;
    const int len_b = a.len[b];
    const int n = min(max(a.n_idx[unit], 0), a.idx_stride);
    const int32_t* irow = a.idx + (int64_t)unit * a.idx_stride;
    const int piece = threadIdx.x % kLpr;
    const int slot0 = blockIdx.x * kReorgSlots + threadIdx.x / kLpr;
    const uint64_t seg0 = (uint64_t)unit * a.idx_stride;

    // 1. index entries
    int pos[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
        const int slot = slot0 + p * kRpp;
        const int e = slot < n ? irow[slot] : -1;
        pos[p] = (e >= 0 && e < len_b) ? e : -1;
    }
    // 2. cache rows (paged: block numbers first).  Every load below is issued unconditionally
    // from an address inside a buffer, so the loads of all passes are in flight together: a
    // slot without a row reads its own destination piece (or the unit's last slot when past
    // the stride) and keeps zeros.
    uint64_t src[kPass];
    if constexpr (PAGED) {
        uint32_t blk[kPass];
#pragma unroll
        for (int p = 0; p < kPass; ++p)
            blk[p] = (uint32_t)a.block_table[(int64_t)b * a.max_blocks +
                                             (max(pos[p], 0) >> a.block_shift)];
        const int bmask = (1 << a.block_shift) - 1;
#pragma unroll
        for (int p = 0; p < kPass; ++p)
            src[p] = (((uint64_t)blk[p] * a.Hkv + h) << a.block_shift) | (uint64_t)(pos[p] & bmask);
    } else {
#pragma unroll
        for (int p = 0; p < kPass; ++p) src[p] = (uint64_t)unit * a.n_cap + pos[p];
    }
    u32x4 kx[kPass], vx[kPass];
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
        const bool has = pos[p] >= 0;
        const uint64_t dst = seg0 + min(slot0 + p * kRpp, a.idx_stride - 1);
        const unsigned char* kb = has ? (const unsigned char*)a.k : (const unsigned char*)a.ck;
        const unsigned char* vb = has ? (const unsigned char*)a.v : (const unsigned char*)a.cv;
        const uint64_t off = (has ? src[p] : dst) * RB + 16 * piece;
        kx[p] = *(const u32x4*)(kb + off);
        vx[p] = *(const u32x4*)(vb + off);
    }
    // 3. the segment
#pragma unroll
    for (int p = 0; p < kPass; ++p) {
        const int slot = slot0 + p * kRpp;
        if (slot < a.idx_stride) {
            const bool has = pos[p] >= 0;
            const uint64_t off = (seg0 + slot) * RB + 16 * piece;
            *(u32x4*)((unsigned char*)a.ck + off) = has ? kx[p] : u32x4{0u, 0u, 0u, 0u};
            *(u32x4*)((unsigned char*)a.cv + off) = has ? vx[p] : u32x4{0u, 0u, 0u, 0u};
            if (piece == 0) a.cpos[seg0 + slot] = pos[p];
        }
    }
}

}  // namespace

hipError_t launch_reorg(const ReorgArgs& a, int B, int row_bytes, hipStream_t s) {
    const dim3 grid((a.idx_stride + kReorgSlots - 1) / kReorgSlots, a.Hkv, B);
    const dim3 block(kReorgThreads);
    const bool paged = a.block_table != nullptr;
    switch (row_bytes * 2 + (paged ? 1 : 0)) {
        case 256: hipLaunchKernelGGL((reorg_kernel<128, false>), grid, block, 0, s, a); break;
        case 257: hipLaunchKernelGGL((reorg_kernel<128, true>), grid, block, 0, s, a); break;
        case 512: hipLaunchKernelGGL((reorg_kernel<256, false>), grid, block, 0, s, a); break;
        case 513: hipLaunchKernelGGL((reorg_kernel<256, true>), grid, block, 0, s, a); break;
        case 1024: hipLaunchKernelGGL((reorg_kernel<512, false>), grid, block, 0, s, a); break;
        case 1025: hipLaunchKernelGGL((reorg_kernel<512, true>), grid, block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace sfi
