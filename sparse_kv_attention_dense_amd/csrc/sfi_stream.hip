// sfi_stream.hip -- measurement yardsticks for the attention kernels: a plain streaming read,
// a gather read of exactly the key and value rows a fast step reads, and the GQA group's dot
// products over a stream of key rows on the vector ALUs or on MFMA.
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
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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


// Group dot yardstick: the dot products q_g . k_j of a GQA group's G query heads with every
// bf16 key row of 128 elements, the rows read in order, on one of three units.  Each wavefront
// takes groups of 16 consecutive rows (4 KB), kDotInFlight groups with every load issued
// before any is used, in all three units, so that only the arithmetic differs:
//   0  no arithmetic: the words are folded into an XOR (as the streaming read does);
//   1  vector ALUs: lane l holds elements 8 (l mod 16) ... + 7 of four rows of a group (the
//      16-byte pieces l, l + 64, l + 128, l + 192 of it); per head 8 FMAs, then the sum over
//      the row's 16 lanes with DPP row shifts (lane 15 of the row ends with the dot product);
//   2  MFMA, in the attention kernels' operand layout: lane (n, q) holds elements
//      32c + 8q ... + 7 of row n of the group for c < 4, and four 16x16x32 bf16 MFMAs against
//      Q^T (heads >= G as zero columns) give the 16 x 16 products.
// Units 1 and 2 add up their dot products per workgroup into part[workgroup], so the two can
// be checked against each other and against a host sum.
constexpr int kDotThreads = 256;
constexpr int kDotInFlight = 2;                      // 16-row groups in flight per wavefront
constexpr int kDotD = 128;                           // elements per row
constexpr int kDotGroupU4 = 16 * kDotD * 2 / 16;     // 16-byte pieces per 16-row group (256)

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

__device__ __forceinline__ float row16_shr_add(float x, int ctrl_sel) {
    const int xi = __float_as_int(x);
    int r;
    switch (ctrl_sel) {                              // row_shr 1, 2, 4, 8 (rows of 16 lanes)
        case 0: r = __builtin_amdgcn_update_dpp(0, xi, 0x111, 0xf, 0xf, false); break;
        case 1: r = __builtin_amdgcn_update_dpp(0, xi, 0x112, 0xf, 0xf, false); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, xi, 0x114, 0xf, 0xf, false); break;
        default: r = __builtin_amdgcn_update_dpp(0, xi, 0x118, 0xf, 0xf, false); break;
    }
    return x + __int_as_float(r);
}

__device__ void dot_part_store(float acc, float* part) {
    __shared__ float s_red[kDotThreads / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kDotThreads / 64; ++w) t += s_red[w];
        part[blockIdx.x] = t;
    }
}

template <int UNIT, int G>
__global__ void __launch_bounds__(kDotThreads)
group_dot_kernel(const u32x4* __restrict__ rows, uint64_t n_groups, const u32x4* __restrict__ q,
                 float* __restrict__ part, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const uint64_t wave = (uint64_t)blockIdx.x * (kDotThreads / 64) + (threadIdx.x >> 6);
    const uint64_t n_waves = (uint64_t)gridDim.x * (kDotThreads / 64);
    const int n16 = lane & 15, q4 = lane >> 4;
    // operands held for the whole stream: unit 1 the lane's 8 elements of each head (fp32),
    // unit 2 the B fragments of Q^T
    float qr[UNIT == 1 ? G : 1][8];
    u32x4 qf[4];
    if constexpr (UNIT == 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const u32x4 x = q[g * (kDotD / 8) + n16];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qr[g][2 * e] = bf16_lo(x[e]);
                qr[g][2 * e + 1] = bf16_hi(x[e]);
            }
        }
    }
    if constexpr (UNIT == 2) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            qf[c] = n16 < G ? q[n16 * (kDotD / 8) + 4 * c + q4] : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t fold = 0;
    float acc = 0.f;
    for (uint64_t s = wave; s < n_groups; s += kDotInFlight * n_waves) {
        u32x4 x[kDotInFlight][4];
        bool ok[kDotInFlight];
#pragma unroll
        for (int t = 0; t < kDotInFlight; ++t) {
            const uint64_t gs = s + t * n_waves;
            ok[t] = gs < n_groups;
            const u32x4* g0 = rows + (ok[t] ? gs : 0) * kDotGroupU4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x[t][i] = UNIT == 2 ? g0[n16 * (kDotD / 8) + 4 * i + q4] : g0[64 * i + lane];
        }
#pragma unroll
        for (int t = 0; t < kDotInFlight; ++t) {
            if constexpr (UNIT == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) fold ^= x[t][i].x ^ x[t][i].y ^ x[t][i].z ^ x[t][i].w;
            } else if constexpr (UNIT == 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float kf[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kf[2 * e] = bf16_lo(x[t][i][e]);
                        kf[2 * e + 1] = bf16_hi(x[t][i][e]);
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        float p = kf[0] * qr[g][0];
#pragma unroll
                        for (int e = 1; e < 8; ++e) p = fmaf(kf[e], qr[g][e], p);
#pragma unroll
                        for (int k = 0; k < 4; ++k) p = row16_shr_add(p, k);
                        acc += (ok[t] && n16 == 15) ? p : 0.f;
                    }
                }
            } else {
                f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x[t][c]),
                                                                __builtin_bit_cast(bf16x8, qf[c]), S,
                                                                0, 0, 0);
                acc += ok[t] ? (S[0] + S[1]) + (S[2] + S[3]) : 0.f;
            }
        }
    }
    if constexpr (UNIT == 0) {
        if (fold == 0x9e3779b9u) sink[blockIdx.x & (kStreamSinkWords - 1)] = fold;
    } else {
        dot_part_store(acc, part);
    }
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


hipError_t launch_group_dot(const void* rows, uint64_t n_rows, const void* q, int G, int unit,
                            int n_wg, float* part, uint32_t* sink, hipStream_t s) {
    const u32x4* r = (const u32x4*)rows;
    const u32x4* qq = (const u32x4*)q;
    const uint64_t n_groups = n_rows / 16;
    const dim3 grid(n_wg), blk(kDotThreads);
#define SFI_DOT(U, GG) hipLaunchKernelGGL((group_dot_kernel<U, GG>), grid, blk, 0, s, r, n_groups, qq, part, sink)
    if (unit == 0) SFI_DOT(0, 1);
    else if (unit == 2) {
        if (G == 1) SFI_DOT(2, 1); else if (G == 2) SFI_DOT(2, 2); else if (G == 4) SFI_DOT(2, 4); else SFI_DOT(2, 8);
    } else {
        if (G == 1) SFI_DOT(1, 1); else if (G == 2) SFI_DOT(1, 2); else if (G == 4) SFI_DOT(1, 4); else SFI_DOT(1, 8);
    }
#undef SFI_DOT
    return hipGetLastError();
}

}  // namespace sfi
