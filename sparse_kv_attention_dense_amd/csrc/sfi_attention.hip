// sfi_attention.hip -- split-K GQA decode attention for gfx950 (dense slow step and sparse
// fast step of Slow-Fast Inference).
//
// attention_kernel: one workgroup (4 wavefronts) owns one (batch b, KV head h, split s): a
// contiguous range of "slots".  A slot is a key position: in the dense step slot ==
// position; in the sparse step slot k < n_idx is idx[k] and the remaining slots walk the
// recent window [r0, len).  In the two-segment fast step (SFI Sec. 4.2) index slot k reads
// its rows from row (b*Hkv + h)*idx_stride + k of the compact segment written by the Reorg;
// the recent window is still read in place.  Each wavefront takes 32-slot tiles (round-robin, or a contiguous
// quarter of the split when the dense step stages its logits) and keeps an online softmax
// (m, l, acc) for the G query heads of the group:
//   - S^T = K_tile * Q^T on MFMA (v_mfma_f32_16x16x32_bf16, or 16x16x4 f32): the 16 rows of
//     the A operand are 16 key rows, read straight from HBM as 16-byte pieces, and the 16
//     columns are the (zero-padded) query heads, so each K row is read once for the group
//     (grouped-query attention without repeating K/V, SinkRouter Sec. 4.3).
//   - the fp32 logits z = S * 1/sqrt(d) go to HBM (dense step only; SFI Sec. 4.2 needs the
//     logits exposed for the Selector): staged per wavefront in LDS and written as runs of
//     at least 1 KB per head (G <= 15 at bf16 d = 128, G <= 8 otherwise), else as float4
//     stores per tile, all nontemporal.
//   - O^T += V_tile^T * P^T on MFMA; bf16 V rows are staged through LDS and read back
//     transposed, and P is split into a bf16 high part and a bf16 residual so the product
//     keeps about 16 bits of the fp32 weight.
// Each workgroup writes one partial record (acc, m, l) per query head of its group.
//
// combine_kernel: one workgroup per query head merges the records of all splits with the
// log-sum-exp rule  M = max_s m_s,  out = sum_s 2^(m_s-M) acc_s / sum_s 2^(m_s-M) l_s
// (m kept in log2 units) and writes out and lse; bypassed heads get the zero surrogate.
// The merge is a second launch on the same stream rather than an in-kernel ticket: the
// kernel boundary makes the partials visible across the chip's XCDs without per-workgroup
// L2 write-back and invalidate fences.
#include <type_traits>

#include "sfi_internal.h"

namespace sfi {
namespace {

// Loads and stores of device memory through the global address space.  The pointers of a
// step descriptor are read from device memory, so the compiler cannot tell that they point to
// global memory and would emit flat accesses for them; a flat load also counts against the LDS
// wait counter, so every LDS wait of the tile loop would then wait for the prefetched tile too.
template <class T>
__device__ __forceinline__ T gld(const T* p) {
    return *(const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ void gst(T* p, T x) {
    *(__attribute__((address_space(1))) T*)p = x;
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Splits of sequence b that hold positions: ceil(len_b / split_len), at most nsplit.
__device__ __forceinline__ int splits_of(const AttnArgs& a, int len_b) {
    return len_b > 0 ? min((len_b + a.split_len - 1) / a.split_len, a.nsplit) : 0;
}

// Finds the (b, r, splits_of(b)) of dense workgroup wg, where r = h * splits_of(b) + split
// counts the active workgroups of sequence b in order; workgroups are numbered sequence by
// sequence.  Returns false when wg is past the last active workgroup.  sh: 8 ints of LDS.
__device__ bool locate_split(const AttnArgs& a, int wg, int* sh, int* loc) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid == 0) sh[4] = -1;
    int off = 0;
    for (int base = 0; base < a.B; base += kThreads) {
        const int bb = base + tid;
        const int ns = bb < a.B ? splits_of(a, a.len[bb]) : 0;
        const int cnt = ns * a.Hkv;
        int inc = cnt;                                     // inclusive scan over the block
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o);
            if (lane >= o) inc += y;
        }
        __syncthreads();
        if (lane == 63) sh[w] = inc;
        __syncthreads();
        int before = off;
        for (int ww = 0; ww < w; ++ww) before += sh[ww];
        const int excl = before + inc - cnt;
        if (cnt > 0 && wg >= excl && wg < excl + cnt) {
            sh[4] = bb;
            sh[5] = wg - excl;
            sh[6] = ns;
        }
        off += sh[0] + sh[1] + sh[2] + sh[3];
        __syncthreads();
        if (sh[4] >= 0) break;
    }
    __syncthreads();
    loc[0] = sh[4];
    loc[1] = sh[5];
    loc[2] = sh[6];
    const bool found = loc[0] >= 0;
    __syncthreads();                                       // sh is reused by the caller
    return found;
}

constexpr int kWideCombine = 1024;                 // combine threads for many splits

// Merges the nsplit partial records of query head i of batch b into out and lse with NT
// threads.  Thread (dim, phase) folds splits phase, phase + R, ... into a running (M, L, A)
// with the log-sum-exp rule, a batch of records at a time; the R phases then merge through
// LDS (s_m, s_l, s_a: NT floats each).
template <int D, bool SPARSE, int NT>
__device__ void merge_head(const AttnArgs& a, int b, int i, float* s_m, float* s_l, float* s_a) {
    constexpr int R = NT / D;
    const int tid = threadIdx.x;
    const int G = a.G, h = i / G, g = i - h * G;
    const int S = SPARSE ? a.nsplit : splits_of(a, a.len[b]), rec = a.rec_floats;
    const float* base = a.part + (int64_t)(b * a.Hkv + h) * a.nsplit * rec;   // nsplit records per unit
    const int dim = tid % D, ph = tid / D;
    // dense step of the fused slow step: the last wavefront folds the splits' (m, l) pairs over
    // J with the same rule, its first batch of loads issued before the main merge
    constexpr int kJB = 4;                           // pairs per lane per batch
    const bool j_merge = !SPARSE && a.lse_j != nullptr && (tid >> 6) == NT / 64 - 1;
    float jm[kJB], jl[kJB];
    if (j_merge) {
#pragma unroll
        for (int u = 0; u < kJB; ++u) {
            const int sp = (tid & 63) + 64 * u;
            const float* r = base + (int64_t)(sp < S ? sp : 0) * rec + G * D + 2 * G + 2 * g;
            jm[u] = sp < S ? r[0] : -INFINITY;
            jl[u] = sp < S ? r[1] : 0.f;
        }
    }
    // Records are merged kMB per thread at a time, all loaded before any is used (one memory
    // round trip per batch); records past S read record 0 and count as empty.  Few splits (a
    // ragged batch has 2 per sequence) take small batches, so no loads are wasted.
    float M = -INFINITY, L = 0.f, A = 0.f;
    auto merge_batches = [&](auto kmb) {
        constexpr int kMB = decltype(kmb)::value;
        for (int s0 = ph; s0 < S; s0 += R * kMB) {
            float m[kMB], l[kMB], x[kMB];
#pragma unroll
            for (int u = 0; u < kMB; ++u) {
                const int s = s0 + u * R;
                const float* r = base + (int64_t)(s < S ? s : 0) * rec;
                m[u] = r[G * D + 2 * g];
                l[u] = r[G * D + 2 * g + 1];
                x[u] = r[g * D + dim];
            }
            float Mb = M;
#pragma unroll
            for (int u = 0; u < kMB; ++u) {
                if (s0 + u * R >= S) m[u] = -INFINITY;
                Mb = fmaxf(Mb, m[u]);
            }
            const float Mu = (Mb == -INFINITY) ? 0.f : Mb;   // nothing attended yet: weights 0
            const float c = exp2_fast(M - Mu);
            L *= c;
            A *= c;
#pragma unroll
            for (int u = 0; u < kMB; ++u) {
                const float w = exp2_fast(m[u] - Mu);
                L += w * l[u];
                A += w * x[u];
            }
            M = Mb;
        }
    };
    if (S <= 2 * R) merge_batches(std::integral_constant<int, 2>{});
    else if (S <= 8 * R) merge_batches(std::integral_constant<int, 8>{});
    else merge_batches(std::integral_constant<int, 16>{});
    s_m[tid] = M;
    s_l[tid] = L;
    s_a[tid] = A;
    __syncthreads();
    if (tid < D) {
        float Mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < R; ++r) Mt = fmaxf(Mt, s_m[tid + r * D]);
        const float Mu = (Mt == -INFINITY) ? 0.f : Mt;
        float Lt = 0.f, At = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float c = exp2_fast(s_m[tid + r * D] - Mu);
            Lt += c * s_l[tid + r * D];
            At += c * s_a[tid + r * D];
        }
        bool zero = !(Lt > 0.f);
        if constexpr (SPARSE) {
            if (a.head_mask) zero |= gld(a.head_mask + b * a.Hq + i) != 0;
        }
        gst(a.out + ((int64_t)b * a.Hq + i) * D + tid, zero ? 0.f : At / Lt);
        if (tid == 0 && a.lse) gst(a.lse + b * a.Hq + i, zero ? -INFINITY : (Mt + log2f(Lt)) * kLn2);
    }
    if constexpr (!SPARSE) {
        if (a.lse_j) {
            // log-sum-exp over the Selector's allowed set: the same merge over the (m, l) pairs
            // the splits kept for positions of J, by the last wavefront (one pass)
            const int lane = tid & 63;
            if (j_merge) {
                float Mj = -INFINITY, Lj = 0.f;
                auto fold = [&](float m, float l) {
                    const float Mn = fmaxf(Mj, m);
                    if (Mn == -INFINITY) return;
                    Lj = Lj * exp2_fast(Mj - Mn) + l * exp2_fast(m - Mn);
                    Mj = Mn;
                };
#pragma unroll
                for (int u = 0; u < kJB; ++u) fold(jm[u], jl[u]);
                // the rest kJB pairs per lane at a time, every load of a batch issued first
                for (int sp0 = lane + 64 * kJB; sp0 < S; sp0 += 64 * kJB) {
#pragma unroll
                    for (int u = 0; u < kJB; ++u) {
                        const int sp = sp0 + 64 * u;
                        const float* r = base + (int64_t)(sp < S ? sp : 0) * rec + G * D + 2 * G + 2 * g;
                        jm[u] = sp < S ? r[0] : -INFINITY;
                        jl[u] = sp < S ? r[1] : 0.f;
                    }
#pragma unroll
                    for (int u = 0; u < kJB; ++u) fold(jm[u], jl[u]);
                }
                for (int o = 32; o >= 1; o >>= 1) fold(__shfl_xor(Mj, o), __shfl_xor(Lj, o));
                if (lane == 0) a.lse_j[b * a.Hq + i] = Lj > 0.f ? (Mj + log2f(Lj)) * kLn2 : -INFINITY;
            }
            // the Selector's digit-0 histogram of this head's KV group starts empty
            if (g == 0 && a.sel_hist) {
                uint32_t* hh = a.sel_hist + (int64_t)(b * a.Hkv + h) * kSelHistBins;
                for (int t = tid; t < kSelHistBins; t += NT) hh[t] = 0u;
            }
        }
    }
    __syncthreads();
}

// Fast step on a device step descriptor: the per-step pointers and the recent window replace
// the launch arguments' (uniform scalar loads at kernel entry).
__device__ __forceinline__ void apply_step(AttnArgs& a) {
    const sfi_step* s = a.step;
    a.k = s->k;
    a.v = s->v;
    a.block_table = s->block_table;
    a.len = s->len;
    a.q = s->q;
    a.idx = s->idx;
    a.n_idx = s->n_idx;
    a.head_mask = s->head_mask;
    a.ck = s->seg_k;
    a.cv = s->seg_v;
    a.out = s->out;
    a.lse = s->lse;
    a.n_recent = s->n_recent;
}

// Orders this wavefront's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

constexpr int kFill = 8;             // sparse row-table slots per thread per batch
constexpr int kPreC = 3;             // index entries per thread loaded at entry (contiguous)

// Group routing of the fast step (SinkRouter Sec. 4.2-4.3): every query head g of KV group h
// is scored against the group's token-0 key, z0_g = (q_g . k_{h,0}) / sqrt(d), and the group is
// sink-dominant when every head satisfies z0_g - route_lse_g >= log(gamma), i.e. its token-0
// attention mass estimated with the cached normaliser reaches gamma.  Thread (g, c) holds 8
// elements of q_g and of k_{h,0}; route_load issues those loads at kernel entry so their latency
// overlaps the other prologue loads, route_decide reduces the D/8 threads of each head by
// shuffles and returns the same answer to every thread of the workgroup.
template <bool BF, int D>
struct RoutePre {
    using V = typename std::conditional<BF, u32x4, f32x4>::type;
    V q[BF ? 1 : 2], k[BF ? 1 : 2];
    float lse;                                         // the head's cached normaliser
};

// Stage 0 (kernel entry): the query elements, and on a contiguous cache with rows the token-0
// key elements.  Stage 1 (once len_b > 0 is known): on a paged cache the token-0 key through
// the block table (its first entry is only defined for a non-empty sequence).
template <bool BF, int D, bool PAGED>
__device__ void route_load(const AttnArgs& a, int b, int h, int hq0, int unit, int stage,
                           RoutePre<BF, D>& r) {
    constexpr int kPer = 8, kLanes = D / kPer;
    const int g = threadIdx.x / kLanes, c = threadIdx.x % kLanes;
    if (g >= a.G) return;
    const bool load_k = PAGED ? stage == 1 : (stage == 0 && a.n_cap > 0);
    if (stage == 0) {
        r.lse = a.route_lse[b * a.Hq + hq0 + g];
        const int64_t qoff = ((int64_t)b * a.Hq + hq0 + g) * D + c * kPer;
        if constexpr (BF) {
            r.q[0] = gld((const u32x4*)((const uint16_t*)a.q + qoff));
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e) r.q[e] = gld((const f32x4*)((const float*)a.q + qoff + 4 * e));
        }
    }
    if (!load_k) return;
    uint32_t row;                                      // the row of position 0
    if constexpr (PAGED)
        row = ((uint32_t)gld(a.block_table + (int64_t)b * a.max_blocks) * (uint32_t)a.Hkv + (uint32_t)h)
              << a.block_shift;
    else
        row = (uint32_t)((int64_t)unit * a.n_cap);
    if constexpr (BF) {
        r.k[0] = gld((const u32x4*)((const uint16_t*)a.k + (uint64_t)row * D + c * kPer));
    } else {
#pragma unroll
        for (int e = 0; e < 2; ++e)
            r.k[e] = gld((const f32x4*)((const float*)a.k + (uint64_t)row * D + c * kPer + 4 * e));
    }
}

template <bool BF, int D>
__device__ bool route_decide(const AttnArgs& a, int b, int hq0, const RoutePre<BF, D>& r, float* sh) {
    constexpr int kPer = 8, kLanes = D / kPer;
    const int tid = threadIdx.x, G = a.G;
    const int g = tid / kLanes, c = tid % kLanes;
    float part = 0.f;
    if (g < G) {
        if constexpr (BF) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part += __uint_as_float(r.q[0][e] << 16) * __uint_as_float(r.k[0][e] << 16);
                part += __uint_as_float(r.q[0][e] & 0xffff0000u) * __uint_as_float(r.k[0][e] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i) part += r.q[e][i] * r.k[e][i];
        }
    }
    for (int o = kLanes / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
    if (g < G && c == 0)
        sh[g] = (part * a.scale - r.lse >= a.route_log_gamma) ? 1.f : 0.f;
    __syncthreads();
    bool all = true;
    for (int gg = 0; gg < G; ++gg) all &= sh[gg] != 0.f;
    __syncthreads();
    return all;
}

// Wavefronts per workgroup: 4 in the dense step (two workgroups per CU); kSparseWaves in the
// fast step, whose launch has about one workgroup per CU, except fp32 at d = 128, whose tile
// registers allow one wavefront per SIMD only.
constexpr int waves_of(bool bf, int d, bool sparse) {
    return (sparse && (bf || d == 64)) ? kSparseWaves : kWaves;
}

template <bool BF, int D, bool PAGED, bool SPARSE>
struct Cfg {
    static constexpr int kNW = waves_of(BF, D, SPARSE);
    static constexpr int kNT = 64 * kNW;
    static constexpr int kVRow = D * 2 + 16;                       // staged bf16 row, bytes
    // The dense step stages V half a tile at a time (16 slots, k = 16 MFMAs) so that its LDS
    // holds longer logit runs; the fast step stages whole tiles (k = 32 MFMAs), which measured
    // faster there (20.2 vs 21.0 us at 128K).
    static constexpr bool kHalfV = BF && !SPARSE;
    static constexpr int kVRows = kHalfV ? kTile / 2 : kTile;      // V rows staged at a time
    static constexpr int kVStage = BF ? kNW * kVRows * kVRow : 0;
    static constexpr int kRed = kNW * kMaxG * (D + 4) * 4;         // cross-wave merge
    // dense: per-wavefront staging of fp32 logits, kZRows (head, tile) rows of 32 positions;
    // 120 rows (15 KB) for bf16 d = 128 keeps two workgroups per CU in 160 KB of LDS
    static constexpr int kZRows = (BF && D == 128) ? 120 : 64;
    static constexpr int kZWave = SPARSE ? 4 : kZRows * kTile;     // floats per wavefront
    // the cross-wave merge reuses the logit staging area when that is large enough (it runs
    // after the last run has been written), else the V staging area
    static constexpr bool kRedInZ = !SPARSE && kNW * kZWave * 4 >= kRed;
    static constexpr int kRaw0 = kRedInZ ? kVStage : (kVStage > kRed ? kVStage : kRed);
    static constexpr int kRaw = kRaw0 > 64 ? kRaw0 : 64;
    static constexpr int kNQ = BF ? D / 32 : D / 16;               // Q / K fragments per row
    static constexpr int kNV = BF ? D / 16 : 2 * 4 * (D / 16);     // V registers per tile
    static constexpr int kRPI = 1024 / (2 * D);                    // bf16 V rows per wave load
    static constexpr int kLPR = 64 / kRPI;                         // lanes per bf16 V row
    using QF = typename std::conditional<BF, u32x4, f32x4>::type;
    using VR = typename std::conditional<BF, u32x4, float>::type;
};

template <bool BF, int D, bool PAGED, bool SPARSE>
struct TileRegs {
    using C = Cfg<BF, D, PAGED, SPARSE>;
    typename C::QF k[2][C::kNQ];
    typename C::VR v[C::kNV];
};

template <bool BF, int D, bool PAGED, bool SPARSE>
__global__ void __launch_bounds__(64 * waves_of(BF, D, SPARSE),
                                  (BF || D == 64) ? 8 / waves_of(BF, D, SPARSE) : 1)
attention_kernel(AttnArgs a_in) {
    using C = Cfg<BF, D, PAGED, SPARSE>;
    AttnArgs a = a_in;
    if constexpr (SPARSE) {
        if (a.step) apply_step(a);
    }
    static_assert(SPARSE || C::kNW == kWaves, "the dense split lookup assumes four wavefronts");
    using Regs = TileRegs<BF, D, PAGED, SPARSE>;
    __shared__ __attribute__((aligned(16))) unsigned char raw[C::kRaw];
    __shared__ __attribute__((aligned(16))) float zstage[C::kNW * C::kZWave];
    // Row table in dynamic LDS, sized by the host for this launch's split length:
    //   sparse: one row per slot, then one "attend" flag byte per slot;
    //   dense paged: one base row per KV block the split touches.
    extern __shared__ __attribute__((aligned(16))) uint32_t tab[];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int q4 = lane >> 4, n16 = lane & 15;
    int split, h, b;
    if constexpr (SPARSE) {
        split = blockIdx.x;
        h = blockIdx.y;
        b = blockIdx.z;
    } else {
        // Dense: the 1-D grid enumerates only the splits that hold positions, sequence by
        // sequence, so a ragged batch does not leave idle workgroups between busy ones.
        int loc[3];
        if (!locate_split(a, blockIdx.x, (int*)raw, loc)) return;
        b = loc[0];
        h = loc[1] / loc[2];
        split = loc[1] - h * loc[2];
    }
    const int G = a.G;
    const int hq0 = h * G;
    const int unit = b * a.Hkv + h;
    const int s0 = split * a.split_len;
    // The index entries of the first kFill * C::kNT slots depend only on the slot, so their
    // loads are issued before the lengths arrive and the latencies overlap.
    int idx_pre[kFill];
    // Table slots per thread in one batch: what the split needs, at most kFill (paged only).
    const int nfill = min(kFill, (a.split_len + C::kNT - 1) / C::kNT);
    if constexpr (SPARSE && !PAGED) {
        // the first kPreC slots of this thread (the whole split up to 3 * 256 slots), so the
        // row table needs no second memory round trip (128K fast step 22.8 -> 22.3 us)
#pragma unroll
        for (int u = 0; u < kPreC; ++u) {
            const int slot = s0 + u * C::kNT + tid;
            idx_pre[u] = (u * C::kNT < a.split_len && slot < a.idx_stride)
                ? gld(a.idx + (int64_t)unit * a.idx_stride + slot) : 0;
        }
    } else if constexpr (SPARSE) {
        const int32_t* irow = a.idx + (int64_t)unit * a.idx_stride;
#pragma unroll
        for (int u = 0; u < kFill; ++u) {
            const int slot = s0 + u * C::kNT + tid;
            idx_pre[u] = (u < nfill && slot < a.idx_stride) ? gld(irow + slot) : 0;
        }
    }
    RoutePre<BF, D> route;
    if constexpr (SPARSE) {
        if (a.route_lse) route_load<BF, D, PAGED>(a, b, h, hq0, unit, 0, route);
    }
    // fast step on a paged cache with a short block table: the sequence's whole table is
    // loaded here, beside the index entries, and staged in LDS below, so the row table costs
    // one memory round trip instead of two (index, then block)
    int bt_pre[kBtPer];
    const bool bt_staged = SPARSE && PAGED && a.bt_off >= 0;
    if constexpr (SPARSE && PAGED) {
        if (bt_staged) {
#pragma unroll
            for (int u = 0; u < kBtPer; ++u) {
                const int e = u * C::kNT + tid;
                bt_pre[u] = e < a.max_blocks ? gld(a.block_table + (int64_t)b * a.max_blocks + e) : 0;
            }
        }
    }
    const int len_b = gld(a.len + b);

    // ---- slot range of this workgroup -------------------------------------------------
    int n_sel = 0, r0 = 0, n_tot = len_b;
    bool all_masked = false;
    if constexpr (SPARSE) {
        n_sel = min(max(gld(a.n_idx + unit), 0), a.idx_stride);
        r0 = max(0, len_b - a.n_recent);
        n_tot = len_b > 0 ? n_sel + (len_b - r0) : 0;
        if (a.head_mask) {
            all_masked = true;
            for (int g = 0; g < G; ++g) all_masked &= gld(a.head_mask + b * a.Hq + hq0 + g) != 0;
        }
        if (a.route_lse) {
            // inline group routing before any key or value row of the group is read
            if (PAGED && len_b > 0) route_load<BF, D, PAGED>(a, b, h, hq0, unit, 1, route);
            const bool sink = len_b > 0 && route_decide<BF, D>(a, b, hq0, route, (float*)raw);
            if (a.routed && split == 0 && tid == 0) a.routed[unit] = sink ? 1 : 0;
            all_masked |= sink;
        }
    }
    int s1 = min(n_tot, s0 + a.split_len);
    if (all_masked || len_b <= 0) s1 = s0;
    const int nslots = max(0, s1 - s0);

    const uint32_t base_row = PAGED ? 0u : (uint32_t)((int64_t)unit * a.n_cap);
    // Two-segment fast step (compact long-range segment): index slot s of the unit reads row
    // unit * idx_stride + s of ck / cv instead of gathering its position from the cache.
    const bool compact = SPARSE && a.ck != nullptr;
    const uint32_t crow0 = (uint32_t)unit * (uint32_t)a.idx_stride;

    const int bmask = (1 << a.block_shift) - 1;
    uint8_t* tab_ok = (uint8_t*)(tab + a.split_len);
    int32_t* s_bt = (int32_t*)((unsigned char*)tab + (a.bt_off > 0 ? a.bt_off : 0));
    if constexpr (SPARSE && PAGED) {
        if (bt_staged) {
#pragma unroll
            for (int u = 0; u < kBtPer; ++u) {
                const int e = u * C::kNT + tid;
                if (e < a.max_blocks) s_bt[e] = bt_pre[u];
            }
        }
        __syncthreads();
    }
    if constexpr (SPARSE) {
        const int32_t* irow = a.idx + (int64_t)unit * a.idx_stride;
        if constexpr (!PAGED) {
            for (int t = tid; t < nslots; t += C::kNT) {
                const int slot = s0 + t;
                int pos;
                bool ok = true;
                if (slot < n_sel) {
                    const int u = (t - tid) / C::kNT;       // this thread's u-th slot
                    bool pre = false;
#pragma unroll
                    for (int v = 0; v < kPreC; ++v)         // static indices: idx_pre stays
                        if (u == v) {                       // in registers
                            pos = idx_pre[v];
                            pre = true;
                        }
                    if (!pre) pos = gld(irow + slot);
                    ok = pos >= 0 && pos < r0;
                    if (!ok) pos = len_b - 1;
                } else {
                    pos = r0 + (slot - n_sel);
                }
                tab_ok[t] = ok;
                tab[t] = (compact && slot < n_sel) ? crow0 + (uint32_t)slot : base_row + (uint32_t)pos;
            }
        }
        // Paged: slots are filled nfill per thread at a time; every index load of a batch is
        // issued before any is used, then every block-table load, so a batch costs two memory
        // round trips however many slots it holds (3% faster fast steps on a ragged batch;
        // on a contiguous cache the plain loop above measured faster).
        for (int t0 = 0; PAGED && t0 < nslots; t0 += nfill * C::kNT) {
            int pos[kFill];
            bool ok[kFill];
#pragma unroll
            for (int u = 0; u < kFill; ++u) {
                const int t = t0 + u * C::kNT + tid;
                const int slot = s0 + t;
                ok[u] = true;
                pos[u] = 0;
                if (u < nfill && t < nslots) {
                    if (slot < n_sel) {
                        pos[u] = t0 == 0 ? idx_pre[u] : gld(irow + slot);
                        ok[u] = pos[u] >= 0 && pos[u] < r0;
                        if (!ok[u]) pos[u] = len_b - 1;
                    } else {
                        pos[u] = r0 + (slot - n_sel);
                    }
                }
            }
            uint32_t row[kFill];
#pragma unroll
            for (int u = 0; u < kFill; ++u) {
                if constexpr (PAGED) {
                    const int t = t0 + u * C::kNT + tid;
                    const bool crow = compact && s0 + t < n_sel;     // compact row: no lookup
                    const int blk = (u < nfill && t < nslots && !crow)
                        ? (bt_staged ? s_bt[pos[u] >> a.block_shift]
                                     : gld(a.block_table + (int64_t)b * a.max_blocks + (pos[u] >> a.block_shift)))
                        : 0;
                    row[u] = crow ? crow0 + (uint32_t)(s0 + t)
                                  : (((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)h) << a.block_shift) |
                                        (uint32_t)(pos[u] & bmask);
                } else {
                    row[u] = base_row + (uint32_t)pos[u];
                }
            }
#pragma unroll
            for (int u = 0; u < kFill; ++u) {
                const int t = t0 + u * C::kNT + tid;
                if (u < nfill && t < nslots) {
                    tab_ok[t] = ok[u];
                    tab[t] = row[u];
                }
            }
        }
        __syncthreads();
    } else if constexpr (PAGED) {
        // blocks [s0 >> shift, (s1 - 1) >> shift] of sequence b
        const int blk0 = s0 >> a.block_shift;
        const int nblk = nslots > 0 ? ((s1 - 1) >> a.block_shift) - blk0 + 1 : 0;
        for (int t = tid; t < nblk; t += C::kNT) {
            const int blk = gld(a.block_table + (int64_t)b * a.max_blocks + blk0 + t);
            tab[t] = ((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)h) << a.block_shift;
        }
        __syncthreads();
    }

    auto slot_row = [&](int slot) -> uint32_t {     // slot in [s0, s1)
        if constexpr (SPARSE) return tab[slot - s0];
        else if constexpr (PAGED)
            return tab[(slot >> a.block_shift) - (s0 >> a.block_shift)] | (uint32_t)(slot & bmask);
        else return base_row + (uint32_t)slot;
    };
    auto slot_ok = [&](int slot) -> bool {
        if (slot >= s1) return false;
        if constexpr (SPARSE) return tab_ok[slot - s0] != 0;
        else return true;
    };

    // ---- query fragments (B operand of S^T = K Q^T); heads >= G are zero columns ---------
    typename C::QF qf[C::kNQ];
    {
        const bool has = n16 < G;
        const int64_t qoff = ((int64_t)b * a.Hq + hq0 + (has ? n16 : 0)) * D;
#pragma unroll
        for (int c = 0; c < C::kNQ; ++c) {
            if constexpr (BF) {
                const uint16_t* qp = (const uint16_t*)a.q + qoff;
                qf[c] = has ? gld((const u32x4*)(qp + 32 * c + 8 * q4)) : u32x4{0u, 0u, 0u, 0u};
            } else {
                const float* qp = (const float*)a.q + qoff;
                qf[c] = has ? gld((const f32x4*)(qp + 16 * c + 4 * q4)) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    // dense step of sfi_slow_step: the same online sums over the positions of the Selector's
    // allowed set J = [n_sink, len_b - n_recent) only (for its log-sum-exp over J)
    const bool track_j = !SPARSE && a.lse_j != nullptr;
    const int j_lo = a.n_sink, j_hi = len_b - a.n_recent;
    float mj_run = -INFINITY, lj_run = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

    unsigned char* vstage = raw + w * C::kVRows * C::kVRow;

    // Tiles of this wavefront.  Logits in runs: when a run holds at least 8 tiles (kZRows / G
    // >= 8: G <= 15 at bf16 d = 128, G <= 8 otherwise) the wavefront takes a contiguous
    // quarter of the split, stages its logits in LDS and writes kZRows / G tiles at a time,
    // runs of 1 KB or more per head instead of 128 B per tile (3.75 KB at G = 4), with
    // nontemporal stores (HBM3E turns short writes mixed into the read stream into lost read
    // bandwidth; on MI355X the runs, the store policy and the half-tile V staging that makes
    // room for them take the dense step at 128K from 428 to about 362 us).  Larger groups
    // would get runs under 1 KB; they take tiles w, w + 4, ... and write each tile's logits
    // directly, as does the sparse kernel (no logits).
    // The tile order depends on G only, so out and lse do not depend on whether logits are
    // requested.
    const int zF = C::kZRows / G;                     // tiles per staged run
    const bool quarters = !SPARSE && zF >= 8;
    const bool staged = quarters && a.logits;
    const int ntiles = (nslots + kTile - 1) / kTile;
    const int tpw = (ntiles + C::kNW - 1) / C::kNW;
    const int t_begin = quarters ? min(ntiles, w * tpw) : w;
    const int t_end = quarters ? min(ntiles, t_begin + tpw) : ntiles;
    const int t_step = quarters ? 1 : C::kNW;
    float* zst = staged ? zstage + w * C::kZWave : nullptr;
    float* logit_row = nullptr;                       // unstaged logits of head n16
    if constexpr (!SPARSE) {
        if (a.logits && !staged && n16 < G) logit_row = a.logits + ((int64_t)b * a.Hq + hq0 + n16) * a.logit_stride;
    }
    // Writes the staged logits of tiles [t_first, t_first + nt) of this wavefront.
    auto flush_logits = [&](int t_first, int nt) {
        wave_lds_sync();
        const int p_first = s0 + t_first * kTile;
        const int n4 = nt * (kTile / 4);              // float4 per head
        for (int e = lane; e < G * n4; e += 64) {
            const int g = e / n4, o4 = e - g * n4;
            const int p = p_first + 4 * o4;
            const f32x4 z = *(const f32x4*)(zst + g * zF * kTile + 4 * o4);
            float* dst = a.logits + ((int64_t)b * a.Hq + hq0 + g) * a.logit_stride + p;
            if (p + 3 < s1) {
                __builtin_nontemporal_store(z, (f32x4*)dst);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (p + i < s1) dst[i] = z[i];
            }
        }
        wave_lds_sync();                              // the run is read before it is reused
    };

    // ---- tile loads (issued one tile ahead of the math) ------------------------------------
    // Cache policy of the V loads, chosen by measurement on MI355X: nontemporal V loads make
    // the dense step 3-4 % faster (128K: 416 -> 403 us; 512K: 466 -> 449).  In the fast step
    // they gain nothing in the benchmark's rotation of layers (contiguous 128K 20.8 us either
    // way, ragged paged batch 31.0 vs 31.1 us), so it keeps ordinary loads.  Nontemporal K
    // loads (the K rows are read in the MFMA operand layout, 64 bytes from each of 16 rows
    // per wavefront load) slowed every step, so K loads stay ordinary.
    constexpr bool kNtV = !SPARSE;
    auto load_k = [](const void* p) -> u32x4 { return gld((const u32x4*)p); };
    auto load_v = [](const void* p) -> u32x4 {
        if constexpr (kNtV)
            return __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)p);
        else return gld((const u32x4*)p);
    };
    using Elem = typename std::conditional<BF, uint16_t, float>::type;
    // first element of the key (or value) row of a slot: the compact segment for index slots
    // of a two-segment step, else the cache
    auto row_ptr = [&](int slot, const void* cache, const void* seg) -> const Elem* {
        const void* base = cache;
        if constexpr (SPARSE) {
            if (compact && slot < n_sel) base = seg;
        }
        return (const Elem*)base + (uint64_t)slot_row(slot) * D;
    };
    // tile < 0: past the wavefront's last tile.  Every lane then reads the split's first row,
    // so the number of loads is the same on every path (the wait before the math covers only
    // the current tile) while the extra loads touch a few cache lines instead of a whole tile.
    auto issue = [&](Regs& r, int tile) {
        const bool idle = tile < 0;
        const int sb = s0 + (idle ? 0 : tile * kTile);
        auto pick = [&](int slot) { return idle ? s0 : min(slot, s1 - 1); };
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            const Elem* kp = row_ptr(pick(sb + 16 * st + n16), a.k, a.ck);
#pragma unroll
            for (int c = 0; c < C::kNQ; ++c) {
                if constexpr (BF) r.k[st][c] = load_k(kp + 32 * c + 8 * q4);
                else r.k[st][c] = gld((const f32x4*)(kp + 16 * c + 4 * q4));
            }
        }
        if constexpr (BF) {
#pragma unroll
            for (int j = 0; j < C::kNV; ++j) {
                const int rr = j * C::kRPI + lane / C::kLPR;
                r.v[j] = load_v(row_ptr(pick(sb + rr), a.v, a.cv) + (lane % C::kLPR) * 8);
            }
        } else {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float* vp = row_ptr(pick(sb + 16 * st + 4 * q4 + i), a.v, a.cv);
#pragma unroll
                    for (int mb = 0; mb < D / 16; ++mb) r.v[(st * 4 + i) * (D / 16) + mb] = gld(vp + 16 * mb + n16);
                }
        }
    };

    // ---- tile math ----------------------------------------------------------------------
    auto compute = [&](Regs& r, int tile) {
        const int sb = s0 + tile * kTile;
        if constexpr (BF) {
#pragma unroll
            for (int j = 0; j < (C::kHalfV ? C::kNV / 2 : C::kNV); ++j) {   // rows staged first
                const int rr = j * C::kRPI + lane / C::kLPR;
                *(u32x4*)(vstage + rr * C::kVRow + (lane % C::kLPR) * 16) = r.v[j];
            }
        }
        f32x4 S[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            S[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < C::kNQ; ++c) {
                if constexpr (BF) {
                    S[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, r.k[st][c]), __builtin_bit_cast(bf16x8, qf[c]),
                        S[st], 0, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[st] = __builtin_amdgcn_mfma_f32_16x16x4f32(r.k[st][c][e], qf[c][e], S[st], 0, 0, 0);
                }
            }
        }
        // scores of this lane: head n16, slots sb + 16*st + 4*q4 + i
        float sv[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = slot_ok(sb + 16 * st + 4 * q4 + i);
                sv[st][i] = ok ? S[st][i] * a.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, sv[st][i]);
            }
        if constexpr (!SPARSE) {
            if (zst) {
                const int slot = (tile - t_begin) % zF;
                if (n16 < G) {
#pragma unroll
                    for (int st = 0; st < 2; ++st)
                        *(f32x4*)(zst + n16 * zF * kTile + slot * kTile + 16 * st + 4 * q4) = S[st] * a.scale;
                }
                if (slot == zF - 1 || tile + 1 == t_end) flush_logits(tile - slot, slot + 1);
            } else if (logit_row) {
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    const int p0 = sb + 16 * st + 4 * q4;
                    const f32x4 z = S[st] * a.scale;
                    if (p0 + 3 < s1) {
                        __builtin_nontemporal_store(z, (f32x4*)(logit_row + p0));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (p0 + i < s1) logit_row[p0 + i] = z[i];
                    }
                }
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_run_prev = m_run;
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_fast(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb) acc[mb] *= alpha;
        float p[2][4];
        float psum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[st][i] = exp2_fast(sv[st][i] - m_use);
                psum += p[st][i];
            }
        l_run += psum;
        // a tile wholly inside J whose head's J maximum so far is the overall one (every tile
        // of a split without sink or recent positions) updates the J sums exactly as the
        // plain ones: same maximum, same weights
        const bool j_same = track_j && sb >= j_lo && sb + kTile <= j_hi && mj_run == m_run_prev;
        if (j_same) {
            lj_run = lj_run * alpha + psum;
            mj_run = m_new;
        } else if (track_j) {
            float tj = -INFINITY;
            bool inj[2][4];
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int slot = sb + 16 * st + 4 * q4 + i;
                    inj[st][i] = slot >= j_lo && slot < j_hi && sv[st][i] != -INFINITY;
                    if (inj[st][i]) tj = fmaxf(tj, sv[st][i]);
                }
            tj = fmaxf(tj, __shfl_xor(tj, 16));
            tj = fmaxf(tj, __shfl_xor(tj, 32));
            const float mj_new = fmaxf(mj_run, tj);
            const float mj_use = (mj_new == -INFINITY) ? 0.f : mj_new;
            lj_run *= exp2_fast(mj_run - mj_use);
            mj_run = mj_new;
            // where J's running maximum is the overall one (every split without sink or recent
            // positions) the weights are the ones just computed
            const bool same = mj_use == m_use;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (inj[st][i]) lj_run += same ? p[st][i] : exp2_fast(sv[st][i] - mj_use);
        }
        if constexpr (BF && !C::kHalfV) {
            // P^T as the B operand: virtual k = 8*q4 + e maps to slot 4*q4 + e of block 0
            // (e < 4) or of block 1 (e >= 4); the V^T A operand uses the same map.
            bf16x8 ph, pl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pv = e < 4 ? p[0][e] : p[1][e - 4];
                const __bf16 hi = (__bf16)pv;
                ph[e] = hi;
                pl[e] = (__bf16)(pv - (float)hi);
            }
            wave_lds_sync();
            const uint16_t* vb16 = (const uint16_t*)vstage;
#pragma unroll
            for (int mb = 0; mb < D / 16; ++mb) {
                u16x8 va;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int tok = e < 4 ? 4 * q4 + e : 16 + 4 * q4 + (e - 4);
                    va[e] = vb16[tok * (C::kVRow / 2) + 16 * mb + n16];
                }
                const bf16x8 vab = __builtin_bit_cast(bf16x8, va);
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vab, ph, acc[mb], 0, 0, 0);
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vab, pl, acc[mb], 0, 0, 0);
            }
        } else if constexpr (BF) {
            // V in two halves of 16 slots, each staged through LDS and read back transposed as
            // the A operand of a k = 16 MFMA whose B operand is P^T for the same slots: lane
            // (q4, n16) holds slots 16*st + 4*q4 + i of head n16.  P is split into a bf16 high
            // part and a bf16 residual (two MFMAs) to keep about 16 bits of the weight.
            const uint16_t* vb16 = (const uint16_t*)vstage;
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if (st == 1) {
                    wave_lds_sync();                    // half 0 is read before it is replaced
#pragma unroll
                    for (int j = C::kNV / 2; j < C::kNV; ++j) {
                        const int rr = j * C::kRPI + lane / C::kLPR - kTile / 2;
                        *(u32x4*)(vstage + rr * C::kVRow + (lane % C::kLPR) * 16) = r.v[j];
                    }
                }
                s16x4 ph, pl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const __bf16 hi = (__bf16)p[st][i];
                    ph[i] = __builtin_bit_cast(short, hi);
                    pl[i] = __builtin_bit_cast(short, (__bf16)(p[st][i] - (float)hi));
                }
                wave_lds_sync();
#pragma unroll
                for (int mb = 0; mb < D / 16; ++mb) {
                    s16x4 va;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        va[i] = (short)vb16[(4 * q4 + i) * (C::kVRow / 2) + 16 * mb + n16];
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, ph, acc[mb], 0, 0, 0);
                    acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pl, acc[mb], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int mb = 0; mb < D / 16; ++mb)
                        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            r.v[(st * 4 + i) * (D / 16) + mb], p[st][i], acc[mb], 0, 0, 0);
        }
    };

    // ---- main loop over [t_begin, t_end) in steps of t_step; loads run one tile ahead --------
    // The next tile's loads are issued unconditionally (past the end as idle loads of one
    // row, see issue), so the number of loads younger than the current tile's is the same on
    // every path and the wait before the math only covers the current tile.
    if (t_begin < t_end) {
        Regs ra, rb;
        int t = t_begin;
        issue(ra, t);
        for (;;) {
            int tn = t + t_step;
            issue(rb, tn < t_end ? tn : -1);
            compute(ra, t);
            if (tn >= t_end) break;
            t = tn;
            tn = t + t_step;
            issue(ra, tn < t_end ? tn : -1);
            compute(rb, t);
            if (tn >= t_end) break;
            t = tn;
        }
    }
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    lj_run += __shfl_xor(lj_run, 16);
    lj_run += __shfl_xor(lj_run, 32);

    // ---- merge the four wavefronts, write this split's partial -----------------------------
    // per wavefront and head: acc [D], (m, l), (m, l) over J
    constexpr int kRS = D + 4;
    __syncthreads();
    float* red = C::kRedInZ ? zstage : (float*)raw;   // [kNW][kMaxG][D+4]
    if (n16 < G) {
        float* rp = red + (w * kMaxG + n16) * kRS;
#pragma unroll
        for (int mb = 0; mb < D / 16; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) rp[16 * mb + 4 * q4 + i] = acc[mb][i];
        if (q4 == 0) {
            rp[D] = m_run;
            rp[D + 1] = l_run;
            rp[D + 2] = mj_run;
            rp[D + 3] = lj_run;
        }
    }
    __syncthreads();
    {
        float* part = a.part + ((int64_t)unit * a.nsplit + split) * a.rec_floats;
        for (int e = tid; e < G * D; e += C::kNT) {
            const int g = e / D, dim = e - g * D;
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < C::kNW; ++ww) M = fmaxf(M, red[(ww * kMaxG + g) * kRS + D]);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            float s = 0.f;
#pragma unroll
            for (int ww = 0; ww < C::kNW; ++ww)
                s += exp2_fast(red[(ww * kMaxG + g) * kRS + D] - Mu) * red[(ww * kMaxG + g) * kRS + dim];
            part[e] = s;
        }
        // (m, l) of every head, and with lse_j the (m, l) over J after them
        const int npair = track_j ? 2 * G : G;
        if (tid < npair) {
            const int g = tid % G, off = tid < G ? D : D + 2;
            float M = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < C::kNW; ++ww) M = fmaxf(M, red[(ww * kMaxG + g) * kRS + off]);
            const float Mu = (M == -INFINITY) ? 0.f : M;
            float L = 0.f;
#pragma unroll
            for (int ww = 0; ww < C::kNW; ++ww)
                L += exp2_fast(red[(ww * kMaxG + g) * kRS + off] - Mu) * red[(ww * kMaxG + g) * kRS + off + 1];
            part[G * D + 2 * tid] = M;
            part[G * D + 2 * tid + 1] = L;
        }
    }
}

// One workgroup of NT threads per query head (blockIdx.x) of batch blockIdx.y merges the
// split records.
template <int D, bool SPARSE, int NT>
__global__ void __launch_bounds__(NT) combine_kernel(AttnArgs a_in) {
    __shared__ float s_m[NT], s_l[NT], s_a[NT];
    AttnArgs a = a_in;
    if constexpr (SPARSE) {
        if (a.step) apply_step(a);
    }
    merge_head<D, SPARSE, NT>(a, blockIdx.y, blockIdx.x, s_m, s_l, s_a);
}

template <bool BF, int D, bool PAGED, bool SPARSE>
hipError_t launch_one(const AttnArgs& a, int B, hipStream_t stream) {
    const dim3 grid = SPARSE ? dim3(a.nsplit, a.Hkv, B) : dim3(a.nsplit * a.Hkv * B);
    hipLaunchKernelGGL((attention_kernel<BF, D, PAGED, SPARSE>), grid,
                       dim3(Cfg<BF, D, PAGED, SPARSE>::kNT),
                       (size_t)a.tab_bytes, stream, a);
    // a head's records merge in one batch of loads per thread up to 16 * NT / D records: past
    // 16 * kThreads / D (32 at d = 128; the dense step of one sequence at 512K has 128 per
    // head, a single KV head's 1024) the merge takes 1024 threads
    if (a.nsplit > 16 * (kThreads / D))
        hipLaunchKernelGGL((combine_kernel<D, SPARSE, kWideCombine>), dim3(a.Hq, B), dim3(kWideCombine), 0, stream, a);
    else
        hipLaunchKernelGGL((combine_kernel<D, SPARSE, kThreads>), dim3(a.Hq, B), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

template <bool BF, int D>
hipError_t launch_layout(const AttnArgs& a, int B, bool paged, bool sparse, hipStream_t s) {
    if (paged) return sparse ? launch_one<BF, D, true, true>(a, B, s) : launch_one<BF, D, true, false>(a, B, s);
    return sparse ? launch_one<BF, D, false, true>(a, B, s) : launch_one<BF, D, false, false>(a, B, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int B, int d, bool bf16, bool paged, bool sparse,
                            hipStream_t stream) {
    if (bf16) {
        if (d == 128) return launch_layout<true, 128>(a, B, paged, sparse, stream);
        if (d == 64) return launch_layout<true, 64>(a, B, paged, sparse, stream);
    } else {
        if (d == 128) return launch_layout<false, 128>(a, B, paged, sparse, stream);
        if (d == 64) return launch_layout<false, 64>(a, B, paged, sparse, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace sfi
