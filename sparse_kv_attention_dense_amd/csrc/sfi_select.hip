// sfi_select.hip -- the Selector of Slow-Fast Inference at decode, and the sink-bypass mask.
//
// Selector (SFI Sec. 3.2, evidence from the slow-step logits over the allowed set J with a
// window of one query; Sec. 3.3, Top-K per KV head; prior and refinements off).  Chunked path
// (long contexts):
//   1. lse_kernel         partial log-sum-exp of each query head's logits over a 4096-wide
//                          chunk of J (also clears the digit-0 histogram of the group); not
//                          launched in the fused slow step, whose dense step already gives the
//                          log-sum-exp over J and clears the histograms
//   2. evidence_kernel    f(j) = sum_{i in group} exp(z_ij - LSE_J,i) for the chunk, stored as
//                          uint32 keys (the bit pattern of a non-negative float orders like
//                          the float), plus a histogram of digit 0 (key bits 30..19)
//   3. candidate_kernel   per chunk: the digit-0 bin that holds the k-th largest key (every
//                          workgroup scans the unit's histogram), then the keys of that bin
//                          compacted into the chunk's region, and the number of keys in
//                          higher bins; when finish_kernel follows, every key of that bin or
//                          above, with its position
//   4'. finish_kernel     (instead of 4 and 5 when a unit's kept keys and candidates fit in
//                          its LDS: k_sel + max_len / 64 <= 16384) one workgroup per unit:
//                          the entries of every chunk copied to LDS in position order, digits
//                          1 and 2 of T over the entries of the digit-0 bin, then the ordered
//                          emit over the entries
//   4. resolve_kernel     one workgroup per unit: digits 1 and 2 (bits 18..9, 8..0) over the
//                          candidates give the key T of the k-th largest evidence and how many
//                          keys equal to T are kept; then the per-chunk numbers of kept keys
//                          above T and equal to T
//   5. emit_kernel        ordered compaction.  Position j of J is kept when key > T, or
//                          key == T and fewer than k_rem earlier positions have key == T (ties
//                          go to the lower position); kept positions are written in ascending
//                          order after the sink positions [0, min(n_sink, N)).
// The one-launch path (select_unit_kernel, short contexts) does the same in one workgroup per
// (b, KV head).
// Full Selector (refine mode, SFI Sec. 3.2 prior and reverse-KL fusion, Sec. 3.3 Soft-NMS and
// cross-head exclusivity; the pages' formulas are lost and the library implements stated
// readings of them): the evidence pass stores log2(f^(1-lam) r^lam) per position and sums
// f^(1-lam) r^lam per chunk instead of building the histogram, then
//   refine_kernel        per sequence and half chunk, for every KV head: s = f^(1-lam) r^lam / Z
//                         per position (from the log2 scores the evidence pass stored, and its two
//                         neighbours'), decayed by 1 - alpha_soft
//                         when a neighbour in J is larger; then every KV head below the largest
//                         at a position is decayed by 1 - alpha_cross; the results are the
//                         keys, and the digit-0 histograms are built from them
// before the candidate pass and the finish (or the resolve and emit passes), which are
// unchanged.
// f is computed without the 1/G factor: a positive common scale does not change the order.
//
// Sink-bypass mask (SinkRouter Sec. 4.2): rank the query heads of each sequence by their
// token-0 log-mass z_i0 - lse_i (the log of p0, same order as p0) and flag the first n_mask.
#include "sfi_internal.h"

namespace sfi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPerThread = kSelChunk / kThreads;     // 16 positions per thread
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
// One-launch path: key digits of 11, 11 and 10 bits (LDS histograms of kRadixBins).
constexpr int kShift[3] = {21, 10, 0};
constexpr uint32_t kDigitMask[3] = {0x7ffu, 0x7ffu, 0x3ffu};
// Chunked path: keys are non-negative floats, so bit 31 is zero; digit 0 is bits 30..19
// (exponent and 4 mantissa bits: bins of 1/16 octave, so the bin at the k-th largest key holds
// few keys), then bits 18..9 and 8..0.
constexpr int kCBins0 = kSelHistBins;
constexpr int kCShift[3] = {19, 9, 0};
constexpr uint32_t kCMask[3] = {0xfffu, 0x3ffu, 0x1ffu};

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
// inclusive prefix sum over the 64 lanes of a wave: DPP row shifts within each row of 16
// lanes, then the broadcasts of lane 15 into row 1 (and row 1's into 2 and 3 via lane 31)
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return x;
}
__device__ __forceinline__ uint32_t wave_sum_u(uint32_t x) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}
// x of the previous lane (lane 0 gets `first`) and of the next lane (lane 63 gets `last`): the
// whole-wave DPP shifts by one lane
__device__ __forceinline__ float lane_prev(float x, float first) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(first), __float_as_int(x),
                                                      0x138, 0xf, 0xf, false));   // wave_shr:1
}
__device__ __forceinline__ float lane_next(float x, float last) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(last), __float_as_int(x),
                                                      0x130, 0xf, 0xf, false));   // wave_shl:1
}

// Exclusive prefix sum over the kW wavefronts of a workgroup in thread order, with the total,
// in one barrier: the wave totals alternate between two rows of wt, and a wave can only reach
// the scan after next once every wave has read this one's totals (at the next scan's barrier).
// parity starts at 0 and is kept by the caller.
template <int kW>
__device__ __forceinline__ uint32_t scan_total(uint32_t x, uint32_t (&wt)[2][kW], int& parity,
                                               uint32_t* tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(x);
    uint32_t* row = wt[parity];
    parity ^= 1;
    if (lane == 63) row[w] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int ww = 0; ww < kW; ++ww) {
        const uint32_t t = row[ww];
        before += ww < w ? t : 0u;
        all += t;
    }
    *tot = all;
    return before + inc - x;
}

// Block-wide reductions over the 256 threads (4 wavefronts).
__device__ float block_max(float x, float* sh) {
    x = wave_max(x);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    x = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
    __syncthreads();
    return x;
}
__device__ float block_sum(float x, float* sh) {
    x = wave_sum(x);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    x = (sh[0] + sh[1]) + (sh[2] + sh[3]);
    __syncthreads();
    return x;
}
__device__ uint32_t block_sum_u(uint32_t x, uint32_t* sh) {
    x = wave_sum_u(x);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = x;
    __syncthreads();
    x = sh[0] + sh[1] + sh[2] + sh[3];
    __syncthreads();
    return x;
}

// Exclusive prefix sum over the 256 threads in thread order.
__device__ uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(x);
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    uint32_t before = 0;
    for (int ww = 0; ww < w; ++ww) before += sh[ww];
    __syncthreads();
    return before + inc - x;
}

struct Range {
    int N, j0, j1, nJ;
};
__device__ __forceinline__ Range j_range(const SelArgs& a, int b) {
    Range r;
    r.N = a.len[b];
    r.j0 = a.n_sink;
    r.j1 = r.N - a.n_recent;
    r.nJ = max(0, r.j1 - r.j0);
    return r;
}

__global__ void __launch_bounds__(kThreads) lse_kernel(SelArgs a) {
    __shared__ float sh[4];
    const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int h = i / a.G;
    const int unit = b * a.Hkv + h;
    if (c == 0 && i % a.G == 0) {
        uint32_t* hh = a.hist + (int64_t)unit * kCBins0;
        for (int t = tid; t < kCBins0; t += kThreads) hh[t] = 0u;
    }
    const Range r = j_range(a, b);
    const int lo = r.j0 + c * kSelChunk;
    const int hi = min(r.j1, lo + kSelChunk);
    // 16-byte loads from the multiple of 4 at or below lo (rows are 16-byte aligned and their
    // stride is a multiple of 4, so every load stays inside the row); positions outside
    // [lo, hi) count as -inf.
    const float* z = a.logits + ((int64_t)b * a.Hq + i) * a.logit_stride;
    const int base = lo & ~3;
    const int n4 = hi > lo ? (hi - base + 3) >> 2 : 0;
    constexpr int kV4 = kPerThread / 4 + 1;             // covers kSelChunk + 3 positions
    f32x4 v[kV4];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < kV4; ++k) {
        const int f = k * kThreads + tid;
        v[k] = f < n4 ? *(const f32x4*)(z + base + 4 * f) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = base + 4 * f + e;
            if (f >= n4 || j < lo || j >= hi) v[k][e] = -INFINITY;
            m = fmaxf(m, v[k][e]);
        }
    }
    m = block_max(m, sh);
    float s = 0.f;
    if (m != -INFINITY) {
        const float m2 = m * kLog2e;
#pragma unroll
        for (int k = 0; k < kV4; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += exp2_hw(fmaf(v[k][e], kLog2e, -m2));
    }
    s = block_sum(s, sh);
    if (tid == 0) a.lse_part[((int64_t)b * a.Hq + i) * a.nchunk + c] = make_float2(m, s);
}

// log2 of the unnormalised prior weight of position j (J = [j0, j0 + nJ)) for unit `unit`:
// a global decay over J, a brake over its last tail_frac, and the inverse key norm.
__device__ __forceinline__ float prior_log2_n(const SelArgs& a, int j, int j0, int nJ, float nrm);
__device__ __forceinline__ float prior_log2(const SelArgs& a, int unit, int j, int j0, int nJ) {
    const float nrm = a.key_norm ? a.key_norm[(int64_t)unit * a.norm_stride + j] : 1.f;
    return prior_log2_n(a, j, j0, nJ, nrm);
}

// the same with the key norm already loaded (1 when there are no norms)
__device__ __forceinline__ float prior_log2_n(const SelArgs& a, int j, int j0, int nJ, float nrm) {
    const float u = ((float)(j - j0) + 0.5f) / (float)nJ;
    float e = -a.prior_decay * u;
    if (a.tail_frac > 0.f) e -= a.tail_brake * fmaxf(0.f, u - (1.f - a.tail_frac)) / a.tail_frac;
    float l = e * kLog2e;
    if (a.key_norm) l -= __log2f(fmaxf(nrm, 1e-6f));
    return l;
}

// log2 of f^(1-lam) r^lam (unnormalised; f without the 1/G factor, r without its sum)
__device__ __forceinline__ float fused_log2(const SelArgs& a, float f, float lr) {
    return (1.f - a.lam) * __log2f(f) + a.lam * lr;
}

// Evidence of one 4096-position chunk of J for one (KV head, sequence): thread t takes the
// position quads t, t + 256, ... (16-byte loads from the multiple of 4 at or below the chunk's
// start), four query heads at a time with every load of the four heads issued before any is
// used; positions outside the chunk are masked.
constexpr int kEvQ = kPerThread / 4 + 1;               // quads per thread (kSelChunk + 3 positions)
template <bool REFINE>
__global__ void __launch_bounds__(kThreads, 4) evidence_kernel(SelArgs a) {
    __shared__ float s_lse[kMaxSelG];
    __shared__ uint32_t lh[kCBins0];
    __shared__ float sh[4];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int G = a.G;
    const int unit = b * a.Hkv + h;
    const Range r = j_range(a, b);
    const int lo = r.j0 + c * kSelChunk;
    const int hi = min(r.j1, lo + kSelChunk);
    if (lo >= hi) return;
    const float* zb = a.logits + ((int64_t)b * a.Hq + h * G) * a.logit_stride;
    const int base = lo & ~3;
    const int n4 = (hi - base + 3) >> 2;
    // the dense step's log-sum-exp over J first (its wait then covers only itself), then the
    // first four heads' quads, in flight before the normalisers are known
    const float lse_j = (!REFINE && a.lse_j && tid < G) ? a.lse_j[(int64_t)b * a.Hq + h * G + tid]
                                                        : 0.f;
    f32x4 v[4][kEvQ];
    auto load4 = [&](int g0) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const float* z = zb + (int64_t)min(g0 + gg, G - 1) * a.logit_stride + base;
#pragma unroll
            for (int k = 0; k < kEvQ; ++k) {
                const int f = k * kThreads + tid;
                v[gg][k] = f < n4 ? *(const f32x4*)(z + 4 * f) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    load4(0);
    if (!REFINE)
        for (int t = tid; t < kCBins0; t += kThreads) lh[t] = 0u;
    // the dense step of the slow step gave the log-sum-exp over J (the full Selector is always
    // called on its own and computes it from the chunks' partial sums)
    const bool have_lse_j = !REFINE && a.lse_j;
    if (have_lse_j && tid < G) s_lse[tid] = lse_j * kLog2e;
    for (int g = w; !have_lse_j && g < G; g += kWaves) {
        const float2* lp = a.lse_part + ((int64_t)b * a.Hq + h * G + g) * a.nchunk;
        float M = -INFINITY;
        for (int k = lane; k < a.nchunk; k += 64) M = fmaxf(M, lp[k].x);
        M = wave_max(M);
        float S = 0.f;
        for (int k = lane; k < a.nchunk; k += 64) {
            const float2 e = lp[k];
            if (e.x != -INFINITY) S += exp2_hw((e.x - M) * kLog2e) * e.y;
        }
        S = wave_sum(S);
        if (lane == 0) s_lse[g] = (M + logf(S)) * kLog2e;   // log2 units
    }
    __syncthreads();
    // f(j) = sum over the group's rows of exp(z - LSE_J) (no 1/G: the order is the same)
    float f[kEvQ][4];
#pragma unroll
    for (int k = 0; k < kEvQ; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) f[k][e] = 0.f;
    for (int g0 = 0; g0 < G; g0 += 4) {
        if (g0 > 0) load4(g0);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            if (g0 + gg >= G) continue;
            const float l = s_lse[g0 + gg];
#pragma unroll
            for (int k = 0; k < kEvQ; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) f[k][e] += exp2_hw(fmaf(v[gg][k][e], kLog2e, -l));
        }
    }
    uint32_t* keys = a.keys + ((int64_t)unit * a.nchunk + c) * kSelChunk;
    if constexpr (REFINE) {
        // log2 of the unnormalised fused score for the refinement pass, and this chunk's share
        // of the fusion normaliser.  The key norms of the prior are loaded here, once the
        // logits' registers are free: 16-byte loads like the logits' when the rows allow them
        // (a.norm_vec), else each clamped into the chunk.
        float nrm[kEvQ][4];
        if (a.key_norm && a.norm_vec) {
            const float* kn = a.key_norm + (int64_t)unit * a.norm_stride + base;
#pragma unroll
            for (int k = 0; k < kEvQ; ++k) {
                const int f = k * kThreads + tid;
                const f32x4 x = f < n4 ? *(const f32x4*)(kn + 4 * f) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) nrm[k][e] = x[e];
            }
        } else if (a.key_norm) {
            const float* kn = a.key_norm + (int64_t)unit * a.norm_stride;
#pragma unroll
            for (int k = 0; k < kEvQ; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    nrm[k][e] = kn[min(max(base + 4 * (k * kThreads + tid) + e, lo), hi - 1)];
        } else {
#pragma unroll
            for (int k = 0; k < kEvQ; ++k)
#pragma unroll
                for (int e = 0; e < 4; ++e) nrm[k][e] = 1.f;
        }
        float* lf = a.lfused + ((int64_t)unit * a.nchunk + c) * kSelChunk;
        float zs = 0.f;
#pragma unroll
        for (int k = 0; k < kEvQ; ++k) {
            const int j = base + 4 * (k * kThreads + tid);
            f32x4 lq;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lq[e] = fused_log2(a, f[k][e], prior_log2_n(a, j + e, r.j0, r.nJ, nrm[k][e]));
                if (j + e >= lo && j + e < hi) zs += exp2_hw(lq[e]);
            }
            // a quad wholly inside the chunk goes out as one 16-byte store when the chunk starts
            // on a multiple of 4; nontemporal, so that little of the 16.8 MB at 128K is left to
            // write back when the kernel ends (the refine pass starts about 1 us sooner)
            if (base == lo && j + 3 < hi) {
                __builtin_nontemporal_store(lq, (f32x4*)(lf + (j - lo)));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e >= lo && j + e < hi) lf[j + e - lo] = lq[e];
            }
        }
        zs = block_sum(zs, sh);
        if (tid == 0) a.zpart[(int64_t)unit * a.nchunk + c] = zs;
        return;
    }
#pragma unroll
    for (int k = 0; k < kEvQ; ++k) {
        // a quad wholly inside the chunk goes out as one 16-byte store when the chunk starts on
        // a multiple of 4
        const int j = base + 4 * (k * kThreads + tid);
        u32x4 kq;
#pragma unroll
        for (int e = 0; e < 4; ++e) kq[e] = __float_as_uint(f[k][e]);
        if (base == lo && j + 3 < hi) {
            *(u32x4*)(keys + (j - lo)) = kq;
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&lh[kq[e] >> kCShift[0]], 1u);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e >= lo && j + e < hi) {
                    keys[j + e - lo] = kq[e];
                    atomicAdd(&lh[kq[e] >> kCShift[0]], 1u);
                }
        }
    }
    __syncthreads();
    uint32_t* hg = a.hist + (int64_t)unit * kCBins0;
    // bins 2t and 2t + 1 as one 64-bit add (the low and high halves of a little-endian word;
    // no count reaches 2^32, so no carry crosses between them); every pair of this thread is
    // read before any is tested
    constexpr int kPairs = kCBins0 / 2 / kThreads;
    uint2 n[kPairs];
#pragma unroll
    for (int u = 0; u < kPairs; ++u) n[u] = *(const uint2*)&lh[2 * (u * kThreads + tid)];
#pragma unroll
    for (int u = 0; u < kPairs; ++u)
        if (n[u].x | n[u].y)
            atomicAdd((unsigned long long*)hg + u * kThreads + tid,
                      (unsigned long long)n[u].x | ((unsigned long long)n[u].y << 32));
}

// Fused score, Soft-NMS and cross-head exclusivity for one quarter of a chunk of J of one
// sequence, every KV head of it.  Thread t takes the 4 consecutive positions lo + 4t ... and
// forms, from the evidence pass's log2 fused scores of those positions and the one on each side,
// the normalised log2 score s = log2(f^(1-lam) r^lam) - log2 Z_h, then the Soft-NMS score
// exp2(s), times keep_soft where a neighbour in J has a strictly larger s.  The loads of up to
// kRefHeads heads (one 16-byte load per lane and the neighbours of the wave's ends, clamped into
// J, per head; the other neighbours come from the adjacent lanes) and of the heads' chunk sums
// are issued together at entry, and the normalisers take one barrier.  At each
// position every head below the largest is then decayed by keep_cross; the results are the keys.
// Each unit's digit-0 histogram is built from them in LDS with two 16-bit counts per word (a
// workgroup counts at most kRefSpan keys per head), every head of the group in one pass, then
// added to the unit's histogram in global memory.  The scores are read from their own buffer, so
// the neighbours' keys written by other workgroups never feed a score.
constexpr int kCrossParts = 2;                         // workgroups per chunk
constexpr int kRefSpan = kSelChunk / kCrossParts;      // positions per workgroup
constexpr int kRefThreads = kRefSpan / 4;              // four positions per thread
constexpr int kRefWaves = kRefThreads / 64;
constexpr int kRefHeads = 8;                           // heads held in registers at a time
constexpr int kRefWords = kCBins0 / 2;                 // packed histogram words per head
constexpr int kRefFlush = 8;                           // histogram words per lane per flush batch
static_assert(kRefThreads % 64 == 0 && kRefThreads <= 1024, "whole waves, one workgroup");
static_assert(kRefSpan < 65536, "a 16-bit count holds every key of a workgroup");
static_assert(kSelChunk % 4 == 0, "16-byte loads of the score buffer");
static_assert((kRefHeads * kRefWords) % (4 * kRefThreads) == 0, "16-byte clears of the histograms");
static_assert((kRefHeads * kRefWords) % (kRefFlush * kRefThreads) == 0, "whole flush batches");
__global__ void __launch_bounds__(kRefThreads) refine_kernel(SelArgs a) {
    __shared__ float s_l2z[kRefHeads];                 // log2 of each head's fusion normaliser
    __shared__ uint32_t lh[kRefHeads][kRefWords];
    const int c = blockIdx.x / kCrossParts, part = blockIdx.x % kCrossParts;
    const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const Range r = j_range(a, b);
    const int lo = r.j0 + c * kSelChunk + part * kRefSpan;
    const int hi = min(r.j1, lo + kRefSpan);
    if (lo >= hi) return;
    const int64_t unit_len = (int64_t)a.nchunk * kSelChunk;
    const int nc = (r.nJ + kSelChunk - 1) / kSelChunk;
    const int pb = lo + 4 * tid;                       // first of this thread's positions
    // offsets into a unit's score buffer: the quad (a multiple of 4, inside the chunk's region
    // even past hi), and the neighbours of the wave's first and last positions, clamped into J
    // (the other neighbours come from the adjacent lanes)
    const int jq = pb - r.j0;
    const int pw = lo + 4 * (tid & ~63);
    const int jl = max(pw - 1, r.j0) - r.j0;
    const int jr = min(pw + 4 * 64, r.j1 - 1) - r.j0;
    float mx[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float sc[kRefHeads][4];
    // heads are taken kRefHeads at a time; with more heads than that, the scores are computed
    // twice (once for the maxima, once for the keys)
    for (int pass = 0; pass < 2; ++pass) {
        for (int h0 = 0; h0 < a.Hkv; h0 += kRefHeads) {
            const int nh = min(kRefHeads, a.Hkv - h0);
            if (pass == 1 && a.Hkv <= kRefHeads) {
                // the scores of pass 0 are still in registers
            } else {
                f32x4 q[kRefHeads];
                float ql[kRefHeads], qr[kRefHeads];
#pragma unroll
                for (int hh = 0; hh < kRefHeads; ++hh) {
                    const int unit = b * a.Hkv + h0 + min(hh, nh - 1);
                    const float* lf = a.lfused + (int64_t)unit * unit_len;
                    q[hh] = *(const f32x4*)(lf + jq);
                    ql[hh] = lf[jl];                   // the same address in every lane
                    qr[hh] = lf[jr];
                }
                // wave w sums the chunk shares of heads w, w + kRefWaves, ...
                for (int hh = w; hh < nh; hh += kRefWaves) {
                    const float* zp = a.zpart + (int64_t)(b * a.Hkv + h0 + hh) * a.nchunk;
                    float zs = 0.f;
                    for (int k = lane; k < nc; k += 64) zs += zp[k];
                    zs = wave_sum(zs);
                    if (lane == 0) s_l2z[hh] = __log2f(zs);
                }
                if (pass == 1) {
                    // the histograms of this group start from zero; the barrier below orders the
                    // clear after the previous group's flush and before any count
                    u32x4* l4 = (u32x4*)&lh[0][0];
                    for (int t = tid; t < kRefHeads * kRefWords / 4; t += kRefThreads)
                        l4[t] = u32x4{0u, 0u, 0u, 0u};
                }
                __syncthreads();
#pragma unroll
                for (int hh = 0; hh < kRefHeads; ++hh) {
                    const float l2z = s_l2z[min(hh, nh - 1)];
                    const float left = lane_prev(q[hh][3], ql[hh]);
                    const float right = lane_next(q[hh][0], qr[hh]);
                    const float ls[6] = {left - l2z,      q[hh][0] - l2z, q[hh][1] - l2z,
                                         q[hh][2] - l2z, q[hh][3] - l2z, right - l2z};
#pragma unroll
                    for (int e = 1; e < 5; ++e) {
                        const int j = pb - 1 + e;
                        const bool lower = (j > r.j0 && ls[e - 1] > ls[e]) ||
                                           (j + 1 < r.j1 && ls[e + 1] > ls[e]);
                        sc[hh][e - 1] = (j < hi) ? exp2_hw(ls[e]) * (lower ? a.keep_soft : 1.f)
                                                 : -INFINITY;
                    }
                }
                if (a.Hkv > kRefHeads) __syncthreads();    // s_l2z is reused by the next group
            }
            if (pass == 0) {
#pragma unroll
                for (int hh = 0; hh < kRefHeads; ++hh)
                    if (hh < nh)
#pragma unroll
                        for (int e = 0; e < 4; ++e) mx[e] = fmaxf(mx[e], sc[hh][e]);
                if (a.Hkv <= kRefHeads) {
                    // pass 1 loads nothing: clear the histograms here, ordered by the barrier
                    // after the maxima
                    u32x4* l4 = (u32x4*)&lh[0][0];
                    for (int t = tid; t < kRefHeads * kRefWords / 4; t += kRefThreads)
                        l4[t] = u32x4{0u, 0u, 0u, 0u};
                    __syncthreads();
                }
                continue;
            }
            // pass 1: exclusivity, keys and the packed histograms of the group
#pragma unroll
            for (int hh = 0; hh < kRefHeads; ++hh) {
                if (hh >= nh) continue;
                const int unit = b * a.Hkv + h0 + hh;
                uint32_t* keys = a.keys + (int64_t)unit * unit_len;
                u32x4 kk;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = sc[hh][e];
                    kk[e] = __float_as_uint(x < mx[e] ? x * a.keep_cross : x);
                }
                // nontemporal (as the scores above): the candidate pass then starts about 1.7 us
                // sooner and reads the keys about 0.8 us slower
                if (pb + 3 < hi) {
                    __builtin_nontemporal_store(kk, (u32x4*)(keys + jq));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (pb + e < hi) keys[jq + e] = kk[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (pb + e < hi) {
                        const uint32_t bin = kk[e] >> kCShift[0];
                        atomicAdd(&lh[hh][bin >> 1], 1u << (16 * (bin & 1u)));
                    }
            }
            __syncthreads();
            // the two counts of a word go to the unit's histogram as one 64-bit add (bins 2i and
            // 2i + 1 are the low and high halves of a little-endian 64-bit word; a count stays far
            // below 2^32, so no carry crosses between them).  One word per lane keeps each wave's
            // adds on the fewest cache lines.
            // kRefFlush words per lane are read before any is tested, so the LDS latency is
            // paid once per batch, not once per word
            for (int t0 = 0; t0 < kRefHeads * kRefWords; t0 += kRefFlush * kRefThreads) {
                uint32_t n[kRefFlush];
#pragma unroll
                for (int u = 0; u < kRefFlush; ++u) n[u] = (&lh[0][0])[t0 + u * kRefThreads + tid];
#pragma unroll
                for (int u = 0; u < kRefFlush; ++u) {
                    const int t = t0 + u * kRefThreads + tid;
                    const int hh = t / kRefWords;
                    if (hh < nh && n[u]) {
                        unsigned long long* hg = (unsigned long long*)(a.hist +
                            (int64_t)(b * a.Hkv + h0 + hh) * kCBins0) + t % kRefWords;
                        atomicAdd(hg, (unsigned long long)(n[u] & 0xffffu) |
                                      ((unsigned long long)(n[u] >> 16) << 32));
                    }
                }
            }
            __syncthreads();
        }
    }
}

// Over bins held kPer per thread in ascending order (thread t holds bins kPer t ... kPer t +
// kPer - 1), finds the bin that holds the k-th largest key (0 < k <= the number of keys):
// s_sel[0] = the bin, s_sel[1] = the number of keys in higher bins.
template <int kPer, int kW>
__device__ void pick_bin(const uint32_t (&bins)[kPer], uint32_t k, uint32_t (&wt)[2][kW],
                         int& parity, uint32_t* s_sel) {
    const int tid = threadIdx.x;
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += bins[j];
    uint32_t total;
    const uint32_t below_incl = scan_total(mine, wt, parity, &total) + mine;
    const uint32_t above = total - below_incl;          // keys in higher bins than this thread's
    if (above < k && k <= above + mine) {
        uint32_t cum = above;
        for (int j = kPer - 1; j >= 0; --j) {
            if (cum + bins[j] >= k) {
                s_sel[0] = (uint32_t)(kPer * tid + j);
                s_sel[1] = cum;
                break;
            }
            cum += bins[j];
        }
    }
    __syncthreads();
}

// state: [0] prefix (bits of T decided so far), [1] k_rem, [2] nJ, [3] take_all
// A unit is active when some but not all of J is kept: !take_all, k_rem > 0 and a prefix
// other than the keep-nothing mark 0xffffffff.
__device__ __forceinline__ bool sel_active(uint32_t prefix, int32_t k_rem, int32_t take_all) {
    return !take_all && k_rem > 0 && prefix != 0xffffffffu;
}

// counts: [unit][chunk][3] = (keys in higher digit-0 bins, candidates above T, kept keys
// equal to T); the first is written by the candidate pass, the others by the resolve pass.
constexpr int kCountSlots = 3;

// Loads the 16 consecutive keys of thread tid in chunk c as four 16-byte loads.  A chunk holds
// kSelChunk keys in the workspace whatever its length, so the loads stay inside it and can be
// issued before the chunk's length is known; the caller masks keys at or past the length.
__device__ __forceinline__ void load_chunk_keys(const SelArgs& a, int unit, int c, uint32_t* kv) {
    const int tid = threadIdx.x;
    const u32x4* keys4 =
        (const u32x4*)(a.keys + ((int64_t)unit * a.nchunk + c) * kSelChunk) + tid * (kPerThread / 4);
#pragma unroll
    for (int k4 = 0; k4 < kPerThread / 4; ++k4) {
        const u32x4 x = keys4[k4];
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[4 * k4 + e] = x[e];
    }
}

// Per chunk, with digit 0 found by every workgroup of the unit from the evidence histogram
// (an L2-resident 16 KB read, so no separate launch is needed; workgroup 0 stores the state):
// compacts the keys of the digit-0 bin that holds the k-th largest key into the chunk's own
// region of the candidate buffer (no cross-workgroup atomics), writes their number to
// cand_n[chunk] and counts[chunk] = (keys in higher digit-0 bins, 0, 0); the resolve pass fills
// in the candidates' share.  Inactive units get their final counts here: everything (take_all)
// or nothing.  The histogram, the keys and the length are loaded together at entry.
__global__ void __launch_bounds__(kThreads) candidate_kernel(SelArgs a) {
    __shared__ uint32_t wt[2][kWaves];
    __shared__ uint32_t s_sel[2];
    __shared__ uint32_t s_key[kSelChunk];             // the chunk's candidates, staged for
    __shared__ int32_t s_pos[kSelChunk];              //   coalesced stores
    int parity = 0;
    constexpr int kPer = kCBins0 / kThreads;          // histogram bins per thread, ascending
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int unit = b * a.Hkv + h;
    // the histogram first: loads complete in order, so the pick below (which runs whether or
    // not the unit is active, so that these loads stay at entry) waits for the histogram only
    // and runs while the chunk's keys are still arriving
    const uint32_t* hg = a.hist + (int64_t)unit * kCBins0;
    uint32_t bins[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) bins[k] = hg[kPer * tid + k];
    uint32_t kv[kPerThread];
    load_chunk_keys(a, unit, c, kv);
    const int32_t nJ = j_range(a, b).nJ;
    const int32_t take_all = a.k_sel >= nJ ? 1 : 0;
    int32_t k_rem = take_all ? nJ : a.k_sel;
    uint32_t prefix = (!take_all && k_rem == 0) ? 0xffffffffu : 0u;   // keep nothing
    const bool active = sel_active(prefix, k_rem, take_all);
    pick_bin<kPer>(bins, active ? (uint32_t)k_rem : 1u, wt, parity, s_sel);
    if (active) {
        prefix = s_sel[0] << kCShift[0];
        k_rem -= (int32_t)s_sel[1];
    }
    if (c == 0 && tid == 0) {
        int32_t* st = a.state + unit * 4;
        st[0] = (int32_t)prefix;
        st[1] = k_rem;
        st[2] = nJ;
        st[3] = take_all;
    }
    const int cnt = max(0, min(kSelChunk, nJ - c * kSelChunk));
    uint32_t* cn = a.counts + ((int64_t)unit * a.nchunk + c) * kCountSlots;
    uint32_t* cand_n = a.cand_n + (int64_t)unit * a.nchunk + c;
    if (!active || cnt == 0) {
        if (tid == 0) {
            cn[0] = take_all ? (uint32_t)cnt : 0u;
            cn[1] = 0u;
            cn[2] = 0u;
            *cand_n = 0u;
        }
        return;
    }
    const uint32_t d0 = prefix >> kCShift[0];
    // candidates: the keys of bin d0, or with finish_kernel to follow, every key of bin d0 or
    // above (with its position), so that the finish reads the kept keys from here
    uint32_t gt = 0, nc = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const bool in = tid * kPerThread + k < cnt;
        const uint32_t d = kv[k] >> kCShift[0];
        gt += (in && d > d0) ? 1u : 0u;
        nc += (in && d == d0) ? 1u : 0u;
    }
    if (a.finish) nc += gt;
    // counts packed as (greater << 16) | candidates: at most kSelChunk each
    uint32_t tot;
    const uint32_t excl = scan_total((gt << 16) | nc, wt, parity, &tot);
    if (tid == 0) {
        *cand_n = tot & 0xffffu;
        cn[0] = tot >> 16;
        cn[1] = 0u;
        cn[2] = 0u;
    }
    uint32_t o = excl & 0xffffu;
    const int jb = a.n_sink + c * kSelChunk + tid * kPerThread;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const uint32_t d = kv[k] >> kCShift[0];
        if (tid * kPerThread + k < cnt && (a.finish ? d >= d0 : d == d0)) {
            s_key[o] = kv[k];
            s_pos[o] = jb + k;
            ++o;
        }
    }
    __syncthreads();
    const int64_t region = ((int64_t)unit * a.nchunk + c) * kSelChunk;
    const uint32_t n = tot & 0xffffu;
    for (uint32_t i = tid; i < n; i += kThreads) {
        a.cand[region + i] = s_key[i];
        if (a.finish) a.epos[region + i] = s_pos[i];
    }
}

__global__ void __launch_bounds__(kThreads) emit_kernel(SelArgs a) {
    __shared__ uint32_t sh[4];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int unit = b * a.Hkv + h;
    // keys, earlier chunks' counts and the state are independent loads: issue them together
    uint32_t kv[kPerThread];
    load_chunk_keys(a, unit, c, kv);
    uint32_t gtb = 0, eqb = 0;                        // kept positions in earlier chunks
    for (int k = tid; k < c; k += kThreads) {
        const uint32_t* ck = a.counts + ((int64_t)unit * a.nchunk + k) * kCountSlots;
        gtb += ck[0] + ck[1];
        eqb += ck[2];
    }
    const int32_t* st = a.state + unit * 4;
    const uint32_t T = (uint32_t)st[0];
    const int32_t k_rem = st[1], nJ = st[2], take_all = st[3];
    const int N = a.len[b];
    const int ns = max(0, min(a.n_sink, N));
    int32_t* row = a.idx + (int64_t)unit * a.idx_stride;
    if (c == 0) {
        for (int t = tid; t < ns; t += kThreads) row[t] = t;
        if (tid == 0) a.n_idx[unit] = ns + (take_all ? nJ : min(a.k_sel, nJ));
    }
    const int lo = c * kSelChunk;
    const int cnt = min(kSelChunk, nJ - lo);
    if (cnt <= 0) return;
    gtb = block_sum_u(gtb, sh);
    eqb = block_sum_u(eqb, sh);
    const uint32_t kr = take_all ? 0u : (uint32_t)k_rem;
    const uint32_t base = (uint32_t)ns + gtb + min(eqb, kr);
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
        if (tid * kPerThread + k >= cnt) kv[k] = 0u;
    uint32_t my_eq = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int t = tid * kPerThread + k;
        my_eq += (t < cnt && !take_all && kv[k] == T) ? 1u : 0u;
    }
    uint32_t eq_rank = eqb + block_exclusive_scan(my_eq, sh);
    uint32_t keep_mask = 0, my_keep = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int t = tid * kPerThread + k;
        bool keep = false;
        if (t < cnt) {
            if (take_all || kv[k] > T) {
                keep = true;
            } else if (kv[k] == T) {
                keep = eq_rank < kr;
                ++eq_rank;
            }
        }
        keep_mask |= keep ? (1u << k) : 0u;
        my_keep += keep ? 1u : 0u;
    }
    uint32_t out = base + block_exclusive_scan(my_keep, sh);
    const int jbase = a.n_sink + lo + tid * kPerThread;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
        if (keep_mask & (1u << k)) row[out++] = jbase + k;
}

// ---- the whole Selector in one launch: one 1024-thread workgroup per (b, KV head) --------
//
// Used when each unit's logits are small enough that one compute unit walks them faster than
// the chunked kernels above can be launched (the host decides from the descriptor).  Same
// result: LSE over J per head, evidence keys, three radix digits of the k-th largest key in
// LDS histograms, then an ordered emit in blocks of 4096 positions with one packed
// (greater, equal) scan per block.  Keys are kept per position in the workspace (L2-resident
// between the passes).

// merge of two partial log-sum-exp pairs (max, sum of 2^(x - max)) in log2 units; max = -inf
// is empty
__device__ __forceinline__ float2 lse2_merge(float2 p, float2 q) {
    const float m = fmaxf(p.x, q.x);
    if (m == -INFINITY) return make_float2(m, 0.f);
    return make_float2(m, p.y * exp2_hw(p.x - m) + q.y * exp2_hw(q.x - m));
}

constexpr int kUT = 1024;                              // threads per workgroup
constexpr int kUW = kUT / 64;                          // wavefronts
constexpr int kUQ = 4;                                 // position quads per thread per batch

struct UnitShared {
    uint32_t hist[kRadixBins];
    uint32_t wtot[kUW];
    float2 red[4 * kUW];
    float lse[kMaxSelG];
    uint32_t sel[2];
};

// exclusive scan over the 1024 threads (ascending thread order); total returned in *tot
__device__ uint32_t unit_scan(uint32_t x, UnitShared& sm, uint32_t* tot) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(x);
    if (lane == 63) sm.wtot[w] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int ww = 0; ww < kUW; ++ww) {
        const uint32_t t = sm.wtot[ww];
        before += ww < w ? t : 0u;
        all += t;
    }
    __syncthreads();
    *tot = all;
    return before + inc - x;
}

// Chooses the digit (bins of sm.hist, ascending) that holds the k_rem-th largest key; keeps
// the digit in prefix at `shift` and subtracts the keys in higher bins from k_rem.
__device__ void unit_resolve(UnitShared& sm, int shift, uint32_t& prefix, int32_t& k_rem) {
    const int tid = threadIdx.x;
    const uint32_t c0 = sm.hist[2 * tid], c1 = sm.hist[2 * tid + 1];
    uint32_t total;
    const uint32_t excl = unit_scan(c0 + c1, sm, &total);
    const uint32_t above = total - excl - c0 - c1;      // keys in higher bins
    const uint32_t k = (uint32_t)k_rem;
    if (above < k && k <= above + c0 + c1) {
        if (above + c1 >= k) {
            sm.sel[0] = 2 * tid + 1;
            sm.sel[1] = above;
        } else {
            sm.sel[0] = 2 * tid;
            sm.sel[1] = above + c1;
        }
    }
    __syncthreads();
    prefix |= sm.sel[0] << shift;
    k_rem -= (int32_t)sm.sel[1];
    __syncthreads();
}

// Digits 1 and 2 over the unit's candidates (all in the digit-0 bin), then the per-chunk
// numbers of candidates above T and equal to T added to the counts of the candidate pass.
// One 1024-thread workgroup per (b, KV head).  Chunks are taken kCntGroup at a time: their
// candidate numbers are scanned in LDS, and candidate i of the group is found in its chunk's
// region by a binary search over the scan.  When a unit's candidates fit (the usual case: a
// digit-0 bin is 1/16 octave of evidence) they are copied to LDS once and the three
// passes run from there; otherwise each pass reads them again, kResolveBatch per thread at a
// time so the loads overlap.
constexpr int kCntGroup = kUT;
constexpr int kCandLds = 16384;
constexpr int kResolveBatch = 4;
struct ResolveShared {
    UnitShared u;
    uint32_t off[kCntGroup + 1];      // exclusive scan of the group's candidate numbers
    uint32_t gt[kCntGroup], eq[kCntGroup];
    uint32_t key[kCandLds];
};

__global__ void __launch_bounds__(kUT) resolve_kernel(SelArgs a) {
    __shared__ ResolveShared rs;
    UnitShared& sm = rs.u;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int unit = b * a.Hkv + h;
    const uint32_t* cand = a.cand + (int64_t)unit * a.nchunk * kSelChunk;
    const uint32_t* cand_n = a.cand_n + (int64_t)unit * a.nchunk;
    // the candidate pass wrote cand_n for all nchunk chunks, so the first group's numbers can
    // be loaded with the state
    const uint32_t n_first = tid < a.nchunk ? cand_n[tid] : 0u;
    int32_t* st = a.state + unit * 4;
    uint32_t prefix = (uint32_t)st[0];
    int32_t k_rem = st[1];
    const int32_t nJ = st[2], take_all = st[3];
    if (!sel_active(prefix, k_rem, take_all)) return;
    const int nch = (nJ + kSelChunk - 1) / kSelChunk;
    // scans the candidate numbers of chunks [g0, g0 + kCntGroup); returns their total
    auto load_group = [&](int g0) -> uint32_t {
        const uint32_t n = g0 == 0 ? (tid < nch ? n_first : 0u) : (g0 + tid < nch ? cand_n[g0 + tid] : 0u);
        uint32_t tot;
        const uint32_t ex = unit_scan(n, sm, &tot);
        rs.off[tid] = ex;
        if (tid == 0) rs.off[kCntGroup] = tot;
        __syncthreads();
        return tot;
    };
    // the chunk (within the group) of candidate i < total: the last c with off[c] <= i
    auto chunk_of = [&](uint32_t i) -> int {
        int lo = 0, hi = kCntGroup;                        // off[lo] <= i < off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (rs.off[mid] <= i) lo = mid; else hi = mid;
        }
        return lo;
    };
    // calls fn(key, chunk in group) for every candidate of the group
    auto for_each = [&](int g0, uint32_t total, bool in_lds, auto&& fn) {
        if (in_lds) {
            for (uint32_t i = tid; i < total; i += kUT) fn(rs.key[i], chunk_of(i));
            return;
        }
        for (uint32_t i0 = tid; i0 < total; i0 += kResolveBatch * kUT) {
            uint32_t kk[kResolveBatch];
            int cc[kResolveBatch];
#pragma unroll
            for (int u = 0; u < kResolveBatch; ++u) {
                const uint32_t i = i0 + u * kUT;
                cc[u] = i < total ? chunk_of(i) : 0;
                kk[u] = i < total ? cand[(int64_t)(g0 + cc[u]) * kSelChunk + (i - rs.off[cc[u]])] : 0u;
            }
#pragma unroll
            for (int u = 0; u < kResolveBatch; ++u)
                if (i0 + u * kUT < total) fn(kk[u], cc[u]);
        }
    };
    const bool one_group = nch <= kCntGroup;
    uint32_t total = one_group ? load_group(0) : 0u;
    const bool in_lds = one_group && total <= (uint32_t)kCandLds;
    if (in_lds) {
        for (uint32_t i0 = tid; i0 < total; i0 += kResolveBatch * kUT) {
            uint32_t kk[kResolveBatch];
#pragma unroll
            for (int u = 0; u < kResolveBatch; ++u) {
                const uint32_t i = i0 + u * kUT;
                const int c = i < total ? chunk_of(i) : 0;
                kk[u] = i < total ? cand[(int64_t)c * kSelChunk + (i - rs.off[c])] : 0u;
            }
#pragma unroll
            for (int u = 0; u < kResolveBatch; ++u)
                if (i0 + u * kUT < total) rs.key[i0 + u * kUT] = kk[u];
        }
        __syncthreads();
    }
#pragma unroll
    for (int pass = 1; pass < 3; ++pass) {
        for (int t = tid; t < kRadixBins; t += kUT) sm.hist[t] = 0u;
        __syncthreads();
        const int hs = kCShift[pass - 1];
        const uint32_t want = prefix >> hs;
        for (int g0 = 0; g0 < nch; g0 += kCntGroup) {
            if (!one_group) total = load_group(g0);
            for_each(g0, total, in_lds, [&](uint32_t key, int) {
                if ((key >> hs) == want) atomicAdd(&sm.hist[(key >> kCShift[pass]) & kCMask[pass]], 1u);
            });
            __syncthreads();
        }
        unit_resolve(sm, kCShift[pass], prefix, k_rem);
    }
    const uint32_t T = prefix;
    for (int g0 = 0; g0 < nch; g0 += kCntGroup) {
        if (!one_group) total = load_group(g0);
        rs.gt[tid] = 0u;
        rs.eq[tid] = 0u;
        __syncthreads();
        for_each(g0, total, in_lds, [&](uint32_t key, int c) {
            if (key > T) atomicAdd(&rs.gt[c], 1u);
            else if (key == T) atomicAdd(&rs.eq[c], 1u);
        });
        __syncthreads();
        if (g0 + tid < nch) {
            uint32_t* cn = a.counts + ((int64_t)unit * a.nchunk + g0 + tid) * kCountSlots;
            cn[1] = rs.gt[tid];
            cn[2] = rs.eq[tid];
        }
        __syncthreads();
    }
    if (tid == 0) {
        st[0] = (int32_t)T;
        st[1] = k_rem;
    }
}

// Finish of the chunked Selector, one 1024-thread workgroup per (b, KV head), after the
// candidate pass has written, per chunk and in position order, every key whose digit 0 is at or
// above the bin d0 of the k-th largest key, with its position.
//   1. The chunks' entry numbers are scanned: chunk c's entries go to [off[c], off[c + 1]).
//   2. Each wavefront copies whole chunks to LDS (chunks w, w + 16, ..., four at a time with
//      every load of the four issued first), so no entry needs a search for its chunk; the keys of
//      bin d0 fill the digit-1 histogram on the way.  Entries past kFinCap stay where they lie
//      (their chunk is then found by a binary search over off).
//   3. Digit 1 of T from that histogram; digit 2 over the entries of T's digit-1 bin.
//   4. The ordered emit: entries above T, and those equal to T while fewer than k_rem came
//      before, after the sink positions, with one packed (greater, equal) scan per 8192 entries.
// It replaces the resolve and emit passes (one launch and one read of all the keys fewer).
constexpr int kFinCap = kFinishCap;                    // entries held in LDS
constexpr int kFinChunks = kUT;                        // chunks per unit (contexts up to 4M)
constexpr int kFinCopy = 4;                            // entries per lane per chunk in flight
constexpr int kFinGroup = 4;                           // chunks per wavefront copied together
constexpr int kFinEmit = 8;                            // consecutive entries per thread in the emit
constexpr int kFinD1 = 1 << (kCShift[0] - kCShift[1]); // digit-1 bins
constexpr int kFinD2 = 1 << kCShift[1];                // digit-2 bins
static_assert((int64_t)kFinishCap * kFinishBinShare <= (int64_t)kFinChunks * kSelChunk,
              "a context the finish takes has its chunk numbers in one scan");
static_assert(kFinD1 == kUT && kFinD2 <= kUT, "one digit-1 bin per thread, at most one digit-2 bin");
static_assert(kFinCap % (kFinEmit * kUT) == 0, "an emit round lies wholly in LDS or wholly past it");
static_assert(kFinEmit * kUT < 65536, "an emit round's counts fit the halves of its packed scan");
struct FinishShared {
    uint32_t wt[2][kUW];
    uint32_t sel[2];
    uint32_t off[kFinChunks + 1];                      // exclusive scan of the entry numbers
    uint32_t h1[kFinD1];
    uint32_t h2[kFinD2];
    __attribute__((aligned(16))) uint32_t key[kFinCap];
    __attribute__((aligned(16))) int32_t pos[kFinCap]; // also the kept positions, staged in place
};

// Over bins held kPer per thread of the 1024-thread workgroup in ascending order, finds the bin
// that holds the k-th largest key (0 < k <= the number of keys): fs.sel = (the bin, the keys in
// higher bins).
template <int kPer>
__device__ void finish_pick(const uint32_t (&bins)[kPer], uint32_t k, FinishShared& fs,
                            int& parity) {
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += bins[j];
    uint32_t total;
    const uint32_t excl = scan_total(mine, fs.wt, parity, &total);
    const uint32_t above = total - excl - mine;        // keys in higher bins than this thread's
    if (above < k && k <= above + mine) {
        uint32_t cum = above;
        for (int j = kPer - 1; j >= 0; --j) {
            if (cum + bins[j] >= k) {
                fs.sel[0] = (uint32_t)(kPer * threadIdx.x + j);
                fs.sel[1] = cum;
                break;
            }
            cum += bins[j];
        }
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kUT) finish_kernel(SelArgs a) {
    __shared__ FinishShared fs;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int unit = b * a.Hkv + h;
    // the entry numbers, the state and the length are independent loads
    const uint32_t n_mine = tid < a.nchunk ? a.cand_n[(int64_t)unit * a.nchunk + tid] : 0u;
    const int32_t* st = a.state + unit * 4;
    uint32_t T = (uint32_t)st[0];
    int32_t k_rem = st[1];
    const int32_t nJ = st[2], take_all = st[3];
    const int N = a.len[b];
    const int ns = max(0, min(a.n_sink, N));
    int32_t* row = a.idx + (int64_t)unit * a.idx_stride;
    for (int t = tid; t < ns; t += kUT) row[t] = t;
    if (tid == 0) a.n_idx[unit] = ns + (take_all ? nJ : min(a.k_sel, nJ));
    if (take_all) {
        for (int t = tid; t < nJ; t += kUT) row[ns + t] = a.n_sink + t;
        return;
    }
    if (!sel_active(T, k_rem, take_all)) return;       // keep nothing
    fs.h1[tid] = 0u;
    if (tid < kFinD2) fs.h2[tid] = 0u;
    if (tid == 0) fs.sel[0] = fs.sel[1] = 0u;
    int parity = 0;
    // 1. chunk c's entries go to [off[c], off[c + 1]); off[nch] = E
    uint32_t E;
    const uint32_t ex = scan_total(n_mine, fs.wt, parity, &E);
    fs.off[tid] = ex;
    if (tid == 0) fs.off[kFinChunks] = E;
    __syncthreads();
    const int nch = (nJ + kSelChunk - 1) / kSelChunk;  // chunks holding positions of J
    const int64_t base = (int64_t)unit * a.nchunk * kSelChunk;
    // 2. copy, kFinGroup chunks per wavefront at a time (chunks w, w + kUW, ...), every load of
    // the group issued before any store; loads clamped into their chunk's region, and none for
    // a chunk past the last or a row of 64 past a chunk's entries (tests that are the same for
    // the whole wavefront)
    const uint32_t d0 = T >> kCShift[0];
    for (int c0 = w; c0 < nch; c0 += kFinGroup * kUW) {
        uint32_t o[kFinGroup], nc[kFinGroup], nmax = 0;
#pragma unroll
        for (int q = 0; q < kFinGroup; ++q) {
            const int c = c0 + q * kUW;
            o[q] = c < nch ? fs.off[c] : 0u;
            nc[q] = c < nch ? fs.off[c + 1] - o[q] : 0u;
            nmax = max(nmax, nc[q]);
        }
        for (uint32_t j0 = 0; j0 < nmax; j0 += 64 * kFinCopy) {
            uint32_t kk[kFinGroup][kFinCopy];
            int32_t pp[kFinGroup][kFinCopy];
#pragma unroll
            for (int q = 0; q < kFinGroup; ++q) {
                const int64_t r = base + (int64_t)(c0 + q * kUW) * kSelChunk;
#pragma unroll
                for (int u = 0; u < kFinCopy; ++u) {
                    // rows of 64 entries that start past the chunk's entries are not loaded (one
                    // CU pulls its unit's entries at a few tens of GB/s, so bytes matter here)
                    if (j0 + 64 * u < nc[q]) {
                        const uint32_t j = min(j0 + lane + 64 * u, (uint32_t)kSelChunk - 1);
                        kk[q][u] = a.cand[r + j];
                        pp[q][u] = a.epos[r + j];
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < kFinGroup; ++q) {
#pragma unroll
                for (int u = 0; u < kFinCopy; ++u) {
                    const uint32_t j = j0 + lane + 64 * u;
                    if (j < nc[q]) {
                        if (o[q] + j < (uint32_t)kFinCap) {
                            fs.key[o[q] + j] = kk[q][u];
                            fs.pos[o[q] + j] = pp[q][u];
                        }
                        if ((kk[q][u] >> kCShift[0]) == d0)
                            atomicAdd(&fs.h1[(kk[q][u] >> kCShift[1]) & kCMask[1]], 1u);
                    }
                }
            }
        }
    }
    __syncthreads();
    // entries past kFinCap: found in their chunk's region (the last c with off[c] <= i)
    auto where = [&](uint32_t i) -> int64_t {
        int lo = 0, hi = nch;                           // off[lo] <= i < off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (fs.off[mid] <= i) lo = mid; else hi = mid;
        }
        return base + (int64_t)lo * kSelChunk + (i - fs.off[lo]);
    };
    // 3. digits 1 and 2 of T
    {
        const uint32_t bins[1] = {fs.h1[tid]};
        finish_pick<1>(bins, (uint32_t)k_rem, fs, parity);
        T |= fs.sel[0] << kCShift[1];
        k_rem -= (int32_t)fs.sel[1];
    }
    // kFinEmit consecutive entries per thread and round (16-byte LDS reads)
    auto entries = [&](uint32_t ib, uint32_t (&kk)[kFinEmit], int32_t (&pp)[kFinEmit], bool pos) {
        if (ib < (uint32_t)kFinCap) {
            const u32x4 k0 = *(const u32x4*)&fs.key[ib], k1 = *(const u32x4*)&fs.key[ib + 4];
            kk[0] = k0[0]; kk[1] = k0[1]; kk[2] = k0[2]; kk[3] = k0[3];
            kk[4] = k1[0]; kk[5] = k1[1]; kk[6] = k1[2]; kk[7] = k1[3];
            if (pos) {
                const int4 p0 = *(const int4*)&fs.pos[ib], p1 = *(const int4*)&fs.pos[ib + 4];
                pp[0] = p0.x; pp[1] = p0.y; pp[2] = p0.z; pp[3] = p0.w;
                pp[4] = p1.x; pp[5] = p1.y; pp[6] = p1.z; pp[7] = p1.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < kFinEmit; ++e) {
                const int64_t at = ib + e < E ? where(ib + e) : base;
                kk[e] = a.cand[at];
                if (pos) pp[e] = a.epos[at];
            }
        }
    };
    {
        const uint32_t want = T >> kCShift[1];
        for (uint32_t i0 = 0; i0 < E; i0 += kFinEmit * kUT) {
            const uint32_t ib = i0 + kFinEmit * tid;
            uint32_t kk[kFinEmit];
            int32_t pp[kFinEmit];
            entries(ib, kk, pp, false);
#pragma unroll
            for (int e = 0; e < kFinEmit; ++e)
                if (ib + e < E && (kk[e] >> kCShift[1]) == want)
                    atomicAdd(&fs.h2[kk[e] & kCMask[2]], 1u);
        }
        __syncthreads();
        const uint32_t bins[1] = {tid < kFinD2 ? fs.h2[tid] : 0u};
        finish_pick<1>(bins, (uint32_t)k_rem, fs, parity);
        T |= fs.sel[0];
        k_rem -= (int32_t)fs.sel[1];
    }
    // 4. ordered emit into LDS; a row never takes more than min(k_sel, nJ) positions.  The kept
    // positions are staged in pos itself: kept entry number `out` is at most the entry's own
    // index, every read of a round's entries comes before the round's scan barrier and every
    // write after it, and later rounds read only entries past this round's.
    const uint32_t kr = (uint32_t)max(k_rem, 0);
    const uint32_t n_out = (uint32_t)min(min(a.k_sel, nJ), kFinCap);
    uint32_t gt_seen = 0, eq_seen = 0;
    for (uint32_t i0 = 0; i0 < E; i0 += kFinEmit * kUT) {
        const uint32_t ib = i0 + kFinEmit * tid;
        uint32_t kk[kFinEmit];
        int32_t pp[kFinEmit];
        entries(ib, kk, pp, true);
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int e = 0; e < kFinEmit; ++e) {
            const bool in = ib + e < E;
            gt += (in && kk[e] > T) ? 1u : 0u;
            eq += (in && kk[e] == T) ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t exc = scan_total((gt << 16) | eq, fs.wt, parity, &tot);
        uint32_t e_before = eq_seen + (exc & 0xffffu);
        uint32_t out = gt_seen + (exc >> 16) + min(e_before, kr);
#pragma unroll
        for (int e = 0; e < kFinEmit; ++e) {
            const bool in = ib + e < E;
            bool keep = in && kk[e] > T;
            if (in && kk[e] == T) {
                keep = e_before < kr;
                ++e_before;
            }
            if (keep) {
                if (out < n_out) fs.pos[out] = pp[e];
                ++out;
            }
        }
        gt_seen += tot >> 16;
        eq_seen += tot & 0xffffu;
    }
    // the staged row, coalesced (n_out <= k_sel <= kFinCap under the finish rule)
    __syncthreads();
    const uint32_t n_kept = min(n_out, gt_seen + min(eq_seen, kr));
    for (uint32_t i = tid; i < n_kept; i += kUT) row[ns + i] = fs.pos[i];
}

__global__ void __launch_bounds__(kUT) select_unit_kernel(SelArgs a) {
    __shared__ UnitShared sm;
    const int h = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = a.G;
    const int unit = b * a.Hkv + h;
    const Range r = j_range(a, b);
    const int ns = max(0, min(a.n_sink, r.N));
    const int nJ = r.nJ;
    int32_t* row = a.idx + (int64_t)unit * a.idx_stride;
    for (int t = tid; t < ns; t += kUT) row[t] = t;
    const bool take_all = a.k_sel >= nJ;
    if (tid == 0) a.n_idx[unit] = ns + (take_all ? nJ : a.k_sel);
    if (take_all) {
        for (int t = tid; t < nJ; t += kUT) row[ns + t] = r.j0 + t;
        return;
    }
    if (a.k_sel == 0) return;

    // Position quads [q0, q1) cover J; logit rows are 16-byte aligned with a stride that is a
    // multiple of 4, so a quad is one float4 load.  Each pass keeps several loads per thread
    // in flight: the passes are bound by memory latency, not bandwidth.
    const int j0 = r.j0, j1 = r.j1;
    const int q0 = j0 >> 2, q1 = (j1 + 3) >> 2;
    const float* zg = a.logits + ((int64_t)b * a.Hq + (int64_t)h * G) * a.logit_stride;
    auto in_j = [&](int qi, int e) { const int j = 4 * qi + e; return qi < q1 && j >= j0 && j < j1; };

    // 1. log-sum-exp over J of each query head, four heads and kUQ quads per thread at a time
    //    (given by the dense step in the fused slow step)
    if (a.lse_j) {
        for (int g = tid; g < G; g += kUT) sm.lse[g] = a.lse_j[(int64_t)b * a.Hq + h * G + g] * kLog2e;
        __syncthreads();
    }
    for (int g0 = 0; !a.lse_j && g0 < G; g0 += 4) {
        float m[4], sum[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            m[gg] = -INFINITY;
            sum[gg] = 0.f;
        }
        for (int qb = q0 + tid; qb < q1; qb += kUQ * kUT) {
            float4 v[4][kUQ];
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const float4* z4 = (const float4*)(zg + (int64_t)min(g0 + gg, G - 1) * a.logit_stride);
#pragma unroll
                for (int u = 0; u < kUQ; ++u) {
                    const int qi = qb + u * kUT;
                    v[gg][u] = qi < q1 ? z4[qi] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                // log2 units: x = z * log2(e), so each exponential is one v_exp_f32
                float x[kUQ][4];
                float mb = -INFINITY;
#pragma unroll
                for (int u = 0; u < kUQ; ++u) {
                    const float vv[4] = {v[gg][u].x, v[gg][u].y, v[gg][u].z, v[gg][u].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[u][e] = in_j(qb + u * kUT, e) ? vv[e] * kLog2e : -INFINITY;
                        mb = fmaxf(mb, x[u][e]);
                    }
                }
                if (mb == -INFINITY) continue;
                const float mn = fmaxf(m[gg], mb);
                float add = 0.f;
#pragma unroll
                for (int u = 0; u < kUQ; ++u)
#pragma unroll
                    for (int e = 0; e < 4; ++e) add += exp2_hw(x[u][e] - mn);
                sum[gg] = (m[gg] == -INFINITY ? 0.f : sum[gg] * exp2_hw(m[gg] - mn)) + add;
                m[gg] = mn;
            }
        }
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            float2 p = make_float2(m[gg], sum[gg]);
            for (int o = 32; o >= 1; o >>= 1)
                p = lse2_merge(p, make_float2(__shfl_xor(p.x, o), __shfl_xor(p.y, o)));
            if (lane == 0) sm.red[gg * kUW + w] = p;
        }
        __syncthreads();
        if (tid < 4 && g0 + tid < G) {
            float2 q = sm.red[tid * kUW];
            for (int ww = 1; ww < kUW; ++ww) q = lse2_merge(q, sm.red[tid * kUW + ww]);
            sm.lse[g0 + tid] = q.x + log2f(q.y);                 // log2 of sum over J
        }
        __syncthreads();
    }

    // 2. evidence keys for every position of J, and the histogram of their top 11 bits
    for (int t = tid; t < kRadixBins; t += kUT) sm.hist[t] = 0u;
    __syncthreads();
    uint4* keys4 = (uint4*)(a.keys + (int64_t)unit * a.nchunk * kSelChunk);
    for (int qb = q0 + tid; qb < q1; qb += kUQ * kUT) {
        float f[kUQ][4];
#pragma unroll
        for (int u = 0; u < kUQ; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) f[u][e] = 0.f;
        for (int g0 = 0; g0 < G; g0 += 4) {
            float4 v[4][kUQ];
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const float4* z4 = (const float4*)(zg + (int64_t)min(g0 + gg, G - 1) * a.logit_stride);
#pragma unroll
                for (int u = 0; u < kUQ; ++u) {
                    const int qi = qb + u * kUT;
                    v[gg][u] = qi < q1 ? z4[qi] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                if (g0 + gg < G) {
                    const float l = sm.lse[g0 + gg];
#pragma unroll
                    for (int u = 0; u < kUQ; ++u) {
                        f[u][0] += exp2_hw(fmaf(v[gg][u].x, kLog2e, -l));
                        f[u][1] += exp2_hw(fmaf(v[gg][u].y, kLog2e, -l));
                        f[u][2] += exp2_hw(fmaf(v[gg][u].z, kLog2e, -l));
                        f[u][3] += exp2_hw(fmaf(v[gg][u].w, kLog2e, -l));
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUQ; ++u) {
            const int qi = qb + u * kUT;
            if (qi >= q1) continue;
            uint4 k;
            k.x = __float_as_uint(f[u][0]);
            k.y = __float_as_uint(f[u][1]);
            k.z = __float_as_uint(f[u][2]);
            k.w = __float_as_uint(f[u][3]);
            keys4[qi] = k;
            const uint32_t kk[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (in_j(qi, e)) atomicAdd(&sm.hist[kk[e] >> kShift[0]], 1u);
        }
    }
    __syncthreads();

    // 3. the key T of the k_sel-th largest evidence, digit by digit
    uint32_t prefix = 0u;
    int32_t k_rem = a.k_sel;
    unit_resolve(sm, kShift[0], prefix, k_rem);
    for (int pass = 1; pass < 3; ++pass) {
        for (int t = tid; t < kRadixBins; t += kUT) sm.hist[t] = 0u;
        __syncthreads();
        const int hs = kShift[pass - 1];
        const uint32_t want = prefix >> hs;
        for (int qb = q0 + tid; qb < q1; qb += 2 * kUQ * kUT) {
            uint4 kq[2 * kUQ];
#pragma unroll
            for (int u = 0; u < 2 * kUQ; ++u) {
                const int qi = qb + u * kUT;
                kq[u] = qi < q1 ? keys4[qi] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < 2 * kUQ; ++u) {
                const uint32_t kk[4] = {kq[u].x, kq[u].y, kq[u].z, kq[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (in_j(qb + u * kUT, e) && (kk[e] >> hs) == want)
                        atomicAdd(&sm.hist[(kk[e] >> kShift[pass]) & kDigitMask[pass]], 1u);
            }
        }
        __syncthreads();
        unit_resolve(sm, kShift[pass], prefix, k_rem);
    }
    const uint32_t T = prefix;

    // 4. ordered emit: position j of J is kept when key > T, or key == T and fewer than k_rem
    //    earlier positions have key == T; its slot after the sinks is (kept before j) =
    //    greater_before + min(equal_before, k_rem).  Thread t takes kUQ consecutive quads of
    //    each block, so thread order is position order for the block scan.
    uint32_t gt_run = 0, eq_run = 0;
    uint4 next[kUQ];                                       // the next block's keys, in flight
#pragma unroll
    for (int u = 0; u < kUQ; ++u) {
        const int qi = q0 + tid * kUQ + u;
        next[u] = qi < q1 ? keys4[qi] : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int qb = q0; qb < q1; qb += kUQ * kUT) {
        const int qt = qb + tid * kUQ;
        uint32_t kk[kUQ][4];
        uint32_t packed = 0;                               // greater | equal << 16
#pragma unroll
        for (int u = 0; u < kUQ; ++u) {
            kk[u][0] = next[u].x; kk[u][1] = next[u].y; kk[u][2] = next[u].z; kk[u][3] = next[u].w;
        }
#pragma unroll
        for (int u = 0; u < kUQ; ++u) {
            const int qi = qt + kUQ * kUT + u;
            next[u] = qi < q1 ? keys4[qi] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kUQ; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = in_j(qt + u, e);
                packed += (in && kk[u][e] > T) ? 1u : 0u;
                packed += (in && kk[u][e] == T) ? (1u << 16) : 0u;
            }
        uint32_t tot;
        const uint32_t excl = unit_scan(packed, sm, &tot);
        uint32_t gt = gt_run + (excl & 0xffffu), eq = eq_run + (excl >> 16);
#pragma unroll
        for (int u = 0; u < kUQ; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (!in_j(qt + u, e)) continue;
                const int j = 4 * (qt + u) + e;
                if (kk[u][e] > T) {
                    row[ns + gt + min(eq, (uint32_t)k_rem)] = j;
                    ++gt;
                } else if (kk[u][e] == T) {
                    if (eq < (uint32_t)k_rem) row[ns + gt + eq] = j;
                    ++eq;
                }
            }
        gt_run += tot & 0xffffu;
        eq_run += tot >> 16;
    }
}

__global__ void __launch_bounds__(kThreads) sink_mask_kernel(MaskArgs a) {
    __shared__ float s_log_p0[1024];
    const int b = blockIdx.x, tid = threadIdx.x;
    for (int i = tid; i < a.Hq; i += kThreads) {
        const int64_t u = (int64_t)b * a.Hq + i;
        s_log_p0[i] = a.logits[u * a.logit_stride] - a.lse[u];
    }
    __syncthreads();
    for (int i = tid; i < a.Hq; i += kThreads) {
        const float x = s_log_p0[i];
        int rank = 0;
        for (int j = 0; j < a.Hq; ++j) {
            const float y = s_log_p0[j];
            rank += (y > x || (y == x && j < i)) ? 1 : 0;
        }
        a.head_mask[(int64_t)b * a.Hq + i] = rank < a.n_mask ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_select(const SelArgs& a, hipStream_t s) {
    if (a.unit_path) {
        hipLaunchKernelGGL(select_unit_kernel, dim3(a.Hkv, a.B), dim3(kUT), 0, s, a);
        return hipGetLastError();
    }
    const dim3 blk(kThreads);
    const dim3 g_head(a.nchunk, a.Hq, a.B);
    const dim3 g_group(a.nchunk, a.Hkv, a.B);
    const dim3 g_unit(a.Hkv, a.B);
    // with lse_j the dense step computed the log-sum-exp over J and cleared the histograms
    if (!a.lse_j) hipLaunchKernelGGL(lse_kernel, g_head, blk, 0, s, a);
    if (a.refine) hipLaunchKernelGGL(evidence_kernel<true>, g_group, blk, 0, s, a);
    else hipLaunchKernelGGL(evidence_kernel<false>, g_group, blk, 0, s, a);
    if (a.refine)
        hipLaunchKernelGGL(refine_kernel, dim3(a.nchunk * kCrossParts, a.B), dim3(kRefThreads), 0, s, a);
    hipLaunchKernelGGL(candidate_kernel, g_group, blk, 0, s, a);
    if (a.finish) {
        hipLaunchKernelGGL(finish_kernel, g_unit, dim3(kUT), 0, s, a);
    } else {
        hipLaunchKernelGGL(resolve_kernel, g_unit, dim3(kUT), 0, s, a);
        hipLaunchKernelGGL(emit_kernel, g_group, blk, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_sink_mask(const MaskArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(sink_mask_kernel, dim3(a.B), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace sfi
