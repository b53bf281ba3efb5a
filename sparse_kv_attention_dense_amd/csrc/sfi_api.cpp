// sfi_api.cpp -- host side of the libsfi.so C ABI (include/sfi.h): argument validation,
// workspace layout and kernel launches.  No allocation, no synchronisation, no device
// queries: the split plan depends only on the descriptor.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "sfi.h"
#include "sfi_internal.h"

#define SFI_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

using namespace sfi;

// Workgroups a launch aims for.  The attention kernel holds two tile buffers in registers
// (about 240 VGPRs), so two 4-wavefront workgroups are resident per CU: 512 on a 256-CU
// MI355X.  Dense steps on a contiguous cache use 1024 equal workgroups (two even rounds; 512
// and 2048 measured slower at 128K), or 256 (one workgroup per CU, one round) when the whole
// step holds at most 2^20 (sequence, KV head, position) triples: each workgroup then has
// only a few tiles, a second round costs more than it balances and fewer, longer workgroups
// amortise their start (one sequence of 32K: 512 workgroups 33.3-33.9 us, 256: 32.0-32.5;
// 64K 56.5 vs 54.8; 128K 105 vs 100.5; 1024 at 32K: 36.6; 128K and 512K batches keep 1024).  The dense grid lists only splits that hold positions,
// so on a paged cache, which usually holds sequences of unequal length, smaller splits
// (about 2048 workgroups at the longest length) even out the rounds: 292 vs 309 us for a
// ragged batch of 16 at 8K-32K.  A fast step moves little data and is bound by latency, so it
// uses about 256 larger workgroups with 32-slot granularity (608 workgroups of 256 slots
// measured 27% slower at 128K).  The plan depends only on the descriptor, so workspace sizes
// are the same on every device.
constexpr int64_t kTargetWorkgroups = 1024;
constexpr int64_t kSmallTargetWorkgroups = 256;
constexpr int64_t kSmallDenseRows = int64_t(1) << 20;    // one round of workgroups below this
constexpr int64_t kPagedTargetWorkgroups = 2048;
constexpr int64_t kSparseTargetWorkgroups = 256;
constexpr int64_t kSparseQuantum = kTile;
constexpr int64_t kSparseManySplits = 64;
constexpr size_t kAlign = 256;
constexpr double kUnitFixedUs = 14.7;           // Selector path estimates, see select_unit_path
constexpr double kUnitUsPerPos = 6.0e-4;
constexpr double kUnitUsPerPosHead = 1.1e-4;
constexpr double kChunkedFixedUs = 31.0;
constexpr double kChunkedUsPerMB = 0.37;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool aligned(const void* p, size_t n) { return ((uintptr_t)p % n) == 0; }

sfi_status check_desc(const sfi_kv_desc* kv, bool need_cache) {
    if (!kv) return SFI_E_INVALID;
    if (kv->batch < 1 || kv->num_q_heads < 1 || kv->num_kv_heads < 1) return SFI_E_INVALID;
    if (kv->num_q_heads % kv->num_kv_heads != 0) return SFI_E_INVALID;
    // the attention kernels hold a group in one MFMA N dimension; the Selector and the mask
    // only read logit rows
    if (kv->num_q_heads / kv->num_kv_heads > (need_cache ? kMaxG : kMaxSelG)) return SFI_E_UNSUPPORTED;
    if (kv->batch > 65535 || kv->num_kv_heads > 65535 || kv->num_q_heads > 65535) return SFI_E_UNSUPPORTED;
    if (kv->head_dim != 64 && kv->head_dim != 128) return SFI_E_UNSUPPORTED;
    if (kv->dtype != SFI_F32 && kv->dtype != SFI_BF16) return SFI_E_UNSUPPORTED;
    if (!kv->len || kv->max_len < 0) return SFI_E_INVALID;
    if (!need_cache) return SFI_OK;
    if (!kv->k || !kv->v || !aligned(kv->k, 16) || !aligned(kv->v, 16)) return SFI_E_INVALID;
    if (kv->block_table) {
        const int bs = kv->block_size;
        if (bs < 1 || bs > 1024 || (bs & (bs - 1)) != 0) return SFI_E_INVALID;
        if (kv->max_blocks < 1 || (int64_t)kv->max_blocks * bs < kv->max_len) return SFI_E_INVALID;
    } else {
        if (kv->n_cap < kv->max_len || kv->n_cap < 0) return SFI_E_INVALID;
        // row numbers are kept in 32 bits
        if ((int64_t)kv->batch * kv->num_kv_heads * kv->n_cap >= (int64_t(1) << 32)) return SFI_E_UNSUPPORTED;
    }
    return SFI_OK;
}

struct AttnPlan {
    int split_len = 0, nsplit = 0, rec = 0, tab_bytes = 0, bt_off = -1;
    size_t bytes = 0;
};

// Split plan: per (b, KV head) unit, nsplit workgroups of split_len slots each, about
// kTargetWorkgroups (dense) or kSparseTargetWorkgroups (sparse) per launch in total.
sfi_status plan_attention(const sfi_kv_desc& kv, bool sparse, int64_t idx_stride, int64_t n_recent,
                          AttnPlan* p, bool lse_j = false) {
    const bool paged = kv.block_table != nullptr;
    const int64_t units = (int64_t)kv.batch * kv.num_kv_heads;
    const int64_t G = kv.num_q_heads / kv.num_kv_heads;
    int64_t slots = sparse ? idx_stride + n_recent : (int64_t)kv.max_len;
    if (slots < 1) slots = 1;
    const int64_t quantum = sparse ? kSparseQuantum : kSplitQuantum;
    const bool small = units * (int64_t)kv.max_len <= kSmallDenseRows;
    const int64_t target = sparse ? kSparseTargetWorkgroups
                                  : (paged ? kPagedTargetWorkgroups
                                           : (small ? kSmallTargetWorkgroups : kTargetWorkgroups));
    const int64_t per_unit = ceil_div(target, units);
    int64_t split = ceil_div(ceil_div(slots, per_unit), quantum) * quantum;
    // a fast step over few KV heads would otherwise cut each head into many splits of one or
    // two tiles (one KV head at 512K: 145 splits of 64 slots, two of four wavefronts idle, 145
    // records to merge); past kSparseManySplits a split holds at least one tile per wavefront
    if (sparse && ceil_div(slots, split) > kSparseManySplits && split < kTile * kWaves)
        split = kTile * kWaves;
    if ((sparse || paged) && split > kTabMax) split = kTabMax;
    int64_t nsplit = ceil_div(slots, split);
    if (nsplit > kMaxSplits) {
        // longer splits, up to the row table's capacity where there is one
        split = ceil_div(ceil_div(slots, kMaxSplits), quantum) * quantum;
        if ((sparse || paged) && split > kTabMax) return SFI_E_UNSUPPORTED;   // > kMaxSplits * kTabMax slots
        nsplit = ceil_div(slots, split);
    }
    if (!sparse && nsplit * units >= (int64_t(1) << 31)) return SFI_E_UNSUPPORTED;   // 1-D grid
    p->split_len = (int)split;
    p->nsplit = (int)nsplit;
    // records: acc [G][d], (m, l) [G], and for the fused slow step (m, l) over J [G]
    p->rec = (int)(ceil_div(G * (kv.head_dim + (lse_j ? 4 : 2)), 4) * 4);
    int64_t tab = 0;
    if (sparse) {
        tab = split * 4 + split;                            // rows, then attend flags
    } else if (paged) {
        int shift = 0;
        while ((1 << shift) < kv.block_size) ++shift;
        tab = ((split >> shift) + 2) * 4;                   // one base row per block touched
    }
    p->tab_bytes = (int)(ceil_div(tab, 16) * 16);
    // fast step on a paged cache: the sequence's block table staged in LDS when it is short
    if (sparse && paged && kv.max_blocks <= kBtPer * kThreads) {
        p->bt_off = p->tab_bytes;                           // the sequence's block table
        p->tab_bytes += (int)(ceil_div((int64_t)kv.max_blocks * 4, 16) * 16);
    }
    // Partial records are sized for a bound on nsplit that never decreases as the length
    // grows (the split itself is rounded, so nsplit alone can), so a workspace sized for the
    // longest step of a cycle serves every shorter one.
    int64_t bound = ceil_div(slots, quantum);
    bound = std::min(bound, std::max(per_unit, (sparse || paged) ? ceil_div(slots, (int64_t)kTabMax) : 1));
    bound = std::min(bound, (int64_t)kMaxSplits);
    p->bytes = align_up((size_t)units * bound * p->rec * sizeof(float));
    return SFI_OK;
}

// Selector path.  One workgroup per (b, KV head) is bound by one compute unit's ALU rate on
// that unit's positions; the chunked kernels spread the work over the chip but pay for six
// launches.  The plan takes whichever is estimated faster from the descriptor alone, with
// linear fits to MI355X measurements of both paths on random logits: one workgroup per unit
// 18 us at 2K positions (G = 4), 42 us at 32K, 126 us at 128K, 209 us at 128K with G = 8,
// 66 us at 64K with G = 1; chunked 30 us at 32 KB of logits in all, 35 us at 4 MB, 37 us at
// 17 MB, 57 us at 67 MB, 81 us at 134 MB.
bool select_unit_path(const sfi_kv_desc& kv) {
    const double G = (double)kv.num_q_heads / kv.num_kv_heads;
    const double all_mb = (double)kv.batch * kv.num_q_heads * kv.max_len * 4.0 / 1e6;
    const double t_unit = kUnitFixedUs + (kUnitUsPerPos + kUnitUsPerPosHead * G) * kv.max_len;
    const double t_chunked = kChunkedFixedUs + kChunkedUsPerMB * all_mb;
    return t_unit < t_chunked;
}

struct SelPlan {
    int nchunk = 0;
    size_t off_lse = 0, off_keys = 0, off_hist = 0, off_state = 0, off_counts = 0;
    size_t off_cand = 0, off_cand_n = 0, off_epos = 0, bytes = 0;
    size_t off_zpart = 0, off_lfused = 0, off_epos_refined = 0, bytes_refined = 0;   // full Selector
};

void plan_select(const sfi_kv_desc& kv, SelPlan* p) {
    const size_t B = kv.batch, Hq = kv.num_q_heads, Hkv = kv.num_kv_heads;
    p->nchunk = (int)(kv.max_len > 0 ? ceil_div(kv.max_len, kSelChunk) : 1);
    const size_t nc = p->nchunk;
    size_t off = 0;
    p->off_lse = off;    off += align_up(B * Hq * nc * sizeof(float2));
    p->off_keys = off;   off += align_up(B * Hkv * nc * kSelChunk * sizeof(uint32_t));
    p->off_hist = off;   off += align_up(B * Hkv * kSelHistBins * sizeof(uint32_t));
    p->off_state = off;  off += align_up(B * Hkv * 4 * sizeof(int32_t));
    p->off_counts = off; off += align_up(B * Hkv * nc * 3 * sizeof(uint32_t));
    p->off_cand = off;   off += align_up(B * Hkv * nc * kSelChunk * sizeof(uint32_t));
    p->off_cand_n = off; off += align_up(B * Hkv * nc * sizeof(uint32_t));
    const size_t common = off;
    const size_t epos_bytes = align_up(B * Hkv * nc * kSelChunk * sizeof(int32_t));
    p->off_epos = off;   off += epos_bytes;
    p->bytes = off;
    // the full Selector's buffers follow the common part, then its own epos region
    off = common;
    p->off_zpart = off;  off += align_up(B * Hkv * nc * sizeof(float));
    p->off_lfused = off; off += align_up(B * Hkv * nc * kSelChunk * sizeof(float));
    p->off_epos_refined = off; off += epos_bytes;
    p->bytes_refined = off;
}

// rows of a compact segment [B][Hkv][idx_stride] (row numbers are kept in 32 bits)
int64_t segment_rows(const sfi_kv_desc& kv, int32_t idx_stride) {
    return (int64_t)kv.batch * kv.num_kv_heads * idx_stride;
}

sfi_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
    if (!ws || !aligned(ws, kAlign) || ws_bytes < need) return SFI_E_WORKSPACE;
    return SFI_OK;
}

void fill_cache_args(const sfi_kv_desc& kv, AttnArgs* a) {
    memset(a, 0, sizeof *a);
    a->k = kv.k;
    a->v = kv.v;
    a->len = kv.len;
    a->block_table = kv.block_table;
    a->n_cap = kv.n_cap;
    a->block_shift = 0;
    if (kv.block_table)
        while ((1 << a->block_shift) < kv.block_size) ++a->block_shift;
    a->max_blocks = kv.max_blocks;
    a->B = kv.batch;
    a->Hq = kv.num_q_heads;
    a->Hkv = kv.num_kv_heads;
    a->G = kv.num_q_heads / kv.num_kv_heads;
    a->scale = (float)(1.0 / sqrt((double)kv.head_dim));
    a->scale_log2 = (float)(1.4426950408889634 / sqrt((double)kv.head_dim));
}

void fill_plan_args(const AttnPlan& p, void* ws, AttnArgs* a) {
    a->split_len = p.split_len;
    a->nsplit = p.nsplit;
    a->tab_bytes = p.tab_bytes;
    a->bt_off = p.bt_off;
    a->rec_floats = p.rec;
    a->part = (float*)ws;
}

// ---- validation + argument packing, shared by the single calls and the layered slow step --

sfi_status prep_dense(const sfi_kv_desc* kv, const void* q, float* out, float* lse, float* logits,
                      int64_t logit_stride, void* ws, size_t ws_bytes, AttnArgs* a) {
    sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return SFI_E_INVALID;
    if (logits && (logit_stride < kv->max_len || logit_stride % 4 != 0 || !aligned(logits, 16)))
        return SFI_E_INVALID;
    AttnPlan plan;
    st = plan_attention(*kv, false, 0, 0, &plan);
    if (st != SFI_OK) return st;
    st = check_ws(ws, ws_bytes, plan.bytes);
    if (st != SFI_OK) return st;
    fill_cache_args(*kv, a);
    fill_plan_args(plan, ws, a);
    a->q = q;
    a->out = out;
    a->lse = lse;
    a->logits = logits;
    a->logit_stride = logit_stride;
    return SFI_OK;
}

sfi_status prep_select(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                       int32_t n_sink, int32_t n_recent, int32_t k_sel, int32_t* idx,
                       int32_t idx_stride, int32_t* n_idx, void* ws, size_t ws_bytes, SelArgs* a) {
    sfi_status st = check_desc(kv, false);
    if (st != SFI_OK) return st;
    if (!logits || !idx || !n_idx || logit_stride < kv->max_len || logit_stride < 1) return SFI_E_INVALID;
    if (logit_stride % 4 != 0 || !aligned(logits, 16)) return SFI_E_INVALID;
    if (n_sink < 0 || n_recent < 0 || k_sel < 0) return SFI_E_INVALID;
    if ((int64_t)idx_stride < (int64_t)n_sink + k_sel || idx_stride < 1) return SFI_E_INVALID;
    SelPlan plan;
    plan_select(*kv, &plan);
    st = check_ws(ws, ws_bytes, plan.bytes);
    if (st != SFI_OK) return st;
    unsigned char* base = (unsigned char*)ws;
    a->logits = logits;
    a->logit_stride = logit_stride;
    a->len = kv->len;
    a->B = kv->batch;
    a->Hq = kv->num_q_heads;
    a->Hkv = kv->num_kv_heads;
    a->G = kv->num_q_heads / kv->num_kv_heads;
    a->n_sink = n_sink;
    a->n_recent = n_recent;
    a->k_sel = k_sel;
    a->nchunk = plan.nchunk;
    a->idx = idx;
    a->idx_stride = idx_stride;
    a->n_idx = n_idx;
    a->lse_part = (float2*)(base + plan.off_lse);
    a->keys = (uint32_t*)(base + plan.off_keys);
    a->hist = (uint32_t*)(base + plan.off_hist);
    a->state = (int32_t*)(base + plan.off_state);
    a->counts = (uint32_t*)(base + plan.off_counts);
    a->cand = (uint32_t*)(base + plan.off_cand);
    a->cand_n = (uint32_t*)(base + plan.off_cand_n);
    a->epos = (int32_t*)(base + plan.off_epos);
    a->unit_path = select_unit_path(*kv) ? 1 : 0;
    a->finish = (int64_t)k_sel + kv->max_len / kFinishBinShare <= kFinishCap ? 1 : 0;
    a->refine = 0;
    a->key_norm = nullptr;
    a->norm_stride = 0;
    a->norm_vec = 0;
    a->lam = 0.f;
    a->keep_soft = a->keep_cross = 1.f;
    a->prior_decay = a->tail_frac = a->tail_brake = 0.f;
    a->zpart = nullptr;
    a->lfused = nullptr;
    a->lse_j = nullptr;
    return SFI_OK;
}

sfi_status prep_mask(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                     const float* lse, float frac, uint8_t* head_mask, MaskArgs* a) {
    sfi_status st = check_desc(kv, false);
    if (st != SFI_OK) return st;
    if (!logits || !lse || !head_mask || logit_stride < 1) return SFI_E_INVALID;
    if (!(frac >= 0.f && frac <= 1.f)) return SFI_E_INVALID;
    if (kv->num_q_heads > 1024) return SFI_E_UNSUPPORTED;
    a->logits = logits;
    a->logit_stride = logit_stride;
    a->lse = lse;
    a->B = kv->batch;
    a->Hq = kv->num_q_heads;
    a->n_mask = (int32_t)floor((double)frac * kv->num_q_heads);
    a->head_mask = head_mask;
    return SFI_OK;
}

sfi_status launch_dense(const sfi_kv_desc* kv, const AttnArgs& a, hipStream_t stream) {
    const hipError_t e = launch_attention(a, kv->batch, kv->head_dim, kv->dtype == SFI_BF16,
                                          kv->block_table != nullptr, false, stream);
    return e == hipSuccess ? SFI_OK : SFI_E_HIP;
}

}  // namespace

SFI_EXPORT sfi_status sfi_dense_decode(const sfi_kv_desc* kv, const void* q, float* out, float* lse,
                                       float* logits, int64_t logit_stride,
                                       void* ws, size_t ws_bytes, hipStream_t stream) {
    AttnArgs a;
    const sfi_status st = prep_dense(kv, q, out, lse, logits, logit_stride, ws, ws_bytes, &a);
    return st == SFI_OK ? launch_dense(kv, a, stream) : st;
}

namespace {

sfi_status sparse_impl(const sfi_kv_desc* kv, const void* q, const int32_t* idx,
                       int32_t idx_stride, const int32_t* n_idx, int32_t n_recent,
                       const uint8_t* head_mask, const float* route_lse, float gamma,
                       uint8_t* routed, const void* ck, const void* cv, float* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
    sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    if (!q || !out || !idx || !n_idx || !aligned(q, 16) || !aligned(out, 16)) return SFI_E_INVALID;
    if (idx_stride < 1 || n_recent < 0) return SFI_E_INVALID;
    if ((ck != nullptr) != (cv != nullptr)) return SFI_E_INVALID;
    if (ck) {
        if (!aligned(ck, 16) || !aligned(cv, 16)) return SFI_E_INVALID;
        if (segment_rows(*kv, idx_stride) >= (int64_t(1) << 32)) return SFI_E_UNSUPPORTED;
    }
    AttnPlan plan;
    st = plan_attention(*kv, true, idx_stride, n_recent, &plan);
    if (st != SFI_OK) return st;
    st = check_ws(ws, ws_bytes, plan.bytes);
    if (st != SFI_OK) return st;
    AttnArgs a;
    fill_cache_args(*kv, &a);
    fill_plan_args(plan, ws, &a);
    a.q = q;
    a.out = out;
    a.lse = lse;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.n_idx = n_idx;
    a.n_recent = n_recent;
    a.head_mask = head_mask;
    a.route_lse = route_lse;
    a.route_log_gamma = route_lse ? (float)log((double)gamma) : 0.f;
    a.routed = routed;
    a.ck = ck;
    a.cv = cv;
    const hipError_t e = launch_attention(a, kv->batch, kv->head_dim, kv->dtype == SFI_BF16,
                                          kv->block_table != nullptr, true, stream);
    return e == hipSuccess ? SFI_OK : SFI_E_HIP;
}

}  // namespace

SFI_EXPORT sfi_status sfi_sparse_decode(const sfi_kv_desc* kv, const void* q,
                                        const int32_t* idx, int32_t idx_stride, const int32_t* n_idx,
                                        int32_t n_recent, const uint8_t* head_mask,
                                        float* out, float* lse,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
    return sparse_impl(kv, q, idx, idx_stride, n_idx, n_recent, head_mask, nullptr, 1.f, nullptr,
                       nullptr, nullptr, out, lse, ws, ws_bytes, stream);
}

namespace {

// ---- the fast step on a library-owned scratch array (sfi_sparse_decode_noalloc) ------------
// Each GPU the library runs on holds its own copy of `scratch` until the process ends.  Host
// code never uses the array's name as an address: the per-device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kScratchBytes = SFI_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kScratchDevices = 256;
std::atomic<void*> g_scratch_addr[kScratchDevices];
std::mutex g_scratch_mutex;

sfi_status scratch_of_current_device(void** addr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return SFI_E_HIP;
    if (dev >= kScratchDevices) return SFI_E_UNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SFI_E_HIP;
            if (((uintptr_t)p % kAlign) != 0) return SFI_E_HIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return SFI_OK;
}

}  // namespace

SFI_EXPORT sfi_status sfi_sparse_decode_noalloc(const sfi_kv_desc* kv, const void* q,
                                                const int32_t* idx, int32_t idx_stride,
                                                const int32_t* n_idx, int32_t n_recent,
                                                const uint8_t* head_mask, float* out, float* lse,
                                                hipStream_t stream) {
    // host-side validation and the size check come before any HIP call
    sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    if (!q || !out || !idx || !n_idx || !aligned(q, 16) || !aligned(out, 16)) return SFI_E_INVALID;
    if (idx_stride < 1 || n_recent < 0) return SFI_E_INVALID;
    AttnPlan plan;
    st = plan_attention(*kv, true, idx_stride, n_recent, &plan);
    if (st != SFI_OK) return st;
    if (plan.bytes > kScratchBytes) return SFI_E_SCRATCH;
    void* ws = nullptr;
    st = scratch_of_current_device(&ws);
    if (st != SFI_OK) return st;
    return sparse_impl(kv, q, idx, idx_stride, n_idx, n_recent, head_mask, nullptr, 1.f, nullptr,
                       nullptr, nullptr, out, lse, ws, kScratchBytes, stream);
}

namespace {

sfi_status prep_reorg(const sfi_kv_desc* kv, const int32_t* idx, int32_t idx_stride,
                      const int32_t* n_idx, void* ck, void* cv, int32_t* cpos, ReorgArgs* out) {
    const sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    if (!idx || !n_idx || !ck || !cv || !cpos || idx_stride < 1) return SFI_E_INVALID;
    if (!aligned(ck, 16) || !aligned(cv, 16) || !aligned(cpos, 4)) return SFI_E_INVALID;
    if (segment_rows(*kv, idx_stride) >= (int64_t(1) << 32)) return SFI_E_UNSUPPORTED;
    ReorgArgs& a = *out;
    a.k = kv->k;
    a.v = kv->v;
    a.len = kv->len;
    a.block_table = kv->block_table;
    a.n_cap = kv->n_cap;
    a.block_shift = 0;
    if (kv->block_table)
        while ((1 << a.block_shift) < kv->block_size) ++a.block_shift;
    a.max_blocks = kv->max_blocks;
    a.Hkv = kv->num_kv_heads;
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.n_idx = n_idx;
    a.ck = ck;
    a.cv = cv;
    a.cpos = cpos;
    return SFI_OK;
}

hipError_t launch_reorg_for(const sfi_kv_desc* kv, const ReorgArgs& a, hipStream_t stream) {
    return launch_reorg(a, kv->batch, kv->head_dim * (kv->dtype == SFI_BF16 ? 2 : 4), stream);
}

}  // namespace

SFI_EXPORT sfi_status sfi_reorg(const sfi_kv_desc* kv, const int32_t* idx, int32_t idx_stride,
                                const int32_t* n_idx, void* ck, void* cv, int32_t* cpos,
                                hipStream_t stream) {
    ReorgArgs a;
    const sfi_status st = prep_reorg(kv, idx, idx_stride, n_idx, ck, cv, cpos, &a);
    if (st != SFI_OK) return st;
    return launch_reorg_for(kv, a, stream) == hipSuccess ? SFI_OK : SFI_E_HIP;
}

SFI_EXPORT sfi_status sfi_sparse_decode_compact(const sfi_kv_desc* kv, const void* q,
                                                const void* ck, const void* cv,
                                                const int32_t* cpos, int32_t idx_stride,
                                                const int32_t* n_idx, int32_t n_recent,
                                                const uint8_t* head_mask, float* out, float* lse,
                                                void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!ck || !cv) return SFI_E_INVALID;
    return sparse_impl(kv, q, cpos, idx_stride, n_idx, n_recent, head_mask, nullptr, 1.f, nullptr,
                       ck, cv, out, lse, ws, ws_bytes, stream);
}

SFI_EXPORT sfi_status sfi_sparse_decode_step(const sfi_kv_desc* kv, const sfi_step* step,
                                             int32_t idx_stride, int32_t max_recent, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
    if (!kv || !step || ((uintptr_t)step % 8) != 0) return SFI_E_INVALID;
    // shapes and capacities from the host descriptor; its pointers are not read (the device
    // descriptor's are), so stand-ins let the common checks run
    sfi_kv_desc hk = *kv;
    hk.k = hk.v = (const void*)kAlign;
    hk.len = (const int32_t*)kAlign;
    hk.max_len = 0;
    sfi_status st = check_desc(&hk, true);
    if (st != SFI_OK) return st;
    if (idx_stride < 1 || max_recent < 0) return SFI_E_INVALID;
    if (segment_rows(hk, idx_stride) >= (int64_t(1) << 32)) return SFI_E_UNSUPPORTED;
    AttnPlan plan;
    st = plan_attention(hk, true, idx_stride, max_recent, &plan);
    if (st != SFI_OK) return st;
    st = check_ws(ws, ws_bytes, plan.bytes);
    if (st != SFI_OK) return st;
    AttnArgs a;
    fill_cache_args(hk, &a);
    fill_plan_args(plan, ws, &a);
    a.idx_stride = idx_stride;
    a.n_recent = max_recent;
    a.step = step;
    const hipError_t e = launch_attention(a, kv->batch, kv->head_dim, kv->dtype == SFI_BF16,
                                          kv->block_table != nullptr, true, stream);
    return e == hipSuccess ? SFI_OK : SFI_E_HIP;
}

SFI_EXPORT sfi_status sfi_sparse_decode_routed(const sfi_kv_desc* kv, const void* q,
                                               const int32_t* idx, int32_t idx_stride,
                                               const int32_t* n_idx, int32_t n_recent,
                                               const uint8_t* head_mask, const float* route_lse,
                                               float gamma, uint8_t* routed, float* out, float* lse,
                                               void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!route_lse || !(gamma > 0.f && gamma <= 1.f)) return SFI_E_INVALID;
    return sparse_impl(kv, q, idx, idx_stride, n_idx, n_recent, head_mask, route_lse, gamma, routed,
                       nullptr, nullptr, out, lse, ws, ws_bytes, stream);
}

SFI_EXPORT sfi_status sfi_select(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                                 int32_t n_sink, int32_t n_recent, int32_t k_sel,
                                 int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
    SelArgs a;
    const sfi_status st = prep_select(kv, logits, logit_stride, n_sink, n_recent, k_sel, idx,
                                      idx_stride, n_idx, ws, ws_bytes, &a);
    if (st != SFI_OK) return st;
    return launch_select(a, stream) == hipSuccess ? SFI_OK : SFI_E_HIP;
}

SFI_EXPORT sfi_status sfi_select_refined(const sfi_kv_desc* kv, const float* logits,
                                         int64_t logit_stride, const float* key_norm,
                                         int64_t norm_stride, int32_t n_sink, int32_t n_recent,
                                         int32_t k_sel, const sfi_refine* params, int32_t* idx,
                                         int32_t idx_stride, int32_t* n_idx, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
    if (!params) return SFI_E_INVALID;
    const sfi_refine& p = *params;
    if (!(p.lambda >= 0.f && p.lambda < 1.f) || !(p.alpha_soft >= 0.f && p.alpha_soft < 1.f) ||
        !(p.alpha_cross >= 0.f && p.alpha_cross < 1.f) || !(p.prior_decay >= 0.f) ||
        !(p.tail_frac >= 0.f && p.tail_frac <= 1.f) || !(p.tail_brake >= 0.f))
        return SFI_E_INVALID;
    if (key_norm && (norm_stride < kv->max_len || norm_stride < 1)) return SFI_E_INVALID;
    SelArgs a;
    sfi_status st = prep_select(kv, logits, logit_stride, n_sink, n_recent, k_sel, idx,
                                idx_stride, n_idx, ws, ws_bytes, &a);
    if (st != SFI_OK) return st;
    SelPlan plan;
    plan_select(*kv, &plan);
    st = check_ws(ws, ws_bytes, plan.bytes_refined);
    if (st != SFI_OK) return st;
    a.unit_path = 0;                        // the exclusivity pass couples the KV heads
    a.refine = 1;
    a.key_norm = key_norm;
    a.norm_stride = norm_stride;
    a.norm_vec = key_norm && aligned(key_norm, 16) && norm_stride % 4 == 0 ? 1 : 0;
    a.lam = p.lambda;
    a.keep_soft = 1.f - p.alpha_soft;
    a.keep_cross = 1.f - p.alpha_cross;
    a.prior_decay = p.prior_decay;
    a.tail_frac = p.tail_frac;
    a.tail_brake = p.tail_brake;
    a.zpart = (float*)((unsigned char*)ws + plan.off_zpart);
    a.lfused = (float*)((unsigned char*)ws + plan.off_lfused);
    a.epos = (int32_t*)((unsigned char*)ws + plan.off_epos_refined);
    return launch_select(a, stream) == hipSuccess ? SFI_OK : SFI_E_HIP;
}

SFI_EXPORT sfi_status sfi_sink_bypass_mask(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                                           const float* lse, float frac, uint8_t* head_mask,
                                           hipStream_t stream) {
    MaskArgs a;
    const sfi_status st = prep_mask(kv, logits, logit_stride, lse, frac, head_mask, &a);
    if (st != SFI_OK) return st;
    return launch_sink_mask(a, stream) == hipSuccess ? SFI_OK : SFI_E_HIP;
}

namespace {

// Slot layout of the layered slow step: the Selector's normaliser over J [B][Hq], then the
// Selector's workspace.
size_t slot_lse_bytes(const sfi_kv_desc& kv) {
    return align_up((size_t)kv.batch * kv.num_q_heads * sizeof(float));
}

// Validation and argument packing of one layer of the layered slow step (the fused form of
// sfi_slow_step, with the dense records in dense_ws and the normaliser and Selector in the
// slot's workspace).
sfi_status prep_layer(const sfi_kv_desc* kv, const void* q, float* out, float* lse, float* logits,
                      int64_t logit_stride, void* dense_ws, size_t dense_ws_bytes, void* sel_ws,
                      size_t sel_ws_bytes, int32_t n_sink, int32_t n_recent, int32_t k_sel,
                      int32_t* idx, int32_t idx_stride, int32_t* n_idx, AttnArgs* da,
                      SelArgs* sa) {
    if (!lse || !logits) return SFI_E_INVALID;
    sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    AttnPlan plan;
    st = plan_attention(*kv, false, 0, 0, &plan, true);
    if (st != SFI_OK) return st;
    st = check_ws(dense_ws, dense_ws_bytes, plan.bytes);
    if (st != SFI_OK) return st;
    st = prep_dense(kv, q, out, lse, logits, logit_stride, dense_ws, dense_ws_bytes, da);
    if (st != SFI_OK) return st;
    const size_t lse_bytes = slot_lse_bytes(*kv);
    if (!sel_ws || sel_ws_bytes < lse_bytes) return SFI_E_WORKSPACE;
    st = prep_select(kv, logits, logit_stride, n_sink, n_recent, k_sel, idx, idx_stride, n_idx,
                     (unsigned char*)sel_ws + lse_bytes, sel_ws_bytes - lse_bytes, sa);
    if (st != SFI_OK) return st;
    fill_plan_args(plan, dense_ws, da);
    da->lse_j = (float*)sel_ws;
    da->n_sink = n_sink;
    da->n_recent = n_recent;
    da->sel_hist = sa->hist;
    sa->lse_j = da->lse_j;
    return SFI_OK;
}

}  // namespace

SFI_EXPORT sfi_status sfi_slow_step_layers(
        int32_t n_layers, const sfi_kv_desc* kv, const void* const* q, float* const* out,
        float* const* lse, int32_t n_slots, float* const* logits, int64_t logit_stride,
        void* const* sel_ws, size_t sel_ws_bytes, void* dense_ws, size_t dense_ws_bytes,
        int32_t n_sink, int32_t n_recent, int32_t k_sel, int32_t* const* idx, int32_t idx_stride,
        int32_t* const* n_idx, float mask_frac, uint8_t* const* head_mask,
        void* const* seg_k, void* const* seg_v, int32_t* const* seg_pos,
        hipStream_t stream, hipStream_t side_stream, hipEvent_t* slot_events,
        hipEvent_t attn_event, hipEvent_t done_event) {
    if (n_layers < 1 || n_slots < 1 || !kv || !q || !out || !lse || !logits || !sel_ws || !idx ||
        !n_idx || !slot_events || !attn_event || !done_event || stream == side_stream)
        return SFI_E_INVALID;
    const bool reorg = seg_k != nullptr;
    if (reorg != (seg_v != nullptr) || reorg != (seg_pos != nullptr)) return SFI_E_INVALID;
    for (int s = 0; s < n_slots; ++s)
        if (!slot_events[s]) return SFI_E_INVALID;
    // Every layer's arguments pass validation before anything is queued.
    for (int l = 0; l < n_layers; ++l) {
        const int s = l % n_slots;
        AttnArgs da;
        SelArgs sa;
        MaskArgs ma;
        sfi_status st = prep_layer(&kv[l], q[l], out[l], lse[l], logits[s], logit_stride,
                                   dense_ws, dense_ws_bytes, sel_ws[s], sel_ws_bytes, n_sink,
                                   n_recent, k_sel, idx[l], idx_stride, n_idx[l], &da, &sa);
        if (st == SFI_OK && head_mask)
            st = prep_mask(&kv[l], logits[s], logit_stride, lse[l], mask_frac, head_mask[l], &ma);
        ReorgArgs ra;
        if (st == SFI_OK && reorg)
            st = prep_reorg(&kv[l], idx[l], idx_stride, n_idx[l], seg_k[l], seg_v[l], seg_pos[l],
                            &ra);
        if (st != SFI_OK) return st;
    }
    for (int l = 0; l < n_layers; ++l) {
        const int s = l % n_slots;
        AttnArgs da;
        SelArgs sa;
        MaskArgs ma;
        prep_layer(&kv[l], q[l], out[l], lse[l], logits[s], logit_stride, dense_ws, dense_ws_bytes,
                   sel_ws[s], sel_ws_bytes, n_sink, n_recent, k_sel, idx[l], idx_stride, n_idx[l],
                   &da, &sa);
        // the slot's logits and Selector workspace are free once layer l - n_slots is selected
        if (l >= n_slots && hipStreamWaitEvent(stream, slot_events[s], 0) != hipSuccess) return SFI_E_HIP;
        if (launch_dense(&kv[l], da, stream) != SFI_OK) return SFI_E_HIP;
        if (hipEventRecord(attn_event, stream) != hipSuccess) return SFI_E_HIP;
        if (hipStreamWaitEvent(side_stream, attn_event, 0) != hipSuccess) return SFI_E_HIP;
        if (launch_select(sa, side_stream) != hipSuccess) return SFI_E_HIP;
        if (head_mask) {
            prep_mask(&kv[l], logits[s], logit_stride, lse[l], mask_frac, head_mask[l], &ma);
            if (launch_sink_mask(ma, side_stream) != hipSuccess) return SFI_E_HIP;
        }
        if (hipEventRecord(slot_events[s], side_stream) != hipSuccess) return SFI_E_HIP;
        // Reorg reads the layer's own cache and indices, not the slot, so it runs after the
        // slot is released
        if (reorg) {
            ReorgArgs ra;
            prep_reorg(&kv[l], idx[l], idx_stride, n_idx[l], seg_k[l], seg_v[l], seg_pos[l], &ra);
            if (launch_reorg_for(&kv[l], ra, side_stream) != hipSuccess) return SFI_E_HIP;
        }
    }
    // one completion barrier: later work on `stream` sees every layer's indices and masks
    if (hipEventRecord(done_event, side_stream) != hipSuccess) return SFI_E_HIP;
    if (hipStreamWaitEvent(stream, done_event, 0) != hipSuccess) return SFI_E_HIP;
    return SFI_OK;
}

namespace {

// Workspace of the fused slow step: the dense records (with the pairs over J), then lse_j
// [B][Hq], then the Selector's own layout.
struct SlowLayout {
    AttnPlan dense;
    SelPlan sel;
    size_t off_lse_j = 0, off_sel = 0, bytes = 0;
};

sfi_status plan_slow(const sfi_kv_desc& kv, SlowLayout* p) {
    const sfi_status st = plan_attention(kv, false, 0, 0, &p->dense, true);
    if (st != SFI_OK) return st;
    plan_select(kv, &p->sel);
    p->off_lse_j = p->dense.bytes;
    p->off_sel = p->off_lse_j + align_up((size_t)kv.batch * kv.num_q_heads * sizeof(float));
    p->bytes = p->off_sel + p->sel.bytes;
    return SFI_OK;
}

}  // namespace

SFI_EXPORT sfi_status sfi_slow_step(const sfi_kv_desc* kv, const void* q, float* out, float* lse,
                                    float* logits, int64_t logit_stride, int32_t n_sink,
                                    int32_t n_recent, int32_t k_sel, int32_t* idx,
                                    int32_t idx_stride, int32_t* n_idx, float mask_frac,
                                    uint8_t* head_mask, void* ws, size_t ws_bytes,
                                    hipEvent_t dense_begin, hipEvent_t dense_done,
                                    hipStream_t stream) {
    sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    if (!logits || !lse) return SFI_E_INVALID;
    if (kv->num_q_heads / kv->num_kv_heads > kMaxG) return SFI_E_UNSUPPORTED;
    SlowLayout lay;
    st = plan_slow(*kv, &lay);
    if (st != SFI_OK) return st;
    st = check_ws(ws, ws_bytes, lay.bytes);
    if (st != SFI_OK) return st;
    unsigned char* base = (unsigned char*)ws;
    AttnArgs da;
    // the dense step validates against its own part of the workspace
    st = prep_dense(kv, q, out, lse, logits, logit_stride, ws, lay.off_lse_j, &da);
    if (st != SFI_OK) return st;
    SelArgs sa;
    st = prep_select(kv, logits, logit_stride, n_sink, n_recent, k_sel, idx, idx_stride, n_idx,
                     base + lay.off_sel, lay.sel.bytes, &sa);
    if (st != SFI_OK) return st;
    MaskArgs ma;
    if (head_mask) {
        st = prep_mask(kv, logits, logit_stride, lse, mask_frac, head_mask, &ma);
        if (st != SFI_OK) return st;
    }
    fill_plan_args(lay.dense, ws, &da);
    da.lse_j = (float*)(base + lay.off_lse_j);
    da.n_sink = n_sink;
    da.n_recent = n_recent;
    da.sel_hist = sa.hist;
    sa.lse_j = da.lse_j;
    if (dense_begin && hipEventRecord(dense_begin, stream) != hipSuccess) return SFI_E_HIP;
    if (launch_dense(kv, da, stream) != SFI_OK) return SFI_E_HIP;
    if (dense_done && hipEventRecord(dense_done, stream) != hipSuccess) return SFI_E_HIP;
    if (launch_select(sa, stream) != hipSuccess) return SFI_E_HIP;
    if (head_mask && launch_sink_mask(ma, stream) != hipSuccess) return SFI_E_HIP;
    return SFI_OK;
}

SFI_EXPORT size_t sfi_workspace_bytes(const sfi_kv_desc* kv, int32_t op, int32_t idx_stride,
                                      int32_t n_recent) {
    if (op == SFI_OP_SLOW) {
        if (check_desc(kv, true) != SFI_OK) return 0;
        if (kv->num_q_heads / kv->num_kv_heads > kMaxG) return 0;
        SlowLayout lay;
        if (plan_slow(*kv, &lay) != SFI_OK) return 0;
        return lay.bytes;
    }
    if (op == SFI_OP_SELECT) {
        if (check_desc(kv, false) != SFI_OK) return 0;
        SelPlan p;
        plan_select(*kv, &p);
        return p.bytes;
    }
    if (op == SFI_OP_SELECT_REFINED) {
        if (check_desc(kv, false) != SFI_OK) return 0;
        SelPlan p;
        plan_select(*kv, &p);
        return p.bytes_refined;
    }
    if (op != SFI_OP_DENSE && op != SFI_OP_SPARSE) return 0;
    if (check_desc(kv, true) != SFI_OK) return 0;
    if (op == SFI_OP_SPARSE && (idx_stride < 1 || n_recent < 0)) return 0;
    AttnPlan p;
    if (plan_attention(*kv, op == SFI_OP_SPARSE, idx_stride, n_recent, &p) != SFI_OK) return 0;
    return p.bytes;
}

SFI_EXPORT sfi_status sfi_stream_read(const void* buf, uint64_t bytes, int32_t n_workgroups,
                                      uint32_t* sink, hipStream_t stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(buf, 16) ||
        !aligned(sink, 4) || n_workgroups < 1 || n_workgroups > (1 << 20))
        return SFI_E_INVALID;
    return launch_stream_read(buf, bytes, n_workgroups, sink, stream) == hipSuccess ? SFI_OK
                                                                                     : SFI_E_HIP;
}

SFI_EXPORT sfi_status sfi_group_dot(const void* rows, int64_t n_rows, const void* q, int32_t G,
                                    int32_t unit, int32_t n_workgroups, float* part,
                                    uint32_t* sink, hipStream_t stream) {
    if (!rows || !q || !sink || n_rows < 16 || n_rows % 16 != 0 || !aligned(rows, 16) ||
        !aligned(q, 16) || !aligned(sink, 4) || unit < 0 || unit > 2 || n_workgroups < 1 ||
        n_workgroups > (1 << 20))
        return SFI_E_INVALID;
    if (unit != 0 && (!part || !aligned(part, 4))) return SFI_E_INVALID;
    if (G != 1 && G != 2 && G != 4 && G != 8) return SFI_E_UNSUPPORTED;
    return launch_group_dot(rows, (uint64_t)n_rows, q, G, unit, n_workgroups, part, sink,
                            stream) == hipSuccess ? SFI_OK : SFI_E_HIP;
}

SFI_EXPORT sfi_status sfi_gather_read(const sfi_kv_desc* kv, const int32_t* idx,
                                      int32_t idx_stride, const int32_t* n_idx, int32_t n_recent,
                                      int32_t n_workgroups, uint32_t* sink, hipStream_t stream) {
    const sfi_status st = check_desc(kv, true);
    if (st != SFI_OK) return st;
    if (!idx || !n_idx || !sink || idx_stride < 1 || n_recent < 0 || !aligned(sink, 4) ||
        n_workgroups < 1 || n_workgroups > (1 << 20))
        return SFI_E_INVALID;
    const int64_t units = (int64_t)kv->batch * kv->num_kv_heads;
    const int64_t slots = (int64_t)idx_stride + n_recent;
    const int64_t per_unit = ceil_div(n_workgroups, units);
    const int64_t split = ceil_div(ceil_div(slots, per_unit), kTile) * kTile;
    const int64_t nsplit = ceil_div(slots, split);
    if (nsplit > 65535) return SFI_E_UNSUPPORTED;
    GatherArgs a;
    memset(&a, 0, sizeof a);
    a.k = kv->k;
    a.v = kv->v;
    a.len = kv->len;
    a.block_table = kv->block_table;
    a.n_cap = kv->n_cap;
    if (kv->block_table)
        while ((1 << a.block_shift) < kv->block_size) ++a.block_shift;
    a.max_blocks = kv->max_blocks;
    a.Hkv = kv->num_kv_heads;
    a.row_bytes = kv->head_dim * (kv->dtype == SFI_BF16 ? 2 : 4);
    a.idx = idx;
    a.idx_stride = idx_stride;
    a.n_idx = n_idx;
    a.n_recent = n_recent;
    a.split_len = (int32_t)split;
    a.sink = sink;
    return launch_gather_read(a, (int)nsplit, kv->batch, stream) == hipSuccess ? SFI_OK : SFI_E_HIP;
}

SFI_EXPORT const char* sfi_status_string(sfi_status s) {
    switch (s) {
        case SFI_OK: return "SFI_OK: success";
        case SFI_E_INVALID: return "SFI_E_INVALID: invalid pointer, size or alignment";
        case SFI_E_UNSUPPORTED: return "SFI_E_UNSUPPORTED: head_dim, dtype, group size or length not supported";
        case SFI_E_WORKSPACE: return "SFI_E_WORKSPACE: workspace missing, misaligned or too small";
        case SFI_E_HIP: return "SFI_E_HIP: HIP runtime error at launch";
        case SFI_E_SCRATCH:
            return "SFI_E_SCRATCH: the step needs more than the library's static scratch array holds";
    }
    return "unknown sfi_status";
}
