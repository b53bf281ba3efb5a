// sfi_internal.h -- launch arguments and plans shared by the HIP sources of libsfi.so.
// Not part of the public ABI (include/sfi.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sfi.h"

namespace sfi {

// ---- attention kernels (dense slow step and sparse fast step share one kernel) ----------

constexpr int kThreads = 256;        // 4 wavefronts of 64
constexpr int kWaves = 4;
constexpr int kSparseWaves = 4;      // wavefronts of a fast-step workgroup
constexpr int kBtPer = 12;           // staged block-table entries per thread (fast step, paged)
constexpr int kTile = 32;            // slots per wavefront iteration (two 16-row MFMA blocks)
constexpr int kSplitQuantum = kTile * kWaves;
constexpr int kTabMax = 4096;        // row-table entries per workgroup (dynamic LDS)
constexpr int kMaxSplits = 1024;     // partial records per (b, h) that the combine merges
constexpr int kMaxG = 16;            // query heads per KV head (MFMA N dimension)
constexpr int kMaxSelG = 64;         // logit rows per KV head that the Selector and the mask
                                     // take (query heads, or query heads x window queries)
// The host stages a fast step's block table when it has at most kBtPer * kThreads entries, and
// the kernel loads kBtPer entries per thread of its own workgroup; the routing prologue gives
// each of the kMaxG * d / 8 (head, 8-element piece) pairs of a group one thread.
static_assert(kSparseWaves * 64 >= kThreads, "a fast-step workgroup stages the whole block table");
static_assert(kSparseWaves * 64 >= kMaxG * 128 / 8, "routing needs one thread per head piece");

struct AttnArgs {
    const void* k;
    const void* v;
    const void* q;
    const int32_t* len;
    const int32_t* block_table;      // paged only
    int64_t n_cap;                   // contiguous only
    int32_t block_shift;             // log2(block_size), paged only
    int32_t max_blocks;
    int32_t B, Hq, Hkv, G;
    float scale;                     // 1/sqrt(d)
    float scale_log2;                // scale * log2(e)
    float* logits;                   // dense only, may be null
    int64_t logit_stride;
    int32_t split_len;               // slots per workgroup, a multiple of kTile
    int32_t nsplit;                  // workgroups per (b, h)
    int32_t tab_bytes;               // dynamic LDS of the row table
    int32_t bt_off;                  // sparse paged: byte offset of the staged block table in
                                     //   the dynamic LDS, or -1 when it is not staged
    int32_t rec_floats;              // floats per partial record (G*(d+2) rounded to 4)
    const int32_t* idx;              // sparse only
    int32_t idx_stride;
    const int32_t* n_idx;
    int32_t n_recent;
    const uint8_t* head_mask;        // sparse only, may be null
    const float* route_lse;          // sparse only, may be null: per-head cached lse for routing
    float route_log_gamma;           // log(gamma) of the routing threshold
    uint8_t* routed;                 // may be null: [B][Hkv] routing decisions
    const void* ck;                  // sparse only, may be null: compact segment of the
    const void* cv;                  //   two-segment step, [B][Hkv][idx_stride][d]
    float* out;
    float* lse;                      // may be null
    float* part;                     // [units][nsplit][rec]: acc [G][d], then (m, l) [G], then
                                     //   (m, l) over the Selector's allowed set [G] (lse_j only)
    // dense step of sfi_slow_step: the log-sum-exp of each query head's logits over the
    // Selector's allowed set J = [n_sink, len - n_recent) goes to lse_j [B][Hq] (natural log),
    // and the combine clears the Selector's digit-0 histograms sel_hist [B*Hkv][kSelHistBins]
    float* lse_j;                    // null: not computed
    int32_t n_sink;                  // with n_recent above: the bounds of J
    uint32_t* sel_hist;
    // fast step of sfi_sparse_decode_step: the per-step pointers and the recent window are
    // read from this device descriptor at kernel entry (null: the fields above hold them)
    const sfi_step* step;
};

hipError_t launch_attention(const AttnArgs& a, int B, int d, bool bf16, bool paged, bool sparse,
                            hipStream_t stream);

// ---- selector -------------------------------------------------------------------------

constexpr int kSelChunk = 4096;      // positions of J per workgroup
constexpr int kRadixBins = 2048;     // LDS histogram bins of the one-launch path
// Entries (kept keys and candidates of one unit) that finish_kernel holds in LDS.  The chunked
// Selector ends in finish_kernel (one launch for the unit's resolve and emit) when
// k_sel + max_len / kFinishBinShare <= kFinishCap: the kept keys and a generous bound on the
// candidates (the digit-0 bin of the k-th largest key held 0.4-0.6 % of J on the benchmark's
// logits) fit in LDS; otherwise in the resolve and emit passes.
constexpr int kFinishCap = 16384;
constexpr int64_t kFinishBinShare = 64;
constexpr int kSelHistBins = 4096;   // digit-0 bins of the chunked path

struct SelArgs {
    const float* logits;
    int64_t logit_stride;
    const int32_t* len;
    int32_t B, Hq, Hkv, G;
    int32_t n_sink, n_recent, k_sel;
    int32_t nchunk;
    int32_t* idx;
    int32_t idx_stride;
    int32_t* n_idx;
    float2* lse_part;                // [B][Hq][nchunk]
    uint32_t* keys;                  // [B][Hkv][nchunk*kSelChunk]
    uint32_t* hist;                  // [B][Hkv][kSelHistBins]: digit 0 of the keys
    int32_t* state;                  // [B][Hkv][4]: prefix, k_rem, nJ, take_all
    uint32_t* counts;                // [B][Hkv][nchunk][3]: keys of higher digit-0 bins,
                                     // candidates > T, kept keys == T, per chunk
    uint32_t* cand;                  // [B][Hkv][nchunk][kSelChunk]: keys of the digit-0 bin
    uint32_t* cand_n;                // [B][Hkv][nchunk]: candidates per chunk
    const float* lse_j;              // [B][Hq] log-sum-exp over J from the dense step (natural
                                     //   log; the histograms are then already cleared), or null
    int32_t unit_path;               // 1: one workgroup per (b, KV head) does everything
    int32_t finish;                  // 1: the chunked path ends in finish_kernel (one launch)
                                     //   instead of the candidate, resolve and emit passes
    int32_t* epos;                   // [B][Hkv][nchunk*kSelChunk]: positions of finish_kernel's
                                     //   entries past its LDS (their keys go to cand)
    // full Selector (refine != 0): prior, reverse-KL fusion, Soft-NMS, cross-head exclusivity
    int32_t refine;
    const float* key_norm;           // [B][Hkv][norm_stride] or null (no key-norm factor)
    int64_t norm_stride;
    int32_t norm_vec;                // 1: key_norm and norm_stride allow 16-byte loads
    float lam;                       // fusion weight of the prior, in [0, 1)
    float keep_soft, keep_cross;     // 1 - alpha_soft, 1 - alpha_cross
    float prior_decay, tail_frac, tail_brake;
    float* zpart;                    // [B][Hkv][nchunk]: partial sums of f^(1-lam) r^lam
    float* lfused;                   // [B][Hkv][nchunk*kSelChunk]: log2 of f^(1-lam) r^lam by
                                     //   j - j0 (unnormalised), written by the evidence pass
};

hipError_t launch_select(const SelArgs& a, hipStream_t stream);

struct MaskArgs {
    const float* logits;
    int64_t logit_stride;
    const float* lse;
    int32_t B, Hq;
    int32_t n_mask;
    uint8_t* head_mask;
};

hipError_t launch_sink_mask(const MaskArgs& a, hipStream_t stream);

// Reorg of the two-segment layout (sfi_reorg.hip): copies the rows named by idx into the
// compact segment ck / cv [B][Hkv][idx_stride][row_bytes] and their positions into cpos.
struct ReorgArgs {
    const void* k;
    const void* v;
    const int32_t* len;
    const int32_t* block_table;      // null when contiguous
    int64_t n_cap;
    int32_t block_shift, max_blocks, Hkv;
    const int32_t* idx;
    int32_t idx_stride;
    const int32_t* n_idx;
    void* ck;
    void* cv;
    int32_t* cpos;
};

hipError_t launch_reorg(const ReorgArgs& a, int B, int row_bytes, hipStream_t stream);

// Streaming-read yardstick (sfi_stream.hip): n_wg workgroups each read a contiguous chunk of
// buf (bytes a multiple of 16); sink is a device buffer of kStreamSinkWords words.
constexpr int kStreamSinkWords = 64;
hipError_t launch_stream_read(const void* buf, uint64_t bytes, int n_wg, uint32_t* sink,
                              hipStream_t stream);

// Gather yardstick (sfi_stream.hip): the key and value rows of a fast step, no arithmetic.
struct GatherArgs {
    const void* k;
    const void* v;
    const int32_t* len;
    const int32_t* block_table;      // null when contiguous
    int64_t n_cap;
    int32_t block_shift, max_blocks, Hkv;
    int32_t row_bytes;               // d * element bytes
    const int32_t* idx;
    int32_t idx_stride;
    const int32_t* n_idx;
    int32_t n_recent;
    int32_t split_len;               // slots per workgroup
    uint32_t* sink;
};
hipError_t launch_gather_read(const GatherArgs& a, int nsplit, int B, hipStream_t stream);

// Group dot yardstick (sfi_stream.hip): the G query heads' dot products with n_rows bf16 rows of
// 128 elements (n_rows a multiple of 16) on unit 0 (none: a read), 1 (vector ALUs) or 2 (MFMA);
// units 1 and 2 write one partial sum per workgroup to part, unit 0 may write sink.
hipError_t launch_group_dot(const void* rows, uint64_t n_rows, const void* q, int G, int unit,
                            int n_wg, float* part, uint32_t* sink, hipStream_t stream);

}  // namespace sfi
