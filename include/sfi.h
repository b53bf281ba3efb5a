/*
 * sfi.h -- C ABI of libsfi.so: Slow-Fast decode attention on AMD Instinct MI355X (gfx950).
 *
 * One decode step of grouped-query attention over a long KV cache, in the slow/fast form
 * of "Slow-Fast Inference" (SFI):
 *   - a slow step runs dense attention over the whole history and exposes the attention
 *     logits (SFI Sec. 1; Sec. 4.2, kernels that expose logits)          -> sfi_dense_decode
 *   - the Selector turns those logits into a per-KV-head Top-K index set
 *     (SFI Sec. 3.2 evidence from slow-step logits, Sec. 3.3 Top-K)      -> sfi_select
 *   - a sink-bypass mask marks query heads whose token-0 attention mass is largest
 *     (SinkRouter Sec. 4.2, target regime and execution policy)          -> sfi_sink_bypass_mask
 *   - the three in one call, the Selector's normaliser over the allowed set kept by the
 *     dense step (SFI Sec. 3.2 and Sec. 4.2)                              -> sfi_slow_step
 *   - a fast step attends only to sink + selected + recent positions
 *     (SFI Sec. 1, the compact cache of fast steps)                       -> sfi_sparse_decode
 *   - the same with its per-step state read from a device step descriptor
 *     (SFI Sec. 4.2, the packed per-step descriptor)                     -> sfi_sparse_decode_step
 *   - the same with its partial records in a library-held device array, for callers that
 *     cannot allocate                                                   -> sfi_sparse_decode_noalloc
 *   - the same with SinkRouter's inline group routing (SinkRouter Sec. 4.2-4.3)
 *                                                                        -> sfi_sparse_decode_routed
 *   - the slow step over a model's layers with the Selector on a second stream
 *     (SFI Sec. 4.1, layer-wise asynchronous execution)                  -> sfi_slow_step_layers
 *   - the Selector with the cache-aware prior, fusion and refinements
 *     (SFI Sec. 3.2-3.3)                                                  -> sfi_select_refined
 *   - the two-segment layout: copy sink + selected rows into a compact segment, then fast
 *     steps that read it (SFI Sec. 4.1-4.2, Reorg and the coalesced
 *     sparse kernel)                          -> sfi_reorg, sfi_sparse_decode_compact
 *   - a plain streaming read, the measured bandwidth yardstick (not a step of the method)
 *                                                                        -> sfi_stream_read
 *   - a read of exactly the rows a fast step gathers, its floor (not a step of the method)
 *                                                                        -> sfi_gather_read
 *   - the GQA group's dot products over a stream of key rows on the vector ALUs or on MFMA,
 *     beside a read of the same rows (not a step of the method)          -> sfi_group_dot
 *
 * Conventions shared by every call
 *   - Every pointer marked "device" is HIP device memory owned by the caller.  The library
 *     never allocates, keeps no pointer after a call returns, and holds no global state;
 *     the one exception is sfi_sparse_decode_noalloc, which runs on a static device array of
 *     the library instead of a caller workspace (see its declaration).
 *   - Calls are asynchronous on `stream` (0 = the null stream) and never synchronise the
 *     host.  A returned SFI_OK means the arguments passed host-side validation and the
 *     launches were queued; device data (lengths, block tables, indices) is trusted.
 *   - Scores use scale 1/sqrt(head_dim) and query head i reads KV head i / G with
 *     G = num_q_heads / num_kv_heads (the grouped-query map of SkipKV Sec. 4.1, token
 *     importance score).  Accumulation is fp32; outputs, logits and lse are fp32.
 *   - Workspace: `ws` (device) must be 256-byte aligned and at least sfi_workspace_bytes()
 *     long; its contents need no initialisation and are scratch between calls.  One buffer
 *     sized for the largest op can serve every call on a descriptor.  Calls that share a
 *     workspace must be ordered (same stream); concurrent calls need separate workspaces.
 *   - The functions are thread-safe.
 */
#ifndef SFI_H
#define SFI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sfi_status {
    SFI_OK = 0,
    SFI_E_INVALID = -1,      /* null pointer, inconsistent sizes, bad alignment */
    SFI_E_UNSUPPORTED = -2,  /* well-formed but not built: head_dim, dtype, group size */
    SFI_E_WORKSPACE = -3,    /* ws is NULL, misaligned or smaller than sfi_workspace_bytes() */
    SFI_E_HIP = -4,          /* the HIP runtime reported an error while launching */
    SFI_E_SCRATCH = -5       /* sfi_sparse_decode_noalloc: the step needs more than the
                                library's static scratch array holds */
} sfi_status;

typedef enum sfi_dtype { SFI_F32 = 0, SFI_BF16 = 1 } sfi_dtype;

typedef enum sfi_op {
    SFI_OP_DENSE = 0, SFI_OP_SELECT = 1, SFI_OP_SPARSE = 2, SFI_OP_SELECT_REFINED = 3,
    SFI_OP_SLOW = 4
} sfi_op;

/* Parameters of the full Selector (sfi_select_refined).  SFI Sec. 5.1 gives lambda_clip = 0.02,
 * alpha_soft = 0.5 and alpha_cross = 0.35; the shape of the position prior is not given there
 * (the tests and the benchmark use prior_decay 1, tail_frac 1/16, tail_brake 1). */
typedef struct sfi_refine {
    float lambda;        /* fusion weight of the prior, 0 <= lambda < 1 */
    float alpha_soft;    /* Soft-NMS decay, 0 <= alpha_soft < 1 */
    float alpha_cross;   /* cross-head exclusivity decay, 0 <= alpha_cross < 1 */
    float prior_decay;   /* global decay of the position prior over J, >= 0 */
    float tail_frac;     /* fraction of J at its end under the tail brake, in [0, 1] */
    float tail_brake;    /* strength of the tail brake, >= 0 */
} sfi_refine;

/* The per-step cache descriptor (SFI Sec. 4.2: one packed description of cache bounds,
 * block tables and layout, read by every kernel of the step).
 *
 *   batch, num_q_heads, num_kv_heads : B, Hq, Hkv; Hq % Hkv == 0 and G = Hq / Hkv <= 16
 *                                     (<= 64 for the calls that read no cache: the Selectors
 *                                     and the mask)
 *   head_dim                          : d, 64 or 128
 *   dtype                             : element type of k, v and q (SFI_F32 or SFI_BF16)
 *   k, v      (device) contiguous: [B][Hkv][n_cap][d]; paged: [num_blocks][Hkv][block_size][d];
 *                      16-byte aligned
 *   n_cap               rows per (b, h) when contiguous (>= max_len); ignored when paged
 *   block_table (device) NULL for contiguous; else int32 [B][max_blocks] of physical block
 *                      numbers, logical position p of sequence b living in block
 *                      block_table[b*max_blocks + p/block_size], row p % block_size
 *   block_size          power of two in [1, 1024] when paged; the paged cache holds fewer than
 *                      2^32 rows (num_blocks * Hkv * block_size), as any cache that fits in
 *                      one MI355X's memory does (a contiguous cache is checked: B*Hkv*n_cap)
 *   len         (device) int32 [B]: current length of each sequence, the current token
 *                      included; 0 <= len[b] <= max_len
 *   max_len             host-side bound of len[] used to size grids (no device read)
 */
typedef struct sfi_kv_desc {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype;
    const void* k;
    const void* v;
    int64_t n_cap;
    const int32_t* block_table;
    int32_t block_size;
    int32_t max_blocks;
    const int32_t* len;
    int32_t max_len;
} sfi_kv_desc;

/* Dense decode step (slow step).  SFI Sec. 1 and Sec. 3: dense full attention over the
 * accessible history, exposing the attention logits the Selector needs (Sec. 4.2).
 * For each b and query head i (h = i / G) over positions j < len[b]:
 *   z_j = (q_i . k_{h,j}) / sqrt(d)
 *   out_i = sum_j softmax(z)_j v_{h,j}             out    (device) fp32 [B][Hq][d]
 *   lse_i = log sum_j exp(z_j)                      lse    (device) fp32 [B][Hq], may be NULL
 *   logits[(b*Hq + i)*logit_stride + j] = z_j       logits (device) fp32, may be NULL; when
 *       given, logit_stride >= max_len, logit_stride % 4 == 0 and logits 16-byte aligned.
 *       Entries j >= len[b] are not written.
 * q (device) [B][Hq][d] in kv->dtype, 16-byte aligned.  len[b] == 0 gives out = 0, lse = -inf.
 * Two kernel launches: split-K partials over the sequence, then their log-sum-exp merge. */
sfi_status sfi_dense_decode(const sfi_kv_desc* kv, const void* q, float* out, float* lse,
                            float* logits, int64_t logit_stride,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Selector (decode window of one query, prior and refinements off).  SFI Sec. 3.2: the
 * slow-step logits over the allowed set J become a per-head distribution; Sec. 3.3: Top-K
 * per KV head.  Per (b, h) with N = len[b]:
 *   S = [0, min(n_sink, N)),  J = [n_sink, N - n_recent)   (empty if N - n_recent <= n_sink)
 *   f(j) = (1/G) sum_{i in group h} exp(z_ij - log sum_{j' in J} exp(z_ij'))
 *   taken = the min(k_sel, |J|) positions of J with the largest f; equal f -> lower j first
 *   idx[(b*Hkv + h)*idx_stride + s], s < n_idx[b*Hkv + h]: ascending positions of S u taken
 * logits (device) fp32 [B][Hq][logit_stride] as written by sfi_dense_decode: 16-byte aligned,
 * logit_stride >= max_len and a multiple of 4.
 * idx (device) int32 [B][Hkv][idx_stride], idx_stride >= n_sink + k_sel.
 * n_idx (device) int32 [B][Hkv] = min(n_sink, N) + min(k_sel, |J|).
 * n_sink, n_recent >= 0, k_sel >= 0.  kv->k and kv->v are not read.
 * Observation window (SFI Sec. 3.2 and Sec. 5.1: evidence averaged over the last W queries, W
 * = 1 at decode, 16 at the end of prefill): pass the logits of W queries per query head as
 * rows i*W + w, w < W, with num_q_heads = Hq*W; the group of KV head h is then its G*W rows
 * and f is their mean.  G*W <= 64. */
sfi_status sfi_select(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                      int32_t n_sink, int32_t n_recent, int32_t k_sel,
                      int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole slow step in one call: sfi_dense_decode with logits, then sfi_select, then (when
 * head_mask is not NULL) sfi_sink_bypass_mask, with the same arguments and results as those
 * three calls up to rounding.  SFI Sec. 4.2 (slow-step kernels expose what the GPU-resident
 * Selector needs) and Sec. 3.2 (the evidence is each head's softmax renormalised over the
 * allowed set J): the dense kernels also keep each split's log-sum-exp over J, so the Selector
 * does not read the logits a second time for it (one pass over the logits of J and one
 * launch fewer than the separate calls).  Because the Selector's normaliser over J comes from
 * the dense accumulators instead of the written logits, its evidence can differ from
 * sfi_select's in the last bits: selections agree except at exact-tie precision.
 * logits and lse are required.  G <= 16 (the dense step's limit).  ws: at least
 * sfi_workspace_bytes(kv, SFI_OP_SLOW, 0, 0) bytes, no initialisation needed.
 * dense_begin, dense_done: HIP events created by the caller, or NULL; when given they are
 * recorded on `stream` right before the dense step's first kernel (after every host-side
 * check) and after its kernels, before the Selector's (for callers that time the dense step,
 * or start other work after it as the layer-wise schedule of SFI Sec. 4.1 does).  Launches:
 * the dense step's two, the Selector's three (four when k_sel + max_len / 64 > 16384; one on
 * short contexts), the mask's one. */
sfi_status sfi_slow_step(const sfi_kv_desc* kv, const void* q, float* out, float* lse,
                         float* logits, int64_t logit_stride,
                         int32_t n_sink, int32_t n_recent, int32_t k_sel,
                         int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                         float mask_frac, uint8_t* head_mask,
                         void* ws, size_t ws_bytes, hipEvent_t dense_begin,
                         hipEvent_t dense_done, hipStream_t stream);

/* The full Selector: sfi_select with the cache-aware prior, reverse-KL fusion and the
 * log-score refinements.  SFI Sec. 3.2 ("Cache-aware prior on allowed positions", "Position
 * factor", "Reverse-KL fusion of evidence and prior", "Choosing lambda") and Sec. 3.3
 * ("Soft-NMS", "Cross-head exclusivity", Top-K).  The page's formulas are lost; this call
 * implements the following readings, per sequence b, KV head h, with J and the evidence f_h as
 * for sfi_select and u_j = (j - n_sink + 1/2)/|J|:
 *   r_h(j) ~ exp(-prior_decay u_j) exp(-tail_brake max(0, u_j - 1 + tail_frac)/tail_frac)
 *            / max(key_norm[b][h][j], 1e-6)              (norm factor only when key_norm given)
 *   s_h    = f_h^(1-lambda) r_h^lambda / Z_h             (the minimiser over distributions on J
 *            of (1 - lambda) KL(s||f_h) + lambda KL(s||r_h))
 *   Soft-NMS: s_h(j) *= 1 - alpha_soft when s_h(j-1) or s_h(j+1) (in J) is strictly larger
 *   exclusivity: s_h(j) *= 1 - alpha_cross when another KV head of b has a strictly larger
 *            score at j after Soft-NMS
 *   then the Top-K of sfi_select on the refined scores (ties to the lower position).
 * With lambda = alpha_soft = alpha_cross = 0 the indices equal sfi_select's.
 * key_norm (device) fp32 [B][Hkv][norm_stride] with norm_stride >= max_len, or NULL: the norms
 * of the cached keys (statistics kept with the cache); when key_norm is 16-byte aligned and
 * norm_stride a multiple of 4 they are read 16 bytes at a time (same result, faster).  ws: sfi_workspace_bytes(kv,
 * SFI_OP_SELECT_REFINED, ...).  Every other argument as for sfi_select.  The chunked Selector
 * plus one refinement pass (five or six kernel launches).  SFI_E_INVALID for parameters outside
 * the stated ranges. */
sfi_status sfi_select_refined(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                              const float* key_norm, int64_t norm_stride,
                              int32_t n_sink, int32_t n_recent, int32_t k_sel,
                              const sfi_refine* params, int32_t* idx, int32_t idx_stride,
                              int32_t* n_idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* Sink-bypass mask.  SinkRouter Sec. 4.2: heads whose attention mass on token 0 is large
 * are in a low-impact regime and are bypassed with a zero surrogate.  Per b:
 *   p0_i = exp(logits[(b*Hq + i)*logit_stride + 0] - lse[b*Hq + i])
 *   head_mask[b*Hq + i] = 1 for the floor(frac * Hq) heads with the largest p0 (equal p0 ->
 *   lower head index first), 0 otherwise.
 * logits, lse (device) fp32 from sfi_dense_decode; head_mask (device) uint8 [B][Hq];
 * 0 <= frac <= 1; every len[b] >= 1.  No workspace. */
sfi_status sfi_sink_bypass_mask(const sfi_kv_desc* kv, const float* logits, int64_t logit_stride,
                                const float* lse, float frac, uint8_t* head_mask,
                                hipStream_t stream);

/* Sparse decode step (fast step).  SFI Sec. 1: attend only to sink + selected + recent, the
 * recent window moving with every step; SinkRouter Sec. 4.2 execution policy: a bypassed
 * head writes the zero surrogate.  Per b and query head i (h = i / G), N = len[b],
 * r0 = max(0, N - n_recent):
 *   I = { idx[(b*Hkv + h)*idx_stride + s] : s < n_idx[b*Hkv + h], the entry < r0 } u [r0, N)
 *   out_i = sum_{j in I} softmax_I(z)_j v_{h,j},  lse_i = log sum_{j in I} exp(z_j)
 *   head_mask[b*Hq + i] != 0  ->  out_i = 0 exactly, lse_i = -inf.
 * idx (device) int32 [B][Hkv][idx_stride]: strictly ascending within each row (as written by
 * sfi_select); entries >= r0 or < 0 are skipped, so the recent run is never counted twice.
 * n_idx (device) int32 [B][Hkv], clamped to idx_stride.  head_mask (device) uint8 [B][Hq] or
 * NULL.  out (device) fp32 [B][Hq][d]; lse (device) fp32 [B][Hq] or NULL.
 * Two kernel launches: partials over splits of the index set, then their merge. */
sfi_status sfi_sparse_decode(const sfi_kv_desc* kv, const void* q,
                             const int32_t* idx, int32_t idx_stride, const int32_t* n_idx,
                             int32_t n_recent, const uint8_t* head_mask,
                             float* out, float* lse,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* The fast step for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same computation, arguments and kernels as
 * sfi_sparse_decode, but the partial records live in a library-owned static device array of
 * SFI_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace: no allocation of any kind
 * happens in the call.  The first call on a device (that device current) looks up the array's
 * device address once; each GPU holds its own array until the process ends.
 *   SFI_E_SCRATCH when the step's partial records need more than SFI_NOALLOC_SCRATCH_BYTES
 *   (sfi_workspace_bytes(kv, SFI_OP_SPARSE, idx_stride, n_recent) tells the need); every
 *   other error as for sfi_sparse_decode.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (other streams,
 * other threads) race and must be ordered by the caller.  The records are written in full by
 * every call before they are read, so nothing needs clearing between calls. */
#define SFI_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
sfi_status sfi_sparse_decode_noalloc(const sfi_kv_desc* kv, const void* q,
                                     const int32_t* idx, int32_t idx_stride, const int32_t* n_idx,
                                     int32_t n_recent, const uint8_t* head_mask,
                                     float* out, float* lse, hipStream_t stream);

/* Step descriptor of the fast step (SFI Sec. 4.2: the host writes a compact packed descriptor
 * once per decoding step, and every kernel of the step reads its per-request cache bounds,
 * block-table pointer and layout offsets from device memory, so steps need no dynamic
 * allocation or extra synchronisation).  One sfi_step lives in device memory (8-byte aligned,
 * caller-owned); the caller writes it before each step, e.g. by a copy from the host, and
 * sfi_sparse_decode_step reads it.  A call captured once in a HIP graph therefore serves every
 * fast step of a cycle: between replays only the descriptor (lengths, query, outputs, index
 * set, mask, segment, recent window) changes.  Field meanings as for sfi_sparse_decode and
 * sfi_sparse_decode_compact:
 *   k, v         cache base pointers, laid out as the host descriptor says (contiguous
 *                [B][Hkv][n_cap][d] or paged [num_blocks][Hkv][block_size][d])
 *   block_table  [B][max_blocks] int32 when the host descriptor is paged, else NULL
 *   len          [B] int32 lengths at this step
 *   q            [B][Hq][d] query of this step; out fp32 [B][Hq][d]; lse fp32 [B][Hq] or NULL
 *   idx, n_idx   index set [B][Hkv][idx_stride] and counts [B][Hkv] (for a two-segment step:
 *                the positions cpos written by sfi_reorg)
 *   head_mask    [B][Hq] uint8 or NULL
 *   seg_k, seg_v compact segment of the two-segment layout ([B][Hkv][idx_stride][d]) or NULL
 *                (both or neither): index slots then read the segment instead of the cache
 *   n_recent     recent window of this step, 0 <= n_recent <= the call's max_recent
 * The device data is trusted, as the other calls trust lengths and indices. */
typedef struct sfi_step {
    const void* k;
    const void* v;
    const int32_t* block_table;
    const int32_t* len;
    const void* q;
    const int32_t* idx;
    const int32_t* n_idx;
    const uint8_t* head_mask;
    const void* seg_k;
    const void* seg_v;
    float* out;
    float* lse;
    int32_t n_recent;
    int32_t reserved;        /* 0 */
} sfi_step;

/* Fast step whose per-step state comes from a device step descriptor (see sfi_step).  The
 * host arguments fix only what the launch plan needs and every step of a cycle shares: kv
 * gives batch, heads, head_dim, dtype and the cache's capacity (n_cap, or block_size and
 * max_blocks with any non-NULL kv->block_table marking a paged cache); kv->k, kv->v,
 * kv->block_table and kv->len are not read (the descriptor's are), and kv->max_len is not
 * used.  idx_stride is the index rows' stride and max_recent bounds the descriptor's
 * n_recent.  step (device) points to the descriptor.  Workspace: sfi_workspace_bytes(kv,
 * SFI_OP_SPARSE, idx_stride, max_recent).  With the descriptor's n_recent equal to max_recent
 * the result equals sfi_sparse_decode (or sfi_sparse_decode_compact, with a segment) called
 * with the descriptor's values bit for bit; a smaller n_recent gives the same attention with the
 * splits planned for max_recent (equal up to rounding).  Two kernel launches, each reading the
 * descriptor at entry.  SFI_E_INVALID for a NULL or misaligned step, idx_stride < 1 or
 * max_recent < 0. */
sfi_status sfi_sparse_decode_step(const sfi_kv_desc* kv, const sfi_step* step,
                                  int32_t idx_stride, int32_t max_recent,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Sparse decode step with inline group routing.  SinkRouter Sec. 4 (decide per KV group,
 * before loading the group's history, whether it is in the sink-dominant regime, and if so
 * write the zero surrogate instead of attending), Sec. 4.2 "Target regime" (token-0 mass at
 * least gamma; the page uses 0.65) and Sec. 4.3 "Inline routing before historical KV loading".
 * The page's routing score (its Eq. 11) is not in the text; this call reads it as the token-0
 * logit of the current query against a normaliser cached from the last slow step:
 *   z0_i = (q_i . k_{h,0}) / sqrt(d),   head i is sink-dominant  <=>  z0_i - route_lse_i >= log(gamma)
 * (exp(z0_i - route_lse_i) estimates head i's token-0 attention mass without scanning the
 * history), and KV group h of sequence b is bypassed when all its G heads are sink-dominant.
 * A bypassed group reads no key or value row and its heads output exactly 0 (lse -inf).  Other
 * groups run exactly as sfi_sparse_decode (head_mask still zeroes its heads).
 * route_lse (device) fp32 [B][Hq], e.g. the lse output of sfi_dense_decode at the slow step;
 * 0 < gamma <= 1; routed (device) uint8 [B][Hkv] or NULL receives 1 for bypassed groups (0 for
 * len[b] == 0).  Every other argument as for sfi_sparse_decode, with the same workspace. */
sfi_status sfi_sparse_decode_routed(const sfi_kv_desc* kv, const void* q,
                                    const int32_t* idx, int32_t idx_stride, const int32_t* n_idx,
                                    int32_t n_recent, const uint8_t* head_mask,
                                    const float* route_lse, float gamma, uint8_t* routed,
                                    float* out, float* lse,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Reorg for the two-segment fast-step layout.  SFI Sec. 4.1 (Reorg_i gathers the sink and
 * selected KV entries of a layer into a contiguous compact buffer after its Selector) and
 * Sec. 4.2 "Coalesced reads with a two-segment KV layout" (fast steps read that long-range
 * segment in order and the recent tokens in place from the cache).  Per b and KV head h, with
 * u = b*Hkv + h and n = n_idx[u] clamped to [0, idx_stride], for every slot s < idx_stride:
 *   p = idx[u*idx_stride + s];  if s < n and 0 <= p < len[b]:  cpos[u*idx_stride + s] = p and
 *   the key and value rows of position p are copied to row u*idx_stride + s of ck and cv;
 *   otherwise cpos = -1 and the rows are zeros.
 * ck, cv (device) [B][Hkv][idx_stride][d] of the cache's dtype, 16-byte aligned; cpos (device)
 * int32 [B][Hkv][idx_stride].  idx and n_idx as for sfi_sparse_decode (e.g. sfi_select's
 * output).  The segment is a snapshot: later writes to the cache do not reach it.  No
 * workspace; one kernel launch.  SFI_E_UNSUPPORTED when B*Hkv*idx_stride >= 2^32. */
sfi_status sfi_reorg(const sfi_kv_desc* kv, const int32_t* idx, int32_t idx_stride,
                     const int32_t* n_idx, void* ck, void* cv, int32_t* cpos, hipStream_t stream);

/* Fast step on the two-segment layout (SFI Sec. 4.2): as sfi_sparse_decode with idx = cpos,
 * except that index slot s of (b, h) reads its key and value rows from row u*idx_stride + s of
 * the compact segment ck, cv written by sfi_reorg instead of from the cache; the recent
 * window [r0, N) is read in place from the cache as before:
 *   I = { cpos[u*idx_stride + s] : s < n_idx[u], 0 <= entry < r0 }  u  [r0, N).
 * With the segment written by sfi_reorg from idx (every entry of idx below len at that call)
 * and the cache rows of those positions unchanged since, the result equals sfi_sparse_decode
 * on idx bit for bit: the same slots in the same order with the same bytes.  n_idx is the
 * array given to sfi_reorg; any value is safe (slots past the reorg's count hold zero rows
 * and cpos -1).  Workspace, head_mask, out and lse as for sfi_sparse_decode (SFI_OP_SPARSE
 * with this idx_stride).  SFI_E_UNSUPPORTED when B*Hkv*idx_stride >= 2^32. */
sfi_status sfi_sparse_decode_compact(const sfi_kv_desc* kv, const void* q,
                                     const void* ck, const void* cv, const int32_t* cpos,
                                     int32_t idx_stride, const int32_t* n_idx, int32_t n_recent,
                                     const uint8_t* head_mask, float* out, float* lse,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Slow step over the layers of a model with the Selector off the critical path.  SFI Sec. 4.1,
 * layer-wise asynchronous execution: the primary stream runs the dense step of layer after
 * layer while the Selector (and the sink mask) of each layer runs on a second stream, with a
 * ring of n_slots maintenance slots and one completion barrier at the end.  For l = 0 ..
 * n_layers - 1, with slot s = l % n_slots:
 *   on `stream`:      if l >= n_slots, wait until slot s is free (slot_events[s]); then
 *                     the dense step of sfi_slow_step(&kv[l], q[l], out[l], lse[l], logits[s],
 *                     logit_stride, ...), its records in dense_ws and its normaliser over J in
 *                     sel_ws[s]
 *   on `side_stream`: wait for that dense step (attn_event); the Selector of sfi_slow_step
 *                     into idx[l], n_idx[l] with workspace sel_ws[s]; when head_mask is not NULL,
 *                     sfi_sink_bypass_mask(&kv[l], logits[s], lse[l], mask_frac, head_mask[l]);
 *                     then record slot_events[s] (slot s free again); when seg_k is not
 *                     NULL, sfi_reorg(&kv[l], idx[l], ..., seg_k[l], seg_v[l], seg_pos[l])
 *                     (SFI Sec. 4.1: Reorg_i follows Sel_i on the maintenance stream).
 * Finally `stream` waits for everything queued on `side_stream` (done_event), so work queued on
 * `stream` after this call sees every layer's indices, masks and compact segments.  Every
 * result equals that of sfi_slow_step (and sfi_reorg) called layer after layer, bit for bit.
 * Arguments: kv, q, out, lse, idx, n_idx (and head_mask, or NULL; seg_k, seg_v, seg_pos, all
 * NULL or all given, laid out as for sfi_reorg with idx_stride) are host arrays of n_layers
 * entries; logits and sel_ws are host arrays of n_slots entries; all the pointers in them are
 * device buffers laid out as for the single calls (lse is required here).  dense_ws serves the
 * dense steps one after another and each sel_ws[s] holds a slot's normaliser and Selector
 * workspace: sfi_workspace_bytes(&kv[l], SFI_OP_SLOW, 0, 0) bytes suffice for both (G <= 16).
 * Measured on MI355X, pipelining pays for a ragged batch of 16 sequences of 8K-32K (294 -> 280
 * us per layer) and is within the run-to-run spread for one 32K sequence (57 -> 52-60 us); at
 * 128K x 4 and 512K, where the dense step alone keeps HBM busy, and on a 2K fp32 layer, where
 * the event hand-offs cost more than the overlap saves, sfi_slow_step layer after layer is
 * faster (406-408 vs 441-443, 476-479 vs 502 and 24 vs 44 us per layer), so that is the
 * default there.  slot_events (n_slots), attn_event and done_event are HIP events created by
 * the caller; the library only records them and waits on them.
 * stream and side_stream must differ; calls that share buffers or events must not overlap.
 * Every layer is validated before anything is queued; on an error nothing has been queued
 * (SFI_E_HIP aside, which may leave earlier layers queued). */
sfi_status sfi_slow_step_layers(
    int32_t n_layers, const sfi_kv_desc* kv, const void* const* q, float* const* out,
    float* const* lse, int32_t n_slots, float* const* logits, int64_t logit_stride,
    void* const* sel_ws, size_t sel_ws_bytes, void* dense_ws, size_t dense_ws_bytes,
    int32_t n_sink, int32_t n_recent, int32_t k_sel, int32_t* const* idx, int32_t idx_stride,
    int32_t* const* n_idx, float mask_frac, uint8_t* const* head_mask,
    void* const* seg_k, void* const* seg_v, int32_t* const* seg_pos,
    hipStream_t stream, hipStream_t side_stream, hipEvent_t* slot_events,
    hipEvent_t attn_event, hipEvent_t done_event);

/* Workspace bytes needed by one call of `op` on this descriptor.  idx_stride and n_recent
 * (index capacity and recent window) are used by SFI_OP_SPARSE only; SFI_OP_DENSE,
 * SFI_OP_SELECT, SFI_OP_SELECT_REFINED and SFI_OP_SLOW (sfi_slow_step) size from the
 * descriptor (max_len) alone.  Returns 0 when the descriptor
 * or op is invalid. */
size_t sfi_workspace_bytes(const sfi_kv_desc* kv, int32_t op, int32_t idx_stride,
                           int32_t n_recent);

/* Measurement yardstick, not a step of the method: a plain sequential read of `bytes` bytes
 * of device memory at `buf` by `n_workgroups` workgroups of 256 threads, each reading one
 * contiguous chunk with 16-byte loads.  Timing it with events on `stream` gives the read
 * bandwidth the memory system delivers on this device, against which the attention kernels'
 * algorithmic rates are also reported (the datasheet peak is not reachable).
 *   buf   (device) 16-byte aligned, bytes > 0 and a multiple of 16; only read
 *   sink  (device) at least 64 uint32 words; written only if the XOR of all words read
 *                  equals a fixed constant (practically never), so its contents are undefined
 *   n_workgroups   1 ... 2^20
 * SFI_E_INVALID for a null pointer, a bad size, alignment or count; asynchronous on stream. */
/* Measurement yardstick, not a step of the method: the key and value rows that
 * sfi_sparse_decode reads for these arguments (index entries below the recent window, a
 * stand-in row for each skipped entry, then the recent window, through the block table when
 * paged), read once each with 16-byte loads by about n_workgroups workgroups in one launch,
 * with no arithmetic, in the fast step's order (row numbers built in LDS once per workgroup,
 * then every load of a 32-slot tile issued together).  Timed with events it is the floor of the fast step's access pattern in
 * one launch (the fast step itself also computes, and merges its splits in a second launch).
 * kv, idx, idx_stride, n_idx, n_recent as for sfi_sparse_decode; sink as for sfi_stream_read.
 * SFI_E_INVALID for a null pointer, a bad size or count; asynchronous on stream. */
sfi_status sfi_gather_read(const sfi_kv_desc* kv, const int32_t* idx, int32_t idx_stride,
                           const int32_t* n_idx, int32_t n_recent, int32_t n_workgroups,
                           uint32_t* sink, hipStream_t stream);

sfi_status sfi_stream_read(const void* buf, uint64_t bytes, int32_t n_workgroups, uint32_t* sink,
                           hipStream_t stream);

/* Measurement yardstick, not a step of the method: the dot products q_g . k_j of a GQA group's
 * G query heads with n_rows bf16 key rows of 128 elements (SinkRouter Sec. 4.3: every key row
 * is read once for the whole group), the rows read in order by n_workgroups workgroups of 256
 * threads, each wavefront taking 16 consecutive rows (4 KB) at a time with two such groups in
 * flight, on one of three units:
 *   unit 0  no arithmetic (the words folded into an XOR), a read of the same rows;
 *   unit 1  the vector ALUs: 8 elements per lane, fp32 FMAs, the 16 lanes of a row summed with
 *           DPP row shifts;
 *   unit 2  MFMA (16x16x32 bf16) in the attention kernels' operand layout, heads >= G as zero
 *           columns of Q^T.
 * Timed with events beside each other they show what the group products cost on each unit
 * next to the read they ride on.
 *   rows  (device) bf16 [n_rows][128], 16-byte aligned, only read; n_rows >= 16, a multiple of 16
 *   q     (device) bf16 [G][128], 16-byte aligned, only read
 *   G     1, 2, 4 or 8
 *   unit  0, 1 or 2
 *   part  (device) float [n_workgroups], 4-byte aligned (may be null for unit 0): units 1 and 2
 *         write workgroup w's sum of q_g . k_j over its rows and the G heads, so the sum of part
 *         is sum_j sum_g q_g . k_j (fp32 accumulation); unit 0 leaves it untouched
 *   sink  as for sfi_stream_read
 * SFI_E_INVALID for a null pointer, a bad size, alignment, unit or count; SFI_E_UNSUPPORTED for
 * another G; asynchronous on stream. */
sfi_status sfi_group_dot(const void* rows, int64_t n_rows, const void* q, int32_t G, int32_t unit,
                         int32_t n_workgroups, float* part, uint32_t* sink, hipStream_t stream);

/* Static description of a status code. */
const char* sfi_status_string(sfi_status status);

#ifdef __cplusplus
}
#endif
#endif /* SFI_H */
