/*
 * sfi_oracle.h -- plain fp64 CPU reference for Slow-Fast decode attention.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The HIP library never calls it and
 * shares no code, header or table with it.
 *
 * Every floating-point step is done in double precision with the C library's exp
 * and log; bf16 inputs are widened exactly (bf16 bits << 16 -> fp32 -> double).
 *
 * Cache addressing (the same bytes the GPU reads):
 *   contiguous: element (b, h, pos, c) at ((b*Hkv + h)*n_cap + pos)*d + c
 *   paged:      element (b, h, pos, c) at ((bt[b*max_blocks + pos/bs]*Hkv + h)*bs + pos%bs)*d + c
 * Query head i reads KV head i / G with G = Hq / Hkv (grouped-query attention as in
 * the SkipKV token-importance equation, Sec. 4.1).
 */
#ifndef SFI_ORACLE_H
#define SFI_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct orc_cache {
    int32_t B, Hq, Hkv, d;
    int32_t is_bf16;               /* 1: K, V, q hold bf16 bits (uint16); 0: fp32 */
    const void* k;
    const void* v;
    int64_t n_cap;                 /* rows per (b, h) when contiguous */
    const int32_t* block_table;    /* NULL when contiguous; [B][max_blocks] when paged */
    int32_t block_size, max_blocks;
    const int32_t* len;            /* [B] current lengths (including the current token) */
} orc_cache;

/* Dense decode (Slow-Fast Inference, Sec. 1 and Sec. 3: a slow step runs full attention
 * over the accessible history and exposes its logits).  For every batch b and query
 * head i:  z_j = (q . k_j)/sqrt(d) for j < len[b];  logits[(b*Hq+i)*logit_stride + j] = z_j;
 * lse = log sum_j exp(z_j);  out = sum_j exp(z_j - lse) v_j.
 * out [B][Hq][d], lse [B][Hq]; logits may be NULL.  len[b] == 0 gives out = 0, lse = -inf. */
int orc_dense(const orc_cache* c, const void* q, double* out, double* lse,
              double* logits, int64_t logit_stride);

/* Selector at decode (Slow-Fast Inference, Sec. 3.2 evidence with a window of one query,
 * Sec. 3.3 Top-K discretization; prior and refinements off).  Per (b, h) with N = len[b]:
 *   S = [0, min(n_sink, N)),  J = [n_sink, N - n_recent)  (empty when N - n_recent <= n_sink)
 *   LSE_i = log sum_{j in J} exp(z_ij)                    for the G query heads i of group h
 *   f(j)  = (1/G) sum_i exp(z_ij - LSE_i)                 for j in J
 *   taken = the min(k_sel, |J|) positions of J with the largest f, ties to the lower j
 *   idx[(b*Hkv+h)*idx_stride ...] = ascending(S u taken), n_idx[b*Hkv+h] = its size.
 * logits are [B][Hq][logit_stride] doubles.  f_out (optional) receives f(j) at
 * f_out[(b*Hkv+h)*logit_stride + j] for j in J and 0 elsewhere.
 * Returns 0, or -1 when idx_stride < min(n_sink,N) + min(k_sel,|J|) for some (b, h). */
int orc_select(int32_t B, int32_t Hq, int32_t Hkv, const int32_t* len,
               const double* logits, int64_t logit_stride,
               int32_t n_sink, int32_t n_recent, int32_t k_sel,
               int32_t* idx, int32_t idx_stride, int32_t* n_idx, double* f_out);

/* Parameters of the full Selector.  lambda: fusion weight of the prior (SFI Sec. 5.1 clips it
 * at 0.02); alpha_soft, alpha_cross: Soft-NMS and cross-head decays (0.5 and 0.35 there);
 * prior_decay, tail_frac, tail_brake: shape of the position prior (not given on the page). */
typedef struct orc_refine {
    double lambda, alpha_soft, alpha_cross, prior_decay, tail_frac, tail_brake;
} orc_refine;

/* The full Selector (Slow-Fast Inference, Sec. 3.2 "Cache-aware prior", "Position factor",
 * "Reverse-KL fusion", Sec. 3.3 "Soft-NMS", "Cross-head exclusivity", Top-K; the pages' formulas
 * are lost, so each step below is a stated reading).  Per sequence b with J = [n_sink,
 * N - n_recent) and u_j = (j - n_sink + 1/2)/|J|:
 *   f_h        the evidence of orc_select
 *   r_h(j)  ~  exp(-prior_decay u_j) * exp(-tail_brake max(0, u_j - 1 + tail_frac)/tail_frac)
 *              / max(key_norm[b][h][j], 1e-6)          (the norm factor only if key_norm given)
 *   s_h     =  argmin over distributions s on J of (1 - lambda) KL(s||f_h) + lambda KL(s||r_h)
 *           =  f_h^(1-lambda) r_h^lambda / Z_h,   ell = log s_h
 *   Soft-NMS:  ell1(j) = ell(j) + log(1 - alpha_soft) if a neighbour j-1 or j+1 in J has a
 *              strictly larger ell, else ell(j)
 *   exclusivity: ell2_h(j) = ell1_h(j) + log(1 - alpha_cross) if some other KV head of b has a
 *              strictly larger ell1 at j, else ell1_h(j)
 *   Top-K of ell2_h as in orc_select (ties to the lower position), emitted after the sinks.
 * key_norm may be NULL ([B][Hkv][norm_stride] otherwise).  fused_out and refined_out (optional,
 * [B][Hkv][logit_stride]) receive ell and ell2 on J and -inf elsewhere.  With lambda =
 * alpha_soft = alpha_cross = 0 the result is that of orc_select.  Returns -1 when idx_stride
 * is too small. */
int orc_select_refined(int32_t B, int32_t Hq, int32_t Hkv, const int32_t* len,
                       const double* logits, int64_t logit_stride,
                       const double* key_norm, int64_t norm_stride,
                       int32_t n_sink, int32_t n_recent, int32_t k_sel, const orc_refine* p,
                       int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                       double* fused_out, double* refined_out);

/* Sparse decode (Slow-Fast Inference, Sec. 1: a fast step attends only to sink + selected
 * + recent tokens, the recent window moving with every step).  Per (b, i), h = i / G,
 * N = len[b], r0 = max(0, N - n_recent):
 *   I = { p in idx[(b*Hkv+h)*idx_stride + s], s < n_idx[b*Hkv+h] : p < r0 }  u  [r0, N)
 * (a set: repeated entries count once), and out = softmax over I of z, applied to V.
 * A query head with head_mask[b*Hq+i] != 0 outputs exact zeros (SinkRouter, Sec. 4.2
 * "Execution policy": a bypassed unit writes a zero surrogate) and lse = -inf.
 * head_mask may be NULL. */
int orc_sparse(const orc_cache* c, const void* q, const int32_t* idx, int32_t idx_stride,
               const int32_t* n_idx, int32_t n_recent, const uint8_t* head_mask,
               double* out, double* lse);

/* Sparse decode with group routing (SinkRouter, Sec. 4.2-4.3: decide per KV group, before
 * attending, whether the group is sink-dominant; a bypassed group outputs the zero surrogate).
 * The page's routing score is not in the text; the reading implemented here: head i of group h
 * is sink-dominant when z0_i - route_lse[b*Hq+i] >= log_gamma, with z0_i = (q_i . k_{h,0})/sqrt(d)
 * (exp of the left side estimates the head's token-0 mass); the group is bypassed (routed[u] =
 * 1, u = b*Hkv + h) when all its heads are.  margin[u] (optional) receives the smallest
 * z0_i - route_lse_i - log_gamma of the group (-inf when len[b] == 0), so callers can tell
 * decisions that rounding could flip.  Outputs as orc_sparse with bypassed heads masked. */
int orc_sparse_routed(const orc_cache* c, const void* q, const int32_t* idx, int32_t idx_stride,
                      const int32_t* n_idx, int32_t n_recent, const uint8_t* head_mask,
                      const double* route_lse, double log_gamma, double* margin,
                      uint8_t* routed, double* out, double* lse);

/* Reorg for the two-segment layout (Slow-Fast Inference, Sec. 4.1: after the Selector the
 * sink and selected KV entries of each (b, h) are gathered into a contiguous compact buffer).
 * Per unit u = b*Hkv + h, n = n_idx[u] clamped to [0, idx_stride], every slot s < idx_stride:
 * if s < n and p = idx[u*idx_stride + s] lies in [0, len[b]), the key and value rows of p are
 * copied byte for byte to slot u*idx_stride + s of ck and cv and cpos[...] = p; otherwise the
 * slot's rows are zero bytes and cpos = -1.  ck, cv hold B*Hkv*idx_stride rows of d elements
 * in the cache's element format. */
int orc_reorg(const orc_cache* c, const int32_t* idx, int32_t idx_stride, const int32_t* n_idx,
              void* ck, void* cv, int32_t* cpos);

/* Fast step on the two-segment layout (Slow-Fast Inference, Sec. 4.2: the long-range
 * segment is read from the compact buffer, the recent tokens in place from the cache).  The
 * attended set is that of orc_sparse with idx = cpos:
 *   I = { cpos[u*idx_stride + s], s < n_idx[u] : 0 <= entry < r0 }  u  [r0, N),
 * but a long-range position's key and value rows are read from its segment slot (the first
 * slot naming it) of ck, cv, and recent positions from the cache.  Masked heads output zeros,
 * lse -inf.  Logits and the weighted sum run over positions in ascending order, as in
 * orc_sparse, so with segment rows equal to the cache rows the two agree exactly. */
int orc_sparse_compact(const orc_cache* c, const void* q, const void* ck, const void* cv,
                       const int32_t* cpos, int32_t idx_stride, const int32_t* n_idx,
                       int32_t n_recent, const uint8_t* head_mask, double* out, double* lse);

/* Sink-bypass mask (SinkRouter, Sec. 4.2 "Target regime": heads whose token-0 attention
 * mass is large are treated as idle).  p0[b,i] = exp(z0[b*Hq+i] - lse[b*Hq+i]); per b the
 * floor(frac*Hq) heads with the largest p0 are masked, ties to the lower head index. */
int orc_sink_mask(int32_t B, int32_t Hq, const double* z0, const double* lse, double frac,
                  uint8_t* head_mask);

/* OpenMP threads the functions above use. */
int orc_threads(void);

#ifdef __cplusplus
}
#endif
#endif
