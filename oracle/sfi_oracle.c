/*
 * sfi_oracle.c -- plain fp64 CPU reference for Slow-Fast decode attention.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark load this file's library; the HIP library shares nothing with it.
 *
 * Written for reading, not speed: one (batch, head) at a time, plain loops, double
 * precision, C library exp/log.  OpenMP only splits independent (batch, head) units.
 * Sources (page titles with section):
 *   - Slow-Fast Inference (SFI), Sec. 1 and Sec. 3: slow steps run dense attention and
 *     expose its logits; the Selector turns slow-step logits over the allowed set J into
 *     a per-head distribution and keeps the Top-K positions per KV head; fast steps
 *     attend to sink + selected + recent.
 *   - SkipKV, Sec. 4.1 "Token Importance Score": softmax(Q K^T / sqrt(d) + M) with query
 *     head i reading KV head g(i) (the scale and the grouped-query map).
 *   - SinkRouter, Sec. 4.2: token-0 attention mass as the idle signal; bypassed units
 *     write a zero surrogate.
 */
#include "sfi_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---- reading the cache ------------------------------------------------------------- */

static double load_elem(const void* base, int is_bf16, int64_t e) {
    if (is_bf16) {
        uint32_t u = (uint32_t)((const uint16_t*)base)[e] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[e];
}

/* first element of row (b, h, pos) */
static int64_t row_start(const orc_cache* c, int b, int h, int64_t pos) {
    if (c->block_table) {
        int64_t blk = c->block_table[(int64_t)b * c->max_blocks + pos / c->block_size];
        return ((blk * c->Hkv + h) * c->block_size + pos % c->block_size) * (int64_t)c->d;
    }
    return (((int64_t)b * c->Hkv + h) * c->n_cap + pos) * (int64_t)c->d;
}

/* z = (q_i . k_pos) / sqrt(d) */
static double logit_of(const orc_cache* c, const double* qi, int b, int h, int64_t pos) {
    int64_t r = row_start(c, b, h, pos);
    double s = 0.0;
    for (int x = 0; x < c->d; ++x) s += qi[x] * load_elem(c->k, c->is_bf16, r + x);
    return s / sqrt((double)c->d);
}

static void load_query(const orc_cache* c, const void* q, int b, int i, double* qi) {
    int64_t base = ((int64_t)b * c->Hq + i) * c->d;
    for (int x = 0; x < c->d; ++x) qi[x] = load_elem(q, c->is_bf16, base + x);
}

/* softmax-weighted sum over a list of positions (given their logits):
 * out = sum_j exp(z_j - lse) v_j, lse = log sum_j exp(z_j).  n == 0 -> out 0, lse -inf. */
static void attend(const orc_cache* c, int b, int h, const int64_t* pos, const double* z,
                   int64_t n, double* out, double* lse) {
    for (int x = 0; x < c->d; ++x) out[x] = 0.0;
    if (n <= 0) {
        *lse = -INFINITY;
        return;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) m = z[j] > m ? z[j] : m;
    double l = 0.0;
    for (int64_t j = 0; j < n; ++j) l += exp(z[j] - m);
    double L = m + log(l);
    for (int64_t j = 0; j < n; ++j) {
        double p = exp(z[j] - L);
        int64_t r = row_start(c, b, h, pos[j]);
        for (int x = 0; x < c->d; ++x) out[x] += p * load_elem(c->v, c->is_bf16, r + x);
    }
    *lse = L;
}

/* ---- dense slow step ---------------------------------------------------------------- */

int orc_dense(const orc_cache* c, const void* q, double* out, double* lse,
              double* logits, int64_t logit_stride) {
    const int G = c->Hq / c->Hkv;
    const int units = c->B * c->Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        int b = u / c->Hq, i = u % c->Hq, h = i / G;
        int64_t N = c->len[b];
        double* qi = (double*)malloc(sizeof(double) * c->d);
        int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
        double* z = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
        load_query(c, q, b, i, qi);
        for (int64_t j = 0; j < N; ++j) {
            pos[j] = j;
            z[j] = logit_of(c, qi, b, h, j);
            if (logits) logits[(int64_t)u * logit_stride + j] = z[j];
        }
        attend(c, b, h, pos, z, N, out + (int64_t)u * c->d, lse + u);
        free(qi);
        free(pos);
        free(z);
    }
    return 0;
}

/* ---- selector ---------------------------------------------------------------------- */

typedef struct { double f; int64_t j; } scored;

/* larger f first; equal f -> lower position first */
static int by_score(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->f > y->f) return -1;
    if (x->f < y->f) return 1;
    return (x->j > y->j) - (x->j < y->j);
}

int orc_select(int32_t B, int32_t Hq, int32_t Hkv, const int32_t* len,
               const double* logits, int64_t logit_stride,
               int32_t n_sink, int32_t n_recent, int32_t k_sel,
               int32_t* idx, int32_t idx_stride, int32_t* n_idx, double* f_out) {
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int u = 0; u < B * Hkv; ++u) {
        int b = u / Hkv, h = u % Hkv;
        int64_t N = len[b];
        int64_t ns = n_sink < N ? n_sink : N;
        int64_t j0 = n_sink, j1 = N - n_recent;
        int64_t nJ = j1 > j0 ? j1 - j0 : 0;
        int64_t take = k_sel < nJ ? k_sel : nJ;
        if (f_out) {
            for (int64_t j = 0; j < logit_stride; ++j) f_out[(int64_t)u * logit_stride + j] = 0.0;
        }
        if (ns + take > idx_stride) {
            bad |= 1;
            n_idx[u] = 0;
            continue;
        }
        scored* s = (scored*)malloc(sizeof(scored) * (nJ > 0 ? nJ : 1));
        for (int64_t t = 0; t < nJ; ++t) {
            s[t].f = 0.0;
            s[t].j = j0 + t;
        }
        for (int g = 0; g < G; ++g) {
            const double* z = logits + ((int64_t)b * Hq + h * G + g) * logit_stride;
            double m = -INFINITY;
            for (int64_t j = j0; j < j1; ++j) m = z[j] > m ? z[j] : m;
            double l = 0.0;
            for (int64_t j = j0; j < j1; ++j) l += exp(z[j] - m);
            double lse_J = m + log(l);
            for (int64_t t = 0; t < nJ; ++t) s[t].f += exp(z[j0 + t] - lse_J) / G;
        }
        if (f_out) {
            for (int64_t t = 0; t < nJ; ++t) f_out[(int64_t)u * logit_stride + j0 + t] = s[t].f;
        }
        qsort(s, (size_t)nJ, sizeof(scored), by_score);
        /* mark the taken positions, then emit S and the marks in ascending order */
        unsigned char* keep = (unsigned char*)calloc((size_t)(nJ > 0 ? nJ : 1), 1);
        for (int64_t t = 0; t < take; ++t) keep[s[t].j - j0] = 1;
        int32_t* row = idx + (int64_t)u * idx_stride;
        int64_t w = 0;
        for (int64_t p = 0; p < ns; ++p) row[w++] = (int32_t)p;
        for (int64_t t = 0; t < nJ; ++t)
            if (keep[t]) row[w++] = (int32_t)(j0 + t);
        n_idx[u] = (int32_t)w;
        free(keep);
        free(s);
    }
    return bad ? -1 : 0;
}

/* ---- full Selector: prior, fusion and log-score refinements ------------------------- */

/* Unnormalised prior weight of position j of J = [j0, j0 + nJ) for a KV head whose key norms
 * are norm_row (NULL: no key-norm factor).  u is the position's place in J, in (0, 1). */
static double prior_weight(const orc_refine* p, const double* norm_row, int64_t j, int64_t j0,
                           int64_t nJ) {
    double u = ((double)(j - j0) + 0.5) / (double)nJ;
    double w = exp(-p->prior_decay * u);                          /* global decay */
    double t0 = 1.0 - p->tail_frac;
    if (p->tail_frac > 0.0 && u > t0) w *= exp(-p->tail_brake * (u - t0) / p->tail_frac);
    if (norm_row) {                                               /* key-norm factor */
        double n = norm_row[j] > 1e-6 ? norm_row[j] : 1e-6;
        w /= n;
    }
    return w;
}

int orc_select_refined(int32_t B, int32_t Hq, int32_t Hkv, const int32_t* len,
                       const double* logits, int64_t logit_stride,
                       const double* key_norm, int64_t norm_stride,
                       int32_t n_sink, int32_t n_recent, int32_t k_sel, const orc_refine* p,
                       int32_t* idx, int32_t idx_stride, int32_t* n_idx,
                       double* fused_out, double* refined_out) {
    const int G = Hq / Hkv;
    int bad = 0;
    for (int b = 0; b < B; ++b) {
        int64_t N = len[b];
        int64_t ns = n_sink < N ? n_sink : N;
        int64_t j0 = n_sink, j1 = N - n_recent;
        int64_t nJ = j1 > j0 ? j1 - j0 : 0;
        int64_t take = k_sel < nJ ? k_sel : nJ;
        int64_t n1 = nJ > 0 ? nJ : 1;
        double* ell = (double*)malloc(sizeof(double) * (size_t)(Hkv * n1));   /* log s_h */
        double* ell1 = (double*)malloc(sizeof(double) * (size_t)(Hkv * n1));  /* after NMS */
        /* 1. evidence f_h (the hot path's), 2. prior r_h, 3. fused s_h = f^(1-l) r^l / Z */
        for (int h = 0; h < Hkv; ++h) {
            double* e = ell + (int64_t)h * n1;
            for (int64_t t = 0; t < nJ; ++t) e[t] = 0.0;
            for (int g = 0; g < G; ++g) {
                const double* z = logits + ((int64_t)b * Hq + h * G + g) * logit_stride;
                double m = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) m = z[j] > m ? z[j] : m;
                double l = 0.0;
                for (int64_t j = j0; j < j1; ++j) l += exp(z[j] - m);
                double lse_J = m + log(l);
                for (int64_t t = 0; t < nJ; ++t) e[t] += exp(z[j0 + t] - lse_J) / G;   /* f */
            }
            const double* nrow = key_norm ? key_norm + ((int64_t)b * Hkv + h) * norm_stride : NULL;
            double R = 0.0;
            for (int64_t t = 0; t < nJ; ++t) R += prior_weight(p, nrow, j0 + t, j0, nJ);
            double Z = 0.0;
            for (int64_t t = 0; t < nJ; ++t) {
                double r = prior_weight(p, nrow, j0 + t, j0, nJ) / R;
                e[t] = pow(e[t], 1.0 - p->lambda) * pow(r, p->lambda);
                Z += e[t];
            }
            for (int64_t t = 0; t < nJ; ++t) e[t] = log(e[t] / Z);
            if (fused_out) {
                double* fo = fused_out + ((int64_t)b * Hkv + h) * logit_stride;
                for (int64_t j = 0; j < logit_stride; ++j) fo[j] = -INFINITY;
                for (int64_t t = 0; t < nJ; ++t) fo[j0 + t] = e[t];
            }
            /* 4. Soft-NMS within the head: a position with a strictly higher neighbour in J is
             *    decayed by log(1 - alpha_soft); local maxima keep their score */
            double* e1 = ell1 + (int64_t)h * n1;
            for (int64_t t = 0; t < nJ; ++t) {
                int lower = (t > 0 && e[t - 1] > e[t]) || (t + 1 < nJ && e[t + 1] > e[t]);
                e1[t] = e[t] + (lower ? log(1.0 - p->alpha_soft) : 0.0);
            }
        }
        /* 5. cross-head exclusivity at each position: every head below the position's best
         *    head is decayed by log(1 - alpha_cross) */
        for (int64_t t = 0; t < nJ; ++t) {
            double M = -INFINITY;
            for (int h = 0; h < Hkv; ++h) M = ell1[(int64_t)h * n1 + t] > M ? ell1[(int64_t)h * n1 + t] : M;
            for (int h = 0; h < Hkv; ++h) {
                double* x = ell + (int64_t)h * n1 + t;            /* ell is reused for the result */
                double v = ell1[(int64_t)h * n1 + t];
                *x = v + (v < M ? log(1.0 - p->alpha_cross) : 0.0);
            }
        }
        /* 6. Top-K per head on the refined log-scores (ties to the lower position), emitted in
         *    ascending order after the sinks */
        for (int h = 0; h < Hkv; ++h) {
            int u = b * Hkv + h;
            const double* e2 = ell + (int64_t)h * n1;
            if (refined_out) {
                double* ro = refined_out + (int64_t)u * logit_stride;
                for (int64_t j = 0; j < logit_stride; ++j) ro[j] = -INFINITY;
                for (int64_t t = 0; t < nJ; ++t) ro[j0 + t] = e2[t];
            }
            if (ns + take > idx_stride) {
                bad = 1;
                n_idx[u] = 0;
                continue;
            }
            scored* sc = (scored*)malloc(sizeof(scored) * (size_t)n1);
            for (int64_t t = 0; t < nJ; ++t) {
                sc[t].f = e2[t];
                sc[t].j = j0 + t;
            }
            qsort(sc, (size_t)nJ, sizeof(scored), by_score);
            unsigned char* keep = (unsigned char*)calloc((size_t)n1, 1);
            for (int64_t t = 0; t < take; ++t) keep[sc[t].j - j0] = 1;
            int32_t* row = idx + (int64_t)u * idx_stride;
            int64_t w = 0;
            for (int64_t q = 0; q < ns; ++q) row[w++] = (int32_t)q;
            for (int64_t t = 0; t < nJ; ++t)
                if (keep[t]) row[w++] = (int32_t)(j0 + t);
            n_idx[u] = (int32_t)w;
            free(keep);
            free(sc);
        }
        free(ell);
        free(ell1);
    }
    return bad ? -1 : 0;
}

/* ---- sparse fast step ---------------------------------------------------------------- */

int orc_sparse(const orc_cache* c, const void* q, const int32_t* idx, int32_t idx_stride,
               const int32_t* n_idx, int32_t n_recent, const uint8_t* head_mask,
               double* out, double* lse) {
    const int G = c->Hq / c->Hkv;
    const int units = c->B * c->Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        int b = u / c->Hq, i = u % c->Hq, h = i / G;
        int64_t N = c->len[b];
        int64_t r0 = N - n_recent > 0 ? N - n_recent : 0;
        double* o = out + (int64_t)u * c->d;
        if (head_mask && head_mask[u]) {
            for (int x = 0; x < c->d; ++x) o[x] = 0.0;
            lse[u] = -INFINITY;
            continue;
        }
        /* the attended set, as a membership array over [0, N) */
        unsigned char* in = (unsigned char*)calloc((size_t)(N > 0 ? N : 1), 1);
        const int32_t* row = idx + ((int64_t)b * c->Hkv + h) * idx_stride;
        for (int32_t s = 0; s < n_idx[b * c->Hkv + h]; ++s)
            if (row[s] >= 0 && row[s] < r0) in[row[s]] = 1;
        for (int64_t p = r0; p < N; ++p) in[p] = 1;
        int64_t n = 0;
        for (int64_t p = 0; p < N; ++p) n += in[p];
        int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
        double* z = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
        double* qi = (double*)malloc(sizeof(double) * c->d);
        load_query(c, q, b, i, qi);
        int64_t w = 0;
        for (int64_t p = 0; p < N; ++p)
            if (in[p]) {
                pos[w] = p;
                z[w] = logit_of(c, qi, b, h, p);
                ++w;
            }
        attend(c, b, h, pos, z, n, o, lse + u);
        free(in);
        free(pos);
        free(z);
        free(qi);
    }
    return 0;
}

/* ---- Reorg and the two-segment fast step ----------------------------------------------- */

int orc_reorg(const orc_cache* c, const int32_t* idx, int32_t idx_stride, const int32_t* n_idx,
              void* ck, void* cv, int32_t* cpos) {
    const size_t es = c->is_bf16 ? 2 : 4;
    const size_t rb = es * (size_t)c->d;
    for (int u = 0; u < c->B * c->Hkv; ++u) {
        int b = u / c->Hkv, h = u % c->Hkv;
        int64_t N = c->len[b];
        int32_t n = n_idx[u] < 0 ? 0 : (n_idx[u] > idx_stride ? idx_stride : n_idx[u]);
        for (int32_t s = 0; s < idx_stride; ++s) {
            int64_t slot = (int64_t)u * idx_stride + s;
            int64_t p = s < n ? idx[slot] : -1;
            unsigned char* dk = (unsigned char*)ck + slot * rb;
            unsigned char* dv = (unsigned char*)cv + slot * rb;
            if (p >= 0 && p < N) {
                int64_t r = row_start(c, b, h, p);
                memcpy(dk, (const unsigned char*)c->k + r * es, rb);
                memcpy(dv, (const unsigned char*)c->v + r * es, rb);
                cpos[slot] = (int32_t)p;
            } else {
                memset(dk, 0, rb);
                memset(dv, 0, rb);
                cpos[slot] = -1;
            }
        }
    }
    return 0;
}

int orc_sparse_compact(const orc_cache* c, const void* q, const void* ck, const void* cv,
                       const int32_t* cpos, int32_t idx_stride, const int32_t* n_idx,
                       int32_t n_recent, const uint8_t* head_mask, double* out, double* lse) {
    const int G = c->Hq / c->Hkv;
    const int units = c->B * c->Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int u = 0; u < units; ++u) {
        int b = u / c->Hq, i = u % c->Hq, h = i / G;
        int64_t N = c->len[b];
        int64_t r0 = N - n_recent > 0 ? N - n_recent : 0;
        double* o = out + (int64_t)u * c->d;
        for (int x = 0; x < c->d; ++x) o[x] = 0.0;
        if (head_mask && head_mask[u]) {
            lse[u] = -INFINITY;
            continue;
        }
        /* where each attended position's rows live: segment slot (>= 0), the cache (-1),
         * or not attended (-2); a position named by several slots counts once */
        int64_t* src = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        for (int64_t p = 0; p < N; ++p) src[p] = p >= r0 ? -1 : -2;
        int64_t seg0 = ((int64_t)b * c->Hkv + h) * idx_stride;
        int32_t n = n_idx[b * c->Hkv + h];
        n = n < 0 ? 0 : (n > idx_stride ? idx_stride : n);
        for (int32_t s = 0; s < n; ++s) {
            int64_t p = cpos[seg0 + s];
            if (p >= 0 && p < r0 && src[p] == -2) src[p] = seg0 + s;
        }
        double* qi = (double*)malloc(sizeof(double) * c->d);
        load_query(c, q, b, i, qi);
        /* logits in ascending position order, then the softmax-weighted sum of V */
        double* z = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        int64_t n_att = 0;
        double m = -INFINITY;
        for (int64_t p = 0; p < N; ++p) {
            if (src[p] == -2) continue;
            const void* kb = src[p] >= 0 ? ck : c->k;
            int64_t r = src[p] >= 0 ? src[p] * c->d : row_start(c, b, h, p);
            double dot = 0.0;
            for (int x = 0; x < c->d; ++x) dot += qi[x] * load_elem(kb, c->is_bf16, r + x);
            z[n_att] = dot / sqrt((double)c->d);
            m = z[n_att] > m ? z[n_att] : m;
            ++n_att;
        }
        if (n_att == 0) {
            lse[u] = -INFINITY;
        } else {
            double l = 0.0;
            for (int64_t j = 0; j < n_att; ++j) l += exp(z[j] - m);
            double L = m + log(l);
            int64_t j = 0;
            for (int64_t p = 0; p < N; ++p) {
                if (src[p] == -2) continue;
                const void* vb = src[p] >= 0 ? cv : c->v;
                int64_t r = src[p] >= 0 ? src[p] * c->d : row_start(c, b, h, p);
                double w = exp(z[j++] - L);
                for (int x = 0; x < c->d; ++x) o[x] += w * load_elem(vb, c->is_bf16, r + x);
            }
            lse[u] = L;
        }
        free(src);
        free(qi);
        free(z);
    }
    return 0;
}

/* ---- sparse fast step with group routing ------------------------------------------------ */

int orc_sparse_routed(const orc_cache* c, const void* q, const int32_t* idx, int32_t idx_stride,
                      const int32_t* n_idx, int32_t n_recent, const uint8_t* head_mask,
                      const double* route_lse, double log_gamma, double* margin,
                      uint8_t* routed, double* out, double* lse) {
    const int G = c->Hq / c->Hkv;
    const int units = c->B * c->Hkv;
    uint8_t* mask = (uint8_t*)malloc((size_t)c->B * c->Hq);
    double* qi = (double*)malloc(sizeof(double) * c->d);
    for (int u = 0; u < units; ++u) {
        int b = u / c->Hkv, h = u % c->Hkv;
        int all = c->len[b] > 0;
        double worst = INFINITY;
        for (int g = 0; g < G; ++g) {
            int i = h * G + g;
            double m = -INFINITY;
            if (c->len[b] > 0) {
                load_query(c, q, b, i, qi);
                m = logit_of(c, qi, b, h, 0) - route_lse[b * c->Hq + i] - log_gamma;
            }
            /* head i is sink-dominant when its estimated token-0 mass reaches gamma */
            if (!(m >= 0.0)) all = 0;
            worst = m < worst ? m : worst;
        }
        routed[u] = (uint8_t)all;
        if (margin) margin[u] = worst;
        for (int g = 0; g < G; ++g) {
            int i = h * G + g;
            mask[b * c->Hq + i] = (uint8_t)(all || (head_mask && head_mask[b * c->Hq + i]));
        }
    }
    int rc = orc_sparse(c, q, idx, idx_stride, n_idx, n_recent, mask, out, lse);
    free(qi);
    free(mask);
    return rc;
}

/* ---- sink-bypass mask ---------------------------------------------------------------- */

int orc_sink_mask(int32_t B, int32_t Hq, const double* z0, const double* lse, double frac,
                  uint8_t* head_mask) {
    if (frac < 0.0 || frac > 1.0) return -1;
    int64_t n_mask = (int64_t)floor(frac * Hq);
    double* p0 = (double*)malloc(sizeof(double) * (Hq > 0 ? Hq : 1));
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < Hq; ++i) p0[i] = exp(z0[b * Hq + i] - lse[b * Hq + i]);
        for (int i = 0; i < Hq; ++i) {
            /* rank = number of heads ahead of i in (p0 descending, index ascending) order */
            int64_t rank = 0;
            for (int j = 0; j < Hq; ++j)
                if (p0[j] > p0[i] || (p0[j] == p0[i] && j < i)) ++rank;
            head_mask[b * Hq + i] = rank < n_mask ? 1 : 0;
        }
    }
    free(p0);
    return 0;
}

/* ---- threads ---------------------------------------------------------------------------- */

int orc_threads(void) { return omp_get_max_threads(); }
