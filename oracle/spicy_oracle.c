/*
 * CPU oracle for SPICY-KV coarse-grained decode — TEST INFRASTRUCTURE ONLY.
 * (See spicy_oracle.h for who may use it and for the cache layout.)
 *
 * Everything here is the definition written out in double precision, one
 * step at a time, in the order the pages give it.  No blocking, no fusion,
 * no reordering beyond the definition.  Rounding to the storage type happens
 * exactly once, when a value is stored.
 */
#include "spicy_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define PAGE 16

/* ------------------------------------------------------------------------ */
/* Storage rounding                                                          */
/* ------------------------------------------------------------------------ */

/* bfloat16 value of a bit pattern: the bits are the top half of a binary32. */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16, ties to even, in one step (no
 * intermediate binary32 rounding).  bfloat16 has 8 significant bits and the
 * binary32 exponent range, so the spacing of representable values around x is
 * 2^(E-7) with E = max(floor(log2|x|), -126).  Scaling by a power of two is
 * exact, rint() rounds to nearest-even, scaling back is exact. */
uint16_t oracle_bf16_round(double x) {
    if (isnan(x)) return (uint16_t)0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;               /* leading bit weight 2^E      */
    if (E < -126) E = -126;       /* subnormal spacing           */
    int lsb = E - 7;
    double q = rint(ldexp(a, -lsb));
    double r = ldexp(q, lsb);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)r;           /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

static double load_elem(int dtype, const void* base, size_t i) {
    switch (dtype) {
    case ORACLE_F32: return (double)((const float*)base)[i];
    case ORACLE_BF16: return oracle_bf16_value(((const uint16_t*)base)[i]);
    default: return ((const double*)base)[i];
    }
}

static void store_elem(int dtype, void* base, size_t i, double x) {
    switch (dtype) {
    case ORACLE_F32: ((float*)base)[i] = (float)x; break;     /* RNE */
    case ORACLE_BF16: ((uint16_t*)base)[i] = oracle_bf16_round(x); break;
    default: ((double*)base)[i] = x; break;
    }
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding                                                 */
/* ------------------------------------------------------------------------ */

/* y = R(pos) x with the half-split pairing (i, i + d/2) and frequencies
 * theta_i = base^(-2i/d).  The position is a real number: macro-nodes are
 * rotated to their mass-weighted anchor (SPICY-KV demo page, Claim 2:
 * "spectral center-of-mass position").  base <= 0 means no rotation. */
void oracle_rope(double* y, const double* x, int32_t d, double pos, double base) {
    int32_t half = d / 2;
    if (!(base > 0.0)) {
        for (int32_t i = 0; i < d; ++i) y[i] = x[i];
        return;
    }
    for (int32_t i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / (double)d);
        double phi = pos * theta;
        double c = cos(phi), s = sin(phi);
        double lo = x[i], hi = x[i + half];
        y[i] = lo * c - hi * s;
        y[i + half] = hi * c + lo * s;
    }
}

/* ------------------------------------------------------------------------ */
/* Coarsening                                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t kind;
    int32_t mass;
    int64_t pos_sum;
} oracle_meta;

typedef struct {
    int dtype;
    int32_t H, d, num_pages, max_pages;
    void *k, *v, *ab;
    oracle_meta* meta;
    const int32_t* table_row;
    void* s2;               /* optional: per-dimension variance sidecar, layout of k */
} cache_view;

/* Offset of element (slot, i) inside a page-head block of 16 x d values:
 * groups of W = min(8, d) dimensions outermost, then the 16 slots, then the
 * W dims of the group (the cache layout the header documents; for d < 8 it
 * is plain entry-major rows). */
static size_t slot_elem(int32_t d, int32_t slot, int32_t i) {
    const int32_t W = d < 8 ? d : 8;
    return ((size_t)(i / W) * PAGE + (size_t)slot) * (size_t)W + (size_t)(i % W);
}

/* Head sizes the grouped layout can hold: below 8, or a multiple of 8. */
static int head_dim_ok(int32_t d) { return d > 0 && (d < 8 || d % 8 == 0); }

/* Store one entry at logical index e of a sequence.  key and val are
 * d-vectors already in their final (rotated) form. */
static int put_entry(const cache_view* c, int32_t h, int64_t e,
                     const double* key, const double* val,
                     double alpha, double beta,
                     int32_t kind, int32_t mass, int64_t pos_sum, const double* s2) {
    int64_t lp = e / PAGE;
    if (lp >= c->max_pages) return 3;
    int32_t P = c->table_row[lp];
    if (P < 0 || P >= c->num_pages) return 2;
    int32_t slot = (int32_t)(e % PAGE);
    size_t ph = (size_t)P * (size_t)c->H + (size_t)h;
    for (int32_t i = 0; i < c->d; ++i) {
        store_elem(c->dtype, c->k, ph * PAGE * (size_t)c->d + slot_elem(c->d, slot, i), key[i]);
        store_elem(c->dtype, c->v, ph * PAGE * (size_t)c->d + slot_elem(c->d, slot, i), val[i]);
        if (c->s2)
            store_elem(c->dtype, c->s2, ph * PAGE * (size_t)c->d + slot_elem(c->d, slot, i), s2 ? s2[i] : 0.0);
    }
    store_elem(c->dtype, c->ab, (ph * PAGE + (size_t)slot) * 2 + 0, alpha);
    store_elem(c->dtype, c->ab, (ph * PAGE + (size_t)slot) * 2 + 1, beta);
    if (c->meta) {
        oracle_meta* m = &c->meta[ph * PAGE + (size_t)slot];
        m->kind = kind;
        m->mass = mass;
        m->pos_sum = pos_sum;
    }
    return 0;
}

/* spicy_coarsen, defined step by step.
 *
 * Per sequence b and KV head h, the caller's segments split the sequence's
 * tokens into contiguous runs.  Inside a segment the protected tokens are
 * C-points (exact, mass 1, own position) and the rest are F-points merged into
 * one macro-node (SPICY-KV demo page, Claim 2; SPICY-KV abstract, item (3)):
 *   m      = |F|                                  conserved mass
 *   kbar   = (1/m) sum_F k_t     (pre-RoPE keys)  mass-weighted mean key
 *   vbar   = (1/m) sum_F v_t                      mean value
 *   sigma2 = (1/(m d)) sum_F ||k_t - kbar||^2     scalar sub-grid variance
 *   tbar   = (1/m) sum_F p_t                      centre-of-mass position
 * stored as key R(tbar) kbar, value vbar, alpha = ln m and
 * beta = sigma2 / (2 d) (demo page, section 2, and Claim 3).
 * A C-point stores R(p_t) k_t, v_t, alpha = 0, beta = 0 (m_c = 1, exact t_c).
 * Order inside a segment: macro-node first, then C-points by position.
 * Heads with fewer entries than the most populous head are padded with null
 * entries (alpha = -inf, zero key and value) up to that count, and the tail
 * of the last page touched is padded with nulls as well.
 * lengths_out[b] = entry_start[b] + max over heads of the entry count. */
static int coarsen_impl(int in_dtype, int dtype, int32_t H_kv, int32_t d,
                   const void* k_pre, const void* v,
                   const int32_t* seq_offsets, const int32_t* pos_base,
                   const int32_t* seg_offsets, const int32_t* seq_seg_ptr,
                   const uint8_t* protected_mask,
                   int32_t B, double rope_base,
                   void* k_pool, void* v_pool, void* ab_pool, void* meta,
                   int32_t num_pages,
                   const int32_t* page_table, int32_t max_pages_per_seq,
                   const int32_t* entry_start, int32_t* lengths_out,
                   int32_t b_begin, int32_t b_end, void* s2_pool, const int64_t* token_weight) {
    if (dtype < 0 || dtype > 2 || in_dtype < 0 || in_dtype > 2) return 1;
    if (H_kv <= 0 || !head_dim_ok(d) || (d % 2) != 0 || B < 0) return 1;
    if (!k_pre || !v || !seq_offsets || !seg_offsets || !seq_seg_ptr || !protected_mask) return 1;
    if (!k_pool || !v_pool || !ab_pool || !page_table || !lengths_out) return 1;
    if (b_begin < 0 || b_end > B || b_begin > b_end) return 1;

    double* key = malloc(sizeof(double) * (size_t)d);
    double* rot = malloc(sizeof(double) * (size_t)d);
    double* val = malloc(sizeof(double) * (size_t)d);
    double* zero = calloc((size_t)d, sizeof(double));
    int64_t* total = malloc(sizeof(int64_t) * (size_t)H_kv);
    double* s2v = malloc(sizeof(double) * (size_t)d);
    double* kt = malloc(sizeof(double) * (size_t)d);
    double* rkt = malloc(sizeof(double) * (size_t)d);
    double* wkey = malloc(sizeof(double) * (size_t)d);
    double* wval = malloc(sizeof(double) * (size_t)d);
    double* rotm = malloc(sizeof(double) * (size_t)d);
    if (!key || !rot || !val || !zero || !total || !s2v || !kt || !rkt || !wkey || !wval || !rotm) {
        free(key); free(rot); free(val); free(zero); free(total); free(s2v); free(kt); free(rkt);
        free(wkey); free(wval); free(rotm);
        return 1;
    }
    int rc = 0;

    for (int32_t b = b_begin; b < b_end && rc == 0; ++b) {
        cache_view c = {dtype, H_kv, d, num_pages, max_pages_per_seq,
                        k_pool, v_pool, ab_pool, (oracle_meta*)meta,
                        page_table + (size_t)b * (size_t)max_pages_per_seq, s2_pool};
        int32_t t0 = seq_offsets[b], t1 = seq_offsets[b + 1];
        int32_t s0 = seq_seg_ptr[b], s1 = seq_seg_ptr[b + 1];
        int64_t e0 = entry_start ? entry_start[b] : 0;
        int64_t p0 = pos_base ? pos_base[b] : 0;
        if (t0 > t1 || s0 > s1 || e0 < 0) { rc = 1; break; }
        if (seg_offsets[s0] != t0 || seg_offsets[s1] != t1) { rc = 1; break; }
        for (int32_t s = s0; s < s1; ++s)
            if (seg_offsets[s] > seg_offsets[s + 1]) { rc = 1; break; }
        if (rc) break;

        for (int32_t h = 0; h < H_kv && rc == 0; ++h) {
            int64_t e = e0;
            for (int32_t s = s0; s < s1 && rc == 0; ++s) {
                int32_t a = seg_offsets[s], z = seg_offsets[s + 1];

                /* F-points: the unprotected tokens of the segment. */
                int32_t m = 0;
                int64_t pos_sum = 0;
                double wsum = 0.0;
                for (int32_t i = 0; i < d; ++i) { key[i] = 0.0; val[i] = 0.0; wkey[i] = 0.0; wval[i] = 0.0; }
                for (int32_t t = a; t < z && rc == 0; ++t) {
                    if (protected_mask[(size_t)t * (size_t)H_kv + (size_t)h]) continue;
                    ++m;
                    pos_sum += p0 + (t - t0);
                    double w = 0.0;
                    if (token_weight) {
                        if (token_weight[t] < 0) { rc = 1; break; }
                        w = (double)token_weight[t];
                        wsum += w;
                    }
                    for (int32_t i = 0; i < d; ++i) {
                        size_t ix = ((size_t)t * (size_t)H_kv + (size_t)h) * (size_t)d + (size_t)i;
                        double kx = load_elem(in_dtype, k_pre, ix), vx = load_elem(in_dtype, v, ix);
                        key[i] += kx;
                        val[i] += vx;
                        if (token_weight) { wkey[i] += w * kx; wval[i] += w * vx; }
                    }
                }
                if (rc) break;
                if (m > 0) {
                    for (int32_t i = 0; i < d; ++i) { key[i] /= (double)m; val[i] /= (double)m; }
                    /* the representative: the plain mean, or with token weights
                     * (the equal-variation page's implementation notes) the
                     * weighted means sum w k / sum w and sum w v / sum w; a
                     * segment whose weights are all zero keeps the plain mean */
                    const double* rkey = key;
                    const double* rval = val;
                    if (token_weight && wsum > 0.0) {
                        for (int32_t i = 0; i < d; ++i) { wkey[i] /= wsum; wval[i] /= wsum; }
                        rkey = wkey;
                        rval = wval;
                    }
                    /* second pass: population variance around the mean */
                    double ss = 0.0;
                    for (int32_t t = a; t < z; ++t) {
                        if (protected_mask[(size_t)t * (size_t)H_kv + (size_t)h]) continue;
                        for (int32_t i = 0; i < d; ++i) {
                            size_t ix = ((size_t)t * (size_t)H_kv + (size_t)h) * (size_t)d + (size_t)i;
                            double dv = load_elem(in_dtype, k_pre, ix) - key[i];
                            ss += dv * dv;
                        }
                    }
                    double sigma2 = ss / ((double)m * (double)d);
                    double tbar = (double)pos_sum / (double)m;
                    oracle_rope(rot, rkey, d, tbar, rope_base);
                    if (s2_pool) {
                        /* diagonal closure: per-dimension population variance
                         * of the member keys rotated to the anchor, the frame
                         * of the stored key (their mean is R(tbar) kbar) */
                        oracle_rope(rotm, key, d, tbar, rope_base);
                        for (int32_t i = 0; i < d; ++i) s2v[i] = 0.0;
                        for (int32_t t = a; t < z; ++t) {
                            if (protected_mask[(size_t)t * (size_t)H_kv + (size_t)h]) continue;
                            for (int32_t i = 0; i < d; ++i) {
                                size_t ix = ((size_t)t * (size_t)H_kv + (size_t)h) * (size_t)d + (size_t)i;
                                kt[i] = load_elem(in_dtype, k_pre, ix);
                            }
                            oracle_rope(rkt, kt, d, tbar, rope_base);
                            for (int32_t i = 0; i < d; ++i) {
                                double dv = rkt[i] - rotm[i];
                                s2v[i] += dv * dv;
                            }
                        }
                        for (int32_t i = 0; i < d; ++i) s2v[i] /= (double)m;
                    }
                    rc = put_entry(&c, h, e, rot, rval, log((double)m),
                                   sigma2 / (2.0 * (double)d), 2, m, pos_sum, s2_pool ? s2v : NULL);
                    ++e;
                }

                /* C-points, ascending position. */
                for (int32_t t = a; t < z && rc == 0; ++t) {
                    if (!protected_mask[(size_t)t * (size_t)H_kv + (size_t)h]) continue;
                    int64_t p = p0 + (t - t0);
                    for (int32_t i = 0; i < d; ++i) {
                        size_t ix = ((size_t)t * (size_t)H_kv + (size_t)h) * (size_t)d + (size_t)i;
                        key[i] = load_elem(in_dtype, k_pre, ix);
                        val[i] = load_elem(in_dtype, v, ix);
                    }
                    oracle_rope(rot, key, d, (double)p, rope_base);
                    rc = put_entry(&c, h, e, rot, val, 0.0, 0.0, 1, 1, p, NULL);
                    ++e;
                }
            }
            total[h] = e - e0;
        }
        if (rc) break;

        int64_t most = 0;
        for (int32_t h = 0; h < H_kv; ++h) if (total[h] > most) most = total[h];
        int64_t len = e0 + most;
        int64_t padded = (len + PAGE - 1) / PAGE * PAGE;
        for (int32_t h = 0; h < H_kv && rc == 0; ++h)
            for (int64_t e = e0 + total[h]; e < padded && rc == 0; ++e)
                rc = put_entry(&c, h, e, zero, zero, -INFINITY, 0.0, 0, 0, 0, NULL);
        if (rc) break;
        lengths_out[b] = (int32_t)len;
    }
    free(key); free(rot); free(val); free(zero); free(total); free(s2v); free(kt); free(rkt);
    free(wkey); free(wval); free(rotm);
    return rc;
}

int oracle_coarsen(int in_dtype, int dtype, int32_t H_kv, int32_t d,
                   const void* k_pre, const void* v,
                   const int32_t* seq_offsets, const int32_t* pos_base,
                   const int32_t* seg_offsets, const int32_t* seq_seg_ptr,
                   const uint8_t* protected_mask,
                   int32_t B, double rope_base,
                   void* k_pool, void* v_pool, void* ab_pool, void* meta,
                   int32_t num_pages,
                   const int32_t* page_table, int32_t max_pages_per_seq,
                   const int32_t* entry_start, int32_t* lengths_out,
                   int32_t b_begin, int32_t b_end) {
    return coarsen_impl(in_dtype, dtype, H_kv, d, k_pre, v, seq_offsets, pos_base, seg_offsets, seq_seg_ptr,
                        protected_mask, B, rope_base, k_pool, v_pool, ab_pool, meta, num_pages, page_table,
                        max_pages_per_seq, entry_start, lengths_out, b_begin, b_end, NULL, NULL);
}

/* The diagonal closure (SPICY-KV demo page, Claim 3: the sub-grid variance
 * as a "diagonal vector"): oracle_coarsen that also stores, per entry, the
 * per-dimension population variance of a macro-node's member keys rotated to
 * its anchor into s2_pool (layout of k_pool); C-points and nulls store 0. */
int oracle_coarsen_diag(int in_dtype, int dtype, int32_t H_kv, int32_t d,
                        const void* k_pre, const void* v,
                        const int32_t* seq_offsets, const int32_t* pos_base,
                        const int32_t* seg_offsets, const int32_t* seq_seg_ptr,
                        const uint8_t* protected_mask,
                        int32_t B, double rope_base,
                        void* k_pool, void* v_pool, void* ab_pool, void* meta, void* s2_pool,
                        int32_t num_pages,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        const int32_t* entry_start, int32_t* lengths_out,
                        int32_t b_begin, int32_t b_end) {
    if (!s2_pool) return 1;
    return coarsen_impl(in_dtype, dtype, H_kv, d, k_pre, v, seq_offsets, pos_base, seg_offsets, seq_seg_ptr,
                        protected_mask, B, rope_base, k_pool, v_pool, ab_pool, meta, num_pages, page_table,
                        max_pages_per_seq, entry_start, lengths_out, b_begin, b_end, s2_pool, NULL);
}

/* Variation-weighted representatives (Equal-Variation KV Cache page,
 * implementation notes): oracle_coarsen (or oracle_coarsen_diag when s2_pool
 * is not NULL) whose macro-node key and value are the token_weight-weighted
 * means of its F-tokens, sum w k / sum w and sum w v / sum w (the plain means
 * when every weight is zero).  token_weight: one non-negative integer per
 * token (the per-token variation d_t), indexed like k_pre's tokens.  Mass,
 * alpha, the anchor, beta and s2 stay the plain statistics. */
int oracle_coarsen_weighted(int in_dtype, int dtype, int32_t H_kv, int32_t d,
                            const void* k_pre, const void* v,
                            const int32_t* seq_offsets, const int32_t* pos_base,
                            const int32_t* seg_offsets, const int32_t* seq_seg_ptr,
                            const uint8_t* protected_mask, const int64_t* token_weight,
                            int32_t B, double rope_base,
                            void* k_pool, void* v_pool, void* ab_pool, void* meta, void* s2_pool,
                            int32_t num_pages,
                            const int32_t* page_table, int32_t max_pages_per_seq,
                            const int32_t* entry_start, int32_t* lengths_out,
                            int32_t b_begin, int32_t b_end) {
    if (!token_weight) return 1;
    return coarsen_impl(in_dtype, dtype, H_kv, d, k_pre, v, seq_offsets, pos_base, seg_offsets, seq_seg_ptr,
                        protected_mask, B, rope_base, k_pool, v_pool, ab_pool, meta, num_pages, page_table,
                        max_pages_per_seq, entry_start, lengths_out, b_begin, b_end, s2_pool, token_weight);
}

/* ------------------------------------------------------------------------ */
/* One level of the dyadic merge cascade                                     */
/* ------------------------------------------------------------------------ */

/* Read entry e of a sequence: key and value rows as stored, alpha, beta and
 * the metadata.  Returns 0, or 2/3 for a page outside the pool / table. */
static int get_entry(const cache_view* c, int32_t h, int64_t e, double* key, double* val,
                     double* alpha, double* beta, oracle_meta* meta) {
    int64_t lp = e / PAGE;
    if (lp >= c->max_pages) return 3;
    int32_t P = c->table_row[lp];
    if (P < 0 || P >= c->num_pages) return 2;
    int32_t slot = (int32_t)(e % PAGE);
    size_t ph = (size_t)P * (size_t)c->H + (size_t)h;
    for (int32_t i = 0; i < c->d; ++i) {
        key[i] = load_elem(c->dtype, c->k, ph * PAGE * (size_t)c->d + slot_elem(c->d, slot, i));
        val[i] = load_elem(c->dtype, c->v, ph * PAGE * (size_t)c->d + slot_elem(c->d, slot, i));
    }
    *alpha = load_elem(c->dtype, c->ab, (ph * PAGE + (size_t)slot) * 2 + 0);
    *beta = load_elem(c->dtype, c->ab, (ph * PAGE + (size_t)slot) * 2 + 1);
    *meta = c->meta[ph * PAGE + (size_t)slot];
    return 0;
}

/* One level of the cascaded dyadic merge (SPICY-KV demo page: the cascaded
 * dyadic ring-buffer pyramid, Claim 12, and the law of total variance across
 * cascades, Claim 10).  For every sequence b and KV head h, the macro-nodes
 * (meta kind 2) among entries [entry_begin[b], entry_end[b]) are paired in
 * entry order, first with second, third with fourth, ...; an odd last one is
 * left alone.  A pair (1, 2) with masses m1, m2, position sums P1, P2 becomes
 * one macro-node of the union of their members:
 *   m = m1 + m2,  P = P1 + P2,  tbar = P / m
 *   mu_i = R(-tbar_i) k_i               (the stored key rotated back to the
 *                                        pre-RoPE mean of its members)
 *   mu = (m1 mu_1 + m2 mu_2) / m,        v = (m1 v_1 + m2 v_2) / m
 *   sigma^2 = (m1 sigma_1^2 + m2 sigma_2^2) / m + m1 m2 ||mu_1 - mu_2||^2 / (m^2 d)
 *             with sigma_i^2 = 2 d beta_i  (the law of total variance)
 * stored at the first entry as key R(tbar) mu, value v, alpha = ln m,
 * beta = sigma^2 / (2 d), meta {2, m, P}; the second entry becomes a null
 * (zero key and value, alpha = -inf, beta = 0, meta {0, 0, 0}).  C-points,
 * nulls and the sequence length are untouched.  The metadata pool is
 * required (it holds the exact masses and anchors); a cache with the
 * diagonal-variance sidecar is not supported (rc 1). */
int oracle_merge_level(int dtype, int32_t H_kv, int32_t d,
                       void* k_pool, void* v_pool, void* ab_pool, void* meta, void* s2_pool,
                       int32_t num_pages, const int32_t* page_table, int32_t max_pages_per_seq,
                       const int32_t* entry_begin, const int32_t* entry_end, int32_t B, double rope_base,
                       int32_t b_begin, int32_t b_end) {
    if (dtype < 0 || dtype > 2 || H_kv <= 0 || !head_dim_ok(d) || (d % 2) != 0 || B < 0) return 1;
    if (!k_pool || !v_pool || !ab_pool || !meta || s2_pool || !page_table || !entry_begin || !entry_end) return 1;
    if (b_begin < 0 || b_end > B || b_begin > b_end) return 1;
    double* k1 = malloc(sizeof(double) * (size_t)d);
    double* k2 = malloc(sizeof(double) * (size_t)d);
    double* v1 = malloc(sizeof(double) * (size_t)d);
    double* v2 = malloc(sizeof(double) * (size_t)d);
    double* mu1 = malloc(sizeof(double) * (size_t)d);
    double* mu2 = malloc(sizeof(double) * (size_t)d);
    double* mu = malloc(sizeof(double) * (size_t)d);
    double* key = malloc(sizeof(double) * (size_t)d);
    double* zero = calloc((size_t)d, sizeof(double));
    int rc = (!k1 || !k2 || !v1 || !v2 || !mu1 || !mu2 || !mu || !key || !zero) ? 1 : 0;
    for (int32_t b = b_begin; b < b_end && rc == 0; ++b) {
        cache_view c = {dtype, H_kv, d, num_pages, max_pages_per_seq, k_pool, v_pool, ab_pool,
                        (oracle_meta*)meta, page_table + (size_t)b * (size_t)max_pages_per_seq, NULL};
        int64_t e0 = entry_begin[b], e1 = entry_end[b];
        if (e0 < 0 || e0 > e1) { rc = 1; break; }
        for (int32_t h = 0; h < H_kv && rc == 0; ++h) {
            int64_t first = -1;                     /* the unpaired macro-node so far */
            for (int64_t e = e0; e < e1 && rc == 0; ++e) {
                double a2, b2;
                oracle_meta m2;
                rc = get_entry(&c, h, e, k2, v2, &a2, &b2, &m2);
                if (rc || m2.kind != 2) continue;
                if (m2.mass <= 0) { rc = 1; break; }
                if (first < 0) { first = e; continue; }
                double a1, b1;
                oracle_meta m1;
                rc = get_entry(&c, h, first, k1, v1, &a1, &b1, &m1);
                if (rc) break;
                const double M1 = (double)m1.mass, M2 = (double)m2.mass;
                const int64_t mass = (int64_t)m1.mass + (int64_t)m2.mass;
                if (mass > INT32_MAX) { rc = 1; break; }
                const double M = (double)mass;
                const int64_t psum = m1.pos_sum + m2.pos_sum;
                oracle_rope(mu1, k1, d, -(double)m1.pos_sum / M1, rope_base);
                oracle_rope(mu2, k2, d, -(double)m2.pos_sum / M2, rope_base);
                double dist = 0.0;
                for (int32_t i = 0; i < d; ++i) {
                    const double dm = mu1[i] - mu2[i];
                    dist += dm * dm;
                    mu[i] = (M1 * mu1[i] + M2 * mu2[i]) / M;
                    v1[i] = (M1 * v1[i] + M2 * v2[i]) / M;
                }
                const double sig1 = 2.0 * (double)d * b1, sig2 = 2.0 * (double)d * b2;
                const double sigma2 = (M1 * sig1 + M2 * sig2) / M + M1 * M2 * dist / (M * M * (double)d);
                oracle_rope(key, mu, d, (double)psum / M, rope_base);
                rc = put_entry(&c, h, first, key, v1, log(M), sigma2 / (2.0 * (double)d), 2, (int32_t)mass, psum,
                               NULL);
                if (!rc) rc = put_entry(&c, h, e, zero, zero, -INFINITY, 0.0, 0, 0, 0, NULL);
                first = -1;
            }
        }
    }
    free(k1); free(k2); free(v1); free(v2); free(mu1); free(mu2); free(mu); free(key); free(zero);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Compaction of a merged range                                              */
/* ------------------------------------------------------------------------ */

static size_t dtype_bytes(int dtype) {
    return dtype == ORACLE_F32 ? 4 : dtype == ORACLE_BF16 ? 2 : 8;
}

/* Copy every stored byte of entry (P_src, slot_src) of head h to
 * (P_dst, slot_dst): key, value and variance rows, (alpha, beta), metadata. */
static void copy_entry_raw(const cache_view* c, int32_t h, int32_t P_src, int32_t s_src,
                           int32_t P_dst, int32_t s_dst) {
    const size_t es = dtype_bytes(c->dtype);
    const size_t src = (size_t)P_src * (size_t)c->H + (size_t)h;
    const size_t dst = (size_t)P_dst * (size_t)c->H + (size_t)h;
    void* rows[3] = {c->k, c->v, c->s2};
    for (int r = 0; r < 3; ++r) {
        if (!rows[r]) continue;
        char* base = (char*)rows[r];
        for (int32_t i = 0; i < c->d; ++i)
            memmove(base + (dst * PAGE * (size_t)c->d + slot_elem(c->d, s_dst, i)) * es,
                    base + (src * PAGE * (size_t)c->d + slot_elem(c->d, s_src, i)) * es, es);
    }
    char* ab = (char*)c->ab;
    memmove(ab + (dst * PAGE + (size_t)s_dst) * 2 * es, ab + (src * PAGE + (size_t)s_src) * 2 * es, 2 * es);
    if (c->meta) c->meta[dst * PAGE + (size_t)s_dst] = c->meta[src * PAGE + (size_t)s_src];
}

/* Give a merged range its freed slots back (SPICY-KV demo page: the cascaded
 * dyadic ring-buffer pyramid, Claim 12, where a level that has merged
 * occupies half its slots; Equal-Variation KV Cache page, implementation
 * notes: the reservoir is split and merged as it streams).  For every
 * sequence b, over logical entries [entry_begin[b], lengths[b]):
 *   - an entry is null when its alpha is -inf (zero softmax weight);
 *   - per KV head h, the c_h entries that are not null keep their order and
 *     move to entries entry_begin[b], entry_begin[b] + 1, ...;
 *   - lengths_out[b] = entry_begin[b] + max over heads of c_h;
 *   - per head, entries from entry_begin[b] + c_h to the end of the page that
 *     holds entry lengths_out[b] - 1 become nulls (zero key, value and
 *     variance, alpha = -inf, beta = 0, meta {0, 0, 0});
 *   - entries before entry_begin[b] and pages after that one are untouched.
 * A moved entry keeps every stored byte.  Attention over the result equals
 * attention over the input: only zero-weight entries are dropped and the
 * others keep their order.  Return codes: 1 for entry_begin outside
 * [0, lengths], 3 for an entry beyond max_pages_per_seq pages, 2 for a page id
 * outside the pool (nothing of that sequence is changed in these cases). */
int oracle_compact_range(int dtype, int32_t H_kv, int32_t d,
                         void* k_pool, void* v_pool, void* ab_pool, void* meta, void* s2_pool,
                         int32_t num_pages, const int32_t* page_table, int32_t max_pages_per_seq,
                         const int32_t* entry_begin, const int32_t* lengths, int32_t B,
                         int32_t* lengths_out, int32_t b_begin, int32_t b_end) {
    if (dtype < 0 || dtype > 2 || H_kv <= 0 || !head_dim_ok(d) || B < 0) return 1;
    if (!k_pool || !v_pool || !ab_pool || !page_table || !entry_begin || !lengths || !lengths_out) return 1;
    if (b_begin < 0 || b_end > B || b_begin > b_end) return 1;
    int rc = 0;
    int64_t* kept = NULL;                 /* source entries of the head being moved */
    int64_t cap = 0;
    int32_t* count = malloc(sizeof(int32_t) * (size_t)H_kv);
    double* zero = calloc((size_t)d, sizeof(double));
    if (!count || !zero) { free(count); free(zero); return 1; }
    for (int32_t b = b_begin; b < b_end && rc == 0; ++b) {
        const int32_t* row = page_table + (size_t)b * (size_t)max_pages_per_seq;
        cache_view c = {dtype, H_kv, d, num_pages, max_pages_per_seq, k_pool, v_pool, ab_pool,
                        (oracle_meta*)meta, row, s2_pool};
        const int64_t e0 = entry_begin[b], L = lengths[b];
        if (e0 < 0 || e0 > L) { rc = 1; break; }
        if ((L + PAGE - 1) / PAGE > max_pages_per_seq) { rc = 3; break; }
        for (int64_t lp = e0 / PAGE; lp < (L + PAGE - 1) / PAGE; ++lp)
            if (row[lp] < 0 || row[lp] >= num_pages) rc = 2;
        if (rc) break;
        if (L - e0 > cap) {
            free(kept);
            cap = L - e0;
            kept = malloc(sizeof(int64_t) * (size_t)cap);
            if (!kept) { rc = 1; break; }
        }
        int32_t longest = 0;
        for (int32_t h = 0; h < H_kv; ++h) {
            count[h] = 0;
            for (int64_t e = e0; e < L; ++e) {
                const size_t ph = (size_t)row[e / PAGE] * (size_t)H_kv + (size_t)h;
                if (load_elem(dtype, ab_pool, (ph * PAGE + (size_t)(e % PAGE)) * 2) != -INFINITY) ++count[h];
            }
            if (count[h] > longest) longest = count[h];
        }
        const int64_t new_len = e0 + longest;
        const int64_t pad_end = (new_len + PAGE - 1) / PAGE * PAGE;
        for (int32_t h = 0; h < H_kv; ++h) {
            int64_t n = 0;
            for (int64_t e = e0; e < L; ++e) {
                const size_t ph = (size_t)row[e / PAGE] * (size_t)H_kv + (size_t)h;
                if (load_elem(dtype, ab_pool, (ph * PAGE + (size_t)(e % PAGE)) * 2) != -INFINITY) kept[n++] = e;
            }
            /* kept[i] >= e0 + i: moving in increasing i never overwrites an
             * entry still to be moved */
            for (int64_t i = 0; i < n; ++i) {
                const int64_t src = kept[i], dst = e0 + i;
                if (src != dst)
                    copy_entry_raw(&c, h, row[src / PAGE], (int32_t)(src % PAGE), row[dst / PAGE],
                                   (int32_t)(dst % PAGE));
            }
            for (int64_t e = e0 + n; e < pad_end && rc == 0; ++e)
                rc = put_entry(&c, h, e, zero, zero, -INFINITY, 0.0, 0, 0, 0, NULL);
        }
        lengths_out[b] = (int32_t)new_len;
    }
    free(kept);
    free(count);
    free(zero);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Decode                                                                    */
/* ------------------------------------------------------------------------ */

/* spicy_decode_attn, defined directly.  For query head g (KV head
 * h = g / (H_q / H_kv)) and every logical entry e < lengths[b]:
 *   s_e = (q . k_e) / sqrt(d) + alpha_e + ||q||^2 beta_e
 * (SPICY-KV demo page, section 2: the logit with log_mass and
 * half_inv_dk_sigma_sq; Claim 3: the closure term ||q||^2 sigma^2 / (2 d_k)).
 *   LSE = ln sum_e exp(s_e),   O = sum_e exp(s_e - LSE) v_e.
 * A null entry (alpha = -inf) has weight zero.  With no entry of non-zero
 * weight: LSE = -inf and O = 0.  o is [B][H_q][d], lse is [B][H_q]. */
static int decode_impl(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                  const void* q,
                  const void* k_pool, const void* v_pool, const void* ab_pool,
                  int32_t num_pages,
                  const int32_t* page_table, int32_t max_pages_per_seq,
                  const int32_t* lengths, int32_t B,
                  double* o, double* lse,
                  int32_t b_begin, int32_t b_end, int32_t g_begin, int32_t g_end, const void* s2_pool) {
    if (dtype < 0 || dtype > 2 || q_dtype < 0 || q_dtype > 2) return 1;
    if (H_q <= 0 || H_kv <= 0 || !head_dim_ok(d) || (H_q % H_kv) != 0) return 1;
    if (!q || !k_pool || !v_pool || !ab_pool || !page_table || !lengths || !o || !lse) return 1;
    if (b_begin < 0 || b_end > B || b_begin > b_end) return 1;
    if (g_begin < 0 || g_end > H_q || g_begin > g_end) return 1;
    int32_t G = H_q / H_kv;
    for (int32_t b = b_begin; b < b_end; ++b) {
        int32_t L = lengths[b];
        if (L < 0) return 1;
        if ((int64_t)(L + PAGE - 1) / PAGE > max_pages_per_seq) return 3;
        for (int32_t lp = 0; lp < (L + PAGE - 1) / PAGE; ++lp) {
            int32_t P = page_table[(size_t)b * (size_t)max_pages_per_seq + (size_t)lp];
            if (P < 0 || P >= num_pages) return 2;
        }
    }

    double* s = malloc(sizeof(double) * 1);
    int32_t cap = 1;
    for (int32_t b = b_begin; b < b_end; ++b) {
        int32_t L = lengths[b];
        if (L > cap) {
            free(s);
            s = malloc(sizeof(double) * (size_t)L);
            cap = L;
        }
        if (!s) return 1;
        const int32_t* row = page_table + (size_t)b * (size_t)max_pages_per_seq;
        for (int32_t g = g_begin; g < g_end; ++g) {
            int32_t h = g / G;
            size_t qo = ((size_t)b * (size_t)H_q + (size_t)g) * (size_t)d;
            double qn2 = 0.0;
            for (int32_t i = 0; i < d; ++i) {
                double qi = load_elem(q_dtype, q, qo + (size_t)i);
                qn2 += qi * qi;
            }
            double smax = -INFINITY;
            for (int32_t e = 0; e < L; ++e) {
                size_t ph = (size_t)row[e / PAGE] * (size_t)H_kv + (size_t)h;
                int32_t slot = e % PAGE;
                double alpha = load_elem(dtype, ab_pool, (ph * PAGE + (size_t)slot) * 2 + 0);
                double beta = load_elem(dtype, ab_pool, (ph * PAGE + (size_t)slot) * 2 + 1);
                if (alpha == -INFINITY) { s[e] = -INFINITY; continue; }
                double dot = 0.0;
                for (int32_t i = 0; i < d; ++i)
                    dot += load_elem(q_dtype, q, qo + (size_t)i) *
                           load_elem(dtype, k_pool, ph * PAGE * (size_t)d + slot_elem(d, slot, i));
                double closure = qn2 * beta;
                if (s2_pool) {
                    /* diagonal closure: sum_i q_i^2 s2_i / (2 d) */
                    double acc = 0.0;
                    for (int32_t i = 0; i < d; ++i) {
                        double qi = load_elem(q_dtype, q, qo + (size_t)i);
                        acc += qi * qi * load_elem(dtype, s2_pool, ph * PAGE * (size_t)d + slot_elem(d, slot, i));
                    }
                    closure = acc / (2.0 * (double)d);
                }
                s[e] = dot / sqrt((double)d) + alpha + closure;
                if (s[e] > smax) smax = s[e];
            }
            double* out = o + qo;
            for (int32_t i = 0; i < d; ++i) out[i] = 0.0;
            if (smax == -INFINITY) {
                lse[(size_t)b * (size_t)H_q + (size_t)g] = -INFINITY;
                continue;
            }
            double z = 0.0;
            for (int32_t e = 0; e < L; ++e) z += exp(s[e] - smax);
            double lz = smax + log(z);
            lse[(size_t)b * (size_t)H_q + (size_t)g] = lz;
            for (int32_t e = 0; e < L; ++e) {
                double w = exp(s[e] - lz);
                if (w == 0.0) continue;
                size_t ph = (size_t)row[e / PAGE] * (size_t)H_kv + (size_t)h;
                int32_t slot = e % PAGE;
                for (int32_t i = 0; i < d; ++i)
                    out[i] += w * load_elem(dtype, v_pool, ph * PAGE * (size_t)d + slot_elem(d, slot, i));
            }
        }
    }
    free(s);
    return 0;
}

int oracle_decode(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                  const void* q,
                  const void* k_pool, const void* v_pool, const void* ab_pool,
                  int32_t num_pages,
                  const int32_t* page_table, int32_t max_pages_per_seq,
                  const int32_t* lengths, int32_t B,
                  double* o, double* lse,
                  int32_t b_begin, int32_t b_end) {
    return decode_impl(q_dtype, dtype, H_q, H_kv, d, q, k_pool, v_pool, ab_pool, num_pages, page_table,
                       max_pages_per_seq, lengths, B, o, lse, b_begin, b_end, 0, H_q, NULL);
}

/* oracle_decode (s2_pool NULL) or oracle_decode_diag for the query heads
 * [g_begin, g_end) of sequences [b_begin, b_end) only: a smaller work item of
 * the same computation (the other rows of o and lse are untouched). */
int oracle_decode_heads(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                        const void* q,
                        const void* k_pool, const void* v_pool, const void* ab_pool, const void* s2_pool,
                        int32_t num_pages,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        const int32_t* lengths, int32_t B,
                        double* o, double* lse,
                        int32_t b_begin, int32_t b_end, int32_t g_begin, int32_t g_end) {
    return decode_impl(q_dtype, dtype, H_q, H_kv, d, q, k_pool, v_pool, ab_pool, num_pages, page_table,
                       max_pages_per_seq, lengths, B, o, lse, b_begin, b_end, g_begin, g_end, s2_pool);
}

/* The diagonal closure at decode: the logit's closure term is
 * sum_i q_i^2 s2_i / (2 d) with the entry's per-dimension variance s2 (the
 * Gaussian second cumulant of q . k / sqrt(d) for a diagonal covariance)
 * instead of ||q||^2 beta; everything else as oracle_decode. */
int oracle_decode_diag(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                       const void* q,
                       const void* k_pool, const void* v_pool, const void* ab_pool, const void* s2_pool,
                       int32_t num_pages,
                       const int32_t* page_table, int32_t max_pages_per_seq,
                       const int32_t* lengths, int32_t B,
                       double* o, double* lse,
                       int32_t b_begin, int32_t b_end) {
    if (!s2_pool) return 1;
    return decode_impl(q_dtype, dtype, H_q, H_kv, d, q, k_pool, v_pool, ab_pool, num_pages, page_table,
                       max_pages_per_seq, lengths, B, o, lse, b_begin, b_end, 0, H_q, s2_pool);
}

/* ------------------------------------------------------------------------
 * Per-step coarsening policy (the step upstream of oracle_coarsen).
 *
 * Equal-variation segments: Equal-Variation KV Cache page, "Mathematical
 * statement" (breakpoints at equal increments of cumulative variation, first
 * hitting time on flat stretches) and "Implementation notes" (feature
 * z_t = P [k_t; v_t] with P a fixed random projection, local variation
 * d_t = ||z_t - z_{t-1}||_2, cumulative c_t, thresholds q_j = j c_T / N,
 * boundary = the first token whose cumulative variation reaches q_j).
 * Landmarks: SPICY-KV demo page, Claim 2 (exact C-points) and section 1
 * (sink and recent tokens kept exact); the landmark rule is the largest key
 * norms per (sequence, KV head).
 *
 * Everything is integer, so the result does not depend on any summation
 * order:
 *   fix(x)   = x * 2^16 rounded to nearest, ties to even, clamped to
 *              [-2^28, 2^28] (bf16 input; NaN -> 0, +-inf -> +-2^28);
 *   z_t[r]   = sum over the entries of row r of P of sign * fix(x_t[c]),
 *              x_t = [k_t (head-major); v_t (head-major)], P ternary and
 *              given as signed column lists;
 *   d_t      = floor(sqrt(sum_r (z_t[r] - z_{t-1}[r])^2)), d = 0 at a
 *              sequence's first token;
 *   C_t      = d_0 + ... + d_t,  Q_j = floor(j * C_T / N), j = 1..N-1;
 *   b_j      = min { t : C_t >= Q_j };   segment j = [b_j, b_{j+1}),
 *              b_0 = 0, b_N = T, so N slots per sequence, empty ones allowed;
 *   norm2    = sum_i fix(k_t,h[i])^2 (uint64), landmarks = the n_landmarks
 *              largest norm2 among positions [sink, T - recent) of the
 *              sequence, ties to the lower position; the mask also holds
 *              the first `sink` and the last `recent` positions.
 * ------------------------------------------------------------------------ */

int64_t oracle_fix16(uint16_t bits) {
    const int64_t lim = (int64_t)1 << 28;
    int neg = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int64_t m = bits & 0x7F;
    int64_t r;
    if (e == 0xFF) {
        if (m) return 0;                                  /* NaN */
        r = lim;                                          /* infinity */
    } else if (e == 0) {
        r = 0;                                            /* |x| < 2^-126: rounds to 0 */
    } else {
        /* x = (128 + m) * 2^(e - 134);  x * 2^16 = (128 + m) * 2^(e - 118) */
        int64_t M = 128 + m;
        int sh = e - 118;
        if (sh >= 0) {
            r = sh > 21 ? lim : (M << sh);                /* M < 2^8: sh > 21 exceeds 2^28 */
            if (r > lim) r = lim;
        } else if (sh < -9) {
            r = 0;                                        /* M / 2^10 < 1/2 */
        } else {
            int64_t q = M >> (-sh);
            int64_t rem = M - (q << (-sh));
            int64_t half = (int64_t)1 << (-sh - 1);
            if (rem > half || (rem == half && (q & 1))) ++q;
            r = q;
        }
    }
    return neg ? -r : r;
}

/* floor(sqrt(x)) for a 128-bit x, by bisection on the answer: the largest
 * r < 2^64 with r * r <= x. */
static uint64_t isqrt_u128(unsigned __int128 x) {
    uint64_t lo = 0, hi = UINT64_MAX;
    while (lo < hi) {
        uint64_t mid = lo + ((hi - lo) >> 1) + ((hi - lo) & 1);     /* upper middle, no overflow */
        unsigned __int128 sq = (unsigned __int128)mid * mid;
        if (sq <= x) lo = mid; else hi = mid - 1;
    }
    return lo;
}

uint64_t oracle_isqrt_u128(uint64_t hi, uint64_t lo) {
    return isqrt_u128(((unsigned __int128)hi << 64) | lo);
}

typedef struct { uint64_t norm2; int32_t pos; } oracle_rank;

static int rank_cmp(const void* a, const void* b) {
    const oracle_rank* x = (const oracle_rank*)a;
    const oracle_rank* y = (const oracle_rank*)b;
    if (x->norm2 != y->norm2) return x->norm2 > y->norm2 ? -1 : 1;   /* larger norm first */
    return (x->pos > y->pos) - (x->pos < y->pos);                     /* then lower position */
}

int oracle_policy(int32_t H_kv, int32_t d, const uint16_t* k_pre, const uint16_t* v,
                  const int32_t* seq_offsets, int32_t B,
                  const int32_t* proj_ptr, const int32_t* proj_idx, int32_t proj_rows,
                  int32_t n_segments, int32_t n_landmarks, int32_t sink, int32_t recent,
                  int32_t* seg_offsets, int32_t* seq_seg_ptr, uint8_t* protected_mask,
                  int64_t* variation_out, uint64_t* norm2_out) {
    if (H_kv <= 0 || d <= 0 || B < 0 || proj_rows <= 0 || proj_rows > 16) return 1;
    if (n_segments <= 0 || n_landmarks < 0 || sink < 0 || recent < 0) return 1;
    if (!k_pre || !v || !seq_offsets || !proj_ptr || !proj_idx || !seg_offsets || !seq_seg_ptr ||
        !protected_mask)
        return 1;
    const int64_t width = (int64_t)H_kv * d;              /* one of k_t, v_t */
    if (proj_ptr[0] != 0) return 2;
    for (int32_t r = 0; r < proj_rows; ++r) {
        if (proj_ptr[r + 1] < proj_ptr[r]) return 2;
        for (int32_t i = proj_ptr[r]; i < proj_ptr[r + 1]; ++i) {
            int64_t c = proj_idx[i] > 0 ? proj_idx[i] - 1 : -(int64_t)proj_idx[i] - 1;
            if (proj_idx[i] == 0 || c >= 2 * width) return 2;
        }
    }
    for (int32_t b = 0; b <= B; ++b) seq_seg_ptr[b] = b * n_segments;

    int64_t z_prev[16], z[16];
    for (int32_t b = 0; b < B; ++b) {
        const int32_t t0 = seq_offsets[b], t1 = seq_offsets[b + 1];
        if (t0 < 0 || t1 < t0) return 2;
        const int32_t T = t1 - t0;
        if (T > (1 << 20)) return 4;
        int64_t* C = (int64_t*)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
        if (!C) return 1;
        /* variation and cumulative variation */
        int64_t acc = 0;
        for (int32_t t = 0; t < T; ++t) {
            const size_t row = (size_t)(t0 + t) * (size_t)width;
            for (int32_t r = 0; r < proj_rows; ++r) {
                int64_t s = 0;
                for (int32_t i = proj_ptr[r]; i < proj_ptr[r + 1]; ++i) {
                    int64_t c = proj_idx[i] > 0 ? proj_idx[i] - 1 : -(int64_t)proj_idx[i] - 1;
                    uint16_t bits = c < width ? k_pre[row + (size_t)c] : v[row + (size_t)(c - width)];
                    int64_t x = oracle_fix16(bits);
                    s += proj_idx[i] > 0 ? x : -x;
                }
                z[r] = s;
            }
            uint64_t dt = 0;
            if (t > 0) {
                unsigned __int128 ss = 0;
                for (int32_t r = 0; r < proj_rows; ++r) {
                    int64_t dz = z[r] - z_prev[r];
                    unsigned __int128 a = (unsigned __int128)(dz < 0 ? -dz : dz);
                    ss += a * a;
                }
                dt = isqrt_u128(ss);
            }
            for (int32_t r = 0; r < proj_rows; ++r) z_prev[r] = z[r];
            acc += (int64_t)dt;
            C[t] = acc;
            if (variation_out) variation_out[t0 + t] = (int64_t)dt;
        }
        const int64_t CT = T > 0 ? C[T - 1] : 0;
        if (CT > 0 && (unsigned __int128)CT * (unsigned __int128)n_segments >= ((unsigned __int128)1 << 62)) {
            free(C);
            return 4;
        }
        /* boundaries: b_j = min { t : C_t >= Q_j } (T if none) */
        int32_t* so = seg_offsets + (size_t)b * (size_t)n_segments;
        so[0] = t0;
        int32_t t = 0;
        for (int32_t j = 1; j < n_segments; ++j) {
            int64_t Q = (int64_t)(((unsigned __int128)j * (unsigned __int128)CT) / (unsigned __int128)n_segments);
            while (t < T && C[t] < Q) ++t;
            so[j] = t0 + t;
        }
        free(C);

        /* protection mask: sink, recent, landmarks per head */
        oracle_rank* cand = (oracle_rank*)malloc(sizeof(oracle_rank) * (size_t)(T > 0 ? T : 1));
        if (!cand) return 1;
        for (int32_t h = 0; h < H_kv; ++h) {
            int32_t n = 0;
            for (int32_t u = 0; u < T; ++u) {
                const size_t row = ((size_t)(t0 + u) * (size_t)H_kv + (size_t)h) * (size_t)d;
                uint64_t n2 = 0;
                for (int32_t i = 0; i < d; ++i) {
                    int64_t x = oracle_fix16(k_pre[row + (size_t)i]);
                    n2 += (uint64_t)(x * x);
                }
                if (norm2_out) norm2_out[(size_t)(t0 + u) * (size_t)H_kv + (size_t)h] = n2;
                int prot = u < sink || u >= T - recent;
                protected_mask[(size_t)(t0 + u) * (size_t)H_kv + (size_t)h] = (uint8_t)prot;
                if (!prot) {
                    cand[n].norm2 = n2;
                    cand[n].pos = u;
                    ++n;
                }
            }
            qsort(cand, (size_t)n, sizeof(oracle_rank), rank_cmp);
            for (int32_t i = 0; i < n && i < n_landmarks; ++i)
                protected_mask[(size_t)(t0 + cand[i].pos) * (size_t)H_kv + (size_t)h] = 1;
        }
        free(cand);
    }
    seg_offsets[(size_t)B * (size_t)n_segments] = seq_offsets[B];
    return 0;
}
