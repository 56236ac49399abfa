/*
 * CPU oracle for SPICY-KV coarse-grained decode — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load or call this library.  The GPU library never links it and shares no
 * code, header, table or helper with it.
 *
 * Plain, slow, definitional C in double precision.  Every function states
 * the passage of the pages it follows:
 *   - "SPICY-KV demo page" = the SPICY-KV demo page ("SPectral Invariant
 *     Coarse-graining with dYadic KV Renormalization"), with its sections
 *     "2. FlashAttention-2/3 & PagedAttention Online-Softmax Kernel Fusion"
 *     and "Patent Pending Notice & Claims 1-20" (Claims 1, 2, 3).
 *   - "SPICY-KV abstract" = the abstract page of the same method, items (1)-(4).
 *
 * in_dtype / q_dtype is the type of the caller's inputs (keys, values,
 * queries); dtype is the storage type of the cache.
 *
 * Storage dtypes: ORACLE_F32 (IEEE binary32), ORACLE_BF16 (bfloat16 bits in a
 * uint16), ORACLE_F64 (no rounding at all: the "exact layer" used by the
 * invariant tests).
 *
 * Cache layout (the same contract the GPU library documents, implemented
 * here independently):
 *   k_pool : [num_pages][H_kv][d/W][16][W]  key rows by groups of W = min(8, d)
 *            dims (d < 8 or d a multiple of 8)
 *   v_pool : [num_pages][H_kv][d/W][16][W]  value rows, the same way
 *   ab_pool: [num_pages][H_kv][16][2]      (alpha, beta) per entry
 *   meta   : [num_pages][H_kv][16] x {int32 kind, int32 mass, int64 pos_sum}
 *            kind 0 = null, 1 = exact C-point, 2 = macro-node
 * Logical entry e of sequence b lives in physical page page_table[b][e/16],
 * slot e%16.
 */
#ifndef SPICY_ORACLE_H
#define SPICY_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Return codes: 0 ok, 1 bad argument, 2 index out of range, 3 capacity. */

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
                   int32_t b_begin, int32_t b_end);

int oracle_decode(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                  const void* q,
                  const void* k_pool, const void* v_pool, const void* ab_pool,
                  int32_t num_pages,
                  const int32_t* page_table, int32_t max_pages_per_seq,
                  const int32_t* lengths, int32_t B,
                  double* o, double* lse,
                  int32_t b_begin, int32_t b_end);

/* The diagonal closure: coarsening also stores each entry's per-dimension
 * variance (of a macro-node's member keys rotated to its anchor; 0 for
 * C-points and nulls) into s2_pool, laid out like k_pool; decoding uses
 * sum_i q_i^2 s2_i / (2 d) as the closure term. */
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
                        int32_t b_begin, int32_t b_end);
/* Variation-weighted representatives: the macro-node key and value are the
 * token_weight-weighted means of its F-tokens (plain means when every weight
 * is zero); everything else as oracle_coarsen.  s2_pool may be NULL. */
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
                            int32_t b_begin, int32_t b_end);
/* One level of the dyadic merge: consecutive macro-node pairs among each
 * (sequence, head)'s entries [entry_begin[b], entry_end[b]) become one
 * macro-node (law of total variance) at the first entry and a null at the
 * second.  Needs the metadata pool; s2_pool must be NULL. */
int oracle_merge_level(int dtype, int32_t H_kv, int32_t d,
                       void* k_pool, void* v_pool, void* ab_pool, void* meta, void* s2_pool,
                       int32_t num_pages, const int32_t* page_table, int32_t max_pages_per_seq,
                       const int32_t* entry_begin, const int32_t* entry_end, int32_t B, double rope_base,
                       int32_t b_begin, int32_t b_end);
/* Compaction after a merge: per (sequence, head) the non-null entries
 * (alpha != -inf) of [entry_begin[b], lengths[b]) move, in order, to the
 * front of the range; lengths_out[b] = entry_begin[b] + the longest head's
 * count; shorter heads and the rest of that last page become nulls. */
int oracle_compact_range(int dtype, int32_t H_kv, int32_t d,
                         void* k_pool, void* v_pool, void* ab_pool, void* meta, void* s2_pool,
                         int32_t num_pages, const int32_t* page_table, int32_t max_pages_per_seq,
                         const int32_t* entry_begin, const int32_t* lengths, int32_t B,
                         int32_t* lengths_out, int32_t b_begin, int32_t b_end);
int oracle_decode_heads(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                        const void* q,
                        const void* k_pool, const void* v_pool, const void* ab_pool, const void* s2_pool,
                        int32_t num_pages,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        const int32_t* lengths, int32_t B,
                        double* o, double* lse,
                        int32_t b_begin, int32_t b_end, int32_t g_begin, int32_t g_end);
int oracle_decode_diag(int q_dtype, int dtype, int32_t H_q, int32_t H_kv, int32_t d,
                       const void* q,
                       const void* k_pool, const void* v_pool, const void* ab_pool, const void* s2_pool,
                       int32_t num_pages,
                       const int32_t* page_table, int32_t max_pages_per_seq,
                       const int32_t* lengths, int32_t B,
                       double* o, double* lse,
                       int32_t b_begin, int32_t b_end);

uint16_t oracle_bf16_round(double x);
double oracle_bf16_value(uint16_t bits);
void oracle_rope(double* y, const double* x, int32_t d, double pos, double base);

/* Per-step coarsening policy: equal-variation segments and key-norm
 * landmarks, in integer arithmetic (see spicy_oracle.c).  Return codes as
 * above, plus 4 = a sequence outside the policy's integer range. */
int64_t oracle_fix16(uint16_t bf16_bits);
uint64_t oracle_isqrt_u128(uint64_t hi, uint64_t lo);
int oracle_policy(int32_t H_kv, int32_t d, const uint16_t* k_pre, const uint16_t* v,
                  const int32_t* seq_offsets, int32_t B,
                  const int32_t* proj_ptr, const int32_t* proj_idx, int32_t proj_rows,
                  int32_t n_segments, int32_t n_landmarks, int32_t sink, int32_t recent,
                  int32_t* seg_offsets, int32_t* seq_seg_ptr, uint8_t* protected_mask,
                  int64_t* variation_out, uint64_t* norm2_out);

#ifdef __cplusplus
}
#endif
#endif
