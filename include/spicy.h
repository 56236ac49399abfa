/*
 * spicy.h — C ABI of the MI355X (gfx950) SPICY-KV coarse-grained decode library.
 *
 * Two core operations, following the pages' statement of the problem:
 *
 *   spicy_coarsen      pre-RoPE keys + values + segment partition + protected
 *                      mask  ->  paged compressed cache
 *                      (SPICY-KV demo page, "Patent Pending Notice & Claims",
 *                      Claim 2: C-points kept exact, F-points merged into
 *                      macro-nodes with mass-weighted mean key, mean value,
 *                      conserved mass and centre-of-mass position; Claim 3:
 *                      scalar sub-grid variance; SPICY-KV abstract, items (1)
 *                      and (3): pre-RoPE tap, C/F splitting)
 *
 *   spicy_decode_attn  query + paged compressed cache -> attention output and
 *                      log-sum-exp (SPICY-KV demo page, section "2.
 *                      FlashAttention-2/3 & PagedAttention Online-Softmax
 *                      Kernel Fusion": logit q.k/sqrt(d_k) + log_mass +
 *                      |q|^2 * half_inv_dk_sigma_sq inside a standard online
 *                      softmax; Claim 3 and abstract item (4): first-order
 *                      log-mass offset and second-order variance closure)
 *
 * and the entry points around them: spicy_decode_attn_shared (a prefix of
 * pages shared by every sequence, read once per KV head), spicy_decode_attn_multi
 * (several query tokens per sequence), spicy_policy (the per-step segments and
 * protection mask computed from the chunk itself), spicy_coarsen_weighted
 * (variation-weighted representatives), spicy_merge_level (one level of the
 * dyadic merge cascade), the optional per-dimension variance sidecar of the
 * cache (diagonal closure), and host helpers for workspace sizes and the
 * split-K plan.
 *
 * Conventions for every entry point
 *   - All buffers are owned and allocated by the caller.  Pointers are DEVICE
 *     pointers unless the comment says host.  The library allocates nothing,
 *     keeps no state between calls and never synchronises; work is enqueued on
 *     the caller's stream (`stream` is a hipStream_t; NULL = default stream).
 *   - Arguments the host can see (sizes, dtypes, null pointers, workspace
 *     size) are validated before anything is launched; on error nothing is
 *     launched and nothing is written.
 *   - Data that live in device memory (offsets, page ids, lengths, masks) are
 *     bounds-checked by the kernels themselves: an index outside its buffer is
 *     never dereferenced; the offending read is skipped (treated as a null
 *     entry / empty segment) and a bit is OR-ed into the sticky device error
 *     word at the start of the workspace (see SPICY_DEVERR_*).  The library
 *     never clears that word: the caller zeroes it (for example with a fill
 *     kernel) when it allocates the workspace and after reading it.
 *   - Kernel faults surface at the caller's next synchronisation; a launch
 *     that fails to enqueue returns SPICY_ERR_HIP.
 *   - Calls on different streams with disjoint outputs may run concurrently;
 *     calls that share a workspace must be ordered by the caller.
 *
 * Paged compressed cache (caller-allocated pool of `num_pages` pages; one page
 * holds PAGE_SIZE = 16 consecutive logical entries of one sequence for all KV
 * heads):
 *   k    : [num_pages][H_kv][d/8][16][8]  key rows, already rotated (RoPE)
 *                                     to the entry's position, cut in 8-dim
 *                                     groups: element (slot s, dim i) of a
 *                                     page-head is at ((i/8)*16 + s)*8 + i%8
 *                                     (so the 16 slots' dims 8g .. 8g+7 are
 *                                     256 contiguous bytes in bf16)
 *   v    : [num_pages][H_kv][d/8][16][8]  value rows, the same way
 *   ab   : [num_pages][H_kv][16][2]   per entry (alpha, beta):
 *                                     alpha = ln(mass), beta = sigma^2/(2d);
 *                                     a null entry has alpha = -inf
 *   s2   : optional (may be NULL), laid out like k: the diagonal closure
 *          (SPICY-KV demo page, Claim 3, the sub-grid variance as a
 *          diagonal vector).  Per entry, the per-dimension population
 *          variance of the member keys rotated to the entry's anchor (the
 *          frame of the stored key); 0 for C-points and nulls.  When set,
 *          spicy_coarsen writes it and every decode entry point uses the
 *          closure sum_i q_i^2 s2_i / (2d) in place of |q|^2 beta.
 *   meta : optional (may be NULL), [num_pages][H_kv][16] x 16 bytes
 *          { int32 kind; int32 mass; int64 pos_sum; }
 *          kind 0 = null, 1 = exact C-point, 2 = macro-node; pos_sum is the sum
 *          of the member positions (anchor = pos_sum / mass).
 *   Element type of k, v, ab, s2: dtype (SPICY_BF16 or SPICY_F32).
 *   Logical entry e of sequence b lives in page page_table[b*max_pages + e/16],
 *   slot e%16.
 */
#ifndef SPICY_H
#define SPICY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPICY_OK = 0,
    SPICY_ERR_ARG = 1,          /* null pointer, negative size, bad enum      */
    SPICY_ERR_RANGE = 2,        /* a host-visible size outside what it indexes */
    SPICY_ERR_CAPACITY = 3,     /* workspace too small                         */
    SPICY_ERR_UNSUPPORTED = 4,  /* head_dim not 64/128, GQA group > 16, ...    */
    SPICY_ERR_HIP = 5           /* a HIP launch failed to enqueue              */
} spicy_status;

typedef enum { SPICY_F32 = 0, SPICY_BF16 = 1 } spicy_dtype;

/* Sticky device error bits (first int32 of every workspace). */
#define SPICY_DEVERR_PAGE_ID     0x1  /* page id outside [0, num_pages)          */
#define SPICY_DEVERR_CAPACITY    0x2  /* entries beyond max_pages_per_seq * 16   */
#define SPICY_DEVERR_SEGMENTS    0x4  /* segment/sequence offsets inconsistent   */
#define SPICY_DEVERR_LENGTH      0x8  /* a length < 0                            */
#define SPICY_DEVERR_SHARED      0x10 /* declared shared prefix pages differ      */
#define SPICY_DEVERR_POLICY      0x20 /* spicy_policy: projection entry outside
                                          [k_t; v_t], bad row pointers, a sequence
                                          longer than 2^20 tokens or one whose
                                          total variation times N reaches 2^62   */
#define SPICY_DEVERR_TICKET      0x40 /* decode or merge: an arrival counter was
                                          not zero when the call started
                                          (workspace not zero-filled, or reused
                                          for more rows or units than it was
                                          zeroed for)                           */

#define SPICY_PAGE_SIZE 16
#define SPICY_WORKSPACE_HEADER 256   /* bytes before any per-call scratch     */

typedef struct {
    int32_t dtype;          /* spicy_dtype                                   */
    int32_t num_kv_heads;   /* H_kv >= 1                                     */
    int32_t head_dim;       /* d: 64 or 128                                  */
    int32_t num_pages;      /* pages in the pool                             */
    void* k;                /* device, see layout above                      */
    void* v;                /* device                                        */
    void* ab;               /* device                                        */
    void* meta;             /* device or NULL                                */
    void* s2;               /* device or NULL: the diagonal closure's
                               per-dimension variance, laid out like k      */
} spicy_cache;

/* Workspace bytes spicy_coarsen needs for `n_seg` segments and
 * `total_tokens` tokens over `B` sequences, `num_kv_heads` heads of
 * `head_dim` dims in cache dtype `dtype` (header, per segment and per
 * (segment, head) plan, a list of C-point items of up to
 * total_tokens x num_kv_heads entries, per (sequence, head) counts, and one
 * macro-node per (segment, head), with its variance row, staged before it
 * is placed).  0 for invalid sizes. */
size_t spicy_coarsen_workspace_bytes(int32_t B, int32_t n_seg, int32_t total_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t dtype);

/* spicy_coarsen — build compressed entries for B sequences.
 *
 * Inputs (device):
 *   k_pre, v        [total_tokens][H_kv][d] in cache->dtype; keys are taken
 *                   before RoPE (demo page Claim 1 (b), pre-RoPE tap).
 *   seq_offsets     int32 [B+1]: tokens of sequence b are
 *                   [seq_offsets[b], seq_offsets[b+1]) of the packed input.
 *   pos_base        int32 [B] or NULL: absolute position of sequence b's first
 *                   token (NULL = 0).  Token t of sequence b sits at position
 *                   pos_base[b] + t - seq_offsets[b].
 *   seg_offsets     int32 [n_seg+1]: segment s covers packed tokens
 *                   [seg_offsets[s], seg_offsets[s+1]).
 *   seq_seg_ptr     int32 [B+1]: segments of sequence b are
 *                   [seq_seg_ptr[b], seq_seg_ptr[b+1]); they must tile that
 *                   sequence's tokens in order (an empty segment emits nothing).
 *   protected_mask  uint8 [total_tokens][H_kv]: non-zero = C-point (kept exact).
 *   page_table      int32 [B][max_pages_per_seq]: physical page of each
 *                   logical page; only the pages this call writes are read.
 *   entry_start     int32 [B] or NULL: first logical entry written for
 *                   sequence b (NULL = 0).  Entries before it are untouched.
 * Output:
 *   Per sequence b and KV head h, segment by segment: if the segment has
 *   unprotected tokens, one macro-node (key R(tbar)·mean, value mean,
 *   alpha = ln m, beta = sigma^2/(2d), sigma^2 = per-dimension population
 *   variance of the member keys, tbar = mean member position); then every
 *   protected token in position order as an exact entry (key R(p)·k, value v,
 *   alpha = beta = 0).  Heads with fewer entries are padded with null entries
 *   to the longest head, and the last page written is padded with nulls to its
 *   end.  lengths_out[b] (int32, device) = entry_start[b] + the longest head's
 *   entry count.  RoPE uses the half-split pairing (i, i+d/2) with
 *   theta_i = rope_base^(-2i/d); rope_base <= 0 means no rotation.  Values are
 *   accumulated in double precision and rounded once, to nearest-even, on store.
 *   With cache->s2 set, each macro-node also gets its per-dimension variance
 *   s2 (see the cache layout), computed from one pass of sums (per dimension,
 *   and per rotary pair the product sum), C-points and nulls get s2 = 0.
 * Workspace: device, >= spicy_coarsen_workspace_bytes(B, n_seg, total_tokens, H_kv, d, dtype) bytes,
 *   first int32 = sticky device error word (not cleared by the library).
 *   Besides the workspace, the library keeps 1 MiB of device memory per
 *   element type and head dim on each GPU (allocated when the library loads)
 *   for hints that let most macro-nodes go straight into the cache; a hint
 *   carries its call's tag, so calls in flight together (on one stream or
 *   several) never take each other's, and a call with more than 2^17
 *   (segment, head) pairs, or a pool of 2^28 pages or more, runs without them.
 *   A call captured into a HIP graph keeps the tag it was captured with, so
 *   replays of one captured call must not be in flight together on one GPU
 *   (which sharing its workspace already rules out).
 * Errors: SPICY_ERR_ARG (null required pointer, B < 0, n_seg < 0, bad dtype),
 *   SPICY_ERR_UNSUPPORTED (head_dim not 64/128, H_kv > 16, max_pages_per_seq > 2^23),
 *   SPICY_ERR_CAPACITY (workspace too small), SPICY_ERR_HIP. */
spicy_status spicy_coarsen(const spicy_cache* cache,              /* host struct */
                           const void* k_pre, const void* v, int32_t total_tokens,
                           const int32_t* seq_offsets, const int32_t* pos_base,
                           const int32_t* seg_offsets, const int32_t* seq_seg_ptr,
                           int32_t n_seg, const uint8_t* protected_mask,
                           int32_t B, double rope_base,
                           const int32_t* page_table, int32_t max_pages_per_seq,
                           const int32_t* entry_start, int32_t* lengths_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* spicy_coarsen_weighted — spicy_coarsen with variation-weighted
 * representatives (Equal-Variation KV Cache page, implementation notes: each
 * segment's representative key and value are the variation-weighted averages
 * sum_r d_r k_r / sum_r d_r and sum_r d_r v_r / sum_r d_r).
 *   token_weight  int64 [total_tokens] (device): one non-negative weight per
 *                 token, indexed like k_pre's tokens; spicy_policy leaves its
 *                 variation d_t in exactly this form in its workspace.
 * A macro-node's key (before rotation) and value are the weighted means of
 * its F-tokens; when every such weight is zero, the plain means.  Mass,
 * alpha, the anchor tbar, beta and the diagonal variances keep their plain
 * definitions; C-points and nulls are unchanged.  The weighted sums are exact
 * in double precision (so the result is rounded once) while weight times
 * |value| sums stay below 2^53 (bf16 inputs, weights below 2^30, segments
 * below 2^14 tokens).  A negative weight is the caller's error (the result is
 * then unspecified, not a fault).  Everything else as spicy_coarsen; the
 * workspace size is the same.
 * Errors: those of spicy_coarsen; SPICY_ERR_ARG also for a null token_weight
 *   when there are tokens. */
spicy_status spicy_coarsen_weighted(const spicy_cache* cache,
                                    const void* k_pre, const void* v, int32_t total_tokens,
                                    const int32_t* seq_offsets, const int32_t* pos_base,
                                    const int32_t* seg_offsets, const int32_t* seq_seg_ptr,
                                    int32_t n_seg, const uint8_t* protected_mask,
                                    const int64_t* token_weight,
                                    int32_t B, double rope_base,
                                    const int32_t* page_table, int32_t max_pages_per_seq,
                                    const int32_t* entry_start, int32_t* lengths_out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * spicy_merge_level — one level of the cascaded dyadic merge, in place.
 *
 * SPICY-KV demo page: the cascaded dyadic ring-buffer pyramid (Claim 12) and
 * the recursive law of total variance across cascades (Claim 10).  For every
 * sequence b and KV head h, the macro-nodes (meta kind 2) among logical
 * entries [entry_begin[b], entry_end[b]) are paired in entry order (first
 * with second, third with fourth, ...; an odd last one is left as it is).
 * A pair with masses m1, m2, position sums P1, P2, stored keys k1, k2,
 * values v1, v2 and betas b1, b2 becomes one macro-node of the union of their
 * members, written at the first entry:
 *   m = m1 + m2, P = P1 + P2, tbar = P / m,
 *   mu_i = R(-P_i / m_i) k_i (pre-RoPE means), mu = (m1 mu_1 + m2 mu_2) / m,
 *   key R(tbar) mu, value (m1 v1 + m2 v2) / m, alpha = ln m,
 *   sigma^2 = (m1 2d b1 + m2 2d b2) / m + m1 m2 |mu_1 - mu_2|^2 / (m^2 d),
 *   beta = sigma^2 / (2d), meta {2, m, P};
 * the second entry becomes a null (zero key and value, alpha = -inf,
 * beta = 0, meta {0, 0, 0}).  C-points, nulls, entries outside the range and
 * the sequence lengths are untouched; attention over the result equals
 * attention over the coarsening of the joined segments up to the storage
 * rounding.  Calling it again merges the next level.  Arithmetic in double
 * precision, one rounding on store.
 *
 * The ranges of different sequences must not share physical pages (merge a
 * shared prefix through one sequence only): calls race on a shared page.
 * Requirements: cache->meta (exact masses and anchors) set; cache->s2 NULL
 * (a diagonal variance does not merge from its own diagonal: the rotated
 * pair covariances are not stored).  rope_base as for spicy_coarsen.
 *   page_table    int32 [B][max_pages_per_seq] (device).
 *   entry_begin, entry_end  int32 [B] (device); end - begin <= max_range.
 * Workspace: device, >= spicy_merge_workspace_bytes(B, H_kv, max_range)
 *   bytes; first int32 = sticky device error word: SPICY_DEVERR_SEGMENTS for
 *   a range outside [0, max_range] or a pair whose metadata is not two
 *   macro-nodes of positive mass (that pair is skipped), SPICY_DEVERR_PAGE_ID
 *   and SPICY_DEVERR_CAPACITY for entries the table or pool cannot hold;
 *   then one int32 arrival counter per (sequence, KV head), which must be
 *   zero when a call starts: allocate the workspace zero-filled (every
 *   completed call leaves the counters at zero); a counter found above its
 *   unit's workgroup count sets SPICY_DEVERR_TICKET.  Calls that overlap on
 *   one workspace race.
 * Errors: SPICY_ERR_ARG (null pointer, B < 0, max_range < 0, meta NULL),
 *   SPICY_ERR_UNSUPPORTED (s2 set, head_dim not 64/128, B * H_kv > 65535),
 *   SPICY_ERR_CAPACITY (workspace too small), SPICY_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t spicy_merge_workspace_bytes(int32_t B, int32_t num_kv_heads, int32_t max_range);

spicy_status spicy_merge_level(const spicy_cache* cache, int32_t B, double rope_base,
                               const int32_t* page_table, int32_t max_pages_per_seq,
                               const int32_t* entry_begin, const int32_t* entry_end,
                               int32_t max_range, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * spicy_compact_range — give a merged range its freed entries back, in place.
 *
 * SPICY-KV demo page, Claim 12: in the cascaded dyadic ring-buffer pyramid a
 * level that has merged holds half as many nodes, so it needs half the
 * storage; spicy_merge_level leaves the second entry of every pair as a null,
 * and this call removes the nulls.  For every sequence b, over logical
 * entries [entry_begin[b], lengths[b]):
 *   - an entry is null when its alpha is -inf (zero weight in the decode);
 *   - per KV head h, the c_h non-null entries keep their order and move to
 *     entries entry_begin[b], entry_begin[b] + 1, ...; a moved entry keeps
 *     every stored byte (key, value, variance row, alpha, beta, metadata);
 *   - lengths_out[b] = entry_begin[b] + max over heads of c_h;
 *   - per head, entries from entry_begin[b] + c_h to the end of the page
 *     holding entry lengths_out[b] - 1 become nulls (zero key, value and
 *     variance, alpha = -inf, beta = 0, meta {0, 0, 0});
 *   - entries before entry_begin[b] and the pages after that last page are
 *     not written: those pages are free for the next appended chunk
 *     (coarsen it at entry_start = lengths_out[b]).
 * The decode over lengths_out equals the decode over lengths up to the
 * order of floating-point additions (only zero-weight entries are dropped);
 * a range with no nulls inside it is left as it is.
 *   page_table    int32 [B][max_pages_per_seq] (device).
 *   entry_begin, lengths  int32 [B] (device); lengths_out int32 [B]
 *                 (device) must not be either of them (it is written before
 *                 the entries move, and they are read again then).
 *   device_error  int32 (device): SPICY_DEVERR_* bits are OR-ed into it:
 *                 SPICY_DEVERR_SEGMENTS for entry_begin[b] outside
 *                 [0, lengths[b]], SPICY_DEVERR_CAPACITY for lengths[b]
 *                 beyond max_pages_per_seq pages, SPICY_DEVERR_PAGE_ID for a
 *                 page id of the range outside the pool; such a sequence is
 *                 left untouched with lengths_out[b] = lengths[b].
 * Ranges of different sequences must not share physical pages.  Needs no
 * workspace: two launches (a count per sequence, then the moves per
 * (sequence, KV head)) on `stream`.
 * Errors: SPICY_ERR_ARG (null pointer, B < 0, max_pages_per_seq < 1,
 *   lengths_out equal to lengths or entry_begin, bad cache),
 *   SPICY_ERR_UNSUPPORTED (B > 65535, head_dim not 64/128), SPICY_ERR_HIP.
 * ------------------------------------------------------------------------ */
spicy_status spicy_compact_range(const spicy_cache* cache, int32_t B,
                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                 const int32_t* entry_begin, const int32_t* lengths,
                                 int32_t* lengths_out, int32_t* device_error, void* stream);

/* Split-K plan: how many splits per (sequence, KV head) spicy_decode_attn
 * uses when asked for `num_splits` (0 = automatic) for a batch of B sequences
 * of at most max_pages_per_seq pages.  Pure host function.  The shared-prefix
 * and multi-token entry points plan over the work of the whole call (prefix
 * chunks and query tiles included): spicy_decode_plan gives their plan. */
int32_t spicy_decode_num_splits(int32_t B, int32_t num_kv_heads, int32_t max_pages_per_seq,
                                int32_t num_splits);

/* The decode's work plan for spicy_decode_attn_multi (and so for
 * spicy_decode_attn: shared_prefix_pages = 0, num_q_tokens = 1; and for
 * spicy_decode_attn_shared: num_q_tokens = 1).  Writes plan[4] (host):
 *   plan[0] shared-prefix chunks (0 without a prefix),
 *   plan[1] prefix pages per chunk (0 without a prefix),
 *   plan[2] splits of each (sequence, KV head)'s private pages (0 if none),
 *   plan[3] private pages per split (0 if none).
 * Pure host function.  Errors: SPICY_ERR_ARG (null plan, counts < 1 where
 * required, negative prefix or num_splits), SPICY_ERR_RANGE (prefix longer
 * than max_pages_per_seq). */
spicy_status spicy_decode_plan(int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_pages_per_seq,
                               int32_t shared_prefix_pages, int32_t num_splits, int32_t num_q_tokens,
                               int32_t* plan);

/* Workspace bytes spicy_decode_attn needs: the header; one int32 arrival
 * counter ("ticket") per query row; per (query row, page group) an fp32
 * partial (max, sum, o[d]).  The tickets must be zero when a call starts:
 * allocate the workspace zero-filled, and zero it again before reusing it
 * for a call with more query rows (B x n_q x H_q) than any earlier call on it
 * (a call finds its tickets right after the header and leaves every ticket
 * it used at zero).  A non-zero ticket sets SPICY_DEVERR_TICKET. */
size_t spicy_decode_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_pages_per_seq,
                                    int32_t num_splits);

/* spicy_decode_attn — one decode query per sequence over the compressed cache.
 *
 * Inputs (device):
 *   q        [B][num_q_heads][d] in cache->dtype, already RoPE-rotated to the
 *            query position.  Query head g reads KV head g / (H_q / H_kv).
 *   lengths  int32 [B]: logical entries of sequence b (null entries inside
 *            count; they get weight zero).  0 = empty sequence.
 *   page_table int32 [B][max_pages_per_seq].
 * Output (device):
 *   o        float32 [B][num_q_heads][d]: sum_e softmax(s)_e v_e with
 *            s_e = q.k_e / sqrt(d) + alpha_e + |q|^2 beta_e (|q|^2 of the
 *            unscaled query); with cache->s2 set the last term is
 *            sum_i q_i^2 s2_e,i / (2d).
 *   lse      float32 [B][num_q_heads]: natural-log log-sum-exp of s; -inf (and
 *            o = 0) when a sequence has no entry of non-zero weight.
 * One launch: the pages of each (sequence, KV head) are cut into page groups
 * (spicy_decode_num_splits(...) of them, each one workgroup, split-K); a row
 * whose pages form a single group is written directly, otherwise every group
 * writes its partial and the last group to arrive at the row (counted with a
 * device-scope atomic ticket) merges the row's partials by log-sum-exp in
 * group order, so the result does not depend on arrival order.
 * Workspace: device, >= spicy_decode_workspace_bytes(...) with the same
 *   num_splits; first int32 = sticky device error word.
 * Errors: SPICY_ERR_ARG, SPICY_ERR_UNSUPPORTED (head_dim not 64/128,
 *   H_q % H_kv != 0, H_q / H_kv > 16), SPICY_ERR_CAPACITY, SPICY_ERR_HIP. */
spicy_status spicy_decode_attn(const spicy_cache* cache,          /* host struct */
                               const void* q, int32_t num_q_heads,
                               const int32_t* page_table, int32_t max_pages_per_seq,
                               const int32_t* lengths, int32_t B,
                               float* o, float* lse,
                               void* workspace, size_t workspace_bytes,
                               int32_t num_splits, void* stream);

/* Workspace bytes spicy_decode_attn_shared needs for the same shapes and a
 * shared prefix of `shared_prefix_pages` pages (either cache dtype). */
size_t spicy_decode_shared_workspace_bytes(int32_t B, int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t max_pages_per_seq,
                                           int32_t shared_prefix_pages, int32_t num_splits);

/* spicy_decode_attn_shared — spicy_decode_attn for a batch whose sequences
 * share a compressed prefix: logical pages [0, shared_prefix_pages) map to the
 * same physical pages in every row of page_table (SPICY-KV demo page, "Patent
 * Pending Notice & Claims", Claim 13: multi-turn shared-prefix reuse; and the
 * page's evaluation list, "4-Turn Shared-Prefix RadixAttention Reuse").  The
 * prefix is compressed once and its pages are referenced by every sequence.
 *
 * Same inputs, outputs, errors and results (up to the order of
 * floating-point additions) as spicy_decode_attn, plus:
 *   shared_prefix_pages  P, host int, 0 <= P <= max_pages_per_seq.  Every row
 *            of page_table must hold the same valid page ids in its first P
 *            entries.  A sequence may be shorter than P pages: entries past its
 *            length get weight zero as usual.
 * On bf16 caches each shared page is read once per KV head and applied to the
 * queries of all B sequences together (rows of 16 query heads x sequences fill
 * the MFMA tiles); the private pages [P, ...) are split as in
 * spicy_decode_attn with `num_splits` (0 = automatic) splits over the longest
 * private part.  Rows whose first P ids differ from row 0's set
 * SPICY_DEVERR_SHARED (the results then follow row 0's ids for the prefix).  On
 * fp32 caches P is only range-checked and every page is read per sequence.
 * Workspace: >= spicy_decode_shared_workspace_bytes(...) with the same P and
 *   num_splits.
 * Errors: those of spicy_decode_attn; SPICY_ERR_ARG if P < 0, SPICY_ERR_RANGE
 *   if P > max_pages_per_seq. */
spicy_status spicy_decode_attn_shared(const spicy_cache* cache,   /* host struct */
                                      const void* q, int32_t num_q_heads,
                                      const int32_t* page_table, int32_t max_pages_per_seq,
                                      const int32_t* lengths, int32_t B,
                                      int32_t shared_prefix_pages,
                                      float* o, float* lse,
                                      void* workspace, size_t workspace_bytes,
                                      int32_t num_splits, void* stream);

/* Workspace bytes spicy_decode_attn_multi needs for the same shapes. */
size_t spicy_decode_multi_workspace_bytes(int32_t B, int32_t num_q_tokens, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, int32_t max_pages_per_seq,
                                          int32_t shared_prefix_pages, int32_t num_splits);

/* spicy_decode_attn_multi — several query tokens per sequence against the
 * compressed cache: every one of the num_q_tokens query tokens of sequence b
 * attends to the same entries [0, lengths[b]) with the logit of
 * spicy_decode_attn (SPICY-KV demo page, section "2. FlashAttention-2/3 &
 * PagedAttention Online-Softmax Kernel Fusion": the tile loop, here with a
 * tile of several query tokens), as in speculative verification or chunked
 * prefill against the compressed history.  The new tokens' own keys and
 * values are not part of this call: merge their attention with the returned
 * LSE.
 *   q    [B][num_q_tokens][num_q_heads][head_dim] (cache dtype), post-RoPE;
 *   o    [B][num_q_tokens][num_q_heads][head_dim] fp32;
 *   lse  [B][num_q_tokens][num_q_heads] fp32 (natural log).
 * Everything else as spicy_decode_attn_shared (shared_prefix_pages = 0 for
 * none).  On bf16 caches the (token, query head) rows of one KV head fill the
 * 16 MFMA columns, so each key and value byte loaded serves up to 16 rows of
 * any tokens; a KV head with more than 16 rows per sequence is processed in
 * several row tiles.  num_q_tokens = 1 is spicy_decode_attn_shared.
 * Workspace: >= spicy_decode_multi_workspace_bytes(...) with the same
 *   arguments.
 * Errors: those of spicy_decode_attn_shared; SPICY_ERR_ARG if num_q_tokens < 1,
 *   SPICY_ERR_UNSUPPORTED if B * num_q_tokens > 65535. */
spicy_status spicy_decode_attn_multi(const spicy_cache* cache,   /* host struct */
                                     const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                                     const int32_t* page_table, int32_t max_pages_per_seq,
                                     const int32_t* lengths, int32_t B, int32_t shared_prefix_pages,
                                     float* o, float* lse, void* workspace, size_t workspace_bytes,
                                     int32_t num_splits, void* stream);

/* ------------------------------------------------------------------------
 * spicy_decode_attn_multi_noalloc — spicy_decode_attn_multi for callers that
 * cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace and calls no
 * allocating routine: the per-row tickets and the partials live in one
 * file-scope device array of the library, spicy_decode_noalloc_max_bytes()
 * bytes on each GPU the library runs on (held until the process ends; its
 * tickets start at zero and every completed call leaves them at zero).
 * Same arguments, results, plan and kernels as spicy_decode_attn_multi,
 * without workspace and workspace_bytes, plus:
 *   device_error  int32 (device) or NULL: the sticky device error word (the
 *                 SPICY_DEVERR_* bits are OR-ed into it; the caller clears
 *                 it); NULL drops device errors.
 * The stream must belong to the current device.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give wrong results; order them.
 * Errors: those of spicy_decode_attn_multi without the workspace ones;
 *   SPICY_ERR_CAPACITY if B x num_q_tokens x num_q_heads > 65536 or the
 *   call's partials do not fit the array; SPICY_ERR_ARG if the stream is on
 *   another device; SPICY_ERR_HIP if the array's address cannot be found.
 * ------------------------------------------------------------------------ */
size_t spicy_decode_noalloc_max_bytes(void);

spicy_status spicy_decode_attn_multi_noalloc(const spicy_cache* cache,   /* host struct */
                                             const void* q, int32_t num_q_tokens, int32_t num_q_heads,
                                             const int32_t* page_table, int32_t max_pages_per_seq,
                                             const int32_t* lengths, int32_t B, int32_t shared_prefix_pages,
                                             float* o, float* lse, int32_t* device_error,
                                             int32_t num_splits, void* stream);

/* Human-readable name of a status code (static string). */
const char* spicy_status_string(spicy_status s);

/* ------------------------------------------------------------------------
 * Per-step policy: the segment partition and the protection mask of a chunk,
 * from the chunk itself, for a following spicy_coarsen call.
 *
 * Equal-Variation KV Cache page, "Mathematical statement" (breakpoints at
 * equal increments of cumulative variation, first hitting time) and
 * "Implementation notes" (feature z_t = P [k_t; v_t] with a fixed random
 * projection P, local variation d_t = ||z_t - z_{t-1}||_2, thresholds
 * q_j = j c_T / N, a boundary at the first token whose cumulative variation
 * reaches the next threshold).  SPICY-KV demo page, Claim 2 (exact
 * C-points) and section 1 (sink and recent tokens kept exact); the landmark
 * rule is the largest key norms per (sequence, KV head).
 *
 * Arithmetic (integer, so the result is exact whatever the order):
 *   fix(x) = x * 2^16 rounded half to even, clamped to [-2^28, 2^28],
 *            NaN -> 0, for each bf16 element x of k_t and v_t;
 *   z_t[r] = sum over row r of P of (+-1) * fix(x_t[c]), with
 *            x_t = [k_t; v_t], each in [H_kv][head_dim] order, so columns
 *            [0, H d) are keys and [H d, 2 H d) values;
 *   d_t    = floor(sqrt(sum_r (z_t[r] - z_{t-1}[r])^2)), 0 at a sequence's
 *            first token;  C_t = d_0 + ... + d_t;
 *   b_j    = min{t : C_t >= floor(j C_T / N)}, j = 1 .. N-1, b_0 = 0,
 *            b_N = T: sequence b gets exactly N segment slots
 *            [b_j, b_{j+1}), empty ones included (spicy_coarsen gives an empty
 *            segment no entry);
 *   mask   = 1 for the first `sink` and the last `recent` tokens of each
 *            sequence, and for the n_landmarks largest
 *            sum_i fix(k_t,h[i])^2 among the others, per KV head h, ties to
 *            the lower position.
 *
 * P is given as signed column lists: row r (r < proj_rows <= 16) has the
 * entries proj_idx[proj_ptr[r] .. proj_ptr[r+1]), value c + 1 for +1 at
 * column c and -(c + 1) for -1; proj_idx has proj_nnz entries.  All device.
 *
 * Inputs (device): k_pre, v [total_tokens][H_kv][head_dim] bf16;
 *   seq_offsets [B+1] (sequence b = tokens [seq_offsets[b], seq_offsets[b+1])).
 * Outputs (device, caller-allocated): seg_offsets [B * n_segments + 1] (global
 *   token indices), seq_seg_ptr [B+1] = b * n_segments, protected_mask
 *   [total_tokens][H_kv] (1 = keep exact), ready to be passed to spicy_coarsen
 *   with n_seg = B * n_segments.  B = 0 writes nothing.
 * Workspace: device, >= spicy_policy_workspace_bytes(total_tokens, H_kv),
 *   first int32 = sticky device error word (SPICY_DEVERR_POLICY).  On return
 *   it holds d_t as int64 [total_tokens] from byte SPICY_WORKSPACE_HEADER:
 *   the token weights spicy_coarsen_weighted takes.
 * Errors: SPICY_ERR_ARG (null pointer, negative count, n_segments < 1,
 *   proj_rows outside [1, 16], B * n_segments + 1 > INT32_MAX),
 *   SPICY_ERR_UNSUPPORTED (dtype not bf16, head_dim not 64/128, H_kv outside
 *   [1, 16]), SPICY_ERR_CAPACITY (workspace too small), SPICY_ERR_HIP.
 * ------------------------------------------------------------------------ */
size_t spicy_policy_workspace_bytes(int32_t total_tokens, int32_t num_kv_heads);

spicy_status spicy_policy(const void* k_pre, const void* v, int32_t total_tokens,
                          int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                          const int32_t* seq_offsets, int32_t B,
                          const int32_t* proj_ptr, const int32_t* proj_idx, int32_t proj_rows,
                          int32_t proj_nnz, int32_t n_segments, int32_t n_landmarks,
                          int32_t sink, int32_t recent,
                          int32_t* seg_offsets, int32_t* seq_seg_ptr, uint8_t* protected_mask,
                          void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPICY_H */
