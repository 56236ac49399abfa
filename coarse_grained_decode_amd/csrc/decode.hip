// SPICY-KV decode attention on gfx950: one launch, split-K over 16-entry pages
// with the log-sum-exp combine fused in.
//
// Logit (SPICY-KV demo page, section "2. FlashAttention-2/3 & PagedAttention
// Online-Softmax Kernel Fusion"; Claim 3):
//     s = q.k / sqrt(d) + alpha + |q|^2 * beta
// followed by an ordinary online softmax.  With the diagonal closure (the
// cache carries a per-dimension variance s2 per entry) the last term is
// sum_i q_i^2 s2_i / (2d) instead.  Everything runs in base 2:
// s2 = s * log2(e), so p = exp2(s2 - m2) and LSE = ln2 * (m2 + log2 l).
//
// bf16 caches (decode_mfma_kernel).  A query "tile" is up to 16 query rows
// that attend to the same KV head.  The rows fill the 16 columns of the MFMA
// tiles, so each key and value byte loaded serves all of them:
//   S^T[16 entries x 16 rows] = K_page[16 x d] . Q^T[d x 16]
//       d/32 x v_mfma_f32_16x16x32_bf16, K rows straight from the page
//       (lane l holds entry l%16, 8 dims of each 32-dim chunk)
//   the accumulator layout of S^T (lane l: entries 4(l/16)+j, row l%16) is
//   exactly the B operand of the next product, so the probabilities go from
//   exp2 to bf16 to MFMA without any lane exchange:
//   O^T[d x 16 rows] += V^T_page[d x 16 entries] . P^T[16 entries x 16 rows]
//       d/16 x v_mfma_f32_16x16x16_bf16.  Values are stored like keys (rows
//       cut in 8-dim groups, so the coarsening writes 16-byte pieces and the
//       operand of a 32-dim chunk of all 16 slots is one sequential 1 KB
//       load); each 32-dim chunk becomes two V^T operand tiles through two MFMAs with
//       0/1 selector matrices (exact), whose accumulator layout is the A
//       operand layout the product needs.
//   diagonal closure: C^T[16 entries x 16 rows] = S2_page . (Q^2)^T, the
//       variance pages loaded like K; q^2 (16 significant bits) is split
//       into two bf16 terms hi + lo that hold it exactly, so the product is
//       d/16 MFMAs with fp32 accumulation of exact bf16 products.
//
// Work decomposition.  A "unit" is a set of query rows and the pages they
// read:
//   shared prefix (only when the caller declares one): a tile-set of the
//       B x n_q x G (sequence, token, query head) rows of one KV head and the
//       first P logical pages, which every sequence maps to the same physical
//       pages;
//   private: a tile-set of the n_q x G rows of one (sequence, KV head) and
//       its pages [P, ceil(length / 16)).
// A unit's pages are cut into page groups; one workgroup of WPG wavefronts
// takes one (unit, group) and its wavefronts take the group's pages in turn
// (wavefront w: pages w, w + WPG, ...), each prefetching its pages NBUF deep
// in registers.  The wavefronts' online-softmax states then merge through LDS
// in a fixed pairwise tree, so a workgroup yields one partial per row.  The
// prefix groups of one (group, KV head) are placed on one XCD, so HBM
// delivers each shared page once to that XCD's L2.
//
// Finishing a row (no second launch).  A row whose unit set has a single
// group in total (prefix groups + its sequence's private groups) is written
// directly as O and LSE.  Otherwise each group writes its partial (running
// max, sum, unnormalised output) to its slot with device-coherent stores
// (sc1: they write through this XCD's L2), waits for them to complete, and
// takes a ticket from the row's counter with a device-scope atomic; the group
// that takes the last ticket reads the row's partials with device-coherent
// loads, merges them by log-sum-exp in slot order (so the result does not
// depend on arrival order), writes O and LSE, and puts the counter back to
// zero for the next call.  Nothing waits on another workgroup.
//
// fp32 caches (decode_f32_kernel): a plain VALU kernel, one workgroup of four
// wavefronts per (sequence, token, query head, page group), lanes = 16
// entries x 4 quarter-rows, the same merge and finishing.  It has no
// shared-prefix role: the host gives it every page as private.
#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;                  // MI355X: workgroups go round-robin over 8 XCDs
constexpr int kF32Waves = 4;              // wavefronts per workgroup of the fp32 kernel

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Clamp a sequence's length (as read from lengths[]) to what its page table
// row can address.
__device__ __forceinline__ int32_t check_length(const DecodeArgs& a, int32_t len) {
    if (len < 0) {
        raise_err(a.err, SPICY_DEVERR_LENGTH);
        len = 0;
    }
    const int64_t cap = static_cast<int64_t>(a.max_pages) * kPage;
    if (len > cap) {
        raise_err(a.err, SPICY_DEVERR_CAPACITY);
        len = static_cast<int32_t>(cap);
    }
    return len;
}

// Partials a row of sequence b receives: one per prefix group, and one per
// private group that holds pages of b (at least one, so that a sequence
// without pages still gets its row written).  len: b's checked length.
__device__ __forceinline__ int32_t row_count(const DecodeArgs& a, int32_t len) {
    if (a.priv_groups == 0) return a.prefix_groups;
    const int32_t priv = max(0, (len + kPage - 1) / kPage - a.prefix_pages);
    const int32_t g = (priv + a.priv_chunk - 1) / a.priv_chunk;
    return a.prefix_groups + min(max(g, 1), a.priv_groups);
}

// Device-coherent 8-byte accesses: relaxed atomics at device scope are
// issued with sc1, which writes through and reads past this XCD's L2.
__device__ __forceinline__ void store2_dev(float* p, float x, float y) {
    const uint64_t v = static_cast<uint64_t>(__float_as_uint(x)) | (static_cast<uint64_t>(__float_as_uint(y)) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 load2_dev(const float* p) {
    const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}

// Wait until every store of this wavefront has completed (for sc1 stores:
// reached the device's point of coherence), and keep the compiler from
// moving memory operations across.
__device__ __forceinline__ void stores_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// One ticket of row prow's counter; returns the counter's previous value.
__device__ __forceinline__ int32_t take_ticket(const DecodeArgs& a, int64_t prow) {
    return __hip_atomic_fetch_add(a.ticket + prow, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void reset_ticket(const DecodeArgs& a, int64_t prow) {
    __hip_atomic_store(a.ticket + prow, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool DIAG>
struct PageRegs {
    bf16x8 k[D / 32];      // K rows: entry lane%16, dims 32i + 8(lane/16) .. +8
    bf16x8 v[D / 32];      // V rows, the same way
    bf16x8 s2[DIAG ? D / 32 : 1];   // per-dimension variances, like K (DIAG only)
    bf16x8 ab;             // (alpha, beta) of entries 4(lane/16) .. +4
    bool ok;               // page id was valid (uniform)
};

// Load KV head h of physical page pid, or of page 0 when pid is invalid
// (then r.ok is false and the page is skipped when processed).
template <int D, bool DIAG>
__device__ __forceinline__ void load_page(const DecodeArgs& a, PageRegs<D, DIAG>& r, int32_t pid, int h) {
    constexpr int KC = D / 32;
    const int lane = threadIdx.x % kWave;
    const int row = lane % 16, grp = lane / 16;
    r.ok = pid >= 0 && pid < a.cache.num_pages;
    if (!r.ok) raise_err(a.err, SPICY_DEVERR_PAGE_ID);
    const int64_t ph = static_cast<int64_t>(r.ok ? pid : 0) * a.cache.H + h;
    // chunk i of all 16 slots is 1 KB: one load per lane covers it
    const uint16_t* kp = static_cast<const uint16_t*>(a.cache.k) + ph * kPage * D + slot_elem(row, 8 * grp);
#pragma unroll
    for (int i = 0; i < KC; ++i) r.k[i] = *reinterpret_cast<const bf16x8*>(kp + kPage * kChunk * i);
    const uint16_t* vp = static_cast<const uint16_t*>(a.cache.v) + ph * kPage * D + slot_elem(row, 8 * grp);
#pragma unroll
    for (int i = 0; i < KC; ++i) r.v[i] = *reinterpret_cast<const bf16x8*>(vp + kPage * kChunk * i);
    if constexpr (DIAG) {
        const uint16_t* sp = static_cast<const uint16_t*>(a.cache.s2) + ph * kPage * D + slot_elem(row, 8 * grp);
#pragma unroll
        for (int i = 0; i < KC; ++i) r.s2[i] = *reinterpret_cast<const bf16x8*>(sp + kPage * kChunk * i);
    }
    r.ab = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.cache.ab) + ph * kPage * 2 + 8 * grp);
}

// Online-softmax state of one query tile; lane l serves query row l%16.
template <int D, bool DIAG>
struct Tile {
    static constexpr int KC = D / 32;
    static constexpr int NT = D / 16;
    bf16x8 q[KC];          // B operand of S^T = K Q^T: 8 dims of each 32-dim chunk
    bf16x8 q2h[DIAG ? KC : 1], q2l[DIAG ? KC : 1];   // q^2 = hi + lo, the same layout (DIAG only)
    bf16x8 sel[2];         // B operands [I; 0] and [0; I] (32 x 16) that transpose V
    float c_beta;          // |q|^2 log2(e) of this lane's row
    int32_t len;           // entries of this row's sequence (0 for a padding row)
    int32_t vlen;          // uniform: largest len of the tile
    float m_run, l_run;    // running max (uniform over a row's lanes); this lane's part of the sum
    f32x4 acc[NT];         // O^T: dims 16t + 4(lane/16) + j of row lane%16

    // rowq: this lane's query row (a padding row passes any valid row).  Only
    // issues the loads, unconditionally, so that nothing waits on them here;
    // init() uses them.
    __device__ __forceinline__ void load_q(const uint16_t* rowq) {
        const int grp = (threadIdx.x % kWave) / 16;
#pragma unroll
        for (int i = 0; i < KC; ++i) q[i] = *reinterpret_cast<const bf16x8*>(rowq + 32 * i + 8 * grp);
    }

    // valid: this lane's row is a real query row (else its query is zeroed);
    // length: entries of that row's sequence, 0 for a padding row
    __device__ __forceinline__ void init(bool valid, int32_t length) {
        const int grp = (threadIdx.x % kWave) / 16;
        float n2 = 0.f;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            if (!valid) q[i] = bf16x8{};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = static_cast<float>(q[i][j]);
                n2 += x * x;
                if constexpr (DIAG) {
                    const float x2 = x * x;                         // exact: 16 significant bits
                    const __bf16 hi = static_cast<__bf16>(x2);
                    q2h[i][j] = hi;
                    q2l[i][j] = static_cast<__bf16>(x2 - static_cast<float>(hi));   // exact remainder
                }
            }
        }
        n2 += __shfl_xor(n2, 16);
        n2 += __shfl_xor(n2, 32);
        c_beta = n2 * kLog2e;
        // lane (column c = lane%16, k-group g) holds rows 8g .. 8g+7 of a
        // selector: [I; 0] has a one at row c, [0; I] at row 16 + c
        const int c = threadIdx.x % 16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sel[0][j] = static_cast<__bf16>(8 * grp + j == c ? 1.f : 0.f);
            sel[1][j] = static_cast<__bf16>(8 * grp + j == 16 + c ? 1.f : 0.f);
        }
        len = length;
        int32_t mx = len;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) mx = max(mx, __shfl_xor(mx, o));
        vlen = __builtin_amdgcn_readfirstlane(mx);
        m_run = -__builtin_huge_valf();
        l_run = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // The logits of logical page lp for this tile's rows and the online-softmax
    // update: returns the factor the running output must be scaled by and the
    // probabilities as the B operand of the P.V product.  A row's entries at
    // or past its length get weight zero.
    __device__ __forceinline__ float softmax(const PageRegs<D, DIAG>& r, int32_t lp, s16x4& pk) {
        const int grp = (threadIdx.x % kWave) / 16;
        const float c_dot = kLog2e / sqrtf(static_cast<float>(D));
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KC; ++i) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[i], q[i], s, 0, 0, 0);
        f32x4 cl = {0.f, 0.f, 0.f, 0.f};
        if constexpr (DIAG) {
#pragma unroll
            for (int i = 0; i < KC; ++i) {
                cl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.s2[i], q2h[i], cl, 0, 0, 0);
                cl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.s2[i], q2l[i], cl, 0, 0, 0);
            }
        }
        const int32_t ebase = lp * kPage + 4 * grp;
        float s2[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float alpha = static_cast<float>(r.ab[2 * j]);
            float x;
            if constexpr (DIAG) {
                constexpr float c_cl = kLog2e / (2.f * D);
                x = s[j] * c_dot + (alpha * kLog2e + cl[j] * c_cl);
            } else {
                const float beta = static_cast<float>(r.ab[2 * j + 1]);
                x = s[j] * c_dot + (alpha * kLog2e + beta * c_beta);
            }
            s2[j] = (ebase + j < len) ? x : -__builtin_huge_valf();
        }
        float pm = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
        pm = fmaxf(pm, __shfl_xor(pm, 16));
        pm = fmaxf(pm, __shfl_xor(pm, 32));
        const float m_new = fmaxf(m_run, pm);
        const float msub = (m_new == -__builtin_huge_valf()) ? 0.f : m_new;
        const float scale = fast_exp2(m_run - msub);
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = fast_exp2(s2[j] - msub);
        l_run = l_run * scale + ((p[0] + p[1]) + (p[2] + p[3]));
        m_run = m_new;
        const bf16x4 pb = {static_cast<__bf16>(p[0]), static_cast<__bf16>(p[1]),
                           static_cast<__bf16>(p[2]), static_cast<__bf16>(p[3])};
        pk = __builtin_bit_cast(s16x4, pb);
        return scale;
    }

    // Merge another state of the same rows (lane by lane: the other state's
    // lane holds the same row and the same part of the sum and the output).
    __device__ __forceinline__ void merge(float m_b, float l_b, const f32x4 (&acc_b)[NT]) {
        const float m_new = fmaxf(m_run, m_b);
        const float msub = (m_new == -__builtin_huge_valf()) ? 0.f : m_new;
        const float sa = fast_exp2(m_run - msub);
        const float sb = fast_exp2(m_b - msub);
        l_run = l_run * sa + l_b * sb;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = acc[t] * sa + acc_b[t] * sb;
        m_run = m_new;
    }
};

// Fold logical page lp into the first `ntile` (uniform, >= 1) of a
// wavefront's TPW tiles; a page whose id was invalid is skipped.  The V^T
// operand tiles are formed once and serve every tile: V_chunk (16 entries x
// 32 dims, loaded as an A operand like K) times a selector gives V^T of 16 of
// its dims in the accumulator layout (lane: entries 4g .. 4g+3 of dim
// lane%16), exactly the A operand layout of O^T += V^T P^T.  The products
// are exact: one bf16 term per output, the rest zeros.  vlen: the largest
// length of the tiles' rows; slots at or past it may hold anything, so their
// values are zeroed (0 * NaN must not poison the product).
template <int D, bool DIAG, int TPW>
__device__ __forceinline__ void fold_page(Tile<D, DIAG> (&T)[TPW], int ntile, const PageRegs<D, DIAG>& r,
                                          int32_t lp, int32_t vlen) {
    constexpr int KC = D / 32;
    if (!r.ok) return;
    s16x4 pk[TPW];
    float scale[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k)
        if (k < ntile) scale[k] = T[k].softmax(r, lp, pk[k]);
    const int grp = (threadIdx.x % kWave) / 16;
    const int32_t ebase = lp * kPage + 4 * grp;
    const bool partial = lp * kPage + kPage > vlen;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
#pragma unroll
        for (int hsel = 0; hsel < 2; ++hsel) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 vtf = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.v[i], T[0].sel[hsel], z, 0, 0, 0);
            uint32_t u[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u[j] = __float_as_uint(vtf[j]);
                if (partial && ebase + j >= vlen) u[j] = 0;
            }
            const uint32_t w0 = __builtin_amdgcn_perm(u[1], u[0], 0x07060302u);
            const uint32_t w1 = __builtin_amdgcn_perm(u[3], u[2], 0x07060302u);
            const s16x4 vt = __builtin_bit_cast(s16x4, make_uint2(w0, w1));
            const int t = 2 * i + hsel;
#pragma unroll
            for (int k = 0; k < TPW; ++k) {
                if (k < ntile) {
                    T[k].acc[t] *= scale[k];
                    T[k].acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pk[k], T[k].acc[t], 0, 0, 0);
                }
            }
        }
    }
}

// The end of a workgroup, for one tile of query rows (every wavefront takes
// part; lane l of a wavefront: row l%16).  Each wavefront's online-softmax
// state of the tile goes to LDS; wavefront w then merges column block w
// (dims 16w .. 16w+15, lane: dims 16w + 4(l/16) .. +4) over the WPG states in
// a fixed order, so the result does not depend on timing, and writes that
// block: as the row's O when the row has a single group (cnt == 1), else as
// this group's partial (slot `slot`, device-coherent stores).  After a
// barrier wavefront 0 takes one ticket per shared row; the rows whose last
// ticket this group took are merged from all their partials (in slot order,
// each wavefront its block), written, and their counters reset.
// valid: the lane's row is a query row; prow: its row index (sequence-token
// * H_q + query head); cnt: the partials the row receives.
template <int D, int WPG>
struct Finish {
    static constexpr int NT = D / 16;
    static constexpr int BPW = (NT + WPG - 1) / WPG;   // column blocks per wavefront: t = wave + WPG i
    f32x4 acc[WPG][NT][kWave];
    float2 ml[WPG][kWave];
    int32_t fin[kWave];              // per row (lanes 0..15): slots to merge, 0 = not finished here

    template <bool DIAG>
    __device__ __forceinline__ void run(const DecodeArgs& a, const Tile<D, DIAG>& T, bool valid, int64_t prow,
                                        int32_t cnt, int slot) {
        constexpr int SB = 8;                // slots whose loads are in flight together
        const int lane = threadIdx.x % kWave;
        const int wave = threadIdx.x / kWave;
        const int row = lane % 16, grp = lane / 16;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[wave][t][lane] = T.acc[t];
        ml[wave][lane] = make_float2(T.m_run, T.l_run);
        __syncthreads();
        // every wavefront: the merged max and the row's sum (the sum over
        // lane groups of the merged per-lane parts)
        float M = -__builtin_huge_valf();
#pragma unroll
        for (int w = 0; w < WPG; ++w) M = fmaxf(M, ml[w][lane].x);
        const float msub = (M == -__builtin_huge_valf()) ? 0.f : M;
        float sc[WPG];
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < WPG; ++w) {
            sc[w] = fast_exp2(ml[w][lane].x - msub);
            L += sc[w] * ml[w][lane].y;
        }
        L += __shfl_xor(L, 16);
        L += __shfl_xor(L, 32);
        const bool shared = valid && cnt > 1;
        const int64_t base = prow * a.slots;
#pragma unroll
        for (int i = 0; i < BPW; ++i) {
            const int t = wave + WPG * i;
            if (t < NT) {
                f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < WPG; ++w) o += sc[w] * acc[w][t][lane];
                if (valid && cnt == 1) {
                    const bool live = L > 0.f;
                    *reinterpret_cast<f32x4*>(a.o + prow * D + 16 * t + 4 * grp) = live ? o * (1.f / L) : f32x4{};
                }
                if (shared) {
                    float* po = a.part_o + (base + slot) * D + 16 * t + 4 * grp;
                    store2_dev(po, o[0], o[1]);
                    store2_dev(po + 2, o[2], o[3]);
                }
            }
        }
        if (wave == 0 && grp == 0) {
            if (valid && cnt == 1) a.lse[prow] = L > 0.f ? (msub + __log2f(L)) * kLn2 : -__builtin_huge_valf();
            if (shared) store2_dev(a.part_ml + 2 * (base + slot), M, L);
        }
        stores_complete();
        __syncthreads();
        if (wave == 0) {
            int32_t old = 0;
            if (shared && grp == 0) old = take_ticket(a, prow);
            if (shared && grp == 0 && old >= cnt) raise_err(a.err, SPICY_DEVERR_TICKET);
            if (lane < 16) fin[lane] = (shared && old == cnt - 1) ? cnt : 0;
        }
        __syncthreads();
        const int32_t n_row = fin[row];
        int32_t n = n_row;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) n = max(n, __shfl_xor(n, o));
        if (n == 0 || wave >= NT) return;        // uniform over the workgroup / this wavefront
        // merge the finished rows' partials: this wavefront's blocks of each
        float M2 = -__builtin_huge_valf(), L2 = 0.f;
        f32x4 o2[BPW];
#pragma unroll
        for (int i = 0; i < BPW; ++i) o2[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < n; s0 += SB) {
            float2 pm[SB];
            f32x4 po[SB][BPW];
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const bool ok = s0 + u < n_row;
                const int64_t ps = base + (ok ? s0 + u : 0);
                pm[u] = ok ? load2_dev(a.part_ml + 2 * ps) : make_float2(-__builtin_huge_valf(), 0.f);
#pragma unroll
                for (int i = 0; i < BPW; ++i) {
                    const int t = wave + WPG * i;
                    const float* src = a.part_o + ps * D + 16 * t + 4 * grp;
                    const bool okt = ok && t < NT;
                    const float2 x = okt ? load2_dev(src) : make_float2(0.f, 0.f);
                    const float2 y = okt ? load2_dev(src + 2) : make_float2(0.f, 0.f);
                    po[u][i] = f32x4{x.x, x.y, y.x, y.y};
                }
            }
            float mc = M2;
#pragma unroll
            for (int u = 0; u < SB; ++u) mc = fmaxf(mc, pm[u].x);
            const float ms = (mc == -__builtin_huge_valf()) ? 0.f : mc;
            const float scale = fast_exp2(M2 - ms);
            L2 *= scale;
#pragma unroll
            for (int i = 0; i < BPW; ++i) o2[i] *= scale;
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const float w = fast_exp2(pm[u].x - ms);     // 0 for a slot past the row's count
                L2 += w * pm[u].y;
#pragma unroll
                for (int i = 0; i < BPW; ++i) o2[i] += w * po[u][i];
            }
            M2 = mc;
        }
        if (n_row > 0) {
            const bool live = L2 > 0.f;
#pragma unroll
            for (int i = 0; i < BPW; ++i) {
                const int t = wave + WPG * i;
                if (t < NT)
                    *reinterpret_cast<f32x4*>(a.o + prow * D + 16 * t + 4 * grp) = live ? o2[i] * (1.f / L2) : f32x4{};
            }
            if (wave == 0 && grp == 0) {
                const float ms = (M2 == -__builtin_huge_valf()) ? 0.f : M2;
                a.lse[prow] = live ? (ms + __log2f(L2)) * kLn2 : -__builtin_huge_valf();
                reset_ticket(a, prow);
            }
        }
    }
};

}  // namespace

// ---------------------------------------------------------------- bf16 MFMA

// Workgroup w (linear over a 2-D grid) of WPG wavefronts takes one (unit,
// page group):
//   w < prefix_blocks: shared-prefix role.  w is first remapped so that the
//       prefix_blocks / 8 consecutive work items of each XCD are contiguous;
//       then (group c, KV head h, tile-set ts): the rows of tiles
//       TPW ts .. TPW ts + TPW-1 of the B x n_q x G rows of h, the pages
//       [c prefix_chunk, ...) of the prefix, with ids from sequence 0's table
//       row.  The tile-sets of one (c, h) are consecutive, so they share an
//       XCD's L2.
//   otherwise: private role, (group s, sequence b, tile-set ts, KV head h),
//       h fastest and s slowest: the rows of tiles TPW ts .. of (b, h), pages
//       [P + s priv_chunk, ...) of sequence b.  A group past b's pages does
//       nothing (group 0 always takes part, so that every row is written).
// Wavefront w of the workgroup takes the group's pages w, w + WPG, ...  Page
// ids come 64 of the wavefront's pages at a time with one vector load, then
// each page's id is read out of its lane (uniform).  Pages past the
// wavefront's last load its last page again (every load is unconditional, so
// each wait covers exactly one page); they are never processed.
template <int D, int NBUF, bool DIAG, int TPW, int WPG>
__global__ __launch_bounds__(WPG * kWave, 8 / WPG) void decode_mfma_kernel(DecodeArgs a) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int row = lane % 16;
    const int H = a.cache.H;
    const int G = a.H_q / H;
    int64_t blk = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;

    int h, ts, slot, ntile;
    int32_t p0, p1;
    int32_t id_end;        // page-id entries the table row holds
    const int32_t* table;
    int64_t prow[TPW];     // this lane's row (sequence-token * H_q + query head) in tile k
    int32_t raw_len[TPW];  // the length of that row's sequence as read, checked below
    bool row_valid[TPW];
    const bool prefix_role = blk < a.prefix_blocks;
    // The query rows and the first window of page ids do not depend on the
    // length: each role issues their loads together with it, so a wavefront
    // waits one memory round trip before its first pages are requested.
    Tile<D, DIAG> T[TPW];
    int32_t ids;
    int64_t prow0;         // a valid query row of the workgroup's KV head
    auto issue_loads = [&]() {
#pragma unroll
        for (int k = 0; k < TPW; ++k)
            T[k].load_q(static_cast<const uint16_t*>(a.q) + (row_valid[k] ? prow[k] : prow0) * D);
        const int32_t pg = p0 + wave + WPG * lane;
        ids = pg < min(p1, id_end) ? table[pg] : 0;
        // keep the compiler from sinking those loads below the length checks
        asm volatile("" ::: "memory");
    };
    if (prefix_role) {
        const int per_xcd = a.prefix_blocks / kXcds;      // prefix_blocks is a multiple of 8
        int w = static_cast<int>(blk % kXcds) * per_xcd + static_cast<int>(blk / kXcds);
        ts = w % a.prefix_sets;
        w /= a.prefix_sets;
        h = w % H;
        const int c = w / H;
        if (c >= a.prefix_groups) return;                 // padding workgroup
        const int rows = a.B * a.n_q * G;                 // rows (sequence, token, query head)
        ntile = min(TPW, (rows - TPW * ts * 16 + 15) / 16);
        slot = c;
        p0 = c * a.prefix_chunk;
        p1 = min(p0 + a.prefix_chunk, a.prefix_pages);
        id_end = a.prefix_pages;
        table = a.page_table;
        prow0 = static_cast<int64_t>(h) * G;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int r = (TPW * ts + k) * 16 + row;
            row_valid[k] = r < rows;
            const int rq = row_valid[k] ? r : 0;
            const int bq = rq / (a.n_q * G);                // sequence
            const int vq = rq / G;                          // sequence * n_q + token
            prow[k] = static_cast<int64_t>(vq) * a.H_q + static_cast<int64_t>(h) * G + rq % G;
            raw_len[k] = row_valid[k] ? a.lengths[bq] : 0;
        }
        issue_loads();
    } else {
        // the split slowest and the KV head fastest: workgroups go round-robin
        // over the XCDs, and this way each XCD gets the same splits of
        // sequences spread over the batch (a split-fastest order would give
        // one XCD every sequence's first, fullest split)
        blk -= a.prefix_blocks;
        const int64_t units = static_cast<int64_t>(a.B) * H * a.priv_sets;
        const int s = static_cast<int>(blk / units);
        if (s >= a.priv_groups) return;
        blk %= units;
        h = static_cast<int>(blk % H);
        blk /= H;
        ts = static_cast<int>(blk % a.priv_sets);
        const int64_t b = blk / a.priv_sets;
        ntile = min(TPW, a.priv_tiles - TPW * ts);
        slot = a.prefix_groups + s;
        p0 = a.prefix_pages + s * a.priv_chunk;
        p1 = p0 + a.priv_chunk;                           // clamped to the length below
        id_end = a.max_pages;
        table = a.page_table + b * a.max_pages;
        prow0 = b * a.n_q * a.H_q + static_cast<int64_t>(h) * G;
        // the tiles' rows: (token, query head) pairs r = token * G + g of this KV head
        const int32_t lb = a.lengths[b];
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int r = (TPW * ts + k) * 16 + row;
            row_valid[k] = r < a.n_q * G;
            const int rq = row_valid[k] ? r : 0;
            prow[k] = (b * a.n_q + rq / G) * a.H_q + static_cast<int64_t>(h) * G + rq % G;
            raw_len[k] = lb;
        }
        issue_loads();
    }
    // the length of each row's sequence; in the private role every lane of
    // the workgroup holds the one sequence's length (padding rows included),
    // so the page range below is uniform
    int32_t len[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) len[k] = (prefix_role && !row_valid[k]) ? 0 : check_length(a, raw_len[k]);
    if (!prefix_role) {
        p1 = min(p1, (len[0] + kPage - 1) / kPage);
        if (p0 >= p1 && slot != a.prefix_groups) return;  // a group past the sequence's pages
    }
    int32_t vlen = 0;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        T[k].init(row_valid[k], row_valid[k] ? len[k] : 0);
        if (k < ntile) vlen = max(vlen, T[k].vlen);
    }

    // This wavefront's pages: p0 + wave + WPG i, i < nmine, in windows of 64
    // (lane i of a window holds the id of its i-th page).
    const int32_t nmine = p1 > p0 + wave ? (p1 - p0 - wave + WPG - 1) / WPG : 0;
    PageRegs<D, DIAG> buf[NBUF];
    for (int32_t i0 = 0; i0 < nmine; i0 += kWave) {
        const int32_t i1 = min(i0 + kWave, nmine);
        if (i0 != 0) ids = (i0 + lane < i1) ? table[p0 + wave + WPG * (i0 + lane)] : 0;
        auto load = [&](PageRegs<D, DIAG>& r, int32_t i) {
            load_page<D, DIAG>(a, r, __builtin_amdgcn_readlane(ids, min(i, i1 - 1) - i0), h);
        };
#pragma unroll
        for (int i = 0; i < NBUF; ++i) load(buf[i], i0 + i);
        for (int32_t i = i0; i < i1; i += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                if (i + u < i1) fold_page<D, DIAG, TPW>(T, ntile, buf[u], p0 + wave + WPG * (i + u), vlen);
                load(buf[u], i + u + NBUF);
            }
        }
    }

    // The KV head 0 prefix groups check that the sequences of their tiles map
    // the group's pages like sequence 0 (each wavefront its own pages).
    if (prefix_role && h == 0) {
        const int rows = a.B * a.n_q * G;
        const int b_first = (TPW * ts * 16) / (a.n_q * G);
        const int b_last = min(rows - 1, (TPW * ts + ntile) * 16 - 1) / (a.n_q * G);
        const int n = (b_last - b_first + 1) * nmine;
        bool bad = false;
        for (int i = lane; i < n; i += kWave) {
            const int32_t pg = p0 + wave + WPG * (i % nmine);
            const int64_t bb = b_first + i / nmine;
            bad |= a.page_table[bb * a.max_pages + pg] != a.page_table[pg];
        }
        if (bad) raise_err(a.err, SPICY_DEVERR_SHARED);
    }

    // The workgroup's rows, one tile at a time through the same LDS.
    __shared__ Finish<D, WPG> fs;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        if (k < ntile) {
            if (k > 0) __syncthreads();          // the previous tile's LDS reads are done
            const int32_t cnt = row_valid[k] ? row_count(a, len[k]) : 0;
            fs.run(a, T[k], row_valid[k], prow[k], cnt, slot);
        }
    }
}

// -------------------------------------------------------------- fp32 VALU

// Workgroup (group s, query head hq, sequence-token bv) of four wavefronts:
// the group's private pages [s priv_chunk, ...) of sequence bv / n_q, taken
// in turn by the wavefronts, merged through LDS, then finished like the MFMA
// kernel's rows.
template <int D>
__global__ __launch_bounds__(kF32Waves * kWave) void decode_f32_kernel(DecodeArgs a) {
    constexpr int QD = D / 4;          // dims per quarter-row
    constexpr int DL = D / kWave;      // output dims per lane
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int ent = lane / 4;
    const int qtr = lane % 4;
    const int s = blockIdx.x;
    const int hq = blockIdx.y;
    const int bv = blockIdx.z;                 // sequence * n_q + token
    const int b = bv / a.n_q;
    const int H = a.cache.H;
    const int G = a.H_q / H;
    const int h = hq / G;

    const int32_t len = check_length(a, a.lengths[b]);
    const int32_t npages = (len + kPage - 1) / kPage;
    const int32_t p0 = s * a.priv_chunk;
    const int32_t p1 = min(p0 + a.priv_chunk, npages);
    if (p0 >= p1 && s != 0) return;            // a group past the sequence's pages (uniform)

    const float* qrow = static_cast<const float*>(a.q) + (static_cast<int64_t>(bv) * a.H_q + hq) * D;
    float qv[QD];
    float n2 = 0.f;
#pragma unroll
    for (int i = 0; i < QD; ++i) {
        qv[i] = qrow[qtr * QD + i];
        n2 += qv[i] * qv[i];
    }
    n2 += __shfl_xor(n2, 1);
    n2 += __shfl_xor(n2, 2);
    const float c_dot = kLog2e / sqrtf(static_cast<float>(D));
    const float c_beta = n2 * kLog2e;
    const float* s2pool = static_cast<const float*>(a.cache.s2);   // diagonal closure when set (uniform)

    const float* kpool = static_cast<const float*>(a.cache.k);
    const float* vpool = static_cast<const float*>(a.cache.v);
    const float* abpool = static_cast<const float*>(a.cache.ab);
    const int32_t* table = a.page_table + static_cast<int64_t>(b) * a.max_pages;

    float m_run = -__builtin_huge_valf();
    float l_run = 0.f;
    float acc[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] = 0.f;

    for (int32_t lp = p0 + wave; lp < p1; lp += kF32Waves) {
        const int32_t pid = table[lp];
        if (pid < 0 || pid >= a.cache.num_pages) {
            raise_err(a.err, SPICY_DEVERR_PAGE_ID);
            continue;
        }
        const int64_t ph = static_cast<int64_t>(pid) * H + h;
        const float* kpage = kpool + ph * kPage * D;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < QD; ++i) dot += qv[i] * kpage[slot_elem(ent, qtr * QD + i)];
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const float alpha = abpool[(ph * kPage + ent) * 2 + 0];
        const float beta = abpool[(ph * kPage + ent) * 2 + 1];
        float closure = beta * c_beta;
        if (s2pool) {
            const float* spage = s2pool + ph * kPage * D;
            float c = 0.f;
#pragma unroll
            for (int i = 0; i < QD; ++i) c += qv[i] * qv[i] * spage[slot_elem(ent, qtr * QD + i)];
            c += __shfl_xor(c, 1);
            c += __shfl_xor(c, 2);
            closure = c * (kLog2e / (2.f * D));
        }
        float s2 = dot * c_dot + (alpha * kLog2e + closure);
        if (lp * kPage + ent >= len) s2 = -__builtin_huge_valf();
        float pm = s2;
#pragma unroll
        for (int o = 4; o < kWave; o <<= 1) pm = fmaxf(pm, __shfl_xor(pm, o));
        const float m_new = fmaxf(m_run, pm);
        const float msub = (m_new == -__builtin_huge_valf()) ? 0.f : m_new;
        const float scale = fast_exp2(m_run - msub);
        const float p = fast_exp2(s2 - msub);
        l_run = l_run * scale + (qtr == 0 ? p : 0.f);
        m_run = m_new;
        const float* vpage = vpool + ph * kPage * D;
#pragma unroll
        for (int j = 0; j < DL; ++j) {
            float o = acc[j] * scale;
#pragma unroll
            for (int e = 0; e < kPage; ++e) {
                const float pe = __shfl(p, 4 * e);
                if (lp * kPage + e < len) o += pe * vpage[slot_elem(e, lane + kWave * j)];
            }
            acc[j] = o;
        }
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) l_run += __shfl_xor(l_run, o);

    // merge the four wavefronts (fixed pairs) through LDS
    __shared__ float red[kF32Waves / 2][DL + 2][kWave];
#pragma unroll
    for (int half = kF32Waves / 2; half >= 1; half /= 2) {
        if (wave >= half && wave < 2 * half) {
#pragma unroll
            for (int j = 0; j < DL; ++j) red[wave - half][j][lane] = acc[j];
            red[wave - half][DL][lane] = m_run;
            red[wave - half][DL + 1][lane] = l_run;
        }
        __syncthreads();
        if (wave < half) {
            const float m_b = red[wave][DL][lane], l_b = red[wave][DL + 1][lane];
            const float m_new = fmaxf(m_run, m_b);
            const float msub = (m_new == -__builtin_huge_valf()) ? 0.f : m_new;
            const float sa = fast_exp2(m_run - msub), sb = fast_exp2(m_b - msub);
            l_run = l_run * sa + l_b * sb;
#pragma unroll
            for (int j = 0; j < DL; ++j) acc[j] = acc[j] * sa + red[wave][j][lane] * sb;
            m_run = m_new;
        }
        if (half > 1) __syncthreads();
    }
    if (wave != 0) return;

    const int64_t prow = static_cast<int64_t>(bv) * a.H_q + hq;
    const int32_t cnt = row_count(a, len);
    float* orow = a.o + prow * D;
    if (cnt == 1) {
        const bool live = l_run > 0.f;
        const float inv = live ? 1.f / l_run : 0.f;
#pragma unroll
        for (int j = 0; j < DL; ++j) orow[lane + kWave * j] = live ? acc[j] * inv : 0.f;
        if (lane == 0) {
            const float msub = (m_run == -__builtin_huge_valf()) ? 0.f : m_run;
            a.lse[prow] = live ? (msub + __log2f(l_run)) * kLn2 : -__builtin_huge_valf();
        }
        return;
    }
    const int64_t base = prow * a.slots;
    float* po = a.part_o + (base + a.prefix_groups + s) * D;
#pragma unroll
    for (int j = 0; j < DL; ++j)
        __hip_atomic_store(po + lane + kWave * j, acc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) store2_dev(a.part_ml + 2 * (base + a.prefix_groups + s), m_run, l_run);
    stores_complete();
    int32_t old = lane == 0 ? take_ticket(a, prow) : 0;
    old = __shfl(old, 0);
    if (old >= cnt) raise_err(a.err, SPICY_DEVERR_TICKET);
    if (old != cnt - 1) return;
    float M = -__builtin_huge_valf(), L = 0.f;
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] = 0.f;
    for (int sl = 0; sl < cnt; ++sl) {
        const float2 ml = load2_dev(a.part_ml + 2 * (base + sl));
        float ov[DL];
#pragma unroll
        for (int j = 0; j < DL; ++j)
            ov[j] = __hip_atomic_load(a.part_o + (base + sl) * D + lane + kWave * j, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        const float mc = fmaxf(M, ml.x);
        const float msub = (mc == -__builtin_huge_valf()) ? 0.f : mc;
        const float sa = fast_exp2(M - msub), sb = fast_exp2(ml.x - msub);
        L = L * sa + ml.y * sb;
#pragma unroll
        for (int j = 0; j < DL; ++j) acc[j] = acc[j] * sa + ov[j] * sb;
        M = mc;
    }
    const bool live = L > 0.f;
    const float inv = live ? 1.f / L : 0.f;
#pragma unroll
    for (int j = 0; j < DL; ++j) orow[lane + kWave * j] = live ? acc[j] * inv : 0.f;
    if (lane == 0) {
        const float msub = (M == -__builtin_huge_valf()) ? 0.f : M;
        a.lse[prow] = live ? (msub + __log2f(L)) * kLn2 : -__builtin_huge_valf();
        reset_ticket(a, prow);
    }
}

// ------------------------------------------------------------------ launch

constexpr int kNbuf = 2;                  // one tile per wavefront (three pages in flight were slower)
constexpr int kNbufPair = 2;              // two tiles per wavefront: their state takes a page's registers
constexpr int kNbufDiag = 2;              // the variance pages add a third page-sized load
constexpr int64_t kMaxGridX = 65536;

// Grid of the bf16 kernel with TPW tiles per wavefront: the shared-prefix
// workgroups (a multiple of 8, see the XCD remap), then the private ones.
template <int TPW>
static dim3 mfma_grid(DecodeArgs& a) {
    const int G = a.H_q / a.cache.H;
    const int tiles = (a.B * a.n_q * G + 15) / 16;
    a.prefix_sets = (tiles + TPW - 1) / TPW;
    const int64_t pb = static_cast<int64_t>(a.prefix_groups) * a.cache.H * a.prefix_sets;
    a.prefix_blocks = static_cast<int32_t>((pb + kXcds - 1) / kXcds * kXcds);
    a.priv_sets = (a.priv_tiles + TPW - 1) / TPW;
    const int64_t nblk = a.prefix_blocks + static_cast<int64_t>(a.priv_groups) * a.priv_sets * a.cache.H * a.B;
    const int64_t gx = nblk < kMaxGridX ? nblk : kMaxGridX;
    const int64_t gy = (nblk + gx - 1) / gx;
    return dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
}

template <int D, int NBUF, bool DIAG, int TPW>
static void launch_mfma(DecodeArgs& a, hipStream_t stream) {
    const dim3 grid = mfma_grid<TPW>(a);
    if (a.wpg == 4)
        hipLaunchKernelGGL((decode_mfma_kernel<D, NBUF, DIAG, TPW, 4>), grid, dim3(4 * kWave), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<D, NBUF, DIAG, TPW, 8>), grid, dim3(8 * kWave), 0, stream, a);
}

template <int D>
static spicy_status launch_decode_t(const DecodeArgs& a0, int dtype, hipStream_t stream) {
    DecodeArgs a = a0;
    if (dtype == SPICY_BF16) {
        if (a.cache.s2) {
            launch_mfma<D, kNbufDiag, true, 1>(a, stream);
        } else if (a.priv_tiles >= 2) {
            // several query tiles per (sequence, KV head): a wavefront takes two,
            // so each page it loads serves both and its V^T is formed once
            launch_mfma<D, kNbufPair, false, 2>(a, stream);
        } else {
            launch_mfma<D, kNbuf, false, 1>(a, stream);
        }
    } else {
        dim3 grid(a.priv_groups, a.H_q, a.B * a.n_q);
        hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(kF32Waves * kWave), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    return SPICY_OK;
}

spicy_status launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t stream) {
    if (a.B == 0) return SPICY_OK;
    return D == 128 ? launch_decode_t<128>(a, dtype, stream) : launch_decode_t<64>(a, dtype, stream);
}

}  // namespace spicy
