// SPICY-KV decode attention on gfx950: split-K over 16-entry pages + a
// log-sum-exp combine.
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
//       cut in 32-dim chunks, so the coarsening writes 64-byte pieces and a
//       chunk of all 16 slots is one contiguous 1 KB load); each
//       32-dim chunk becomes two V^T operand tiles through two MFMAs with
//       0/1 selector matrices (exact), whose accumulator layout is the A
//       operand layout the product needs.
//   diagonal closure: C^T[16 entries x 16 rows] = S2_page . (Q^2)^T, the
//       variance pages loaded like K; q^2 (16 significant bits) is split
//       into two bf16 terms hi + lo that hold it exactly, so the product is
//       d/16 MFMAs with fp32 accumulation of exact bf16 products.
// One launch holds two kinds of workgroups:
//   split-K: one wavefront per (sequence, KV head, split, query tile).  A
//       query row is a (query token, query head of that KV head) pair: with
//       n_q query tokens per sequence a KV head has n_q x G rows in
//       ceil(n_q G / 16) tiles (one tile of G rows for single-token decode).
//       The wavefronts of a workgroup are the tiles of one split (1, 2 or 4
//       of them), so they read its pages together through one L2; each
//       prefetches its pages NBUF deep in registers.
//   shared prefix (only when the caller declares one): the first P logical
//       pages map to the same physical pages in every sequence.  One wavefront
//       applies a chunk of them to a tile of 16 rows drawn from all sequences
//       (B x n_q x G rows per KV head).  The wavefronts of one (chunk, KV
//       head) run on one XCD, so HBM delivers each shared page once to its L2.
// Both kinds write partials (running max, sum, unnormalised output) to the
// workspace.  combine_kernel merges the partials of each (sequence, query
// token, query head) by log-sum-exp and writes O (fp32) and LSE (natural
// log).
//
// fp32 caches (decode_f32_kernel): a plain VALU kernel, one wavefront per
// (sequence, query head, split), lanes = 16 entries x 4 quarter-rows.  It has
// no shared-prefix role: the host gives it every page as private.
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
constexpr int kWavesPerBlock = 4;
constexpr int kXcds = 8;                  // MI355X: workgroups go round-robin over 8 XCDs

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

__device__ __forceinline__ int32_t checked_length(const DecodeArgs& a, int b) { return check_length(a, a.lengths[b]); }

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
    float m_run, l_run;
    f32x4 acc[NT];

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

    // Finish the row sums (held per lane group) and store this lane's row as
    // partial `slot` of partial row `prow` (= sequence * H_q + query head).
    __device__ __forceinline__ void store(const DecodeArgs& a, bool row_valid, int64_t prow, int slot) {
        const int grp = (threadIdx.x % kWave) / 16;
        float l = l_run;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        if (!row_valid) return;
        const int64_t idx = prow * a.splits + slot;
        if (grp == 0) {
            a.part_ml[2 * idx + 0] = m_run;
            a.part_ml[2 * idx + 1] = l;
        }
        float* po = a.part_o + idx * D + 4 * grp;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(po + 16 * t) = acc[t];
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

}  // namespace

// ---------------------------------------------------------------- bf16 MFMA

// Workgroup w (linear over a 2-D grid) of 4 wavefronts.  Both roles run the
// same page pipeline; they differ in the rows of their tile, the page range
// and where its page ids come from.
//   w < prefix_blocks: shared-prefix role, work item (chunk c, KV head h, tile
//       t).  Tile t holds rows r = 16t .. 16t+15 of the B x G (sequence,
//       query head of h) rows; its pages are [c * prefix_chunk, ...) of the
//       shared prefix, with ids from sequence 0's table row.  w is first
//       remapped so that the prefix_blocks / 8 consecutive work items of each
//       XCD are contiguous: the tiles of one (chunk, KV head) share an L2.
//   otherwise: split-K role, work item (split, KV head h, sequence b).  The
//       tile is the G query heads of h; the pages are private pages
//       [page_begin + split * pages_per_split, ...) of sequence b.
// Pages are prefetched NBUF deep in registers.  Page ids are read 64 at a
// time with one vector load, then each page's id is read out of its lane
// (uniform).  Pages past the window's end load its last page again (every
// load is unconditional, so each wait covers exactly one page); they are
// never processed.
template <int D, int NBUF, bool DIAG, int TPW>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(DecodeArgs a) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int row = lane % 16;
    const int H = a.cache.H;
    const int G = a.H_q / H;
    int64_t blk = static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x;

    // The wavefront's TPW query tiles are tiles TPW * wt + k, k < ntile
    // (ntile: the ones that hold rows); per tile, this lane's row.
    int h, slot, wt = 0, ntile = 1;
    int32_t p0, p1;
    int32_t id_end;        // page-id entries this wavefront's table row holds
    const int32_t* table;
    int64_t prow[TPW];     // this lane's partial row (sequence * H_q + query head) in tile k
    int32_t raw_len[TPW];  // that row's sequence length as read, checked below
    bool row_valid[TPW];
    const bool prefix_role = blk < a.prefix_blocks;
    // The query rows and the first window of page ids do not depend on the
    // length: each role issues their loads together with it, so the wavefront
    // waits one memory round trip before its first pages are requested.
    Tile<D, DIAG> T[TPW];
    int32_t ids;
    int64_t prow0;         // a valid query row of the wavefront's KV head
    auto issue_loads = [&]() {
#pragma unroll
        for (int k = 0; k < TPW; ++k)
            T[k].load_q(static_cast<const uint16_t*>(a.q) + (row_valid[k] ? prow[k] : prow0) * D);
        ids = (p0 + lane < min(p0 + kWave, id_end)) ? table[p0 + lane] : 0;
        // keep the compiler from sinking those loads below the exit test
        asm volatile("" ::: "memory");
    };
    if (prefix_role) {
        const int per_xcd = a.prefix_blocks / kXcds;      // prefix_blocks is a multiple of 8
        int w = static_cast<int>(blk % kXcds) * per_xcd + static_cast<int>(blk / kXcds);
        const int tgb = a.prefix_tile_blocks;
        wt = (w % tgb) * kWavesPerBlock + wave;
        w /= tgb;
        h = w % H;
        const int c = w / H;
        const int rows = a.B * a.n_q * G;                  // rows (sequence, token, query head)
        if (c >= a.prefix_splits || TPW * wt * 16 >= rows) return;
        ntile = min(TPW, (rows - TPW * wt * 16 + 15) / 16);
        slot = c;
        p0 = c * a.prefix_chunk;
        p1 = min(p0 + a.prefix_chunk, a.prefix_pages);
        id_end = a.prefix_pages;
        table = a.page_table;
        prow0 = static_cast<int64_t>(h) * G;
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int r = (TPW * wt + k) * 16 + row;
            row_valid[k] = r < rows;
            const int rq = row_valid[k] ? r : 0;
            const int bq = rq / (a.n_q * G);                // sequence
            const int vq = rq / G;                          // sequence * n_q + token
            prow[k] = static_cast<int64_t>(vq) * a.H_q + static_cast<int64_t>(h) * G + rq % G;
            raw_len[k] = row_valid[k] ? a.lengths[bq] : 0;
        }
        issue_loads();
    } else {
        blk -= a.prefix_blocks;
        // a workgroup's wavefronts: kWavesPerBlock / wpt splits x wpt
        // wavefronts of each, so the tiles of one split read its pages
        // together (one L2)
        const int wtiles = (a.priv_tiles + TPW - 1) / TPW;   // wavefronts per split
        const int wpt = a.priv_wpt;
        const int spb = kWavesPerBlock / wpt;
        const int sgb = (a.priv_splits + spb - 1) / spb;
        const int ntg = (wtiles + wpt - 1) / wpt;
        const int split = static_cast<int>(blk % sgb) * spb + wave / wpt;
        blk /= sgb;
        wt = static_cast<int>(blk % ntg) * wpt + wave % wpt;
        blk /= ntg;
        h = static_cast<int>(blk % H);
        const int64_t b = blk / H;
        if (split >= a.priv_splits || wt >= wtiles || b >= a.B) return;
        ntile = min(TPW, a.priv_tiles - TPW * wt);
        slot = a.prefix_splits + split;
        p0 = a.page_begin + split * a.pages_per_split;
        p1 = p0 + a.pages_per_split;                      // clamped to the length below
        id_end = a.max_pages;
        table = a.page_table + b * a.max_pages;
        prow0 = b * a.n_q * a.H_q + static_cast<int64_t>(h) * G;
        // the tiles' rows: (token, query head) pairs r = token * G + g of this KV head
        const int32_t lb = a.lengths[b];
#pragma unroll
        for (int k = 0; k < TPW; ++k) {
            const int r = (TPW * wt + k) * 16 + row;
            row_valid[k] = r < a.n_q * G;
            const int rq = row_valid[k] ? r : 0;
            prow[k] = (b * a.n_q + rq / G) * a.H_q + static_cast<int64_t>(h) * G + rq % G;
            raw_len[k] = lb;
        }
        issue_loads();
    }
    int32_t len[TPW];
#pragma unroll
    for (int k = 0; k < TPW; ++k) len[k] = (prefix_role && !row_valid[k]) ? 0 : check_length(a, raw_len[k]);
    if (!prefix_role) p1 = min(p1, (len[0] + kPage - 1) / kPage);
    if (p0 >= p1) return;
    int32_t vlen = 0;
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
        T[k].init(row_valid[k], row_valid[k] ? len[k] : 0);
        if (k < ntile) vlen = max(vlen, T[k].vlen);
    }

    // Pages go in windows of 64: one vector load brings the window's page ids
    // (lane i: page w0 + i) before its pipeline starts, so no wait inside the
    // pipeline depends on it.
    PageRegs<D, DIAG> buf[NBUF];
    for (int32_t w0 = p0; w0 < p1; w0 += kWave) {
        const int32_t w1 = min(w0 + kWave, p1);
        if (w0 != p0) ids = (w0 + lane < w1) ? table[w0 + lane] : 0;
        auto load = [&](PageRegs<D, DIAG>& r, int32_t lp) {
            load_page<D, DIAG>(a, r, __builtin_amdgcn_readlane(ids, min(lp, w1 - 1) - w0), h);
        };
#pragma unroll
        for (int i = 0; i < NBUF; ++i) load(buf[i], w0 + i);
        for (int32_t lp = w0; lp < w1; lp += NBUF) {
#pragma unroll
            for (int i = 0; i < NBUF; ++i) {
                if (lp + i < w1) fold_page<D, DIAG, TPW>(T, ntile, buf[i], lp + i, vlen);
                load(buf[i], lp + i + NBUF);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < TPW; ++k)
        if (k < ntile) T[k].store(a, row_valid[k], prow[k], slot);

    // The KV head 0 wavefronts of the shared prefix check that the sequences
    // of their tiles map the chunk's pages like sequence 0 (independent loads,
    // one flag).  It is done last, off the path to the first pages.
    if (prefix_role && h == 0) {
        const int rows = a.B * a.n_q * G;
        const int b_first = (TPW * wt * 16) / (a.n_q * G);
        const int b_last = min(rows - 1, (TPW * wt + ntile) * 16 - 1) / (a.n_q * G);
        const int npg = p1 - p0;
        const int n = (b_last - b_first + 1) * npg;
        bool bad = false;
        for (int i = lane; i < n; i += kWave) {
            const int32_t pg = p0 + i % npg;
            const int64_t bb = b_first + i / npg;
            bad |= a.page_table[bb * a.max_pages + pg] != a.page_table[pg];
        }
        if (bad) raise_err(a.err, SPICY_DEVERR_SHARED);
    }
}

// -------------------------------------------------------------- fp32 VALU

template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeArgs a) {
    constexpr int QD = D / 4;          // dims per quarter-row
    constexpr int DL = D / kWave;      // output dims per lane
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int ent = lane / 4;
    const int qtr = lane % 4;
    const int split = blockIdx.x * (blockDim.x / kWave) + wave;
    const int hq = blockIdx.y;
    const int bv = blockIdx.z;                 // sequence * n_q + token
    const int b = bv / a.n_q;
    const int H = a.cache.H;
    const int G = a.H_q / H;
    const int h = hq / G;
    if (split >= a.priv_splits) return;

    const int32_t len = checked_length(a, b);
    const int32_t npages = (len + kPage - 1) / kPage;
    const int32_t p0 = a.page_begin + split * a.pages_per_split;
    const int32_t p1 = min(p0 + a.pages_per_split, npages);
    if (p0 >= p1) return;

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

    for (int32_t lp = p0; lp < p1; ++lp) {
        const int32_t pid = table[lp];
        if (pid < 0 || pid >= a.cache.num_pages) {
            raise_err(a.err, SPICY_DEVERR_PAGE_ID);
            continue;
        }
        const int64_t ph = static_cast<int64_t>(pid) * H + h;
        const float* krow = kpool + ph * kPage * D + slot_elem(ent, qtr * QD);   // QD <= 32: one chunk
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < QD; ++i) dot += qv[i] * krow[i];
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const float alpha = abpool[(ph * kPage + ent) * 2 + 0];
        const float beta = abpool[(ph * kPage + ent) * 2 + 1];
        float closure = beta * c_beta;
        if (s2pool) {
            const float* srow = s2pool + ph * kPage * D + slot_elem(ent, qtr * QD);
            float c = 0.f;
#pragma unroll
            for (int i = 0; i < QD; ++i) c += qv[i] * qv[i] * srow[i];
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
    const int64_t idx = (static_cast<int64_t>(bv) * a.H_q + hq) * a.splits + a.prefix_splits + split;
    if (lane == 0) {
        a.part_ml[2 * idx + 0] = m_run;
        a.part_ml[2 * idx + 1] = l_run;
    }
#pragma unroll
    for (int j = 0; j < DL; ++j) a.part_o[idx * D + lane + kWave * j] = acc[j];
}

// ----------------------------------------------------------------- combine

// One wavefront per (sequence, query head): merge its partials (prefix chunks
// first, then the private splits that hold pages) by log-sum-exp, in one
// pass with a running maximum: the loads of kChunk partials are issued
// together and nothing waits for a separate maximum pass.  Every lane reads
// the same (m, l) of a partial, so the maximum needs no lane exchange; lanes
// own D/64 dimensions.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs a) {
    constexpr int DL = D / kWave;
    constexpr int kChunk = 32;
    const int lane = threadIdx.x;
    const int hq = blockIdx.x;
    const int bv = blockIdx.y;                 // sequence * n_q + token
    const int32_t len = checked_length(a, bv / a.n_q);
    const int32_t npages = (len + kPage - 1) / kPage;
    const int32_t priv = max(0, npages - a.page_begin);
    const int nsplit = a.prefix_splits + min(a.priv_splits, (priv + a.pages_per_split - 1) / a.pages_per_split);
    const int64_t base = (static_cast<int64_t>(bv) * a.H_q + hq) * a.splits;

    float M = -__builtin_huge_valf();
    float L = 0.f;
    float acc[DL];
#pragma unroll
    for (int j = 0; j < DL; ++j) acc[j] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kChunk) {
        float w[kChunk], l[kChunk], ov[kChunk][DL];
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const int s = min(s0 + u, nsplit - 1);
            w[u] = a.part_ml[2 * (base + s)];
            l[u] = a.part_ml[2 * (base + s) + 1];
#pragma unroll
            for (int j = 0; j < DL; ++j) ov[u][j] = a.part_o[(base + s) * D + lane + kWave * j];
        }
        float mc = M;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) mc = fmaxf(mc, w[u]);     // repeats of the last partial change nothing
        const float msub = (mc == -__builtin_huge_valf()) ? 0.f : mc;
        const float scale = fast_exp2(M - msub);                   // 0 while M is -inf
        L *= scale;
#pragma unroll
        for (int j = 0; j < DL; ++j) acc[j] *= scale;
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float wu = (s0 + u < nsplit) ? fast_exp2(w[u] - msub) : 0.f;
            L += wu * l[u];
#pragma unroll
            for (int j = 0; j < DL; ++j) acc[j] += wu * ov[u][j];
        }
        M = mc;
    }
    const float msub = (M == -__builtin_huge_valf()) ? 0.f : M;
    float* orow = a.o + (static_cast<int64_t>(bv) * a.H_q + hq) * D;
    const bool live = L > 0.f;
    const float inv = live ? 1.f / L : 0.f;
#pragma unroll
    for (int j = 0; j < DL; ++j) orow[lane + kWave * j] = live ? acc[j] * inv : 0.f;
    if (lane == 0)
        a.lse[static_cast<int64_t>(bv) * a.H_q + hq] = live ? (msub + __log2f(L)) * kLn2 : -__builtin_huge_valf();
}

// ------------------------------------------------------------------ launch

constexpr int kNbuf = 4;                  // one tile per wavefront
constexpr int kNbufPair = 2;              // two tiles per wavefront: their state takes a page's registers
constexpr int kNbufDiag = 2;              // the variance pages add a third page-sized load
constexpr int64_t kMaxGridX = 65536;

// Grid of the bf16 kernel with TPW tiles per wavefront: the shared-prefix
// workgroups (a multiple of 8, see the XCD remap), then the split-K ones.
template <int TPW>
static dim3 mfma_grid(DecodeArgs& a) {
    const int G = a.H_q / a.cache.H;
    const int tiles = (a.B * a.n_q * G + 15) / 16;
    const int wtiles = (tiles + TPW - 1) / TPW;
    a.prefix_tile_blocks = (wtiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t pb = static_cast<int64_t>(a.prefix_splits) * a.cache.H * a.prefix_tile_blocks;
    a.prefix_blocks = static_cast<int32_t>((pb + kXcds - 1) / kXcds * kXcds);
    const int pw = (a.priv_tiles + TPW - 1) / TPW;   // wavefronts per split
    a.priv_wpt = pw >= 3 ? 4 : pw;
    const int64_t spb = kWavesPerBlock / a.priv_wpt;
    const int64_t sgb = (a.priv_splits + spb - 1) / spb;
    const int64_t ntg = (pw + a.priv_wpt - 1) / a.priv_wpt;
    const int64_t nblk = a.prefix_blocks + sgb * ntg * a.cache.H * a.B;
    const int64_t gx = nblk < kMaxGridX ? nblk : kMaxGridX;
    const int64_t gy = (nblk + gx - 1) / gx;
    return dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy));
}

template <int D>
static spicy_status launch_decode_t(const DecodeArgs& a0, int dtype, hipStream_t stream) {
    DecodeArgs a = a0;
    if (dtype == SPICY_BF16) {
        const dim3 block(kWavesPerBlock * kWave);
        if (a.cache.s2) {
            const dim3 grid = mfma_grid<1>(a);
            hipLaunchKernelGGL((decode_mfma_kernel<D, kNbufDiag, true, 1>), grid, block, 0, stream, a);
        } else if (a.priv_tiles >= 2) {
            // several query tiles per (sequence, KV head): a wavefront takes two,
            // so each page it loads serves both and its V^T is formed once
            const dim3 grid = mfma_grid<2>(a);
            hipLaunchKernelGGL((decode_mfma_kernel<D, kNbufPair, false, 2>), grid, block, 0, stream, a);
        } else {
            const dim3 grid = mfma_grid<1>(a);
            hipLaunchKernelGGL((decode_mfma_kernel<D, kNbuf, false, 1>), grid, block, 0, stream, a);
        }
    } else {
        const int wpb = a.priv_splits < 4 ? a.priv_splits : 4;
        dim3 grid((a.priv_splits + wpb - 1) / wpb, a.H_q, a.B * a.n_q);
        hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(wpb * kWave), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    hipLaunchKernelGGL((combine_kernel<D>), dim3(a.H_q, a.B * a.n_q), dim3(kWave), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    return SPICY_OK;
}

spicy_status launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t stream) {
    if (a.B == 0) return SPICY_OK;
    return D == 128 ? launch_decode_t<128>(a, dtype, stream) : launch_decode_t<64>(a, dtype, stream);
}

}  // namespace spicy
