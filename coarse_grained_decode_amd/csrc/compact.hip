// Compaction of a merged range of the paged SPICY-KV cache on gfx950.
//
// What is computed (SPICY-KV demo page, Claim 12: in the cascaded dyadic
// ring-buffer pyramid a merged level holds half as many nodes, so it holds
// half the storage): for every sequence b, over logical entries
// [entry_begin[b], lengths[b]),
//   - per KV head h, the c_h entries whose alpha is not -inf keep their order
//     and move to entries entry_begin[b], entry_begin[b] + 1, ...;
//   - lengths_out[b] = entry_begin[b] + max over heads of c_h;
//   - per head, entries from entry_begin[b] + c_h to the end of the page that
//     holds entry lengths_out[b] - 1 become nulls;
//   - nothing before entry_begin[b] or past that page is written.
// A moved entry keeps every stored byte (key, value and variance rows, alpha
// and beta, metadata).
//
// Two launches, in place:
//   compact_count  one workgroup per sequence: checks the range and its page
//                  ids, counts every head's non-null entries and writes
//                  lengths_out (the range's length itself when the range or a
//                  page id is bad, with the error bit).  The count has to be
//                  done before any head moves: a head that is being moved
//                  cannot be counted.
//   compact_move   one workgroup per (KV head, sequence), 8 wavefronts:
//     1. the range's page ids are read once and kept in LDS (the first
//        kPageCache of them);
//     2. rounds of 512 source entries: a ballot scan gives each non-null
//        entry its destination; the entries that move (those after the
//        range's first null) are listed in LDS with their source and
//        destination slots;
//     3. the listed entries are copied in batches of 16-byte pieces: every
//        piece of a batch is loaded and the loads have completed (vmcnt 0)
//        before the workgroup barrier, and only then is any piece stored;
//     4. nulls from the head's last entry to the end of the new last page.
// Why in place is safe: the destinations rise with the sources and never
// pass them (dst(j) <= src(j), both increasing in j), so a store can only hit
// the source of an earlier entry of the same head, whose load finished before
// the barrier of its own batch; destinations of later batches and rounds are
// above every source already read.  Heads are separate page-head blocks, so
// workgroups never touch each other's bytes.
#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kPageCache = 1024;   // page ids of the range kept in LDS
constexpr int kBatch = 8;          // 16-byte pieces per thread per batch

struct Slot {                      // one listed move
    int32_t src_page, src_slot, dst_page, dst_slot;
};

// Byte layout of one entry's pieces for element size ES and head size D:
// rows (key, value, then the variance sidecar when present) of D / 8 groups
// of 8 elements, each group ES / 2 pieces of 16 bytes; then (alpha, beta);
// then the 16-byte metadata record when present.
struct Pieces {
    int32_t per_row;     // 16-byte pieces per row
    int32_t rows;        // 2 or 3
    int32_t total;       // pieces per entry
    bool meta;
};

template <int ES>
__device__ __forceinline__ Pieces pieces_of(const CompactArgs& a) {
    Pieces p;
    p.per_row = a.D / 8 * (ES / 2);
    p.rows = a.cache.s2 ? 3 : 2;
    p.meta = a.cache.meta != nullptr;
    p.total = p.rows * p.per_row + 1 + (p.meta ? 1 : 0);
    return p;
}

// Address and width (bytes) of piece `piece` of entry (page P, slot s) of
// head h.
template <int ES>
__device__ __forceinline__ char* piece_addr(const CompactArgs& a, const Pieces& pc, int64_t P, int s, int h,
                                            int piece, int* width) {
    const int64_t ph = P * a.cache.H + h;
    if (piece < pc.rows * pc.per_row) {
        const int row = piece / pc.per_row;
        const int c = piece % pc.per_row;
        const int g = c / (ES / 2), half = c % (ES / 2);
        char* base = static_cast<char*>(row == 0 ? a.cache.k : row == 1 ? a.cache.v : a.cache.s2);
        *width = 16;
        return base + (ph * kPage * a.D + (static_cast<int64_t>(g) * kPage + s) * kGroup) * ES + half * 16;
    }
    if (piece == pc.rows * pc.per_row) {
        *width = 2 * ES;
        return static_cast<char*>(a.cache.ab) + (ph * kPage + s) * 2 * ES;
    }
    *width = 16;
    return static_cast<char*>(a.cache.meta) + (ph * kPage + s) * 16;
}

__device__ __forceinline__ uint4 load_piece(const char* p, int width) {
    if (width == 16) return *reinterpret_cast<const uint4*>(p);
    if (width == 8) {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        return make_uint4(x.x, x.y, 0u, 0u);
    }
    return make_uint4(*reinterpret_cast<const uint32_t*>(p), 0u, 0u, 0u);
}

__device__ __forceinline__ void store_piece(char* p, int width, uint4 x) {
    if (width == 16) *reinterpret_cast<uint4*>(p) = x;
    else if (width == 8) *reinterpret_cast<uint2*>(p) = make_uint2(x.x, x.y);
    else *reinterpret_cast<uint32_t*>(p) = x.x;
}

// alpha == -inf, read as bits (bfloat16 0xFF80, binary32 0xFF800000)
template <int ES>
__device__ __forceinline__ bool alpha_null(const CompactArgs& a, int64_t P, int s, int h) {
    const int64_t at = ((P * a.cache.H + h) * kPage + s) * 2;
    if (ES == 2) return static_cast<const uint16_t*>(a.cache.ab)[at] == 0xFF80u;
    return static_cast<const uint32_t*>(a.cache.ab)[at] == 0xFF800000u;
}

// The range of sequence b and whether it can be compacted: 0, or the error bit.
__device__ __forceinline__ int32_t range_error(const CompactArgs& a, int32_t e0, int32_t L) {
    if (e0 < 0 || e0 > L) return SPICY_DEVERR_SEGMENTS;
    if ((static_cast<int64_t>(L) + kPage - 1) / kPage > a.max_pages) return SPICY_DEVERR_CAPACITY;
    return 0;
}

template <int ES>
__global__ __launch_bounds__(kThreads) void compact_count_kernel(CompactArgs a) {
    __shared__ int32_t counts[16];
    __shared__ int32_t bad;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int H = a.cache.H;
    const int32_t e0 = a.entry_begin[b];
    const int32_t L = a.lengths[b];
    const int32_t* row = a.page_table + static_cast<int64_t>(b) * a.max_pages;
    int32_t err = range_error(a, e0, L);
    if (t < 16) counts[t] = 0;
    if (t == 0) bad = 0;
    __syncthreads();
    int32_t n[16];
#pragma unroll
    for (int hh = 0; hh < 16; ++hh) n[hh] = 0;
    if (!err) {
        for (int32_t lp = e0 / kPage + t; lp < (L + kPage - 1) / kPage; lp += kThreads) {
            const int32_t P = row[lp];
            if (P < 0 || P >= a.cache.num_pages) bad = 1;
        }
        __syncthreads();
        if (bad) err = SPICY_DEVERR_PAGE_ID;
    }
    if (!err) {
        for (int64_t e = static_cast<int64_t>(e0) + t; e < L; e += kThreads) {
            const int64_t P = row[e / kPage];
#pragma unroll
            for (int hh = 0; hh < 16; ++hh)
                if (hh < H) n[hh] += alpha_null<ES>(a, P, static_cast<int>(e % kPage), hh) ? 0 : 1;
        }
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) {
            if (hh >= H) break;
            int32_t x = n[hh];
            for (int off = kWave / 2; off > 0; off /= 2) x += __shfl_xor(x, off);
            if (threadIdx.x % kWave == 0 && x) atomicAdd(&counts[hh], x);
        }
        __syncthreads();
    }
    if (t == 0) {
        int32_t longest = 0;
        for (int hh = 0; hh < H; ++hh) longest = max(longest, counts[hh]);
        if (err) raise_err(a.err, err);
        a.lengths_out[b] = err ? L : e0 + longest;
    }
}

template <int ES>
__global__ __launch_bounds__(kThreads) void compact_move_kernel(CompactArgs a) {
    __shared__ int32_t pages[kPageCache];
    __shared__ Slot list[kThreads];
    __shared__ int32_t wsum[kWaves];
    __shared__ int32_t fixed;
    __shared__ int32_t bad;

    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int lane = t % kWave, wave = t / kWave;
    const int32_t e0 = a.entry_begin[b];
    const int32_t L = a.lengths[b];
    const int32_t* row = a.page_table + static_cast<int64_t>(b) * a.max_pages;

    // ---- the range and its pages (the count launch reported any problem;
    // then nothing moves)
    if (range_error(a, e0, L)) return;
    if (t == 0) bad = 0;
    __syncthreads();
    const int32_t lp0 = e0 / kPage;
    const int32_t lp1 = (L + kPage - 1) / kPage;
    for (int32_t lp = lp0 + t; lp < lp1; lp += kThreads) {
        const int32_t P = row[lp];
        if (P < 0 || P >= a.cache.num_pages) bad = 1;
        if (lp - lp0 < kPageCache) pages[lp - lp0] = P;
    }
    __syncthreads();
    if (bad) return;
    const int32_t new_len = a.lengths_out[b];
    auto page_at = [&](int32_t e) -> int64_t {
        const int32_t lp = e / kPage;
        return lp - lp0 < kPageCache ? pages[lp - lp0] : row[lp];
    };

    // ---- rounds: scan, list the moves, copy them
    const Pieces pc = pieces_of<ES>(a);
    int32_t base = 0;                     // non-null entries of this head before the round
    for (int64_t s0 = e0; s0 < L; s0 += kThreads) {
        const int32_t e = static_cast<int32_t>(min(s0 + t, static_cast<int64_t>(L)));   // L: past the range
        int64_t P = 0;
        bool keep = false;
        if (e < L) {
            P = page_at(e);
            keep = !alpha_null<ES>(a, P, e % kPage, h);
        }
        const uint64_t m = __ballot(keep);
        const int32_t below = __popcll(m & ((1ull << lane) - 1ull));
        if (t == 0) fixed = 0;
        if (lane == 0) wsum[wave] = __popcll(m);
        __syncthreads();
        int32_t before = 0, round_n = 0;
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? wsum[w] : 0;
            round_n += wsum[w];
        }
        const int32_t rank = before + below;             // among this round's non-null entries
        const int32_t dst = e0 + base + rank;
        const bool stays = keep && dst == e;             // no null before it in the range
        const uint64_t ms = __ballot(stays);
        if (lane == 0 && ms) atomicAdd(&fixed, __popcll(ms));
        __syncthreads();
        const int32_t n_fixed = fixed;                   // they are the round's first non-null entries
        if (keep && !stays) {
            const int64_t Pd = page_at(dst);
            list[rank - n_fixed] = Slot{static_cast<int32_t>(P), e % kPage, static_cast<int32_t>(Pd), dst % kPage};
        }
        __syncthreads();
        const int32_t items = (round_n - n_fixed) * pc.total;
        for (int32_t i0 = 0; i0 < items; i0 += kBatch * kThreads) {
            uint4 x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int32_t i = i0 + u * kThreads + t;
                if (i < items) {
                    const Slot sl = list[i / pc.total];
                    int wd;
                    const char* p = piece_addr<ES>(a, pc, sl.src_page, sl.src_slot, h, i % pc.total, &wd);
                    x[u] = load_piece(p, wd);
                }
            }
            // every load of the batch has returned before any store below
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int32_t i = i0 + u * kThreads + t;
                if (i < items) {
                    const Slot sl = list[i / pc.total];
                    int wd;
                    char* p = piece_addr<ES>(a, pc, sl.dst_page, sl.dst_slot, h, i % pc.total, &wd);
                    store_piece(p, wd, x[u]);
                }
            }
        }
        base += round_n;
        __syncthreads();                                 // the list is rewritten by the next round
    }

    // ---- nulls from the end of this head's entries to the end of the new
    // last page (every load above has completed before its batch's barrier)
    const int64_t pad_end = min((static_cast<int64_t>(new_len) + kPage - 1) / kPage,
                                static_cast<int64_t>(lp1)) * kPage;       // within the range's pages
    const int64_t items = (pad_end - (e0 + base)) * pc.total;
    for (int64_t i = t; i < items; i += kThreads) {
        const int32_t e = static_cast<int32_t>(e0 + base + i / pc.total);
        const int piece = static_cast<int>(i % pc.total);
        int wd;
        char* p = piece_addr<ES>(a, pc, page_at(e), e % kPage, h, piece, &wd);
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (piece == pc.rows * pc.per_row) x.x = ES == 2 ? 0xFF80u : 0xFF800000u;   // alpha -inf, beta +0
        store_piece(p, wd, x);
    }
}

}  // namespace

spicy_status launch_compact(const CompactArgs& a, int dtype, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.cache.H), static_cast<unsigned>(a.B));
    if (dtype == SPICY_BF16) {
        hipLaunchKernelGGL(compact_count_kernel<2>, dim3(a.B), dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(compact_move_kernel<2>, grid, dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(compact_count_kernel<4>, dim3(a.B), dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(compact_move_kernel<4>, grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? SPICY_OK : SPICY_ERR_HIP;
}

}  // namespace spicy
