// SPICY-KV coarsening on gfx950.
//
// What is computed (SPICY-KV demo page, Claims 2 and 3; SPICY-KV abstract,
// items (1) and (3)): per sequence, KV head and caller segment, the
// unprotected ("F") tokens merge into one macro-node carrying their mass m,
// mean pre-RoPE key rotated to the mean position, mean value, alpha = ln m and
// beta = sigma^2 / (2d) (sigma^2 = per-dimension population variance of the
// member keys); protected ("C") tokens stay exact (mass 1, own position).
//
// Two kernels:
//   coarsen_main   two roles that share nothing, so they run side by side.
//     plan role:   one 256-thread workgroup per sequence, one thread per
//                  segment: counts the protected tokens of each (segment,
//                  head) with 32 mask rows in flight, block-scans the per-head
//                  entry counts into entry offsets (and the C-point counts
//                  into item offsets), writes a compact descriptor per
//                  segment, then lists the segment's C-points as items
//                  {token, entry, head} in position order per head; records
//                  the sequence's length and where each head's null padding
//                  starts.
//     streaming:   persistent workgroups, one wavefront per segment and group
//                  of KV heads (4 heads at d = 128).  A lane owns 8
//                  consecutive dimensions of one head, so one 16-byte load per
//                  lane reads a whole token row of the wave's heads; tokens
//                  stream through a register ring.  F-tokens are accumulated
//                  branch-free in double precision (mask as a 0/1 weight) and
//                  the macro-node is staged at the segment end.  Bound by
//                  reading K and V from HBM.
//     The plan workgroups then place the C-points they listed (key rotated
//     to the token's position) and each head's null padding while the
//     streaming role is still running.
//   coarsen_cpoint the staged macro-nodes of every sequence, one per 16-lane
//                  group, copied to the entries the plan gave them.
// Variants of the streaming role: the diagonal closure (per-dimension
// variances of the rotated member keys, when the cache has that sidecar) and
// variation-weighted representatives (per-token weights, from
// spicy_coarsen_weighted); they are described where they are summed.
//
// Exactness: inputs are bf16 (8 significant bits).  Sums of bf16 values and
// of their squares are exact in double precision for any realistic segment,
// so the mean is one correctly rounded division, as in a sequential sum, and
// the variance sum (k^2) - (sum k)^2 / m is zero for a segment of identical
// keys.  Every stored value is rounded once, to nearest-even.
#include <algorithm>

#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kCpointBlocksPerSeq = 64;
constexpr int kMaxH = 16;
constexpr int kRing = 3;
// streaming workgroups: twice the 512 that coarsen_main's register use fits
// at once (2 of 4 waves per CU); the later ones start as earlier ones finish
constexpr int kResidentBlocks = 1024;
// coarsen_cpoint's register use allows 8 waves per SIMD: 8 workgroups of 4
// waves per CU, 2048 on the chip; its grid stays within one such round.
constexpr int kCpointResident = 2048;
constexpr int32_t kWindow = 65536;      // tokens per buffer resource (< 4 GiB)

struct Meta {
    int32_t kind;
    int32_t mass;
    int64_t pos_sum;
};

// Resolve logical entry e of sequence b to its physical page; -1 on error.
__device__ __forceinline__ int32_t entry_page(const CoarsenArgs& a, int b, int64_t e) {
    const int64_t lp = e / kPage;
    if (e < 0 || lp >= a.max_pages) {
        raise_err(a.err, SPICY_DEVERR_CAPACITY);
        return -1;
    }
    const int32_t P = a.page_table[static_cast<int64_t>(b) * a.max_pages + lp];
    if (P < 0 || P >= a.cache.num_pages) {
        raise_err(a.err, SPICY_DEVERR_PAGE_ID);
        return -1;
    }
    return P;
}

// Destination hints.  The plan role knows where each (segment, head)
// macro-node goes; the streaming role computes the macro-node.  When the plan
// has already published the destination by the time the streaming role
// finishes the segment, the streaming role writes the macro-node straight
// into the cache; otherwise it stages it and coarsen_cpoint copies it there
// from the plan's record in the workspace (seg_head), which alone is
// authoritative.  A hint is one 64-bit word, gen << 32 | page << 4 | slot,
// published and read with single device-scope atomic accesses; gen is the
// call's nonzero tag, so a word left by another call (on this or another
// stream) never matches and only sends its macro-node down the staged path.
// The array starts zero, only the library writes it, and coarsen_cpoint
// clears every word of its call.
__device__ uint64_t g_dest_hint[kDestHintWords];

__device__ __forceinline__ uint64_t dest_word(int32_t page, int64_t entry, uint32_t gen) {
    return (static_cast<uint64_t>(gen) << 32) | (static_cast<uint64_t>(static_cast<uint32_t>(page)) << 4) |
           static_cast<uint64_t>(entry % kPage);
}

struct Dest {
    int32_t page;
    int slot;
    bool ok;
};

__device__ __forceinline__ Dest read_dest(uint64_t w, uint32_t gen) {
    Dest d;
    d.page = static_cast<int32_t>((w >> 4) & 0x0FFFFFFFu);
    d.slot = static_cast<int>(w & 15u);
    d.ok = gen != 0 && static_cast<uint32_t>(w >> 32) == gen;
    return d;
}

// 8 consecutive elements of one row: a 16-byte (bf16) or 32-byte (fp32) load
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
    uint4 x;
    __device__ __forceinline__ void load(const uint16_t* p) { x = *reinterpret_cast<const uint4*>(p); }
    static __device__ __forceinline__ void load_buf(Row8& r, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff), soff, 0);
        r.x = make_uint4(v[0], v[1], v[2], v[3]);
    }
    __device__ __forceinline__ uint32_t word(int i) const {
        return (i < 2) ? x.x : (i < 4) ? x.y : (i < 6) ? x.z : x.w;
    }
    __device__ __forceinline__ uint16_t raw(int i) const {
        const uint32_t w = word(i);
        return static_cast<uint16_t>((i & 1) ? (w >> 16) : (w & 0xFFFFu));
    }
    __device__ __forceinline__ double f64(int i) const {
        const uint32_t w = word(i);
        const uint32_t bits = (i & 1) ? (w & 0xFFFF0000u) : (w << 16);
        return static_cast<double>(__uint_as_float(bits));
    }
    // the row held by lane (this lane xor P), P = 4 or 8
    template <int P>
    __device__ __forceinline__ Row8 lane_xor() const {
        Row8 r;
        r.x = make_uint4(dpp_xor<P>(x.x), dpp_xor<P>(x.y), dpp_xor<P>(x.z), dpp_xor<P>(x.w));
        return r;
    }
};
template <> struct Row8<float> {
    float4 x, y;
    __device__ __forceinline__ void load(const float* p) {
        x = *reinterpret_cast<const float4*>(p);
        y = *reinterpret_cast<const float4*>(p + 4);
    }
    static __device__ __forceinline__ void load_buf(Row8& r, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff), soff, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(voff + 16), soff, 0);
        r.x = make_float4(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3]));
        r.y = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
    }
    __device__ __forceinline__ float raw(int i) const {
        const float4& q = i < 4 ? x : y;
        const int j = i & 3;
        return j == 0 ? q.x : j == 1 ? q.y : j == 2 ? q.z : q.w;
    }
    __device__ __forceinline__ double f64(int i) const { return static_cast<double>(raw(i)); }
    template <int P>
    __device__ __forceinline__ Row8 lane_xor() const {
        auto sw = [](float f) { return __uint_as_float(dpp_xor<P>(__float_as_uint(f))); };
        Row8 r;
        r.x = make_float4(sw(x.x), sw(x.y), sw(x.z), sw(x.w));
        r.y = make_float4(sw(y.x), sw(y.y), sw(y.z), sw(y.w));
        return r;
    }
};

template <typename T> struct Pack8;
template <> struct Pack8<uint16_t> {
    __device__ __forceinline__ static void store(uint16_t* p, const double (&y)[8]) {
        uint4 o;
        o.x = f64_to_bf16(y[0]) | (static_cast<uint32_t>(f64_to_bf16(y[1])) << 16);
        o.y = f64_to_bf16(y[2]) | (static_cast<uint32_t>(f64_to_bf16(y[3])) << 16);
        o.z = f64_to_bf16(y[4]) | (static_cast<uint32_t>(f64_to_bf16(y[5])) << 16);
        o.w = f64_to_bf16(y[6]) | (static_cast<uint32_t>(f64_to_bf16(y[7])) << 16);
        *reinterpret_cast<uint4*>(p) = o;
    }
};
template <> struct Pack8<float> {
    __device__ __forceinline__ static void store(float* p, const double (&y)[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(static_cast<float>(y[0]), static_cast<float>(y[1]),
                                                    static_cast<float>(y[2]), static_cast<float>(y[3]));
        *reinterpret_cast<float4*>(p + 4) = make_float4(static_cast<float>(y[4]), static_cast<float>(y[5]),
                                                        static_cast<float>(y[6]), static_cast<float>(y[7]));
    }
};

// 8 consecutive elements given one by one, stored with one (bf16) or two
// (fp32) 16-byte writes.
template <typename T> struct Store8;
template <> struct Store8<uint16_t> {
    template <typename F>
    __device__ __forceinline__ static void store(uint16_t* p, const F& f) {
        uint4 o;
        o.x = f(0) | (static_cast<uint32_t>(f(1)) << 16);
        o.y = f(2) | (static_cast<uint32_t>(f(3)) << 16);
        o.z = f(4) | (static_cast<uint32_t>(f(5)) << 16);
        o.w = f(6) | (static_cast<uint32_t>(f(7)) << 16);
        *reinterpret_cast<uint4*>(p) = o;
    }
};
template <> struct Store8<float> {
    template <typename F>
    __device__ __forceinline__ static void store(float* p, const F& f) {
        *reinterpret_cast<float4*>(p) = make_float4(f(0), f(1), f(2), f(3));
        *reinterpret_cast<float4*>(p + 4) = make_float4(f(4), f(5), f(6), f(7));
    }
};

}  // namespace

// ------------------------------------------------------------------- plan

// Protection bits of token t (bit h = head h) from its mask row.  NQ > 0:
// the row is NQ dwords (H = 4 NQ); NQ = 0: H bytes, read one by one (the
// clamped index keeps every load unconditional).
template <int NQ>
__device__ __forceinline__ uint32_t row_bits(const CoarsenArgs& a, int32_t t) {
    const int H = a.cache.H;
    const uint8_t* row = a.mask + static_cast<int64_t>(t) * H;
    uint32_t bits = 0;
    if constexpr (NQ > 0) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(row)[q];
#pragma unroll
            for (int y = 0; y < 4; ++y)
                if ((w >> (8 * y)) & 0xFFu) bits |= 1u << (4 * q + y);
        }
    } else {
#pragma unroll
        for (int q = 0; q < kMaxH; ++q) {
            const uint8_t x = row[min(q, H - 1)];
            if (q < H && x) bits |= 1u << q;
        }
    }
    return bits;
}

// Inclusive sum over the workgroup's threads (in thread order) of x, given
// the wave-level scratch; returns this thread's inclusive prefix and leaves
// the workgroup total in *total.  All threads must call it.
__device__ __forceinline__ int block_inclusive_scan(int x, int32_t* s_wave, int* total) {
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    int incl = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
        before += w < wave ? s_wave[w] : 0;
        tot += s_wave[w];
    }
    __syncthreads();
    *total = tot;
    return before + incl;
}

// kRound mask rows of tokens tb .. tb+kRound-1 of a segment ending at sz,
// all loads in flight together (indexes clamped into the segment and the
// input, so every load is unconditional and in bounds).
template <int NQ, int kRound>
__device__ __forceinline__ void load_round(const CoarsenArgs& a, int32_t tb, int32_t sz, uint32_t (&w)[kRound]) {
    const int32_t last = min(sz, a.total_tokens) - 1;
#pragma unroll
    for (int u = 0; u < kRound; ++u) w[u] = row_bits<NQ>(a, max(min(tb + u, last), 0));
}

template <typename T, int D>
__device__ __forceinline__ void place_listed(const CoarsenArgs& a, int b, int32_t t0, int32_t t1, int64_t pos_off,
                                             const int2* items, int32_t n_cp, int64_t padded);

// One workgroup plans sequence b: per segment (one thread each) the
// protected tokens of every head, block scans into entry and item offsets,
// descriptors, and the C-point items in position order per head.
// What placing the listed entries needs from the plan (ok false: the
// sequence failed its checks and gets nothing).
struct PlanOut {
    bool ok;
    int32_t t0, t1;
    int32_t n_cp;
    int64_t padded;
};

template <typename T, int D, int NQ>
__device__ __forceinline__ void plan_sequence(const CoarsenArgs& a, int32_t (*s_wave)[kPlanWaves], int32_t& s_ok,
                                              PlanOut& out) {
    constexpr int NH = NQ > 0 ? 4 * NQ : kMaxH;      // heads a mask row can hold
    constexpr int kRound = NQ > 0 ? 64 / NQ : 8;     // mask rows in flight per thread
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int H = a.cache.H;

    const int32_t t0 = a.seq_offsets[b], t1 = a.seq_offsets[b + 1];
    const int32_t s0 = a.seq_seg_ptr[b], s1 = a.seq_seg_ptr[b + 1];
    const int32_t e0 = a.entry_start ? a.entry_start[b] : 0;
    const bool ranges_sane = 0 <= s0 && s0 <= s1 && s1 <= a.n_seg;
    // this thread's first segment and its first mask rows are read before the
    // sequence is validated (every index is bounded by the array it reads)
    int32_t sa = 0, sz = 0;
    uint32_t w[kRound];
    if (ranges_sane && s0 + tid < s1) {
        sa = a.seg_offsets[s0 + tid];
        sz = a.seg_offsets[s0 + tid + 1];
    }
    load_round<NQ, kRound>(a, sa, sz, w);
    if (tid == 0) {
        bool ok = ranges_sane && 0 <= t0 && t0 <= t1 && t1 <= a.total_tokens && e0 >= 0;
        if (ok) ok = a.seg_offsets[s0] == t0 && a.seg_offsets[s1] == t1;
        s_ok = ok;
        if (!ok) {
            raise_err(a.err, SPICY_DEVERR_SEGMENTS);
            a.lengths_out[b] = e0 < 0 ? 0 : e0;
            a.cp_count[b] = 0;
        }
        if (b == a.B - 1 && a.seq_seg_ptr[a.B] != a.n_seg) raise_err(a.err, SPICY_DEVERR_SEGMENTS);
        if (b == 0 && a.seq_seg_ptr[0] != 0) raise_err(a.err, SPICY_DEVERR_SEGMENTS);
    }
    __syncthreads();
    // segments no valid sequence owns are marked so that coarsen_main skips them
    if (b == a.B - 1) {
        const int32_t first = max(a.seq_seg_ptr[a.B], 0);
        for (int32_t s = first + tid; s < a.n_seg; s += kPlanThreads) a.seg_desc[s] = make_int4(-1, 0, 0, 0);
    }
    if (b == 0) {
        const int32_t last = min(a.seq_seg_ptr[0], a.n_seg);
        for (int32_t s = tid; s < last; s += kPlanThreads) a.seg_desc[s] = make_int4(-1, 0, 0, 0);
    }
    if (!s_ok) {
        if (ranges_sane)
            for (int32_t s = s0 + tid; s < s1; s += kPlanThreads) a.seg_desc[s] = make_int4(-1, 0, 0, 0);
        if (tid < H) a.null_from[static_cast<int64_t>(b) * H + tid] = INT32_MAX;
        return;
    }

    const int32_t pos_off = (a.pos_base ? a.pos_base[b] : 0) - t0;
    int2* items = a.cp_items + static_cast<int64_t>(t0) * H;
    const int32_t cap = a.max_pages * kPage;
    int carry[kMaxH + 1];                      // entries per head, then C-point items, so far
#pragma unroll
    for (int h = 0; h <= kMaxH; ++h) carry[h] = 0;

    for (int32_t base = s0; base < s1; base += kPlanThreads) {
        const int32_t s = base + tid;
        if (base != s0) {                      // later rounds of segments: read now
            sa = sz = 0;
            if (s < s1) {
                sa = a.seg_offsets[s];
                sz = a.seg_offsets[s + 1];
            }
            load_round<NQ, kRound>(a, sa, sz, w);
        }
        int cnt[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) cnt[h] = 0;
        if (s < s1) {
            if (!(t0 <= sa && sa <= sz && sz <= t1)) {
                raise_err(a.err, SPICY_DEVERR_SEGMENTS);
                sa = sz = t0;
            }
            // protected tokens per head; w holds the segment's first round
            for (int32_t tb = sa; tb < sz; tb += kRound) {
                if (tb != sa) load_round<NQ, kRound>(a, tb, sz, w);
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    const uint32_t bits = tb + u < sz ? w[u] : 0u;
#pragma unroll
                    for (int h = 0; h < NH; ++h) cnt[h] += (bits >> h) & 1u;
                }
            }
            a.seg_desc[s] = make_int4(b, sa, sz, pos_off);
        }
        // entries per head: protected tokens + one macro-node if any F-token;
        // C-point items: protected (token, head) pairs of the segment
        int first[NH], has_f[NH];
        int ncount = 0, item0 = 0;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const bool live = s < s1 && h < H;
            has_f[h] = live && (sz - sa - cnt[h]) > 0 ? 1 : 0;
            ncount += live ? cnt[h] : 0;
            first[h] = 0;
        }
#pragma unroll
        for (int h = 0; h <= NH; ++h) {
            if (h < H || h == NH) {            // uniform: every thread scans alike
                const int x = h == NH ? ncount : (s < s1 ? cnt[h] + has_f[h] : 0);
                int tot;
                const int incl = block_inclusive_scan(x, s_wave[h], &tot);
                if (h < NH) {
                    first[h] = e0 + carry[h] + incl - x;
                    carry[h] += tot;
                } else {
                    item0 = carry[kMaxH] + incl - x;
                    carry[kMaxH] += tot;
                }
            }
        }
        if (s < s1) {
#pragma unroll
            for (int h = 0; h < NH; ++h)
                if (h < H) {
                    // the macro-node's physical page, resolved here so that
                    // placing it needs no table lookup (-1: none, or an
                    // entry the table cannot hold, reported here), and
                    // published as a hint for the streaming role
                    const int32_t Pg = has_f[h] ? entry_page(a, b, first[h]) : -1;
                    const int64_t idx = static_cast<int64_t>(s) * H + h;
                    a.seg_head[idx] = make_int2(first[h], Pg);
                    if (a.gen != 0 && Pg >= 0)
                        __hip_atomic_store(&g_dest_hint[idx], dest_word(Pg, first[h], a.gen), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            // the segment's C-point items, in position order within each head
            int nxt[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h) nxt[h] = first[h] + has_f[h];
            int64_t k = item0;
            for (int32_t tb = sa; tb < sz && ncount > 0; tb += kRound) {
                if (sz - sa > kRound) load_round<NQ, kRound>(a, tb, sz, w);   // else still in w
#pragma unroll
                for (int u = 0; u < kRound; ++u) {
                    uint32_t bits = tb + u < sz ? w[u] : 0u;
                    while (bits) {
                        const int h = __builtin_ctz(bits);
                        bits &= bits - 1;
                        int32_t e = 0;
#pragma unroll
                        for (int q = 0; q < NH; ++q) {
                            if (q == h) {
                                e = nxt[q];
                                nxt[q] = e + 1;
                            }
                        }
                        // an entry past the table's capacity is clamped to its
                        // end, which the storing kernel reports
                        items[k] = make_int2(tb + u, (min(e, cap) << 4) | h);
                        k += 1;
                    }
                }
            }
        }
    }

    // length, C-point count and where each head's null padding starts
    // (coarsen_cpoint writes the nulls)
    int32_t most = 0;
#pragma unroll
    for (int h = 0; h < NH; ++h)
        if (h < H) most = max(most, carry[h]);
    const int64_t len = static_cast<int64_t>(e0) + most;
    const int64_t padded = (len + kPage - 1) / kPage * kPage;
    if (tid == 0) {
        a.lengths_out[b] = static_cast<int32_t>(len);
        a.cp_count[b] = carry[kMaxH];
        if (padded / kPage > a.max_pages) raise_err(a.err, SPICY_DEVERR_CAPACITY);
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
        if (h < H && tid == h) a.null_from[static_cast<int64_t>(b) * H + h] = e0 + carry[h];
    out.ok = true;
    out.t0 = t0;
    out.t1 = t1;
    out.n_cp = carry[kMaxH];
    out.padded = padded;
}

template <typename T, int D>
__device__ __forceinline__ void plan_role(const CoarsenArgs& a) {
    __shared__ int32_t s_wave[kMaxH + 1][kPlanWaves];
    __shared__ int32_t s_ok;
    PlanOut out{false, 0, 0, 0, 0};
    // mask rows read as H / 4 dwords when H is a multiple of 4, else as bytes
    switch (a.cache.H % 4 == 0 ? a.cache.H / 4 : 0) {
    case 1: plan_sequence<T, D, 1>(a, s_wave, s_ok, out); break;
    case 2: plan_sequence<T, D, 2>(a, s_wave, s_ok, out); break;
    case 3: plan_sequence<T, D, 3>(a, s_wave, s_ok, out); break;
    case 4: plan_sequence<T, D, 4>(a, s_wave, s_ok, out); break;
    default: plan_sequence<T, D, 0>(a, s_wave, s_ok, out); break;
    }
    if (!out.ok) return;                               // the same for the whole workgroup
    // the listed C-points and the null padding are placed now, while the
    // streaming role runs (they need nothing from it); every thread's items
    // and null starts are visible to the workgroup after the barrier
    __syncthreads();
    const int b = blockIdx.x;
    const int64_t pos_off = static_cast<int64_t>(a.pos_base ? a.pos_base[b] : 0) - out.t0;
    place_listed<T, D>(a, b, out.t0, out.t1, pos_off, a.cp_items + static_cast<int64_t>(out.t0) * a.cache.H,
                       out.n_cp, out.padded);
}

// ---------------------------------------------------------- main + C-points

// Lane layout shared by coarsen_main and coarsen_cpoint: one wavefront covers
// HW heads of one token; lane (hl, j) owns dims 8j .. 8j+7 of head hl.  RoPE
// pairs dims (i, i + D/2), held by lanes j and j + PARTNER.
template <typename T, int D>
struct Lanes {
    static constexpr int LPH = D / 8;         // lanes per head
    static constexpr int HW = kWave / LPH;    // heads per wavefront
    static constexpr int PARTNER = LPH / 2;   // lane distance to the rotary partner
    int lane, hl, j, h, hh, hbase, d0;
    bool active, hi_half, rotate;
    double theta[4];                          // the 4 frequencies this lane evaluates

    __device__ __forceinline__ Lanes(const CoarsenArgs& a) {
        lane = threadIdx.x % kWave;
        hl = lane / LPH;
        j = lane % LPH;
        hbase = blockIdx.y * HW;
        h = hbase + hl;
        active = h < a.cache.H;
        hh = active ? h : 0;
        hi_half = j >= PARTNER;
        d0 = 8 * j;
        rotate = a.rope_base > 0.0;
        const int pair0 = 8 * (hi_half ? j - PARTNER : j) + (hi_half ? 4 : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            theta[r] = a.theta[pair0 + r];
    }

    // cos and sin of pos * theta for the rotary pairs of this lane's
    // dimensions q and 4 + q (all lanes of the wave must call it together).
    __device__ __forceinline__ void angle(double pos, int q, double& ca, double& sa, double& cb, double& sb) const {
        double sq, cq;
        sincos_f64(pos * theta[q], &sq, &cq);          // index (hi ? 4 : 0) + q
        const double oc = __shfl_xor(cq, PARTNER);      // index (hi ? 0 : 4) + q
        const double os = __shfl_xor(sq, PARTNER);
        ca = hi_half ? oc : cq;
        sa = hi_half ? os : sq;
        cb = hi_half ? cq : oc;
        sb = hi_half ? sq : os;
    }

    // Rotate this lane's 8 key values to position pos (all lanes of the wave
    // must call it together: it exchanges sin/cos and partner values).  One
    // rotary pair index q at a time, to keep few double-precision values live.
    template <typename GetX>
    __device__ __forceinline__ void rope(const GetX& x, double pos, double (&y)[8]) const {
        if (!rotate) {
#pragma unroll
            for (int r = 0; r < 8; ++r) y[r] = x(r);
            return;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            double sq, cq;
            sincos_f64(pos * theta[q], &sq, &cq);          // angle of index (hi ? 4 : 0) + q
            const double oc = __shfl_xor(cq, PARTNER);      // angle of index (hi ? 0 : 4) + q
            const double os = __shfl_xor(sq, PARTNER);
            const double xa = x(q), xb = x(4 + q);
            const double pa = __shfl_xor(xa, PARTNER), pb = __shfl_xor(xb, PARTNER);
            const double ca = hi_half ? oc : cq, sa_ = hi_half ? os : sq;   // index q
            const double cb = hi_half ? cq : oc, sb = hi_half ? sq : os;    // index 4 + q
            y[q] = hi_half ? xa * ca + pa * sa_ : xa * ca - pa * sa_;
            y[4 + q] = hi_half ? xb * cb + pb * sb : xb * cb - pb * sb;
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// Sequence that owns segment s: the last b with seq_seg_ptr[b] <= s, found
// with one ballot per 64 entries of seq_seg_ptr; -1 if none (or s lies past
// every sequence).
__device__ __forceinline__ int32_t find_sequence(const CoarsenArgs& a, int32_t s) {
    const int lane = threadIdx.x % kWave;
    int32_t cnt = 0;
    for (int32_t base = 0; base <= a.B; base += kWave) {
        const int32_t i = base + lane;
        const bool le = i <= a.B && a.seq_seg_ptr[min(i, a.B)] <= s;
        cnt += __popcll(__ballot(le));
    }
    return cnt - 1 < a.B ? cnt - 1 : -1;
}

// Streaming role: one segment's F-tokens summed in double precision, then the
// macro-node (mean key rotated to the mean position, mean value, alpha,
// beta) written to the staging area at (segment, head).  Needs nothing from
// the plan role, which runs at the same time.
//
// DIAG (diagonal closure, SPICY-KV demo page, Claim 3: the sub-grid variance
// as a diagonal vector): also the per-dimension variance of the member keys
// rotated to the anchor tbar.  Rotation mixes only the dimensions of one
// rotary pair (i, i + d/2), so with c, s the cosine and sine of tbar * theta_i
// and the pair's pre-rotation variances and covariance,
//     s2_i       = c^2 Var_i + s^2 Var_(i+d/2) - 2 c s Cov
//     s2_(i+d/2) = s^2 Var_i + c^2 Var_(i+d/2) + 2 c s Cov;
// one pass suffices: each lane also sums the product of its values with its
// rotary partner's (exchanged lane to lane), exact in double precision for
// bf16 inputs like the other sums.
//
// WEIGHTED (Equal-Variation KV Cache page, implementation notes: variation-
// weighted representatives): the key and value of the macro-node are
// sum w k / sum w and sum w v / sum w with one integer weight per token (the
// plain means when every weight of the segment's F-tokens is zero); mass,
// anchor, beta and s2 keep the plain sums.  w k is exact in double precision
// for bf16 k and w < 2^45, and so are the sums while they stay below 2^53.
template <typename T, int D, bool DIAG, bool WEIGHTED>
__device__ __forceinline__ void stream_segment(const CoarsenArgs& a, const Lanes<T, D>& L, int32_t s) {
    const int H = a.cache.H;
    // the segment bounds are the same for the whole wave: keep them in scalar registers
    const int32_t sa = __builtin_amdgcn_readfirstlane(a.seg_offsets[s]);
    const int32_t sz = __builtin_amdgcn_readfirstlane(a.seg_offsets[s + 1]);
    if (!(0 <= sa && sa < sz && sz <= a.total_tokens)) return;     // reported by the plan role
    const T* kin = static_cast<const T*>(a.k_pre);
    const T* vin = static_cast<const T*>(a.v);

    // masked sums of the F-tokens, double-buffered: block B (kRing tokens)
    // is in flight while block A is accumulated and vice versa.  Rows are read
    // through buffer resources spanning the segment (rebased every kWindow
    // tokens), the whole offset in the vector offset, which the hardware
    // range-checks: reads past the segment's end return zeros and touch no
    // memory.  A token that is not taken (protected, or past the end)
    // contributes through selects, not products with a zero weight, so
    // whatever its bytes hold (NaN, inf) adds nothing.  Positions are summed
    // relative to the segment's first token.
    constexpr int RING = kRing;
    double sk[8], sq[8], sv[8], sx[8], skw[8], svw[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) sk[r] = sq[r] = sv[r] = sx[r] = skw[r] = svw[r] = 0.0;
    double sw = 0.0;
    int32_t m = 0;
    int64_t prel = 0;
    struct Block {
        Row8<T> k[RING], v[RING];
        uint8_t mk[RING];
        int64_t wt[WEIGHTED ? RING : 1];
    };
    Block A, Bk;
    constexpr uint32_t kRow = static_cast<uint32_t>(D * sizeof(T));      // one head's row
    const uint32_t tok_bytes = static_cast<uint32_t>(H) * kRow;
    const uint32_t lane_off = static_cast<uint32_t>(L.hh) * kRow + static_cast<uint32_t>(L.d0 * sizeof(T));
    for (int32_t w0 = sa; w0 < sz; w0 += kWindow) {
        const int32_t wn = min(sz - w0, kWindow);
        const int64_t row0 = static_cast<int64_t>(w0) * H;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kin + row0 * D, static_cast<uint32_t>(wn) * tok_bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vin + row0 * D, static_cast<uint32_t>(wn) * tok_bytes);
        const __amdgpu_buffer_rsrc_t rm = make_rsrc(a.mask + row0, static_cast<uint32_t>(wn * H));
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(WEIGHTED ? a.token_weight + w0 : nullptr, WEIGHTED ? static_cast<uint32_t>(wn) * 8u : 0u);
        auto fetch = [&](Block& X, int32_t u0) {
#pragma unroll
            for (int u = 0; u < RING; ++u) {
                const uint32_t to = static_cast<uint32_t>(u0 + u) * tok_bytes;
                Row8<T>::load_buf(X.k[u], rk, lane_off + to, 0);
                Row8<T>::load_buf(X.v[u], rv, lane_off + to, 0);
                X.mk[u] = __builtin_amdgcn_raw_buffer_load_b8(rm, L.hh + (u0 + u) * H, 0, 0);
                if constexpr (WEIGHTED) {
                    // the token's weight, the same for every lane (0 past the window)
                    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 wv = __builtin_amdgcn_raw_buffer_load_b64(rw, (u0 + u) * 8, 0, 0);
                    X.wt[u] = static_cast<int64_t>((static_cast<uint64_t>(wv[1]) << 32) | wv[0]);
                }
            }
        };
        auto accumulate = [&](const Block& X, int32_t u0) {
            const int nvalid = min(RING, wn - u0);
#pragma unroll
            for (int u = 0; u < RING; ++u) {
                const bool take = (u < nvalid) && !X.mk[u];
                double tw = 0.0;
                if constexpr (WEIGHTED) {
                    tw = take ? static_cast<double>(X.wt[u]) : 0.0;
                    sw += tw;
                }
                Row8<T> kp;
                if constexpr (DIAG) kp = X.k[u].template lane_xor<Lanes<T, D>::PARTNER>();
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const double xw = take ? X.k[u].f64(r) : 0.0;
                    const double vw = take ? X.v[u].f64(r) : 0.0;
                    sk[r] += xw;
                    sq[r] = fma(xw, xw, sq[r]);
                    sv[r] += vw;
                    if constexpr (DIAG) sx[r] = fma(xw, take ? kp.f64(r) : 0.0, sx[r]);
                    if constexpr (WEIGHTED) {
                        skw[r] = fma(xw, tw, skw[r]);
                        svw[r] = fma(vw, tw, svw[r]);
                    }
                }
                m += take ? 1 : 0;
                prel += take ? static_cast<int64_t>(w0 - sa) + u0 + u : 0;
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // the barriers keep every load of one block ahead of the next block's,
        // so each wait covers only the token about to be accumulated
        fetch(A, 0);
        __builtin_amdgcn_sched_barrier(0);
        fetch(Bk, RING);
        __builtin_amdgcn_sched_barrier(0);
        // steady state refills a block only while it starts inside the
        // window; the last two blocks are drained without refills
        int32_t u0 = 0;
        for (; u0 + 2 * RING < wn; u0 += 2 * RING) {
            accumulate(A, u0);
            fetch(A, u0 + 2 * RING);
            __builtin_amdgcn_sched_barrier(0);
            accumulate(Bk, u0 + RING);
            fetch(Bk, u0 + 3 * RING);
            __builtin_amdgcn_sched_barrier(0);
        }
        accumulate(A, u0);
        if (u0 + RING < wn) accumulate(Bk, u0 + RING);
    }

    // the macro-node (all lanes take part in the shuffles)
    const int32_t b = find_sequence(a, s);
    if (b < 0) return;
    const int64_t pos_off = static_cast<int64_t>(a.pos_base ? a.pos_base[b] : 0) - a.seq_offsets[b];
    const int64_t psum = prel + static_cast<int64_t>(m) * (sa + pos_off);
    const double md = m > 0 ? static_cast<double>(m) : 1.0;
    double part = 0.0;
#pragma unroll
    for (int r = 0; r < 8; ++r) part += sq[r] - sk[r] * sk[r] / md;
#pragma unroll
    for (int o = 1; o < Lanes<T, D>::LPH; o <<= 1) part += __shfl_xor(part, o);
    const bool mine = L.active && m > 0;
    if (!__any(mine)) return;
    double y[8];
    const double tbar = static_cast<double>(psum) / md;
    // the representative: weighted means when the segment's weights are not all zero
    const bool wmean = WEIGHTED && sw > 0.0;
    L.rope([&](int r) { return wmean ? skw[r] / sw : sk[r] / md; }, tbar, y);
    double s2[8];
    if constexpr (DIAG) {
        constexpr int P = Lanes<T, D>::PARTNER;
        double var[8], cov[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const double skp = __shfl_xor(sk[r], P);
            var[r] = (sq[r] - sk[r] * sk[r] / md) / md;
            cov[r] = (sx[r] - sk[r] * skp / md) / md;     // the same value in both partner lanes
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            double c[2] = {1.0, 1.0}, sn[2] = {0.0, 0.0};
            if (L.rotate) L.angle(tbar, q, c[0], sn[0], c[1], sn[1]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int r = q + 4 * u;
                const double varp = __shfl_xor(var[r], P);
                const double c2s = 2.0 * c[u] * sn[u] * cov[r];
                const double v2 = c[u] * c[u] * var[r] + sn[u] * sn[u] * varp + (L.hi_half ? c2s : -c2s);
                s2[r] = v2 > 0.0 ? v2 : 0.0;
            }
        }
    }
    const int64_t idx = static_cast<int64_t>(s) * H + L.hh;
    // if the plan role has already published where this macro-node goes, it
    // is written there; otherwise it is staged for coarsen_cpoint.  The word
    // of the head's first lane decides for all 16 lanes of the head.
    const uint64_t w0 =
        a.gen != 0 ? __hip_atomic_load(&g_dest_hint[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
    const uint64_t w = static_cast<uint64_t>(__shfl(static_cast<long long>(w0), L.lane - L.j));
    if (!mine) return;
    const Dest dst = read_dest(w, a.gen);
    const double sigma2 = (part > 0.0 ? part : 0.0) / (md * D);
    const int64_t ph = static_cast<int64_t>(dst.ok ? dst.page : 0) * H + L.h;
    const int64_t row = dst.ok ? ph * kPage * D + slot_elem(dst.slot, L.d0) : idx * D + L.d0;
    if constexpr (DIAG) Pack8<T>::store(static_cast<T*>(dst.ok ? a.cache.s2 : a.stage_s2) + row, s2);
    Pack8<T>::store(static_cast<T*>(dst.ok ? a.cache.k : a.stage_k) + row, y);
    Store8<T>::store(static_cast<T*>(dst.ok ? a.cache.v : a.stage_v) + row,
                     [&](int r) { return Elem<T>::from_f64(wmean ? svw[r] / sw : sv[r] / md); });
    if (L.j == 0) {
        const int64_t ab_at = dst.ok ? ph * kPage + dst.slot : idx;
        T* ab = static_cast<T*>(dst.ok ? a.cache.ab : a.stage_ab);
        ab[ab_at * 2 + 0] = Elem<T>::from_f64(log(md));
        ab[ab_at * 2 + 1] = Elem<T>::from_f64(sigma2 / (2.0 * D));
        if (dst.ok && a.cache.meta) static_cast<Meta*>(a.cache.meta)[ab_at] = Meta{2, m, psum};
        // mass 0 tells coarsen_cpoint the macro-node is already in place
        a.stage_meta[idx] = make_int4(dst.ok ? 0 : m, b, static_cast<int32_t>(psum & 0xFFFFFFFF),
                                      static_cast<int32_t>(psum >> 32));
    }
}

// coarsen_main: workgroups x < B plan sequence x (with head group 0); the
// others are persistent streaming workgroups: wave w takes segments w,
// w + W, w + 2W, ...  The two roles share nothing, so they run side by side.
template <typename T, int D, bool DIAG, bool WEIGHTED>
__global__ __launch_bounds__(256, 2) void coarsen_main_kernel(CoarsenArgs a) {
    if (static_cast<int>(blockIdx.x) < a.B) {
        if (blockIdx.y == 0) plan_role<T, D>(a);
        return;
    }
    const int wave = threadIdx.x / kWave;
    const Lanes<T, D> L(a);
    const int32_t nstream = gridDim.x - a.B;
    const int32_t stride = nstream * (blockDim.x / kWave);
    for (int32_t s = (blockIdx.x - a.B) * (blockDim.x / kWave) + wave; s < a.n_seg; s += stride)
        stream_segment<T, D, DIAG, WEIGHTED>(a, L, s);
}

// Placing entries.  The plan role places the C-points it listed and each
// head's null padding (place_listed, below) while the streaming role runs;
// coarsen_cpoint then places the staged macro-nodes, spread over workgroups
// (x, b) and their 16-lane groups (8 at d = 64), unit u = (head, segment)
// head-major: the groups of a wavefront take consecutive segments of one
// head, whose entries are mostly consecutive slots, so their 16-byte pieces
// of each 8-dim group of the page land side by side.
template <typename T, int D>
__device__ __forceinline__ void place_macro(const CoarsenArgs& a, int b, int32_t s0, int32_t nseg, int64_t u, int d0,
                                            int j) {
    const int H = a.cache.H;
    const int32_t sg = s0 + static_cast<int32_t>(u % nseg);
    const int h = static_cast<int>(u / nseg);
    const int64_t idx = static_cast<int64_t>(sg) * H + h;
    // every read of the unit is independent: issue them together; the hint
    // is cleared once read (the array starts every call zero)
    const int32_t owner = a.seg_desc[sg].x;
    const int2 hd = a.seg_head[idx];
    const int4 mt = a.stage_meta[idx];
    if (a.gen != 0 && j == 0) __hip_atomic_store(&g_dest_hint[idx], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (owner != b) return;                             // sequence failed its checks
    const int32_t Pg = hd.y;                            // -1: no F-token in this head, or no page
    if (Pg < 0) return;
    if (mt.y != b || mt.x < 0) {
        raise_err(a.err, SPICY_DEVERR_SEGMENTS);
        return;
    }
    if (mt.x == 0) return;                              // written in place by the streaming role
    Row8<T> kx, vx, sx;
    kx.load(static_cast<const T*>(a.stage_k) + idx * D + d0);
    vx.load(static_cast<const T*>(a.stage_v) + idx * D + d0);
    if (a.cache.s2) sx.load(static_cast<const T*>(a.stage_s2) + idx * D + d0);
    const int slot = hd.x % kPage;
    const int64_t ph = static_cast<int64_t>(Pg) * H + h;
    Store8<T>::store(static_cast<T*>(a.cache.k) + ph * kPage * D + slot_elem(slot, d0),
                     [&](int r) { return kx.raw(r); });
    Store8<T>::store(static_cast<T*>(a.cache.v) + ph * kPage * D + slot_elem(slot, d0),
                     [&](int r) { return vx.raw(r); });
    if (a.cache.s2)
        Store8<T>::store(static_cast<T*>(a.cache.s2) + ph * kPage * D + slot_elem(slot, d0),
                         [&](int r) { return sx.raw(r); });
    if (j == 0) {
        const T* sab = static_cast<const T*>(a.stage_ab);
        T* abc = static_cast<T*>(a.cache.ab);
        abc[(ph * kPage + slot) * 2 + 0] = sab[idx * 2 + 0];
        abc[(ph * kPage + slot) * 2 + 1] = sab[idx * 2 + 1];
        if (a.cache.meta) {
            const int64_t ps = static_cast<int64_t>(static_cast<uint32_t>(mt.z)) |
                               (static_cast<int64_t>(mt.w) << 32);
            static_cast<Meta*>(a.cache.meta)[ph * kPage + slot] = Meta{2, mt.x, ps};
        }
    }
}

// A listed C-point {token, entry << 4 | head}: its rows and page are loaded
// by cp_fetch (indexes clamped, so a bad item never reads out of bounds) and
// stored exact by cp_store (value bits copied, key rotated to the token's own
// position, alpha = beta = 0).
template <typename T>
struct CpFetch {
    Row8<T> kx, vx;
    int32_t Pg;            // -1: nothing to store
    int32_t t;
    int h;
    int64_t e;
};

template <typename T, int D>
__device__ __forceinline__ CpFetch<T> cp_fetch(const CoarsenArgs& a, int b, int2 it, int32_t t0, int32_t t1, int d0) {
    const int H = a.cache.H;
    CpFetch<T> f;
    f.t = it.x;
    f.h = it.y & 15;
    f.e = static_cast<uint32_t>(it.y) >> 4;
    const bool sane = f.t >= t0 && f.t < t1 && f.h < H;
    const int64_t base = (static_cast<int64_t>(min(max(f.t, t0), t1 - 1)) * H + min(f.h, H - 1)) * D + d0;
    f.kx.load(static_cast<const T*>(a.k_pre) + base);
    f.vx.load(static_cast<const T*>(a.v) + base);
    if (!sane) raise_err(a.err, SPICY_DEVERR_SEGMENTS);
    f.Pg = sane ? entry_page(a, b, f.e) : -1;
    return f;
}

template <typename T, int D>
__device__ __forceinline__ void cp_store(const CoarsenArgs& a, const CpFetch<T>& f, int64_t pos_off,
                                         const double (&theta)[4], int d0, int j) {
    constexpr int PARTNER = D / 16;
    const int H = a.cache.H;
    const bool hi_half = j >= PARTNER;
    double y[8];
    if (a.rope_base > 0.0) {
        const double pos = static_cast<double>(f.t + pos_off);
        double c4[4], s4[4], cs[8], sn[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) sincos_f64(pos * theta[r], &s4[r], &c4[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const double oc = __shfl_xor(c4[r], PARTNER);
            const double os = __shfl_xor(s4[r], PARTNER);
            cs[r] = hi_half ? oc : c4[r];
            sn[r] = hi_half ? os : s4[r];
            cs[4 + r] = hi_half ? c4[r] : oc;
            sn[4 + r] = hi_half ? s4[r] : os;
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const double x = f.kx.f64(r);
            const double other = __shfl_xor(x, PARTNER);
            y[r] = hi_half ? x * cs[r] + other * sn[r] : x * cs[r] - other * sn[r];
        }
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) y[r] = f.kx.f64(r);
    }
    if (f.Pg < 0) return;
    const int slot = static_cast<int>(f.e % kPage);
    const int64_t ph = static_cast<int64_t>(f.Pg) * H + f.h;
    Pack8<T>::store(static_cast<T*>(a.cache.k) + ph * kPage * D + slot_elem(slot, d0), y);
    Store8<T>::store(static_cast<T*>(a.cache.v) + ph * kPage * D + slot_elem(slot, d0),
                     [&](int r) { return f.vx.raw(r); });
    const double zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (a.cache.s2) Pack8<T>::store(static_cast<T*>(a.cache.s2) + ph * kPage * D + slot_elem(slot, d0), zero);
    if (j == 0) {
        T* abc = static_cast<T*>(a.cache.ab);
        abc[(ph * kPage + slot) * 2 + 0] = Elem<T>::from_f32(0.f);
        abc[(ph * kPage + slot) * 2 + 1] = Elem<T>::from_f32(0.f);
        if (a.cache.meta) static_cast<Meta*>(a.cache.meta)[ph * kPage + slot] = Meta{1, 1, f.t + pos_off};
    }
}

template <typename T, int D>
__device__ __forceinline__ void place_null(const CoarsenArgs& a, int b, int h, int64_t e, int d0, int j) {
    const int H = a.cache.H;
    const int32_t Pg = entry_page(a, b, e);
    if (Pg < 0) return;
    const int slot = static_cast<int>(e % kPage);
    const int64_t ph = static_cast<int64_t>(Pg) * H + h;
    const double zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    Pack8<T>::store(static_cast<T*>(a.cache.k) + ph * kPage * D + slot_elem(slot, d0), zero);
    Pack8<T>::store(static_cast<T*>(a.cache.v) + ph * kPage * D + slot_elem(slot, d0), zero);
    if (a.cache.s2) Pack8<T>::store(static_cast<T*>(a.cache.s2) + ph * kPage * D + slot_elem(slot, d0), zero);
    if (j == 0) {
        T* abc = static_cast<T*>(a.cache.ab);
        abc[(ph * kPage + slot) * 2 + 0] = Elem<T>::from_f32(-__builtin_huge_valf());
        abc[(ph * kPage + slot) * 2 + 1] = Elem<T>::from_f32(0.f);
        if (a.cache.meta) static_cast<Meta*>(a.cache.meta)[ph * kPage + slot] = Meta{0, 0, 0};
    }
}

// The plan workgroup of sequence b places its n_cp listed C-points, a batch
// of kCpBatch per 16-lane group (8 at d = 64) with every load of the batch
// issued before any store, then each head's nulls from its own end up to
// `padded` (the end of the sequence's last page).
constexpr int kCpBatch = 4;

template <typename T, int D>
__device__ __forceinline__ void place_listed(const CoarsenArgs& a, int b, int32_t t0, int32_t t1, int64_t pos_off,
                                             const int2* items, int32_t n_cp, int64_t padded) {
    constexpr int LPH = D / 8;                // lanes per item
    constexpr int IPW = kWave / LPH;          // items per wavefront step
    constexpr int NG = kPlanWaves * IPW;      // groups of the workgroup
    constexpr int PARTNER = LPH / 2;
    const int H = a.cache.H;
    const int lane = threadIdx.x % kWave;
    const int grp = (threadIdx.x / kWave) * IPW + lane / LPH;
    const int j = lane % LPH;
    const int d0 = 8 * j;
    double theta[4];
    {
        const bool hi_half = j >= PARTNER;
        const int pair0 = 8 * (hi_half ? j - PARTNER : j) + (hi_half ? 4 : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) theta[r] = a.theta[pair0 + r];
    }
    for (int32_t k0 = 0; k0 < n_cp; k0 += kCpBatch * NG) {
        int2 it[kCpBatch];
#pragma unroll
        for (int i = 0; i < kCpBatch; ++i) {
            const int32_t k = k0 + i * NG + grp;
            it[i] = k < n_cp ? items[k] : make_int2(t0, 0);
        }
        CpFetch<T> f[kCpBatch];
#pragma unroll
        for (int i = 0; i < kCpBatch; ++i) f[i] = cp_fetch<T, D>(a, b, it[i], t0, t1, d0);
#pragma unroll
        for (int i = 0; i < kCpBatch; ++i) {
            if (k0 + i * NG + grp >= n_cp) f[i].Pg = -1;       // past the list: nothing to store
            cp_store<T, D>(a, f[i], pos_off, theta, d0, j);
        }
    }
    int64_t n_null = 0;
    for (int h = 0; h < H; ++h) {
        const int64_t c = padded - a.null_from[static_cast<int64_t>(b) * H + h];
        n_null += c > 0 ? c : 0;
    }
    for (int64_t u = grp; u < n_null; u += NG) {
        int64_t rem = u, e = 0;
        int h = 0;
        for (int q = 0; q < H; ++q) {
            const int64_t nf = a.null_from[static_cast<int64_t>(b) * H + q];
            const int64_t cnt = padded - nf > 0 ? padded - nf : 0;
            if (rem < cnt) {
                h = q;
                e = nf + rem;
                break;
            }
            rem -= cnt;
        }
        place_null<T, D>(a, b, h, e, d0, j);
    }
}

// coarsen_cpoint: the staged macro-nodes of sequence b, unit u = (head,
// segment) with a grid stride over the workgroups (x, b).
template <typename T, int D>
__global__ __launch_bounds__(256) void coarsen_cpoint_kernel(CoarsenArgs a) {
    constexpr int LPH = D / 8;                // lanes per item
    constexpr int IPW = kWave / LPH;          // items per wavefront step
    const int b = blockIdx.y;
    const int H = a.cache.H;
    const int32_t s0 = a.seq_seg_ptr[b], s1 = a.seq_seg_ptr[b + 1];
    const int64_t n_mac = (0 <= s0 && s0 <= s1 && s1 <= a.n_seg) ? static_cast<int64_t>(s1 - s0) * H : 0;
    const int lane = threadIdx.x % kWave;
    const int grp = (threadIdx.x / kWave) * IPW + lane / LPH;
    const int ngrp = (blockDim.x / kWave) * IPW;
    const int j = lane % LPH;
    const int d0 = 8 * j;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * ngrp;
    for (int64_t u = static_cast<int64_t>(blockIdx.x) * ngrp + grp; u < n_mac; u += stride)
        place_macro<T, D>(a, b, s0, s1 - s0, u, d0, j);
}

// ------------------------------------------------------------------ launch

template <typename T, int D>
spicy_status launch_coarsen_t(const CoarsenArgs& a, hipStream_t stream) {
    constexpr int HW = kWave / (D / 8);
    // plan workgroups (one per sequence) + persistent streaming workgroups
    const int wpb = 4;
    const int nstream = max(1, min((a.n_seg + wpb - 1) / wpb, kResidentBlocks));
    dim3 grid(a.B + nstream, (a.cache.H + HW - 1) / HW);
    const dim3 block(wpb * kWave);
    if (a.cache.s2 && a.token_weight)
        hipLaunchKernelGGL((coarsen_main_kernel<T, D, true, true>), grid, block, 0, stream, a);
    else if (a.cache.s2)
        hipLaunchKernelGGL((coarsen_main_kernel<T, D, true, false>), grid, block, 0, stream, a);
    else if (a.token_weight)
        hipLaunchKernelGGL((coarsen_main_kernel<T, D, false, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((coarsen_main_kernel<T, D, false, false>), grid, block, 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    // entries: the resident workgroups shared by the sequences
    // macro-nodes: about n_seg * H / B per sequence, one per 16-lane group
    // (16 groups per workgroup at d = 128, 32 at d = 64)
    const int per_wg = 4 * (kWave / (D / 8));
    const int64_t want = (static_cast<int64_t>(a.n_seg) * a.cache.H / std::max(a.B, 1) + per_wg - 1) / per_wg;
    const int64_t cap = std::min(kCpointBlocksPerSeq, kCpointResident / std::max(a.B, 1));
    const int cx = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(want, cap)));
    hipLaunchKernelGGL((coarsen_cpoint_kernel<T, D>), dim3(cx, a.B), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    return SPICY_OK;
}

// The library compiles this file once per (element type, head dim), with
// SPICY_COARSEN_PART = 0 .. 3; each object instantiates its own launcher
// (and kernels), and part 0 also holds the dispatcher.
#ifndef SPICY_COARSEN_PART
#define SPICY_COARSEN_PART 0
#endif
#if SPICY_COARSEN_PART == 0
template spicy_status launch_coarsen_t<uint16_t, 128>(const CoarsenArgs&, hipStream_t);
extern template spicy_status launch_coarsen_t<uint16_t, 64>(const CoarsenArgs&, hipStream_t);
extern template spicy_status launch_coarsen_t<float, 128>(const CoarsenArgs&, hipStream_t);
extern template spicy_status launch_coarsen_t<float, 64>(const CoarsenArgs&, hipStream_t);

spicy_status launch_coarsen(const CoarsenArgs& a, int dtype, int D, hipStream_t stream) {
    if (a.B == 0) return SPICY_OK;
    if (dtype == SPICY_BF16) {
        return D == 128 ? launch_coarsen_t<uint16_t, 128>(a, stream) : launch_coarsen_t<uint16_t, 64>(a, stream);
    }
    return D == 128 ? launch_coarsen_t<float, 128>(a, stream) : launch_coarsen_t<float, 64>(a, stream);
}

#elif SPICY_COARSEN_PART == 1
template spicy_status launch_coarsen_t<uint16_t, 64>(const CoarsenArgs&, hipStream_t);
#elif SPICY_COARSEN_PART == 2
template spicy_status launch_coarsen_t<float, 128>(const CoarsenArgs&, hipStream_t);
#elif SPICY_COARSEN_PART == 3
template spicy_status launch_coarsen_t<float, 64>(const CoarsenArgs&, hipStream_t);
#endif

}  // namespace spicy
