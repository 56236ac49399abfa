// One level of the SPICY-KV dyadic merge cascade on gfx950.
//
// What is computed (SPICY-KV demo page: the cascaded dyadic ring-buffer
// pyramid, Claim 12; the law of total variance across cascades, Claim 10):
// for every sequence b and KV head h, the macro-nodes among entries
// [entry_begin[b], entry_end[b]) are paired in entry order (first with
// second, third with fourth, ...; an odd last one stays).  A pair with masses
// m1, m2, position sums P1, P2, stored keys k1, k2 (rotated to their anchors
// P_i / m_i), values v1, v2 and betas b1, b2 becomes, at the first entry,
//     m = m1 + m2, P = P1 + P2, tbar = P / m,
//     mu_i = R(-P_i / m_i) k_i,  mu = (m1 mu_1 + m2 mu_2) / m,
//     (computed as R(tbar) mu = (m1 R(tbar - tbar_1) k1 + m2 R(tbar - tbar_2) k2) / m)
//     v = (m1 v1 + m2 v2) / m,
//     sigma^2 = (m1 2d b1 + m2 2d b2) / m + m1 m2 |mu_1 - mu_2|^2 / (m^2 d),
//     key R(tbar) mu, alpha = ln m, beta = sigma^2 / (2d), meta {2, m, P},
// and the second entry becomes a null.  Everything in double precision,
// rounded once on store.  The sequence lengths do not change.
//
// One kernel, workgroups (x, sequence * H + head) of 4 wavefronts, cx of them
// per (sequence, head) unit:
//   every workgroup lists its unit's range itself, in windows of 1024
//   entries: page ids and entry kinds are read (one entry per thread per
//   round, every load of the window in flight together), a workgroup scan
//   ranks the macro-nodes, and pair i (macro-nodes 2i and 2i + 1 of the
//   range, the odd one of a window carried into the next) goes to LDS with
//   both entries and both pages.  Pairs come in blocks of one per 16-lane
//   group (8 at d = 64); block k belongs to workgroup k mod cx, and a group
//   takes its pairs two at a time, both pairs' rows loaded before either is
//   computed, a lane owning 8 dims as in the coarsening.  A workgroup writes
//   the merged key, value, alpha and beta and the null's key, value and
//   alpha, but no entry metadata: the kinds stay as they were while any
//   workgroup of the unit may still be listing.  Each workgroup then takes a
//   ticket from its unit's counter (device-scope atomic, after every load and
//   store of the workgroup has completed); the one that takes the last ticket
//   writes the metadata of every pair of the unit from the original records
//   ({2, m, P} at the first entry, a null record at the second, the same
//   checks as the merge itself), then resets the counter.  Nothing waits for
//   another workgroup.
#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kWin = 1024;                  // entries listed per window
constexpr int kResident = 512;              // merge_level workgroups resident at once (2 per CU)

struct MetaRec {
    int32_t kind;
    int32_t mass;
    int64_t pos_sum;
};

// Physical page of logical entry e of sequence b; -1 (and an error bit) when
// the table or the pool cannot hold it.
__device__ __forceinline__ int32_t page_of(const MergeArgs& a, int b, int64_t e) {
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

// 8 consecutive elements of a row as doubles, and back (one rounding).
template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, double (&x)[8]) {
        const uint4 w = *reinterpret_cast<const uint4*>(p);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = static_cast<double>(__uint_as_float(u[i] << 16));
            x[2 * i + 1] = static_cast<double>(__uint_as_float(u[i] & 0xFFFF0000u));
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const double (&y)[8]) {
        uint4 o;
        o.x = f64_to_bf16(y[0]) | (static_cast<uint32_t>(f64_to_bf16(y[1])) << 16);
        o.y = f64_to_bf16(y[2]) | (static_cast<uint32_t>(f64_to_bf16(y[3])) << 16);
        o.z = f64_to_bf16(y[4]) | (static_cast<uint32_t>(f64_to_bf16(y[5])) << 16);
        o.w = f64_to_bf16(y[6]) | (static_cast<uint32_t>(f64_to_bf16(y[7])) << 16);
        *reinterpret_cast<uint4*>(p) = o;
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, double (&x)[8]) {
        const float4 lo = *reinterpret_cast<const float4*>(p);
        const float4 hi = *reinterpret_cast<const float4*>(p + 4);
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w;
        x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    }
    static __device__ __forceinline__ void store(float* p, const double (&y)[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(static_cast<float>(y[0]), static_cast<float>(y[1]),
                                                    static_cast<float>(y[2]), static_cast<float>(y[3]));
        *reinterpret_cast<float4*>(p + 4) = make_float4(static_cast<float>(y[4]), static_cast<float>(y[5]),
                                                        static_cast<float>(y[6]), static_cast<float>(y[7]));
    }
};

// 8 consecutive elements of a row as stored (converted to double when used).
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
    uint4 x;
    __device__ __forceinline__ void load(const uint16_t* p) { x = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void zero() { x = make_uint4(0u, 0u, 0u, 0u); }
    __device__ __forceinline__ void f64(double (&y)[8]) const {
        const uint32_t u[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[2 * i] = static_cast<double>(__uint_as_float(u[i] << 16));
            y[2 * i + 1] = static_cast<double>(__uint_as_float(u[i] & 0xFFFF0000u));
        }
    }
};
template <> struct Raw8<float> {
    float4 lo, hi;
    __device__ __forceinline__ void load(const float* p) {
        lo = *reinterpret_cast<const float4*>(p);
        hi = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void zero() { lo = hi = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void f64(double (&y)[8]) const {
        y[0] = lo.x; y[1] = lo.y; y[2] = lo.z; y[3] = lo.w;
        y[4] = hi.x; y[5] = hi.y; y[6] = hi.z; y[7] = hi.w;
    }
};

// One listed pair's inputs, loaded by pair_load and merged by pair_store.
template <typename T>
struct PairIn {
    Raw8<T> k1, k2, v1, v2;
    T b1, b2;
    MetaRec r1, r2;
    int64_t ph1, ph2;
    int s1, s2;
    bool ok;
};

// A pair's records are merged when both are macro-nodes of positive mass
// whose mass sum fits int32 (else the pair is skipped and flagged).
__device__ __forceinline__ bool pair_ok(const MetaRec& r1, const MetaRec& r2) {
    return r1.kind == 2 && r2.kind == 2 && r1.mass > 0 && r2.mass > 0 &&
           static_cast<int64_t>(r1.mass) + r2.mass <= 0x7FFFFFFF;
}

template <typename T, int D>
__device__ __forceinline__ void pair_load(const MergeArgs& a, int h, bool live, int32_t e1, int32_t P1, int32_t e2,
                                          int32_t P2, const MetaRec& r1, const MetaRec& r2, int d0, PairIn<T>& in) {
    const int H = a.cache.H;
    in.ok = live && P1 >= 0 && P2 >= 0;
    in.ph1 = static_cast<int64_t>(in.ok ? P1 : 0) * H + h;
    in.ph2 = static_cast<int64_t>(in.ok ? P2 : 0) * H + h;
    in.s1 = e1 % kPage;
    in.s2 = e2 % kPage;
    in.b1 = in.b2 = T(0);
    in.r1 = in.r2 = MetaRec{0, 0, 0};
    if (in.ok) {
        const T* kp = static_cast<const T*>(a.cache.k);
        const T* vp = static_cast<const T*>(a.cache.v);
        const T* ab = static_cast<const T*>(a.cache.ab);
        in.k1.load(kp + in.ph1 * kPage * D + slot_elem(in.s1, d0));
        in.k2.load(kp + in.ph2 * kPage * D + slot_elem(in.s2, d0));
        in.v1.load(vp + in.ph1 * kPage * D + slot_elem(in.s1, d0));
        in.v2.load(vp + in.ph2 * kPage * D + slot_elem(in.s2, d0));
        in.b1 = ab[(in.ph1 * kPage + in.s1) * 2 + 1];
        in.b2 = ab[(in.ph2 * kPage + in.s2) * 2 + 1];
        in.r1 = r1;
        in.r2 = r2;
    } else {
        in.k1.zero();
        in.k2.zero();
        in.v1.zero();
        in.v2.zero();
    }
}

// The merge of one pair (every lane of the wavefront takes part in the
// shuffles, live or not).
template <typename T, int D>
__device__ __forceinline__ void pair_store(const MergeArgs& a, const PairIn<T>& in, int j, bool hi_half,
                                           bool rotate, const double (&theta)[4]) {
    constexpr int LPH = D / 8;                // lanes per pair
    constexpr int PARTNER = LPH / 2;          // lane distance to the rotary partner
    int32_t i1 = in.r1.mass, i2 = in.r2.mass;
    if (in.ok && !pair_ok(in.r1, in.r2)) {
        raise_err(a.err, SPICY_DEVERR_SEGMENTS);
        i1 = i2 = 0;                                          // not stored
    }
    const double m1 = in.ok && i1 > 0 ? static_cast<double>(i1) : 1.0;
    const double m2 = in.ok && i2 > 0 ? static_cast<double>(i2) : 1.0;
    const int64_t q1 = in.ok ? in.r1.pos_sum : 0, q2 = in.ok ? in.r2.pos_sum : 0;
    // cos and sin at pos for the rotary pair of each of this lane's 8 dims
    // (the partner's values through DPP lane moves)
    auto angles = [&](double pos, double (&cs)[8], double (&sn)[8]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            double sq, cq;
            sincos_f64(pos * theta[q], &sq, &cq);
            const double oc = dpp_xor_f64<PARTNER>(cq), os = dpp_xor_f64<PARTNER>(sq);
            cs[q] = hi_half ? oc : cq;
            sn[q] = hi_half ? os : sq;
            cs[4 + q] = hi_half ? cq : oc;
            sn[4 + q] = hi_half ? sq : os;
        }
    };
    // y = R(angle) x for this lane's dims
    auto rot = [&](const double (&x)[8], const double (&cs)[8], const double (&sn)[8], double (&y)[8]) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const double ps = dpp_xor_f64<PARTNER>(x[r]) * sn[r];
            y[r] = hi_half ? x[r] * cs[r] + ps : x[r] * cs[r] - ps;
        }
    };
    const double m = m1 + m2;
    const int64_t P = q1 + q2;
    double k1[8], k2[8];
    in.k1.f64(k1);
    in.k2.f64(k2);
    const double b1 = Elem<T>::to_f64(in.b1), b2 = Elem<T>::to_f64(in.b2);
    // R(tbar) mu = (m1 R(tbar - tbar_1) k1 + m2 R(tbar - tbar_2) k2) / m, and
    // |mu_1 - mu_2| is the norm of the difference of the two rotated keys
    // (rotations keep norms): two sets of angles instead of three
    const double tb = static_cast<double>(P) / m;
    double y1[8], y2[8], key[8], val[8], cs[8], sn[8];
    if (rotate) {
        angles(tb - static_cast<double>(q1) / m1, cs, sn);
        rot(k1, cs, sn, y1);
        angles(tb - static_cast<double>(q2) / m2, cs, sn);
        rot(k2, cs, sn, y2);
    } else {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            y1[r] = k1[r];
            y2[r] = k2[r];
        }
    }
    // the weighted means with one reciprocal of m (the double-precision
    // value moves by at most an ulp of double before the storage rounding)
    const double inv_m = 1.0 / m;
    double dist = 0.0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const double dm = y1[r] - y2[r];
        dist += dm * dm;
        key[r] = (m1 * y1[r] + m2 * y2[r]) * inv_m;
    }
    {
        double v1[8], v2[8];
        in.v1.f64(v1);
        in.v2.f64(v2);
#pragma unroll
        for (int r = 0; r < 8; ++r) val[r] = (m1 * v1[r] + m2 * v2[r]) * inv_m;
    }
    // sum over the pair's lanes (LPH = 16 or 8)
    dist += dpp_xor_f64<1>(dist);
    dist += dpp_xor_f64<2>(dist);
    dist += dpp_xor_f64<4>(dist);
    if constexpr (LPH == 16) dist += dpp_xor_f64<8>(dist);
    if (!in.ok || i1 <= 0) return;
    const double sig = (m1 * (2.0 * D * b1) + m2 * (2.0 * D * b2)) / m + m1 * m2 * dist / (m * m * D);
    T* kp = static_cast<T*>(a.cache.k);
    T* vp = static_cast<T*>(a.cache.v);
    const int d0 = 8 * j;
    Vec8<T>::store(kp + in.ph1 * kPage * D + slot_elem(in.s1, d0), key);
    Vec8<T>::store(vp + in.ph1 * kPage * D + slot_elem(in.s1, d0), val);
    const double zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    Vec8<T>::store(kp + in.ph2 * kPage * D + slot_elem(in.s2, d0), zero);
    Vec8<T>::store(vp + in.ph2 * kPage * D + slot_elem(in.s2, d0), zero);
    if (j == 0) {
        T* ab = static_cast<T*>(a.cache.ab);
        ab[(in.ph1 * kPage + in.s1) * 2 + 0] = Elem<T>::from_f64(log(m));
        ab[(in.ph1 * kPage + in.s1) * 2 + 1] = Elem<T>::from_f64(sig / (2.0 * D));
        ab[(in.ph2 * kPage + in.s2) * 2 + 0] = Elem<T>::from_f32(-__builtin_huge_valf());
        ab[(in.ph2 * kPage + in.s2) * 2 + 1] = Elem<T>::from_f32(0.f);
    }
}

// Lists the macro-nodes of the window [w0, min(w0 + kWin, e1)) of sequence b,
// head h, after the carried one (slot 0 when `carried`): entries in l_e,
// pages in l_p, metadata records in l_r, in entry order.  Returns their
// number, the carried one included.  Every thread of the workgroup calls it.
__device__ __forceinline__ int32_t list_window(const MergeArgs& a, int b, int h, int32_t w0, int32_t e1,
                                               int32_t carried, int32_t* l_e, int32_t* l_p, MetaRec* l_r,
                                               int32_t* w_cnt) {
    constexpr int kRounds = kWin / kThreads;
    const int H = a.cache.H;
    const int t = threadIdx.x, lane = t % kWave, wave = t / kWave;
    const MetaRec* meta = static_cast<const MetaRec*>(a.cache.meta);
    int32_t pg[kRounds];
    MetaRec rec[kRounds];
    bool mac[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const int32_t e = w0 + r * kThreads + t;
        pg[r] = e < e1 ? page_of(a, b, e) : -1;
    }
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const int32_t e = w0 + r * kThreads + t;
        rec[r] = pg[r] >= 0 ? meta[(static_cast<int64_t>(pg[r]) * H + h) * kPage + e % kPage] : MetaRec{0, 0, 0};
        mac[r] = rec[r].kind == 2;
    }
    int32_t base = carried;                   // list slot of this round's first macro-node
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
        const uint64_t M = __ballot(mac[r]);
        if (lane == 0) w_cnt[wave] = __popcll(M);
        __syncthreads();
        int32_t before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            before += w < wave ? w_cnt[w] : 0;
            total += w_cnt[w];
        }
        if (mac[r]) {
            const int32_t slot = base + before + __popcll(M & ((1ull << lane) - 1ull));
            l_e[slot] = w0 + r * kThreads + t;
            l_p[slot] = pg[r];
            l_r[slot] = rec[r];
        }
        base += total;
        __syncthreads();                      // w_cnt is rewritten by the next round; the list is complete
    }
    return base;
}

// The odd last macro-node of a window becomes slot 0 of the next one.
__device__ __forceinline__ void carry_last(int32_t n, int32_t* l_e, int32_t* l_p, MetaRec* l_r) {
    const int32_t odd = n & 1;
    const int32_t last_e = odd ? l_e[n - 1] : 0, last_p = odd ? l_p[n - 1] : 0;
    const MetaRec last_r = odd ? l_r[n - 1] : MetaRec{0, 0, 0};
    __syncthreads();                          // every read of the list is done
    if (odd && threadIdx.x == 0) {
        l_e[0] = last_e;
        l_p[0] = last_p;
        l_r[0] = last_r;
    }
    __syncthreads();
}

// The metadata of the listed pairs 0 .. np-1 (one pair per thread), from
// their records as listed: the merged record at the first entry, a null
// record at the second.
__device__ __forceinline__ void write_meta(const MergeArgs& a, int h, const int32_t* l_e, const int32_t* l_p,
                                           const MetaRec* l_r, int32_t np) {
    const int H = a.cache.H;
    MetaRec* meta = static_cast<MetaRec*>(a.cache.meta);
    for (int32_t i = threadIdx.x; i < np; i += kThreads) {
        const int32_t P1 = l_p[2 * i], P2 = l_p[2 * i + 1];
        if (P1 < 0 || P2 < 0) continue;
        const int64_t x1 = (static_cast<int64_t>(P1) * H + h) * kPage + l_e[2 * i] % kPage;
        const int64_t x2 = (static_cast<int64_t>(P2) * H + h) * kPage + l_e[2 * i + 1] % kPage;
        const MetaRec r1 = l_r[2 * i], r2 = l_r[2 * i + 1];
        if (!pair_ok(r1, r2)) continue;
        meta[x1] = MetaRec{2, r1.mass + r2.mass, r1.pos_sum + r2.pos_sum};
        meta[x2] = MetaRec{0, 0, 0};
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_level_kernel(MergeArgs a) {
    constexpr int LPH = D / 8;                // lanes per pair
    constexpr int PPW = kWave / LPH;          // pairs per wavefront round
    constexpr int NG = kWaves * PPW;          // groups of the workgroup: pairs per block
    constexpr int PARTNER = LPH / 2;
    __shared__ int32_t l_e[kWin + 1];         // the window's macro-nodes in order (slot 0: the carried one)
    __shared__ int32_t l_p[kWin + 1];         // their pages
    __shared__ MetaRec l_r[kWin + 1];         // their metadata records
    __shared__ int32_t w_cnt[kWaves];
    __shared__ int32_t s_last;
    const int H = a.cache.H;
    const int64_t unit = blockIdx.y;          // sequence * H + head
    const int b = static_cast<int>(unit / H);
    const int h = static_cast<int>(unit % H);
    const int lane = threadIdx.x % kWave;
    const int j = lane % LPH;
    const int d0 = 8 * j;
    const bool hi_half = j >= PARTNER;
    const int grp = (threadIdx.x / kWave) * PPW + lane / LPH;
    const bool rotate = a.rope_base > 0.0;
    const int32_t cx = static_cast<int32_t>(gridDim.x), x = static_cast<int32_t>(blockIdx.x);
    double theta[4];
    {
        const int pair0 = 8 * (hi_half ? j - PARTNER : j) + (hi_half ? 4 : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) theta[r] = a.theta[pair0 + r];
    }
    const int32_t e0 = a.entry_begin[b], e1 = a.entry_end[b];
    if (e0 < 0 || e0 > e1 || e1 - e0 > a.max_range) {
        if (threadIdx.x == 0 && x == 0) raise_err(a.err, SPICY_DEVERR_SEGMENTS);
        return;                               // uniform over the unit's workgroups: no ticket taken
    }
    int32_t carried = 0;
    int32_t done = 0;                         // pairs of the range before this window
    int32_t n = 0;
    for (int32_t w0 = e0; w0 < e1; w0 += kWin) {
        n = list_window(a, b, h, w0, e1, carried, l_e, l_p, l_r, w_cnt);
        const int32_t q_lo = done, q_hi = done + n / 2;
        // this workgroup's blocks k = x, x + cx, ... of the window's pairs,
        // two blocks per pass (uniform over the workgroup)
        int32_t k = q_lo / NG;
        k += ((x - k % cx) % cx + cx) % cx;
        for (; static_cast<int64_t>(k) * NG < q_hi; k += 2 * cx) {
            PairIn<T> in[2];
            bool any[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int64_t q = (static_cast<int64_t>(k) + u * cx) * NG + grp;
                const bool live = q >= q_lo && q < q_hi;
                any[u] = __any(live);             // uniform over the wavefront
                const int32_t i = live ? static_cast<int32_t>(q - q_lo) : 0;
                pair_load<T, D>(a, h, live, l_e[2 * i], l_p[2 * i], l_e[2 * i + 1], l_p[2 * i + 1], l_r[2 * i],
                                l_r[2 * i + 1], d0, in[u]);
            }
            // a wavefront whose pairs of this pass are all past the count
            // skips their arithmetic (its lanes only ever exchange values
            // among themselves), which leaves the SIMD's fp64 unit to the others
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (any[u]) pair_store<T, D>(a, in[u], j, hi_half, rotate, theta);
        }
        done = q_hi;
        carried = n & 1;
        if (w0 + kWin < e1) carry_last(n, l_e, l_p, l_r);
    }
    // arrival: every load and store of this workgroup has completed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int32_t old = __hip_atomic_fetch_add(a.ticket + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old >= cx) raise_err(a.err, SPICY_DEVERR_TICKET);
        s_last = old == cx - 1;
    }
    __syncthreads();
    if (!s_last) return;
    // the last workgroup of the unit: every listing is done, so the records
    // can change now (a range of one window is still listed in LDS; a
    // longer one is listed again, from the unchanged records)
    if (e1 - e0 <= kWin) {
        write_meta(a, h, l_e, l_p, l_r, n / 2);
    } else {
        carried = 0;
        for (int32_t w0 = e0; w0 < e1; w0 += kWin) {
            n = list_window(a, b, h, w0, e1, carried, l_e, l_p, l_r, w_cnt);
            write_meta(a, h, l_e, l_p, l_r, n / 2);
            carried = n & 1;
            if (w0 + kWin < e1) carry_last(n, l_e, l_p, l_r);
        }
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.ticket + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, int D>
spicy_status launch_merge_t(const MergeArgs& a, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(a.B) * a.cache.H;
    // at most kResident workgroups over all (sequence, head) units, so that
    // they all run at once (a second round of workgroups doubles the time);
    // each takes 2 x 16 (d = 128) or 2 x 32 (d = 64) pairs per pass
    constexpr int ngrp = kWaves * (kWave / (D / 8));
    const int64_t want = (static_cast<int64_t>(a.cap) + 2 * ngrp - 1) / (2 * ngrp);
    const int64_t fill = kResident / units > 1 ? kResident / units : 1;
    const int64_t cx = want < 1 ? 1 : (want < fill ? want : fill);
    hipLaunchKernelGGL((merge_level_kernel<T, D>), dim3(static_cast<unsigned>(cx), static_cast<unsigned>(units)),
                       dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    return SPICY_OK;
}

}  // namespace

spicy_status launch_merge(const MergeArgs& a, int dtype, int D, hipStream_t stream) {
    if (a.B == 0) return SPICY_OK;                 // with cap = 0 the listing still flags non-empty ranges
    if (dtype == SPICY_BF16) return D == 128 ? launch_merge_t<uint16_t, 128>(a, stream) : launch_merge_t<uint16_t, 64>(a, stream);
    return D == 128 ? launch_merge_t<float, 128>(a, stream) : launch_merge_t<float, 64>(a, stream);
}

}  // namespace spicy
