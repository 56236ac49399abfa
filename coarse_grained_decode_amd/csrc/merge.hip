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
// Two kernels:
//   merge_list  one wavefront per (sequence, head): reads the entry kinds 64
//               at a time (one ballot), pairs the macro-nodes in order with
//               a carried odd one, and lists the pairs in the workspace.
//   merge_pair  workgroups (x, sequence * H + head); every 16-lane group (8
//               at d = 64) merges one listed pair per round, a lane owning 8
//               dims as in the coarsening; the rounds of a wavefront are
//               uniform so that the rotary-partner shuffles see every lane.
#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

constexpr int kListWaves = 4;
constexpr int kResident = 1024;

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

__global__ __launch_bounds__(kListWaves * kWave) void merge_list_kernel(MergeArgs a) {
    const int lane = threadIdx.x % kWave;
    const int H = a.cache.H;
    const int64_t unit = static_cast<int64_t>(blockIdx.x) * kListWaves + threadIdx.x / kWave;
    if (unit >= static_cast<int64_t>(a.B) * H) return;
    const int b = static_cast<int>(unit / H);
    const int h = static_cast<int>(unit % H);
    const int32_t e0 = a.entry_begin[b], e1 = a.entry_end[b];
    int32_t npairs = 0;
    if (e0 < 0 || e0 > e1 || e1 - e0 > a.max_range) {
        if (lane == 0) {
            raise_err(a.err, SPICY_DEVERR_SEGMENTS);
            a.pair_count[unit] = 0;
        }
        return;
    }
    const MetaRec* meta = static_cast<const MetaRec*>(a.cache.meta);
    int2* out = a.pairs + unit * a.cap;
    int32_t carry = -1;                                  // the unpaired macro-node so far (uniform)
    // kBatch windows of 64 entries at a time: their page ids, then their
    // kinds, are requested together before the windows are paired in order
    constexpr int kBatch = 4;
    for (int32_t base0 = e0; base0 < e1; base0 += kBatch * kWave) {
        int32_t pg[kBatch];
        int32_t kind[kBatch];
#pragma unroll
        for (int w = 0; w < kBatch; ++w) {
            const int32_t e = base0 + w * kWave + lane;
            pg[w] = e < e1 ? page_of(a, b, e) : -1;
        }
#pragma unroll
        for (int w = 0; w < kBatch; ++w) {
            const int32_t e = base0 + w * kWave + lane;
            kind[w] = pg[w] >= 0 ? meta[(static_cast<int64_t>(pg[w]) * H + h) * kPage + e % kPage].kind : 0;
        }
#pragma unroll
        for (int w = 0; w < kBatch; ++w) {
            const int32_t base = base0 + w * kWave;
            const int32_t e = base + lane;
            const bool mac = kind[w] == 2;
            const uint64_t M = __ballot(mac);
            const int c = carry >= 0 ? 1 : 0;
            const int n = __popcll(M);
            if (mac) {
                const int r = __popcll(M & ((1ull << lane) - 1));   // rank among this window's macro-nodes
                const int p = c + r;                                 // place in the sequence carry, m_0, m_1, ...
                if (p & 1) {
                    const uint64_t below = M & ((1ull << lane) - 1);
                    const int32_t first = (r == 0) ? carry : base + (63 - __clzll(below));
                    const int32_t j = npairs + (p >> 1);
                    if (j < a.cap) out[j] = make_int2(first, e);
                    else raise_err(a.err, SPICY_DEVERR_CAPACITY);
                }
            }
            npairs += (c + n) >> 1;
            if ((c + n) & 1) carry = n > 0 ? base + (63 - __clzll(M)) : carry;
            else carry = -1;
        }
    }
    if (lane == 0) a.pair_count[unit] = npairs < a.cap ? npairs : a.cap;
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

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_pair_kernel(MergeArgs a) {
    constexpr int LPH = D / 8;                // lanes per pair
    constexpr int PPW = kWave / LPH;          // pairs per wavefront round
    constexpr int PARTNER = LPH / 2;          // lane distance to the rotary partner
    const int H = a.cache.H;
    const int64_t unit = blockIdx.y;          // sequence * H + head
    const int b = static_cast<int>(unit / H);
    const int h = static_cast<int>(unit % H);
    const int lane = threadIdx.x % kWave;
    const int j = lane % LPH;
    const int d0 = 8 * j;
    const bool hi_half = j >= PARTNER;
    const int wave_grp = (threadIdx.x / kWave) * PPW;
    const int ngrp = (blockDim.x / kWave) * PPW;
    const bool rotate = a.rope_base > 0.0;
    double theta[4];
    {
        const int pair0 = 8 * (hi_half ? j - PARTNER : j) + (hi_half ? 4 : 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) theta[r] = a.theta[pair0 + r];
    }
    // cos and sin at pos for the rotary pair of each of this lane's 8 dims
    auto angles = [&](double pos, double (&cs)[8], double (&sn)[8]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            double sq, cq;
            sincos_f64(pos * theta[q], &sq, &cq);
            const double oc = __shfl_xor(cq, PARTNER), os = __shfl_xor(sq, PARTNER);
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
            const double ps = __shfl_xor(x[r], PARTNER) * sn[r];
            y[r] = hi_half ? x[r] * cs[r] + ps : x[r] * cs[r] - ps;
        }
    };

    const int32_t count = a.pair_count[unit];
    const int64_t start = static_cast<int64_t>(blockIdx.x) * ngrp;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * ngrp;
    const MetaRec* meta = static_cast<const MetaRec*>(a.cache.meta);
    for (int64_t r0 = start; r0 < count; r0 += stride) {              // uniform over the workgroup
        const int64_t pj = r0 + wave_grp + lane / LPH;
        const bool live = pj < count;
        int32_t P1 = -1, P2 = -1, e1 = 0, e2 = 0;
        if (live) {
            const int2 pr = a.pairs[unit * a.cap + pj];
            e1 = pr.x;
            e2 = pr.y;
            P1 = page_of(a, b, e1);
            P2 = page_of(a, b, e2);
        }
        const bool ok = live && P1 >= 0 && P2 >= 0;
        const int64_t ph1 = static_cast<int64_t>(ok ? P1 : 0) * H + h, ph2 = static_cast<int64_t>(ok ? P2 : 0) * H + h;
        const int s1 = e1 % kPage, s2 = e2 % kPage;
        double k1[8], k2[8], v1[8], v2[8];
        double m1 = 1.0, m2 = 1.0, b1 = 0.0, b2 = 0.0;
        int64_t q1 = 0, q2 = 0;
        int32_t i1 = 1, i2 = 1;
        if (ok) {
            const T* kp = static_cast<const T*>(a.cache.k);
            const T* vp = static_cast<const T*>(a.cache.v);
            const T* ab = static_cast<const T*>(a.cache.ab);
            Vec8<T>::load(kp + ph1 * kPage * D + slot_elem(s1, d0), k1);
            Vec8<T>::load(kp + ph2 * kPage * D + slot_elem(s2, d0), k2);
            Vec8<T>::load(vp + ph1 * kPage * D + slot_elem(s1, d0), v1);
            Vec8<T>::load(vp + ph2 * kPage * D + slot_elem(s2, d0), v2);
            b1 = Elem<T>::to_f64(ab[(ph1 * kPage + s1) * 2 + 1]);
            b2 = Elem<T>::to_f64(ab[(ph2 * kPage + s2) * 2 + 1]);
            const MetaRec r1 = meta[ph1 * kPage + s1], r2 = meta[ph2 * kPage + s2];
            i1 = r1.mass;
            i2 = r2.mass;
            q1 = r1.pos_sum;
            q2 = r2.pos_sum;
            if (r1.kind != 2 || r2.kind != 2 || r1.mass <= 0 || r2.mass <= 0 ||
                static_cast<int64_t>(r1.mass) + r2.mass > 0x7FFFFFFF) {
                raise_err(a.err, SPICY_DEVERR_SEGMENTS);
                i1 = i2 = 0;                                  // not stored
            }
            m1 = i1 > 0 ? static_cast<double>(i1) : 1.0;
            m2 = i2 > 0 ? static_cast<double>(i2) : 1.0;
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r) k1[r] = k2[r] = v1[r] = v2[r] = 0.0;
        }
        const double m = m1 + m2;
        const int64_t P = q1 + q2;
        // R(tbar) mu = (m1 R(tbar - tbar_1) k1 + m2 R(tbar - tbar_2) k2) / m, and
        // |mu_1 - mu_2| is the norm of the difference of the two rotated keys
        // (rotations keep norms): two sets of angles instead of three
        const double tb = static_cast<double>(P) / m;
        double y1[8], y2[8], key[8], cs[8], sn[8];
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
        double dist = 0.0;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const double dm = y1[r] - y2[r];
            dist += dm * dm;
            key[r] = (m1 * y1[r] + m2 * y2[r]) / m;
            v1[r] = (m1 * v1[r] + m2 * v2[r]) / m;
        }
#pragma unroll
        for (int o = 1; o < LPH; o <<= 1) dist += __shfl_xor(dist, o);
        if (!ok || i1 <= 0) continue;
        const double sig = (m1 * (2.0 * D * b1) + m2 * (2.0 * D * b2)) / m + m1 * m2 * dist / (m * m * D);
        T* kp = static_cast<T*>(a.cache.k);
        T* vp = static_cast<T*>(a.cache.v);
        Vec8<T>::store(kp + ph1 * kPage * D + slot_elem(s1, d0), key);
        Vec8<T>::store(vp + ph1 * kPage * D + slot_elem(s1, d0), v1);
        const double zero[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        Vec8<T>::store(kp + ph2 * kPage * D + slot_elem(s2, d0), zero);
        Vec8<T>::store(vp + ph2 * kPage * D + slot_elem(s2, d0), zero);
        if (j == 0) {
            T* ab = static_cast<T*>(a.cache.ab);
            ab[(ph1 * kPage + s1) * 2 + 0] = Elem<T>::from_f64(log(m));
            ab[(ph1 * kPage + s1) * 2 + 1] = Elem<T>::from_f64(sig / (2.0 * D));
            ab[(ph2 * kPage + s2) * 2 + 0] = Elem<T>::from_f32(-__builtin_huge_valf());
            ab[(ph2 * kPage + s2) * 2 + 1] = Elem<T>::from_f32(0.f);
            MetaRec* mt = static_cast<MetaRec*>(a.cache.meta);
            mt[ph1 * kPage + s1] = MetaRec{2, i1 + i2, P};
            mt[ph2 * kPage + s2] = MetaRec{0, 0, 0};
        }
    }
}

template <typename T, int D>
spicy_status launch_merge_t(const MergeArgs& a, hipStream_t stream) {
    const int64_t units = static_cast<int64_t>(a.B) * a.cache.H;
    const int64_t lb = (units + kListWaves - 1) / kListWaves;
    hipLaunchKernelGGL(merge_list_kernel, dim3(static_cast<unsigned>(lb)), dim3(kListWaves * kWave), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    // about kResident workgroups over all (sequence, head) units; each takes
    // 16 (d = 128) or 32 (d = 64) pairs per round
    constexpr int ngrp = 4 * (kWave / (D / 8));
    const int64_t want = (static_cast<int64_t>(a.cap) + ngrp - 1) / ngrp;
    const int64_t cx = want < 1 ? 1 : (want < kResident / units + 1 ? want : kResident / units + 1);
    hipLaunchKernelGGL((merge_pair_kernel<T, D>), dim3(static_cast<unsigned>(cx), static_cast<unsigned>(units)),
                       dim3(256), 0, stream, a);
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
