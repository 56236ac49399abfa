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
//   coarsen_plan  one workgroup per sequence: counts the protected tokens of
//                 every (segment, head), scans the per-head entry counts into
//                 entry offsets, writes lengths_out and the null padding.
//   coarsen_main  one wavefront per segment and pair of KV heads: streams
//                 the segment's keys and values once (32 lanes per head, each
//                 lane owning d/64 rotary pairs), accumulates in double
//                 precision, writes C-points as they pass and the macro-node
//                 at the end.  The work is bound by reading K and V from HBM.
//
// Variance without a second pass: with c the first merged key of the
// segment, sum (k - mean)^2 = sum (k - c)^2 - (sum k - m c)^2 / m per
// dimension.  Inputs are bf16 (8 significant bits), so sum k, m c and
// sum (k - c)^2 are exact in double precision for any realistic segment and a
// segment of identical keys gives exactly zero.
#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

constexpr int kPlanThreads = 256;
constexpr int kHeadsPerWave = 2;
constexpr int kLanesPerHead = 32;
constexpr int kUnroll = 8;

struct Meta {
    int32_t kind;
    int32_t mass;
    int64_t pos_sum;
};

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Resolve logical entry e of sequence b to (physical page, slot); -1 on error.
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

template <typename T, int D>
__device__ void write_null(const CoarsenArgs& a, int b, int h, int64_t e, int elem) {
    // one thread writes element `elem` of the key row and value column;
    // element 0 also writes the sidecars and the metadata.
    const int32_t P = entry_page(a, b, e);
    if (P < 0) return;
    const int slot = static_cast<int>(e % kPage);
    const int64_t ph = static_cast<int64_t>(P) * a.cache.H + h;
    T* k = static_cast<T*>(a.cache.k);
    T* v = static_cast<T*>(a.cache.v);
    k[(ph * kPage + slot) * D + elem] = Elem<T>::from_f32(0.f);
    v[(ph * D + elem) * kPage + slot] = Elem<T>::from_f32(0.f);
    if (elem == 0) {
        T* ab = static_cast<T*>(a.cache.ab);
        ab[(ph * kPage + slot) * 2 + 0] = Elem<T>::from_f32(-__builtin_huge_valf());
        ab[(ph * kPage + slot) * 2 + 1] = Elem<T>::from_f32(0.f);
        if (a.cache.meta) {
            Meta* m = static_cast<Meta*>(a.cache.meta);
            m[ph * kPage + slot] = Meta{0, 0, 0};
        }
    }
}

}  // namespace

// ------------------------------------------------------------------- plan

template <typename T, int D>
__global__ __launch_bounds__(kPlanThreads) void coarsen_plan_kernel(CoarsenArgs a) {
    __shared__ int32_t s_total[64];
    __shared__ int32_t s_ok;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int nwaves = blockDim.x / kWave;
    const int H = a.cache.H;

    const int32_t t0 = a.seq_offsets[b], t1 = a.seq_offsets[b + 1];
    const int32_t s0 = a.seq_seg_ptr[b], s1 = a.seq_seg_ptr[b + 1];
    const int32_t e0 = a.entry_start ? a.entry_start[b] : 0;
    if (tid == 0) {
        bool ok = 0 <= t0 && t0 <= t1 && t1 <= a.total_tokens && 0 <= s0 && s0 <= s1 &&
                  s1 <= a.n_seg && e0 >= 0;
        if (ok) ok = a.seg_offsets[s0] == t0 && a.seg_offsets[s1] == t1;
        s_ok = ok;
        if (!ok) {
            raise_err(a.err, SPICY_DEVERR_SEGMENTS);
            a.lengths_out[b] = e0 < 0 ? 0 : e0;
        }
    }
    __syncthreads();
    if (!s_ok) return;

    // 1. protected-token count and entry count per (segment, head)
    for (int32_t s = s0 + wave; s < s1; s += nwaves) {
        int32_t sa = a.seg_offsets[s], sz = a.seg_offsets[s + 1];
        if (!(t0 <= sa && sa <= sz && sz <= t1)) {
            if (lane == 0) raise_err(a.err, SPICY_DEVERR_SEGMENTS);
            sa = sz = t0;                 // treated as empty by both kernels
        }
        for (int h = 0; h < H; ++h) {
            int c = 0;
            for (int32_t t = sa + lane; t < sz; t += kWave)
                c += a.mask[static_cast<int64_t>(t) * H + h] != 0;
            c = wave_sum(c);
            if (lane == 0) {
                a.seg_ncnt[static_cast<int64_t>(s) * H + h] = c;
                a.seg_start[static_cast<int64_t>(s) * H + h] = c + ((sz - sa - c) > 0 ? 1 : 0);
            }
        }
        if (lane == 0) a.seg_seq[s] = b;
    }
    __threadfence_block();
    __syncthreads();

    // 2. exclusive scan of the counts per head (one wave per head)
    for (int h = wave; h < H; h += nwaves) {
        int32_t running = e0;
        for (int32_t base = s0; base < s1; base += kWave) {
            const int32_t s = base + lane;
            const int c = s < s1 ? a.seg_start[static_cast<int64_t>(s) * H + h] : 0;
            int incl = c;
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            if (s < s1) a.seg_start[static_cast<int64_t>(s) * H + h] = running + incl - c;
            running += __shfl(incl, kWave - 1);
        }
        if (lane == 0) s_total[h] = running - e0;
    }
    __threadfence_block();
    __syncthreads();

    // 3. length and null padding
    int32_t most = 0;
    for (int h = 0; h < H; ++h) most = max(most, s_total[h]);
    const int64_t len = static_cast<int64_t>(e0) + most;
    const int64_t padded = (len + kPage - 1) / kPage * kPage;
    if (tid == 0) {
        a.lengths_out[b] = static_cast<int32_t>(len);
        if (padded / kPage > a.max_pages) raise_err(a.err, SPICY_DEVERR_CAPACITY);
    }
    for (int h = 0; h < H; ++h) {
        const int64_t first = static_cast<int64_t>(e0) + s_total[h];
        const int64_t n = (padded - first) * D;
        for (int64_t i = tid; i < n; i += blockDim.x)
            write_null<T, D>(a, b, h, first + i / D, static_cast<int>(i % D));
    }
}

// ------------------------------------------------------------------- main

template <typename T, int D>
__global__ __launch_bounds__(256) void coarsen_main_kernel(CoarsenArgs a) {
    constexpr int P = D / (2 * kLanesPerHead);   // rotary pairs per lane
    constexpr int HALF = D / 2;
    typedef T vecP __attribute__((ext_vector_type(P)));

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int32_t s = blockIdx.x * (blockDim.x / kWave) + wave;
    if (s >= a.n_seg) return;
    const int H = a.cache.H;
    const int hs = lane / kLanesPerHead;
    const int ql = lane % kLanesPerHead;
    const int h = blockIdx.y * kHeadsPerWave + hs;
    const bool active = h < H;

    // which sequence owns this segment; give up on anything inconsistent
    // (the same checks the plan kernel made, so that a segment is only
    // processed when its plan entries were written by this call)
    const int32_t b = a.seg_seq[s];
    if (b < 0 || b >= a.B) return;
    const int32_t s0 = a.seq_seg_ptr[b], s1 = a.seq_seg_ptr[b + 1];
    if (!(0 <= s0 && s0 <= s && s < s1 && s1 <= a.n_seg)) return;
    const int32_t t0 = a.seq_offsets[b], t1 = a.seq_offsets[b + 1];
    if (!(0 <= t0 && t0 <= t1 && t1 <= a.total_tokens)) return;
    if (a.seg_offsets[s0] != t0 || a.seg_offsets[s1] != t1) return;
    if (a.entry_start && a.entry_start[b] < 0) return;
    const int32_t sa = a.seg_offsets[s], sz = a.seg_offsets[s + 1];
    if (!(t0 <= sa && sa <= sz && sz <= t1)) return;
    const int64_t pos0 = a.pos_base ? a.pos_base[b] : 0;

    const int hh = active ? h : 0;
    const int32_t start = a.seg_start[static_cast<int64_t>(s) * H + hh];
    const int32_t ncnt = a.seg_ncnt[static_cast<int64_t>(s) * H + hh];
    const int hasF = (sz - sa - ncnt) > 0 ? 1 : 0;

    // frequencies of this lane's rotary pairs
    double theta[P];
    const bool rotate = a.rope_base > 0.0;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int pair = P * ql + i;
        theta[i] = rotate ? pow(a.rope_base, -2.0 * static_cast<double>(pair) / static_cast<double>(D)) : 0.0;
    }

    const T* kin = static_cast<const T*>(a.k_pre);
    const T* vin = static_cast<const T*>(a.v);
    T* kc = static_cast<T*>(a.cache.k);
    T* vc = static_cast<T*>(a.cache.v);
    T* abc = static_cast<T*>(a.cache.ab);
    Meta* meta = static_cast<Meta*>(a.cache.meta);

    double sk[2 * P], sv[2 * P], qk[2 * P];
#pragma unroll
    for (int i = 0; i < 2 * P; ++i) sk[i] = sv[i] = qk[i] = 0.0;
    vecP shift_lo = {}, shift_hi = {};
    int32_t m = 0;
    int64_t pos_sum = 0;
    int32_t rank = 0;

    auto rotate_store = [&](const double (&x)[2 * P], double pos, int64_t e, int32_t kind,
                            int32_t mass, int64_t psum, double alpha, double beta,
                            const T (&vraw)[2 * P], const double (&vmean)[2 * P], bool raw_v) {
        const int32_t Pg = entry_page(a, b, e);
        if (Pg < 0) return;
        const int slot = static_cast<int>(e % kPage);
        const int64_t ph = static_cast<int64_t>(Pg) * H + h;
        vecP lo, hi;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            double yl = x[i], yh = x[P + i];
            if (rotate) {
                double sn, cs;
                sincos(pos * theta[i], &sn, &cs);
                yl = x[i] * cs - x[P + i] * sn;
                yh = x[P + i] * cs + x[i] * sn;
            }
            lo[i] = Elem<T>::from_f64(yl);
            hi[i] = Elem<T>::from_f64(yh);
        }
        T* krow = kc + (ph * kPage + slot) * D;
        *reinterpret_cast<vecP*>(krow + P * ql) = lo;
        *reinterpret_cast<vecP*>(krow + HALF + P * ql) = hi;
        T* vcol = vc + ph * D * kPage + slot;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            vcol[(P * ql + i) * kPage] = raw_v ? vraw[i] : Elem<T>::from_f64(vmean[i]);
            vcol[(HALF + P * ql + i) * kPage] = raw_v ? vraw[P + i] : Elem<T>::from_f64(vmean[P + i]);
        }
        if (ql == 0) {
            abc[(ph * kPage + slot) * 2 + 0] = Elem<T>::from_f64(alpha);
            abc[(ph * kPage + slot) * 2 + 1] = Elem<T>::from_f64(beta);
            if (meta) meta[ph * kPage + slot] = Meta{kind, mass, psum};
        }
    };

    for (int32_t tb = sa; tb < sz; tb += kUnroll) {
        vecP klo[kUnroll], khi[kUnroll], vlo[kUnroll], vhi[kUnroll];
        uint8_t msk[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int32_t t = tb + u;
            if (active && t < sz) {
                const int64_t base = (static_cast<int64_t>(t) * H + h) * D;
                klo[u] = *reinterpret_cast<const vecP*>(kin + base + P * ql);
                khi[u] = *reinterpret_cast<const vecP*>(kin + base + HALF + P * ql);
                vlo[u] = *reinterpret_cast<const vecP*>(vin + base + P * ql);
                vhi[u] = *reinterpret_cast<const vecP*>(vin + base + HALF + P * ql);
                msk[u] = a.mask[static_cast<int64_t>(t) * H + h];
            } else {
                msk[u] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int32_t t = tb + u;
            if (!(active && t < sz)) continue;
            const int64_t pos = pos0 + (t - t0);
            double x[2 * P];
            T vr[2 * P];
#pragma unroll
            for (int i = 0; i < P; ++i) {
                x[i] = Elem<T>::to_f64(klo[u][i]);
                x[P + i] = Elem<T>::to_f64(khi[u][i]);
                vr[i] = vlo[u][i];
                vr[P + i] = vhi[u][i];
            }
            if (msk[u]) {
                // C-point: exact entry after the macro-node of this segment
                const int64_t e = static_cast<int64_t>(start) + hasF + rank;
                ++rank;
                rotate_store(x, static_cast<double>(pos), e, 1, 1, pos, 0.0, 0.0, vr, sv, true);
            } else {
                ++m;
                pos_sum += pos;
                if (m == 1) {
                    shift_lo = klo[u];
                    shift_hi = khi[u];
                }
#pragma unroll
                for (int i = 0; i < 2 * P; ++i) {
                    sk[i] += x[i];
                    const double c = Elem<T>::to_f64(i < P ? shift_lo[i] : shift_hi[i - P]);
                    const double dd = x[i] - c;
                    qk[i] += dd * dd;
                    sv[i] += Elem<T>::to_f64(vr[i]);
                }
            }
        }
    }

    // variance of the merged keys: per lane sum_i (Q_i - D_i^2/m) with
    // D_i = sum k_i - m c_i, then over the lanes of the head
    double part = 0.0;
    if (active && m > 0) {
#pragma unroll
        for (int i = 0; i < 2 * P; ++i) {
            const double c = Elem<T>::to_f64(i < P ? shift_lo[i] : shift_hi[i - P]);
            const double dsum = sk[i] - static_cast<double>(m) * c;
            part += qk[i] - dsum * dsum / static_cast<double>(m);
        }
    }
#pragma unroll
    for (int o = 1; o < kLanesPerHead; o <<= 1) part += __shfl_xor(part, o);

    if (active && m > 0) {
        double mean_k[2 * P], mean_v[2 * P];
#pragma unroll
        for (int i = 0; i < 2 * P; ++i) {
            mean_k[i] = sk[i] / static_cast<double>(m);
            mean_v[i] = sv[i] / static_cast<double>(m);
        }
        const double sigma2 = (part > 0.0 ? part : 0.0) / (static_cast<double>(m) * D);
        const double tbar = static_cast<double>(pos_sum) / static_cast<double>(m);
        T unused[2 * P];
        rotate_store(mean_k, tbar, start, 2, m, pos_sum, log(static_cast<double>(m)),
                     sigma2 / (2.0 * D), unused, mean_v, false);
    }
}

// ------------------------------------------------------------------ launch

template <typename T, int D>
static spicy_status launch_coarsen_t(const CoarsenArgs& a, hipStream_t stream) {
    if (a.B > 0) {
        hipLaunchKernelGGL((coarsen_plan_kernel<T, D>), dim3(a.B), dim3(kPlanThreads), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    }
    if (a.n_seg > 0) {
        const int wpb = 4;
        dim3 grid((a.n_seg + wpb - 1) / wpb, (a.cache.H + kHeadsPerWave - 1) / kHeadsPerWave);
        hipLaunchKernelGGL((coarsen_main_kernel<T, D>), grid, dim3(wpb * kWave), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    }
    return SPICY_OK;
}

spicy_status launch_coarsen(const CoarsenArgs& a, int dtype, int D, hipStream_t stream) {
    if (dtype == SPICY_BF16) {
        return D == 128 ? launch_coarsen_t<uint16_t, 128>(a, stream) : launch_coarsen_t<uint16_t, 64>(a, stream);
    }
    return D == 128 ? launch_coarsen_t<float, 128>(a, stream) : launch_coarsen_t<float, 64>(a, stream);
}

}  // namespace spicy
