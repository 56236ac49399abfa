// SPICY-KV decode attention on gfx950: split-K over 16-entry pages + a
// log-sum-exp combine.
//
// Logit (SPICY-KV demo page, section "2. FlashAttention-2/3 & PagedAttention
// Online-Softmax Kernel Fusion"; Claim 3):
//     s = q.k / sqrt(d) + alpha + |q|^2 * beta
// followed by an ordinary online softmax.  Everything runs in base 2:
// s2 = s * log2(e), so p = exp2(s2 - m2) and LSE = ln2 * (m2 + log2 l).
//
// bf16 caches (decode_mfma_kernel): one wavefront owns one (sequence, KV head,
// split).  The G = H_q / H_kv query heads sharing the KV head are packed into
// the 16 columns of MFMA tiles, so every key and value byte is read from HBM
// once per KV head:
//   S^T[16 entries x 16 heads] = K_page[16 x d] . Q^T[d x 16]
//       d/32 x v_mfma_f32_16x16x32_bf16, K rows straight from the page
//       (lane l holds entry l%16, 8 dims of each 32-dim chunk)
//   the accumulator layout of S^T (lane l: entries 4(l/16)+j, head l%16) is
//   exactly the B operand of the next product, so the probabilities go from
//   exp2 to bf16 to MFMA without any lane exchange:
//   O^T[d x 16 heads] += V^T_page[d x 16 entries] . P^T[16 entries x 16 heads]
//       d/16 x v_mfma_f32_16x16x16_bf16, value tiles stored dim-major in the
//       page so each lane's 4 entries of one dimension are 8 contiguous bytes.
// Pages are prefetched NBUF deep in registers; page ids are scalar loads.
//
// fp32 caches (decode_f32_kernel): a plain VALU kernel, one wavefront per
// (sequence, query head, split), lanes = 16 entries x 4 quarter-rows.
//
// combine_kernel merges the splits of each (sequence, query head) by
// log-sum-exp and writes O (fp32) and LSE (natural log).
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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Clamp a sequence's length to what its page table row can address.
__device__ __forceinline__ int32_t checked_length(const DecodeArgs& a, int b) {
    int32_t len = a.lengths[b];
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

template <int D>
struct PageRegs {
    bf16x8 k[D / 32];      // K rows: entry lane%16, dims 32i + 8(lane/16) .. +8
    s16x4 v[D / 16];       // V^T tile t: dim 16t + lane%16, entries 4(lane/16) .. +4
    bf16x8 ab;             // (alpha, beta) of entries 4(lane/16) .. +4
    bool ok;
};

}  // namespace

// ---------------------------------------------------------------- bf16 MFMA

template <int D, int NBUF>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
    constexpr int KC = D / 32;
    constexpr int NT = D / 16;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int row = lane % 16;     // entry (A rows) / query head (B, C columns)
    const int grp = lane / 16;
    const int split = blockIdx.x * (blockDim.x / kWave) + wave;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int H = a.cache.H;
    const int G = a.H_q / H;
    if (split >= a.splits) return;

    const int32_t len = checked_length(a, b);
    const int32_t npages = (len + kPage - 1) / kPage;
    const int32_t p0 = split * a.pages_per_split;
    const int32_t p1 = min(p0 + a.pages_per_split, npages);
    if (p0 >= p1) return;

    // query operand (B of S^T = K Q^T): lane holds head `row`, 8 dims per chunk
    const uint16_t* qbase = static_cast<const uint16_t*>(a.q) +
                            (static_cast<int64_t>(b) * a.H_q + static_cast<int64_t>(h) * G + row) * D;
    bf16x8 qv[KC];
    float n2 = 0.f;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        if (row < G) {
            qv[i] = *reinterpret_cast<const bf16x8*>(qbase + 32 * i + 8 * grp);
        } else {
            qv[i] = bf16x8{};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float x = static_cast<float>(qv[i][j]);
            n2 += x * x;
        }
    }
    n2 += __shfl_xor(n2, 16);
    n2 += __shfl_xor(n2, 32);
    const float c_dot = kLog2e / sqrtf(static_cast<float>(D));
    const float c_beta = n2 * kLog2e;

    const uint16_t* kpool = static_cast<const uint16_t*>(a.cache.k);
    const uint16_t* vpool = static_cast<const uint16_t*>(a.cache.v);
    const uint16_t* abpool = static_cast<const uint16_t*>(a.cache.ab);
    const int32_t* table = a.page_table + static_cast<int64_t>(b) * a.max_pages;

    // Page ids of the split, 64 at a time: one vector load, then each page's
    // id is read out of its lane (uniform).  Pages past the split's end and
    // invalid ids load a valid page (so that every load is unconditional and
    // each wait covers exactly one page); they are skipped when processed.
    int32_t ids = 0;
    int32_t ids_base = -kWave;
    auto page_id = [&](int32_t lp) {
        const int32_t q = min(lp, p1 - 1);
        if (q - ids_base >= kWave) {            // uniform
            ids_base = q;
            ids = (q + lane < p1) ? table[q + lane] : 0;
        }
        return __builtin_amdgcn_readlane(ids, q - ids_base);
    };
    auto load = [&](PageRegs<D>& r, int32_t lp) {
        const int32_t pid = page_id(lp);
        r.ok = pid >= 0 && pid < a.cache.num_pages;
        if (!r.ok) raise_err(a.err, SPICY_DEVERR_PAGE_ID);
        const int64_t ph = static_cast<int64_t>(r.ok ? pid : 0) * H + h;
        const uint16_t* kp = kpool + ph * kPage * D + row * D + 8 * grp;
#pragma unroll
        for (int i = 0; i < KC; ++i) r.k[i] = *reinterpret_cast<const bf16x8*>(kp + 32 * i);
        const uint16_t* vp = vpool + ph * D * kPage + row * kPage + 4 * grp;
#pragma unroll
        for (int t = 0; t < NT; ++t) r.v[t] = *reinterpret_cast<const s16x4*>(vp + 16 * kPage * t);
        r.ab = *reinterpret_cast<const bf16x8*>(abpool + ph * kPage * 2 + 8 * grp);
    };

    float m_run = -__builtin_huge_valf();
    float l_run = 0.f;
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto process = [&](const PageRegs<D>& r, int32_t lp) {
        if (!r.ok) return;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KC; ++i) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.k[i], qv[i], s, 0, 0, 0);
        float s2[4];
        const int32_t ebase = lp * kPage + 4 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float alpha = static_cast<float>(r.ab[2 * j]);
            const float beta = static_cast<float>(r.ab[2 * j + 1]);
            const float x = s[j] * c_dot + (alpha * kLog2e + beta * c_beta);
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
        const s16x4 pk = __builtin_bit_cast(s16x4, pb);
        if (lp * kPage + kPage <= len) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                acc[t] *= scale;
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(r.v[t], pk, acc[t], 0, 0, 0);
            }
        } else {
            // last, partly used page: slots past the length may hold anything,
            // so their values are zeroed (0 * NaN would poison the product)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                s16x4 vt = r.v[t];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (ebase + j >= len) vt[j] = 0;
                acc[t] *= scale;
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, pk, acc[t], 0, 0, 0);
            }
        }
    };

    PageRegs<D> buf[NBUF];
#pragma unroll
    for (int i = 0; i < NBUF; ++i) load(buf[i], p0 + i);
    for (int32_t lp = p0; lp < p1; lp += NBUF) {
#pragma unroll
        for (int i = 0; i < NBUF; ++i) {
            if (lp + i < p1) process(buf[i], lp + i);
            load(buf[i], lp + i + NBUF);
        }
    }

    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (row < G) {
        const int64_t idx = (static_cast<int64_t>(b) * a.H_q + static_cast<int64_t>(h) * G + row) * a.splits + split;
        if (grp == 0) {
            a.part_ml[2 * idx + 0] = m_run;
            a.part_ml[2 * idx + 1] = l_run;
        }
        float* po = a.part_o + idx * D + 4 * grp;
#pragma unroll
        for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(po + 16 * t) = acc[t];
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
    const int b = blockIdx.z;
    const int H = a.cache.H;
    const int G = a.H_q / H;
    const int h = hq / G;
    if (split >= a.splits) return;

    const int32_t len = checked_length(a, b);
    const int32_t npages = (len + kPage - 1) / kPage;
    const int32_t p0 = split * a.pages_per_split;
    const int32_t p1 = min(p0 + a.pages_per_split, npages);
    if (p0 >= p1) return;

    const float* qrow = static_cast<const float*>(a.q) + (static_cast<int64_t>(b) * a.H_q + hq) * D;
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
        const float* krow = kpool + (ph * kPage + ent) * D + qtr * QD;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < QD; ++i) dot += qv[i] * krow[i];
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const float alpha = abpool[(ph * kPage + ent) * 2 + 0];
        const float beta = abpool[(ph * kPage + ent) * 2 + 1];
        float s2 = dot * c_dot + (alpha * kLog2e + beta * c_beta);
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
#pragma unroll
        for (int j = 0; j < DL; ++j) {
            const float* vrow = vpool + (ph * D + lane + kWave * j) * kPage;
            float o = acc[j] * scale;
#pragma unroll
            for (int e = 0; e < kPage; ++e) {
                const float pe = __shfl(p, 4 * e);
                if (lp * kPage + e < len) o += pe * vrow[e];
            }
            acc[j] = o;
        }
    }
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) l_run += __shfl_xor(l_run, o);
    const int64_t idx = (static_cast<int64_t>(b) * a.H_q + hq) * a.splits + split;
    if (lane == 0) {
        a.part_ml[2 * idx + 0] = m_run;
        a.part_ml[2 * idx + 1] = l_run;
    }
#pragma unroll
    for (int j = 0; j < DL; ++j) a.part_o[idx * D + lane + kWave * j] = acc[j];
}

// ----------------------------------------------------------------- combine

// One wavefront per (sequence, query head): merge the splits by log-sum-exp.
// Loads of kChunk splits are issued together; lanes own D/64 dimensions.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(DecodeArgs a) {
    constexpr int DL = D / kWave;
    constexpr int kChunk = 16;
    const int lane = threadIdx.x;
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int32_t len = checked_length(a, b);
    const int32_t npages = (len + kPage - 1) / kPage;
    const int nsplit = min(a.splits, (npages + a.pages_per_split - 1) / a.pages_per_split);
    const int64_t base = (static_cast<int64_t>(b) * a.H_q + hq) * a.splits;

    float M = -__builtin_huge_valf();
    for (int s = lane; s < nsplit; s += kWave) M = fmaxf(M, a.part_ml[2 * (base + s)]);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float msub = (M == -__builtin_huge_valf()) ? 0.f : M;

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
#pragma unroll
        for (int u = 0; u < kChunk; ++u) {
            const float wu = (s0 + u < nsplit) ? fast_exp2(w[u] - msub) : 0.f;
            L += wu * l[u];
#pragma unroll
            for (int j = 0; j < DL; ++j) acc[j] += wu * ov[u][j];
        }
    }
    float* orow = a.o + (static_cast<int64_t>(b) * a.H_q + hq) * D;
    const bool live = L > 0.f;
    const float inv = live ? 1.f / L : 0.f;
#pragma unroll
    for (int j = 0; j < DL; ++j) orow[lane + kWave * j] = live ? acc[j] * inv : 0.f;
    if (lane == 0)
        a.lse[static_cast<int64_t>(b) * a.H_q + hq] = live ? (msub + __log2f(L)) * kLn2 : -__builtin_huge_valf();
}

// ------------------------------------------------------------------ launch

constexpr int kNbuf = 4;

template <int D>
static spicy_status launch_decode_t(const DecodeArgs& a, int dtype, hipStream_t stream) {
    const int wpb = a.splits < 4 ? a.splits : 4;
    if (dtype == SPICY_BF16) {
        dim3 grid((a.splits + wpb - 1) / wpb, a.cache.H, a.B);
        hipLaunchKernelGGL((decode_mfma_kernel<D, kNbuf>), grid, dim3(wpb * kWave), 0, stream, a);
    } else {
        dim3 grid((a.splits + wpb - 1) / wpb, a.H_q, a.B);
        hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(wpb * kWave), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    hipLaunchKernelGGL((combine_kernel<D>), dim3(a.H_q, a.B), dim3(kWave), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPICY_ERR_HIP;
    return SPICY_OK;
}

spicy_status launch_decode(const DecodeArgs& a, int dtype, int D, hipStream_t stream) {
    if (a.B == 0) return SPICY_OK;
    return D == 128 ? launch_decode_t<128>(a, dtype, stream) : launch_decode_t<64>(a, dtype, stream);
}

}  // namespace spicy
