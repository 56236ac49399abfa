// SPICY-KV per-step policy on gfx950: the segment partition and the
// protection mask of a freshly appended chunk, computed from the chunk itself
// (the inputs spicy_coarsen then consumes).
//
// Equal-Variation KV Cache page, "Mathematical statement" and "Implementation
// notes": a feature z_t = P [k_t; v_t] with P a fixed random projection, the
// local variation d_t = ||z_t - z_{t-1}||_2, the cumulative variation, the
// thresholds q_j = j c_T / N and each boundary at the first token whose
// cumulative variation reaches the next threshold (first hitting time).
// SPICY-KV demo page, Claim 2 and section 1: exact C-points (the landmarks:
// here the largest key norms per KV head) and protected sink / recent tokens.
//
// The arithmetic is integer end to end, so every order of summation gives
// the same bits:
//   fix(x)  = x * 2^16 rounded half to even, clamped to +-2^28, NaN -> 0.
//             Done in fp32, which is exact here: bf16 -> fp32 is exact, the
//             scaling by 2^16 is exact and v_rndne_f32 rounds that exact
//             value half to even.
//   z_t[r]  = sum of sign * fix(x_t[c]) over the entries of row r (int64);
//   d_t     = floor(sqrt(sum_r (z_t[r] - z_{t-1}[r])^2)), the square sum in
//             128 bits, the root from an fp64 estimate corrected with exact
//             integer comparisons; d = 0 at a sequence's first token;
//   C_t     = prefix sums of d, and with
//             cnt(C) = #{j in [1, N-1] : floor(j C_T / N) <= C}
//                    = clamp(floor(((C + 1) N - 1) / C_T), 0, N - 1)
//             token t is boundary b_j = min{t : C_t >= floor(j C_T / N)} of
//             every j in (cnt(C_{t-1}), cnt(C_t)] (cnt(C_{-1}) = 0);
//   norm2   = sum_i fix(k_t,h[i])^2 (uint64); the landmarks of (sequence,
//             head) are its L largest among the positions [sink, T - recent),
//             ties to the lower position: an 8-bit radix select finds the
//             L-th largest value, a position-ordered scan takes its ties.
//
// policy_token_kernel: one wavefront per run of kRun consecutive tokens (it
//   recomputes z of the token before its run); token rows stream through a
//   ring of kRing prefetched tokens, and each row is staged as fixed-point
//   int32 in the wavefront's LDS slice for the projection's gathers: lanes
//   4r .. 4r+3 own row r of P, each every fourth entry.  Writes d_t and
//   norm2[t][h].
// policy_seq_kernel: workgroup (b, y).  y < H: landmarks of head y of
//   sequence b, written into that head's mask column.  y == H: the scan of
//   d over the sequence and its N segment offsets.
#include "launch.h"
#include "spicy_device.h"

namespace spicy {

namespace {

constexpr int kRun = 32;             // tokens per wavefront
constexpr int kRing = 3;             // token rows in flight per wavefront (3: 128 VGPRs, 4 waves per SIMD)
constexpr int kMaxEnt = 16;          // projection entries a lane keeps in registers
constexpr int kTokWaves = 4;         // wavefronts per token workgroup
constexpr int kSeqThreads = 512;
constexpr int kPer = 16;             // tokens (or candidates) a sequence-kernel thread holds
constexpr int64_t kRangeLimit = int64_t(1) << 62;

// fix(x): x * 2^16 rounded half to even (exact in fp32), then the hardware
// conversion to int32, which saturates out-of-range values and turns NaN into
// 0 (written as the instruction itself: a C++ conversion of NaN or of an
// out-of-range value is undefined), then the clamp to +-2^28.
__device__ __forceinline__ int32_t fix16(uint32_t bf16_bits) {
    const float y = __builtin_rintf(__uint_as_float(bf16_bits << 16) * 65536.0f);
    int32_t i;
    asm("v_cvt_i32_f32 %0, %1" : "=v"(i) : "v"(y));
    return min(max(i, -268435456), 268435456);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x & 0xFFFFFFFFu), m));
    const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x >> 32), m));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t x, int d) {
    const uint32_t lo = static_cast<uint32_t>(__shfl_up(static_cast<int>(x & 0xFFFFFFFFu), d));
    const uint32_t hi = static_cast<uint32_t>(__shfl_up(static_cast<int>(x >> 32), d));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t isqrt_u128(unsigned __int128 s) {
    const double est = static_cast<double>(static_cast<uint64_t>(s >> 64)) * 18446744073709551616.0 +
                       static_cast<double>(static_cast<uint64_t>(s));
    uint64_t r = static_cast<uint64_t>(sqrt(est));
    while (static_cast<unsigned __int128>(r) * r > s) --r;
    while (static_cast<unsigned __int128>(r + 1) * (r + 1) <= s) ++r;
    return r;
}

// A projection entry, checked: returned as is when its column lies inside
// [k_t; v_t], else 0 (skipped) with the error bit raised.
__device__ __forceinline__ int32_t checked_entry(const PolicyArgs& a, int32_t e, int32_t width2) {
    const int32_t c = e > 0 ? e - 1 : -e - 1;
    if (e == 0 || c >= width2) {
        raise_err(a.err, SPICY_DEVERR_POLICY);
        return 0;
    }
    return e;
}

template <int CPL>
struct TokRow {
    uint4 k[CPL], v[CPL];
};

// DPP moves (within rows of 16 lanes); 64-bit values move as two halves.
constexpr int kQuadXor1 = 0xB1;       // quad_perm(1, 0, 3, 2)
constexpr int kQuadXor2 = 0x4E;       // quad_perm(2, 3, 0, 1)
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kHalfMirror = 0x141;    // lane i <-> 7 - i within each half row

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x & 0xFFFFFFFFu), CTRL, 0xF, 0xF, false));
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(x >> 32), CTRL, 0xF, 0xF, false));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    return __builtin_bit_cast(double, dpp_u64<CTRL>(__builtin_bit_cast(uint64_t, x)));
}

// Sum over aligned groups of 16 lanes (D = 128: one head) or 8 lanes (D = 64).
template <int G>
__device__ __forceinline__ uint64_t group_sum_u64(uint64_t v) {
    if constexpr (G == 16) {
        v += dpp_u64<kRowRor8>(v);
        v += dpp_u64<kRowRor4>(v);
    } else {
        v += dpp_u64<kHalfMirror>(v);
    }
    v += dpp_u64<kQuadXor2>(v);
    v += dpp_u64<kQuadXor1>(v);
    return v;
}

// floor(sqrt(s)) for s < 2^62, from the reciprocal square root estimate.
__device__ __forceinline__ uint64_t isqrt_u64(uint64_t s) {
    if (s == 0) return 0;
    const double e = static_cast<double>(s);
    uint64_t r = static_cast<uint64_t>(e * __builtin_amdgcn_rsq(e));
    while (r * r > s) --r;
    while ((r + 1) * (r + 1) <= s) ++r;
    return r;
}

template <int D, int CPL>
__global__ __launch_bounds__(kTokWaves * kWave) void policy_token_kernel(PolicyArgs a) {
    extern __shared__ int32_t lds[];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int H = a.H;
    const int W = H * D;                 // elements of k_t (and of v_t)
    const int nch = W / 8;               // 16-byte chunks of one row
    int32_t* xs = lds + static_cast<int64_t>(wave) * (2 * W + 4);   // + a zero slot at 2W
    const int64_t run = static_cast<int64_t>(blockIdx.x) * kTokWaves + wave;
    const int64_t t_begin = run * kRun;
    if (t_begin >= a.total_tokens) return;
    const int64_t t_end = min(t_begin + kRun, static_cast<int64_t>(a.total_tokens));
    if (lane == 0) xs[2 * W] = 0;

    // this lane's projection entries: row r = lane / 4, entries q, q + 4, ...
    // kept as (LDS index, sign); missing or invalid entries read the zero slot
    const int r = lane / 4, q = lane % 4;
    int32_t e0 = 0, n_own = 0;
    if (r < a.R) {
        e0 = a.proj_ptr[r];
        const int32_t e1 = a.proj_ptr[r + 1];
        if (e0 < 0 || e1 < e0 || e1 > a.nnz) {
            raise_err(a.err, SPICY_DEVERR_POLICY);
            e0 = 0;
        } else {
            n_own = max(0, (e1 - e0 - q + 3) / 4);
        }
    }
    int32_t goff[kMaxEnt];
    double gsgn[kMaxEnt];
#pragma unroll
    for (int i = 0; i < kMaxEnt; ++i) {
        const int32_t e = i < n_own ? checked_entry(a, a.proj_idx[e0 + q + 4 * i], 2 * W) : 0;
        goff[i] = e == 0 ? 2 * W : (e > 0 ? e - 1 : -e - 1);
        gsgn[i] = e < 0 ? -1.0 : 1.0;
    }
    int32_t nmax = n_own;                // entries the wavefront loops over (uniform)
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) nmax = max(nmax, __shfl_xor(nmax, o));
    nmax = __builtin_amdgcn_readfirstlane(nmax);

    // the sequence holding t_begin: the largest b with seq_offsets[b] <= t_begin
    int32_t lo = 0, hi = a.B;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) / 2;
        if (a.seq_offsets[mid] <= t_begin) lo = mid; else hi = mid - 1;
    }
    int32_t b = lo;
    int64_t cur_start = a.seq_offsets[b];
    int64_t next_start = b < a.B ? a.seq_offsets[b + 1] : INT64_MAX;
    // z of the token before the run, unless the run starts a sequence
    const int64_t t_first = (t_begin == cur_start || t_begin == 0) ? t_begin : t_begin - 1;

    const uint16_t* kin = a.k;
    const uint16_t* vin = a.v;
    auto load = [&](TokRow<CPL>& x, int64_t t) {
        const int64_t tc = min(t, t_end - 1);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = min(lane + kWave * j, nch - 1);
            x.k[j] = *reinterpret_cast<const uint4*>(kin + tc * W + 8 * c);
            x.v[j] = *reinterpret_cast<const uint4*>(vin + tc * W + 8 * c);
        }
    };

    double zprev = 0.0;
    auto process = [&](const TokRow<CPL>& x, int64_t t) {
        while (b < a.B && t >= next_start) {          // sequences are contiguous: step to t's
            ++b;
            cur_start = next_start;
            next_start = b < a.B ? a.seq_offsets[b + 1] : INT64_MAX;
        }
        const bool first = (b >= a.B) || t == cur_start;
        const bool out = t >= t_begin;
        // fixed point, staged in LDS; squared norms per head
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + kWave * j;
            uint64_t n2 = 0;
            if (c < nch) {
                const uint32_t kw[4] = {x.k[j].x, x.k[j].y, x.k[j].z, x.k[j].w};
                const uint32_t vw[4] = {x.v[j].x, x.v[j].y, x.v[j].z, x.v[j].w};
                int32_t xk[8], xv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xk[e] = fix16((e & 1) ? (kw[e / 2] >> 16) : (kw[e / 2] & 0xFFFFu));
                    xv[e] = fix16((e & 1) ? (vw[e / 2] >> 16) : (vw[e / 2] & 0xFFFFu));
                    n2 += static_cast<uint64_t>(static_cast<int64_t>(xk[e]) * xk[e]);
                }
                *reinterpret_cast<int4*>(xs + 8 * c) = make_int4(xk[0], xk[1], xk[2], xk[3]);
                *reinterpret_cast<int4*>(xs + 8 * c + 4) = make_int4(xk[4], xk[5], xk[6], xk[7]);
                *reinterpret_cast<int4*>(xs + W + 8 * c) = make_int4(xv[0], xv[1], xv[2], xv[3]);
                *reinterpret_cast<int4*>(xs + W + 8 * c + 4) = make_int4(xv[4], xv[5], xv[6], xv[7]);
            }
            n2 = group_sum_u64<D / 8>(n2);              // lanes of one head: D/8 consecutive chunks
            if (out && c < nch && (c % (D / 8)) == 0) a.norm2[t * H + (8 * c) / D] = n2;
        }
        __builtin_amdgcn_wave_barrier();
        // projection row r: this lane's entries (exact in double: every
        // partial sum is an integer below 2^53), then the quad's sum
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < kMaxEnt; ++i)
            if (i < nmax) acc = fma(gsgn[i], static_cast<double>(xs[goff[i]]), acc);
        for (int32_t i = kMaxEnt; i < nmax; ++i) {
            if (i < n_own) {
                const int32_t e = checked_entry(a, a.proj_idx[e0 + q + 4 * i], 2 * W);
                const double v = static_cast<double>(xs[e == 0 ? 2 * W : (e > 0 ? e - 1 : -e - 1)]);
                acc += e < 0 ? -v : v;
            }
        }
        acc += dpp_f64<kQuadXor1>(acc);
        acc += dpp_f64<kQuadXor2>(acc);
        const double z = r < a.R ? acc : 0.0;
        const double dzd = z - zprev;
        zprev = z;
        const uint64_t adz = static_cast<uint64_t>(dzd < 0.0 ? -dzd : dzd);
        uint64_t d;
        if (!__any(adz >= (uint64_t(1) << 29))) {
            // every |dz| < 2^29: the 16 squares sum below 2^62 in 64 bits
            const uint32_t a32 = static_cast<uint32_t>(adz);
            uint64_t sq = q == 0 ? static_cast<uint64_t>(a32) * a32 : 0;
            sq = group_sum_u64<16>(sq);
            // row totals sit in lanes 0, 16, 32, 48 (words read as uint32: no sign extension)
            uint64_t tot = 0;
#pragma unroll
            for (int rr = 0; rr < kWave / 16; ++rr) {
                const uint32_t lo32 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sq), 16 * rr));
                const uint32_t hi32 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sq >> 32), 16 * rr));
                tot += (static_cast<uint64_t>(hi32) << 32) | lo32;
            }
            d = isqrt_u64(tot);
        } else {
            unsigned __int128 sq = (q == 0) ? static_cast<unsigned __int128>(adz) * adz : 0;
            uint64_t sl = static_cast<uint64_t>(sq), sh = static_cast<uint64_t>(sq >> 64);
#pragma unroll
            for (int o = 4; o < kWave; o <<= 1) {
                const uint64_t ol = shfl_xor_u64(sl, o), oh = shfl_xor_u64(sh, o);
                const uint64_t nl = sl + ol;
                sh = sh + oh + (nl < sl ? 1 : 0);
                sl = nl;
            }
            d = isqrt_u128((static_cast<unsigned __int128>(sh) << 64) | sl);
        }
        if (first) d = 0;
        if (out && lane == 0) a.var[t] = static_cast<int64_t>(d);
        __builtin_amdgcn_wave_barrier();
    };

    TokRow<CPL> ring[kRing];
#pragma unroll
    for (int u = 0; u < kRing; ++u) load(ring[u], t_first + u);
    for (int64_t tt = t_first; tt < t_end; tt += kRing) {
#pragma unroll
        for (int u = 0; u < kRing; ++u) {
            if (tt + u < t_end) process(ring[u], tt + u);
            load(ring[u], tt + u + kRing);
        }
    }
}

// Exclusive prefix sum over the workgroup (kSeqThreads threads) and the total.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t x, int64_t* total, int64_t* scratch) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int64_t incl = x;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int64_t y = static_cast<int64_t>(shfl_up_u64(static_cast<uint64_t>(incl), o));
        if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    int64_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSeqThreads / kWave; ++w) {
        const int64_t s = scratch[w];
        if (w < wave) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + incl - x;
}

// cnt(C) = #{j in [1, N-1] : floor(j CT / N) <= C} = clamp(floor(((C+1) N - 1) / CT), 0, N - 1).
// The quotient comes from an fp64 estimate (off by at most one: the operands
// are below 2^63 and the quotient below 2N) corrected with exact products.
__device__ __forceinline__ int32_t cnt_below(int64_t C, int64_t CT, int32_t N, double inv_ct) {
    if (C < 0) return 0;
    if (CT == 0) return N - 1;
    const uint64_t num = static_cast<uint64_t>(C + 1) * static_cast<uint64_t>(N) - 1;
    const uint64_t ct = static_cast<uint64_t>(CT);
    uint64_t j = static_cast<uint64_t>(static_cast<double>(num) * inv_ct);
    j = min(j, static_cast<uint64_t>(2) * static_cast<uint64_t>(N));
    while (j > 0 && j * ct > num) --j;
    while ((j + 1) * ct <= num) ++j;
    return static_cast<int32_t>(min(j, static_cast<uint64_t>(N - 1)));
}

__global__ __launch_bounds__(kSeqThreads) void policy_seq_kernel(PolicyArgs a) {
    __shared__ int64_t scratch[kSeqThreads / kWave];
    __shared__ uint32_t hist[256];
    __shared__ uint32_t s_digit;
    __shared__ int64_t s_above;
    __shared__ unsigned long long s_or;
    constexpr int64_t kRound = static_cast<int64_t>(kSeqThreads) * kPer;   // tokens per round
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int y = blockIdx.y;
    const int H = a.H;
    const int64_t t0 = a.seq_offsets[b], t1 = a.seq_offsets[b + 1];
    const bool bad = t0 < 0 || t1 < t0 || t1 > a.total_tokens || t1 - t0 > (int64_t(1) << 20);
    const int64_t T = bad ? 0 : t1 - t0;

    if (y == H) {
        // ---- segment boundaries.  Round r covers tokens [r kRound, (r+1) kRound);
        // thread tid owns the kPer consecutive tokens starting at tid * kPer.
        const int32_t N = a.N;
        int32_t* so = a.seg_offsets + static_cast<int64_t>(b) * N;
        if (bad && tid == 0) raise_err(a.err, SPICY_DEVERR_POLICY);
        const int32_t base = bad ? 0 : static_cast<int32_t>(t0);
        if (tid == 0) {
            so[0] = base;
            a.seq_seg_ptr[b] = b * N;
            if (b == a.B - 1) {
                a.seq_seg_ptr[a.B] = a.B * N;
                a.seg_offsets[static_cast<int64_t>(a.B) * N] = a.seq_offsets[a.B];
            }
        }
        if (T == 0) {
            for (int32_t j = 1 + tid; j < N; j += kSeqThreads) so[j] = base;
            return;
        }
        int64_t dv[kPer];
        auto load_round = [&](int64_t r0) {
#pragma unroll
            for (int m = 0; m < kPer; ++m) {
                const int64_t u = r0 + static_cast<int64_t>(tid) * kPer + m;
                dv[m] = u < T ? a.var[t0 + u] : 0;
            }
        };
        // total variation
        int64_t CT = 0;
        for (int64_t r0 = 0; r0 < T; r0 += kRound) {
            load_round(r0);
            int64_t local = 0;
#pragma unroll
            for (int m = 0; m < kPer; ++m) local += dv[m];
            int64_t tot;
            block_exclusive_scan(local, &tot, scratch);
            CT += tot;
        }
        if (CT >= kRangeLimit / N) {
            if (tid == 0) raise_err(a.err, SPICY_DEVERR_POLICY);
            CT = 0;
        }
        const double inv_ct = CT > 0 ? 1.0 / static_cast<double>(CT) : 0.0;
        // boundaries: token t is b_j for every j in (cnt(C_{t-1}), cnt(C_t)]
        int64_t carry = 0;
        for (int64_t r0 = 0; r0 < T; r0 += kRound) {
            if (r0 != 0 || T > kRound) load_round(r0);
            int64_t local = 0;
#pragma unroll
            for (int m = 0; m < kPer; ++m) local += dv[m];
            int64_t tot;
            int64_t C = carry + block_exclusive_scan(local, &tot, scratch);
            carry += tot;
#pragma unroll
            for (int m = 0; m < kPer; ++m) {
                const int64_t u = r0 + static_cast<int64_t>(tid) * kPer + m;
                if (u < T) {
                    const int32_t cp = u == 0 ? 0 : cnt_below(C, CT, N, inv_ct);
                    C += dv[m];
                    const int32_t cc = cnt_below(C, CT, N, inv_ct);
                    for (int32_t j = cp + 1; j <= cc; ++j) so[j] = static_cast<int32_t>(t0 + u);
                }
            }
        }
        return;
    }

    // ---- landmarks of head y
    const int h = y;
    if (bad) return;                                   // reported by the boundary workgroup
    const int64_t c_lo = min(static_cast<int64_t>(a.sink), T);
    const int64_t c_hi = max(c_lo, T - a.recent);
    const int64_t n_cand = c_hi - c_lo;
    const int64_t Lsel = min(static_cast<int64_t>(a.L), n_cand);
    uint64_t tau;
    int64_t take_eq;                                   // ties of tau to take, lowest positions first
    if (Lsel == n_cand) {
        tau = 0;
        take_eq = INT64_MAX;                           // every candidate
    } else if (Lsel == 0) {
        tau = UINT64_MAX;
        take_eq = 0;                                   // none
    } else {
        uint64_t prefix = 0, pmask = 0;
        int64_t k = Lsel;                              // rank of the wanted value from the top
        // candidates c_lo + tid + kSeqThreads m stay in registers when they fit
        const bool in_regs = n_cand <= kRound;
        uint64_t vals[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int64_t u = c_lo + tid + static_cast<int64_t>(kSeqThreads) * m;
            vals[m] = (in_regs && u < c_hi) ? a.norm2[(t0 + u) * H + h] : 0;
        }
        // digits above the largest candidate's top byte are 0 for every
        // candidate: those passes would select digit 0 and change nothing, so
        // the select starts at that byte
        unsigned long long vor = 0;
        if (in_regs) {
#pragma unroll
            for (int m = 0; m < kPer; ++m) vor |= vals[m];
        } else {
            for (int64_t u = c_lo + tid; u < c_hi; u += kSeqThreads) vor |= a.norm2[(t0 + u) * H + h];
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) vor |= shfl_xor_u64(vor, o);
        if (tid == 0) s_or = 0;
        __syncthreads();
        if ((threadIdx.x % kWave) == 0) atomicOr(&s_or, vor);
        __syncthreads();
        const uint64_t top = s_or;
        const int shift0 = top ? (63 - __clzll(top)) / 8 * 8 : 0;
        for (int shift = shift0; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            if (in_regs) {
#pragma unroll
                for (int m = 0; m < kPer; ++m) {
                    const int64_t u = c_lo + tid + static_cast<int64_t>(kSeqThreads) * m;
                    const uint64_t v = vals[m];
                    const bool hit = u < c_hi && (v & pmask) == prefix;
                    const uint32_t dg = static_cast<uint32_t>(v >> shift) & 255u;
                    // one atomic per wavefront when all its hits share the digit
                    const uint32_t d0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(dg)));
                    if (__all(!hit || dg == d0)) {
                        const uint64_t hits = __ballot(hit);
                        if ((threadIdx.x % kWave) == 0 && hits)
                            atomicAdd(&hist[d0], static_cast<uint32_t>(__popcll(hits)));
                    } else if (hit) {
                        atomicAdd(&hist[dg], 1u);
                    }
                }
            } else {
                for (int64_t u = c_lo + tid; u < c_hi; u += kSeqThreads) {
                    const uint64_t v = a.norm2[(t0 + u) * H + h];
                    if ((v & pmask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1u);
                }
            }
            __syncthreads();
            // counts above each bin, high digit first: thread i < 256 holds bin 255 - i
            const int bin = 255 - tid;
            const int64_t cntb = tid < 256 ? hist[bin] : 0;
            int64_t dummy;
            const int64_t above = block_exclusive_scan(cntb, &dummy, scratch);
            if (tid < 256 && above < k && above + cntb >= k) {
                s_digit = static_cast<uint32_t>(bin);
                s_above = above;
            }
            __syncthreads();
            prefix |= static_cast<uint64_t>(s_digit) << shift;
            pmask |= uint64_t(255) << shift;
            k -= s_above;
            __syncthreads();
        }
        tau = prefix;
        take_eq = k;
    }
    // the mask, in rounds: thread tid owns kPer consecutive positions; ties of
    // tau are ranked in position order by a block scan with a running carry
    int64_t eq_carry = 0;
    for (int64_t r0 = 0; r0 < T; r0 += kRound) {
        uint64_t nv[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int64_t u = r0 + static_cast<int64_t>(tid) * kPer + m;
            nv[m] = (u >= c_lo && u < c_hi) ? a.norm2[(t0 + u) * H + h] : 0;
        }
        int64_t eq_local = 0;
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int64_t u = r0 + static_cast<int64_t>(tid) * kPer + m;
            eq_local += (u >= c_lo && u < c_hi && nv[m] == tau) ? 1 : 0;
        }
        int64_t eq_tot;
        int64_t eq_rank = eq_carry + block_exclusive_scan(eq_local, &eq_tot, scratch);
        eq_carry += eq_tot;
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int64_t u = r0 + static_cast<int64_t>(tid) * kPer + m;
            if (u < T) {
                uint8_t mk = 1;
                if (u >= c_lo && u < c_hi) {
                    mk = nv[m] > tau ? 1 : 0;
                    if (nv[m] == tau) {
                        mk = eq_rank < take_eq ? 1 : 0;
                        ++eq_rank;
                    }
                }
                a.mask[(t0 + u) * H + h] = mk;
            }
        }
    }
}

template <int D, int CPL>
spicy_status launch_token(const PolicyArgs& a, hipStream_t stream) {
    const int64_t runs = (static_cast<int64_t>(a.total_tokens) + kRun - 1) / kRun;
    const int64_t blocks = (runs + kTokWaves - 1) / kTokWaves;
    const size_t lds = static_cast<size_t>(kTokWaves) * (2 * a.H * D + 4) * sizeof(int32_t);
    hipLaunchKernelGGL((policy_token_kernel<D, CPL>), dim3(static_cast<unsigned>(blocks)), dim3(kTokWaves * kWave),
                       lds, stream, a);
    return hipGetLastError() == hipSuccess ? SPICY_OK : SPICY_ERR_HIP;
}

}  // namespace

spicy_status launch_policy(const PolicyArgs& a, hipStream_t stream) {
    if (a.B == 0) return SPICY_OK;
    if (a.total_tokens > 0) {
        const int chunks = a.H * a.d / 8;
        const int cpl = (chunks + kWave - 1) / kWave;
        spicy_status st;
        if (a.d == 128) {
            st = cpl == 1 ? launch_token<128, 1>(a, stream) : cpl == 2 ? launch_token<128, 2>(a, stream)
                                                                      : launch_token<128, 4>(a, stream);
        } else {
            st = cpl == 1 ? launch_token<64, 1>(a, stream) : launch_token<64, 2>(a, stream);
        }
        if (st != SPICY_OK) return st;
    }
    hipLaunchKernelGGL(policy_seq_kernel, dim3(static_cast<unsigned>(a.B), static_cast<unsigned>(a.H + 1)),
                       dim3(kSeqThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SPICY_OK : SPICY_ERR_HIP;
}

}  // namespace spicy
