// Device-side helpers and kernel argument blocks shared by the coarsen and
// decode kernels of the gfx950 SPICY-KV library.  (Private to the library.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spicy.h"

namespace spicy {

constexpr int kPage = 16;      // entries per page
constexpr int kWave = 64;      // gfx950 wavefront
constexpr int kGroup = 8;      // dims per group of a key/value page row
constexpr int kChunk = 32;     // dims of one MFMA operand chunk (4 groups)

// Offset of element (slot s, dim i) inside a page-head's 16 x d key or value
// block: 8-dim groups outermost, then the 16 slots, then the group's dims.
// The MFMA operand of a 32-dim chunk (lane 16g + r: slot r, dims
// 32c + 8g .. +8) is then the 1 KB at 512c elements with lane l reading the
// l-th 16 bytes: every wavefront-wide load is one sequential 1 KB run.
__device__ __forceinline__ int slot_elem(int s, int i) {
    return ((i / kGroup) * kPage + s) * kGroup + i % kGroup;
}

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// binary32 -> bfloat16, nearest-even (inputs here are never NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// binary64 -> bfloat16 in a single nearest-even rounding.  The double is
// first rounded to binary32 "to odd" (truncate, then set the last bit if
// anything was lost), then binary32 -> bfloat16 rounds to nearest-even.
// Because binary32 keeps at least two more bits than bfloat16, the two steps
// give exactly the nearest-even bfloat16 of the double (Boldo & Melquiond,
// rounding to odd).  The truncation is recovered from the hardware's
// nearest-even conversion: if it rounded away from zero, step one unit back.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    if (x != x) return 0x7FC0;                                         // NaN
    const float f = static_cast<float>(x);
    uint32_t u = __float_as_uint(f);
    const double d = static_cast<double>(f);
    if (d != x) {
        if (fabs(d) > fabs(x)) u -= 1u;                                // toward zero
        u |= 1u;                                                       // sticky
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// sin and cos of a double-precision angle, accurate to a few units in the
// last place for |x| up to ~1e9.  Cody-Waite reduction by pi/2 with pi/2 split
// into two 32-bit pieces and a double tail (each product with the quadrant
// number is exact for |k| < 2^21), then Taylor series of sin and cos on
// |r| <= pi/4 up to r^17 / r^16 (the first omitted terms are below 1e-17).
__device__ __forceinline__ void sincos_f64(double x, double* s, double* c) {
    constexpr double kTwoOverPi = 0.6366197723675814;
    constexpr double kPio2Hi = 1.5707963267341256;      // first 32 bits of pi/2
    constexpr double kPio2Mid = 6.077100506303966e-11;  // next 32 bits
    constexpr double kPio2Lo = 2.0222662487959506e-21;  // the rest
    const double k = rint(x * kTwoOverPi);
    const double r = ((x - k * kPio2Hi) - k * kPio2Mid) - k * kPio2Lo;
    const double z = r * r;
    // 1/n! for n = 3, 5, ..., 17 and n = 2, 4, ..., 16
    double ps = 1.0 / 355687428096000.0;                 // 1/17!
    ps = fma(ps, z, -1.0 / 1307674368000.0);             // 1/15!
    ps = fma(ps, z, 1.0 / 6227020800.0);                 // 1/13!
    ps = fma(ps, z, -1.0 / 39916800.0);                  // 1/11!
    ps = fma(ps, z, 1.0 / 362880.0);                     // 1/9!
    ps = fma(ps, z, -1.0 / 5040.0);                      // 1/7!
    ps = fma(ps, z, 1.0 / 120.0);                        // 1/5!
    ps = fma(ps, z, -1.0 / 6.0);                         // 1/3!
    const double sr = fma(r * z, ps, r);
    double pc = 1.0 / 20922789888000.0;                  // 1/16!
    pc = fma(pc, z, -1.0 / 87178291200.0);               // 1/14!
    pc = fma(pc, z, 1.0 / 479001600.0);                  // 1/12!
    pc = fma(pc, z, -1.0 / 3628800.0);                   // 1/10!
    pc = fma(pc, z, 1.0 / 40320.0);                      // 1/8!
    pc = fma(pc, z, -1.0 / 720.0);                       // 1/6!
    pc = fma(pc, z, 1.0 / 24.0);                         // 1/4!
    pc = fma(pc, z, -0.5);                               // 1/2!
    const double cr = fma(z, pc, 1.0);
    const int q = static_cast<int>(static_cast<long long>(k) & 3);
    const double ss = (q & 1) ? cr : sr;
    const double cc = (q & 1) ? sr : cr;
    *s = (q & 2) ? -ss : ss;
    *c = ((q + 1) & 2) ? -cc : cc;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {   // bfloat16 bits
    static __device__ __forceinline__ double to_f64(uint16_t b) { return static_cast<double>(bf16_to_f32(b)); }
    static __device__ __forceinline__ float to_f32(uint16_t b) { return bf16_to_f32(b); }
    static __device__ __forceinline__ uint16_t from_f64(double x) { return f64_to_bf16(x); }
    static __device__ __forceinline__ uint16_t from_f32(float x) { return f32_to_bf16(x); }
};
template <> struct Elem<float> {
    static __device__ __forceinline__ double to_f64(float b) { return static_cast<double>(b); }
    static __device__ __forceinline__ float to_f32(float b) { return b; }
    static __device__ __forceinline__ float from_f64(double x) { return static_cast<float>(x); }
    static __device__ __forceinline__ float from_f32(float x) { return x; }
};

// ------------------------------------------------------------- lane moves

// The value of lane (this lane xor P), P = 1, 2, 4 or 8, through DPP moves
// (VALU only, no LDS round trip): P = 1 and 2 are quad permutations; P = 8 is
// a rotation by 8 inside each 16-lane row; P = 4 is a reversal inside each
// quad (lane xor 3) followed by a mirror inside each half-row of 8 (lane xor 7).
template <int P>
__device__ __forceinline__ uint32_t dpp_xor(uint32_t v) {
    static_assert(P == 1 || P == 2 || P == 4 || P == 8, "lane distance");
    const int x = static_cast<int>(v);
    if constexpr (P == 1) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));     // quad_perm [1,0,3,2]
    } else if constexpr (P == 2) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));     // quad_perm [2,3,0,1]
    } else if constexpr (P == 8) {
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));    // row_ror:8
    } else {
        const int r = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false);                      // quad_perm [3,2,1,0]
        return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, false));     // row_half_mirror
    }
}

template <int P>
__device__ __forceinline__ double dpp_xor_f64(double v) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
    const uint32_t lo = dpp_xor<P>(static_cast<uint32_t>(u)), hi = dpp_xor<P>(static_cast<uint32_t>(u >> 32));
    return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// ------------------------------------------------------------ buffer loads

// Raw buffer resource over `bytes` bytes at p: loads at offsets >= bytes
// return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// --------------------------------------------------------- error reporting

__device__ __forceinline__ void raise_err(int32_t* err, int32_t bit) {
    if (err) atomicOr(err, bit);
}

// ----------------------------------------------------------- argument blocks

struct CacheArgs {
    void* k;
    void* v;
    void* ab;
    void* meta;
    int32_t num_pages;
    int32_t H;      // KV heads
    void* s2;       // diagonal closure: per-dimension variance, layout of k (nullptr: scalar closure)
};

// spicy_policy: per-step segments and protection mask from the chunk itself.
struct PolicyArgs {
    const uint16_t* k;           // [total_tokens][H][d] bf16 keys (pre-RoPE)
    const uint16_t* v;           // [total_tokens][H][d] bf16 values
    const int32_t* seq_offsets;  // [B+1]
    const int32_t* proj_ptr;     // [R+1]  row r of P: proj_idx[proj_ptr[r] .. proj_ptr[r+1])
    const int32_t* proj_idx;     // [nnz]  +(c+1) / -(c+1): +-1 at column c of [k_t; v_t]
    int32_t* seg_offsets;        // [B*N + 1] out
    int32_t* seq_seg_ptr;        // [B+1]     out
    uint8_t* mask;               // [total_tokens][H] out
    int64_t* var;                // [total_tokens]    workspace: d_t
    uint64_t* norm2;             // [total_tokens][H] workspace: squared fixed-point key norms
    int32_t* err;
    int32_t total_tokens, B, H, d, R, nnz, N, L, sink, recent;
};

// Destination hints of the coarsening: one 64-bit word per (segment, head)
// of a call, in a device array of this many words that the library owns.
// Calls with more (segment, head) pairs, or pools of 2^28 pages or more, run
// without hints.
constexpr int64_t kDestHintWords = int64_t{1} << 17;

struct CoarsenArgs {
    CacheArgs cache;
    const void* k_pre;
    const void* v;
    const int32_t* seq_offsets;
    const int32_t* pos_base;
    const int32_t* seg_offsets;
    const int32_t* seq_seg_ptr;
    const uint8_t* mask;
    const int32_t* page_table;
    const int32_t* entry_start;
    const int64_t* token_weight;   // [total_tokens] or null: weights of the representatives
    int32_t* lengths_out;
    int32_t* err;          // workspace header word
    int4* seg_desc;        // [n_seg]     {sequence (-1 = skip), first token, end token, position offset}
    int2* seg_head;        // [n_seg][H]  {first entry of the segment, physical page of its macro-node (-1: none)}
    int2* cp_items;        // C-points of sequence b at [seq_offsets[b] * H, + cp_count[b]):
                           //   {token, entry << 4 | head}
    int32_t* cp_count;     // [B]
    int32_t* null_from;    // [B][H]      first null-padding entry of each head (INT32_MAX: none)
    void* stage_k;         // [n_seg][H][d]  macro-node keys (rotated, rounded), as streamed
    void* stage_v;         // [n_seg][H][d]  macro-node values
    void* stage_ab;        // [n_seg][H][2]  alpha, beta
    int4* stage_meta;      // [n_seg][H]     {mass, sequence, pos_sum lo, pos_sum hi}
    void* stage_s2;        // [n_seg][H][d]  macro-node per-dimension variances (diagonal closure)
    int32_t total_tokens;
    int32_t n_seg;
    int32_t B;
    int32_t max_pages;
    uint32_t gen;          // this call's tag in the destination hints (0: no hints this call)
    double rope_base;
    double theta[64];      // rotary frequencies rope_base^(-2i/d), i < d/2 (host libm pow)
};

// spicy_merge_level: one level of the dyadic merge cascade.
struct MergeArgs {
    CacheArgs cache;
    const int32_t* page_table;    // [B][max_pages]
    const int32_t* entry_begin;   // [B]
    const int32_t* entry_end;     // [B]
    int32_t* err;
    int32_t* ticket;              // [B*H]  workspace: arrivals per (sequence, head), zero between calls
    int32_t cap;                  // pairs per (sequence, head) at most = (max_range + 1) / 2
    int32_t B;
    int32_t max_pages;
    int32_t max_range;
    double rope_base;
    double theta[64];             // rotary frequencies rope_base^(-2i/d), i < d/2 (host libm pow)
};

// spicy_compact_range: non-null entries of [entry_begin, lengths) moved to
// the front of the range, per head.
struct CompactArgs {
    CacheArgs cache;
    const int32_t* page_table;    // [B][max_pages]
    const int32_t* entry_begin;   // [B]
    const int32_t* lengths;       // [B]
    int32_t* lengths_out;         // [B]
    int32_t* err;
    int32_t B;
    int32_t max_pages;
    int32_t D;
};

struct DecodeArgs {
    CacheArgs cache;
    const void* q;
    const int32_t* page_table;
    const int32_t* lengths;
    float* o;
    float* lse;
    int32_t* err;
    int32_t* ticket;       // [B][n_q][H_q]        arrivals per query row (zero between calls)
    float* part_ml;        // [B][n_q][H_q][S][2]  running max (log2 units) and sum of a page group
    float* part_o;         // [B][n_q][H_q][S][d]  its unnormalised output
    int32_t B;
    int32_t H_q;
    int32_t max_pages;
    int32_t n_q;               // query tokens per sequence (rows: (b * n_q + token) * H_q + head)
    int32_t slots;             // S = prefix_groups + priv_groups partial slots per row
    int32_t prefix_pages;      // P shared logical pages (0 = none)
    int32_t prefix_groups;     // page groups of the shared prefix (slots 0 .. prefix_groups-1)
    int32_t prefix_chunk;      // prefix pages per group
    int32_t priv_groups;       // page groups of each (sequence, KV head)'s private pages [P, ...)
    int32_t priv_chunk;        // private pages per group
    int32_t priv_tiles;        // 16-row tiles of one (sequence, KV head): ceil(n_q * G / 16)
    int32_t wpg;               // wavefronts per workgroup of the MFMA kernel (4 or 8)
    int32_t prefix_sets;       // set by the launcher: tile-sets of one KV head's prefix rows
    int32_t priv_sets;         // set by the launcher: tile-sets of one (sequence, KV head)
    int32_t prefix_blocks;     // set by the launcher: workgroups of the prefix role (a multiple of 8)
};

}  // namespace spicy
