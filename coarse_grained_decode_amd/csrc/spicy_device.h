// Device-side helpers and kernel argument blocks shared by the coarsen and
// decode kernels of the gfx950 SPICY-KV library.  (Private to the library.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spicy.h"

namespace spicy {

constexpr int kPage = 16;      // entries per page
constexpr int kWave = 64;      // gfx950 wavefront

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

// binary64 -> bfloat16 in a single nearest-even rounding, on the bit pattern:
// bfloat16 keeps 8 significant bits and the binary32 exponent range, so the
// result is the 64-bit significand shifted to the bf16 spacing with a sticky
// round-half-even on the bits shifted out.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    const uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
    const uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
    if (a > 0x7FF0000000000000ull) return 0x7FC0;                      // NaN
    if (a == 0x7FF0000000000000ull) return sign | 0x7F80;              // inf
    if (a == 0) return sign;
    int be = static_cast<int>(a >> 52);
    uint64_t mant = a & 0x000FFFFFFFFFFFFFull;
    if (be != 0) mant |= 0x0010000000000000ull; else be = 1;           // subnormal double
    const int E = be - 1023;                                           // exponent of bit 52
    const int lsb = (E < -126 ? -126 : E) - 7;                         // bf16 spacing
    const int sh = lsb - (be - 1075);                                  // >= 45
    uint64_t q;
    if (sh >= 54) {
        q = 0;                                                         // below half the spacing
    } else {
        q = mant >> sh;
        const uint64_t rem = mant & ((1ull << sh) - 1);
        const uint64_t half = 1ull << (sh - 1);
        if (rem > half || (rem == half && (q & 1))) ++q;
    }
    if (E < -126) return sign | static_cast<uint16_t>(q);            // subnormal (q==128: min normal)
    int Eo = E;
    if (q == 256) { q = 128; ++Eo; }
    if (Eo > 127) return sign | 0x7F80;
    return sign | static_cast<uint16_t>(((Eo + 127) << 7) | (q & 0x7F));
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
};

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
    int32_t* lengths_out;
    int32_t* err;          // workspace header word
    int32_t* seg_seq;      // [n_seg]           owning sequence of each segment
    int32_t* seg_start;    // [n_seg][H]        first entry of the segment per head
    int32_t* seg_ncnt;     // [n_seg][H]        protected tokens of the segment per head
    int32_t total_tokens;
    int32_t n_seg;
    int32_t B;
    int32_t max_pages;
    double rope_base;
};

struct DecodeArgs {
    CacheArgs cache;
    const void* q;
    const int32_t* page_table;
    const int32_t* lengths;
    float* o;
    float* lse;
    int32_t* err;
    float* part_ml;        // [B][H_q][S][2]    running max (log2 units) and sum
    float* part_o;         // [B][H_q][S][d]    unnormalised output
    int32_t B;
    int32_t H_q;
    int32_t max_pages;
    int32_t splits;        // S
    int32_t pages_per_split;
};

}  // namespace spicy
