// Streaming-read reference for the benchmark (not part of the SPICY-KV
// library): one launch reads `bytes` bytes with 16-byte loads in a grid-stride
// loop and keeps an XOR of the data so the loads cannot be dropped.  The
// benchmark reports the fastest configuration beside each kernel's rate as
// the plain streaming-read ceiling at that byte count.  Built as its own
// shared library (libspicy_probe.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, uint64_t n16, uint32_t* sink) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * blockDim.x;
    uint64_t i = static_cast<uint64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    // never true for data the caller fills with a constant pattern other
    // than this value; keeps the loads live
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Read `bytes` bytes (a multiple of 16) at device pointer p with `blocks`
// workgroups of 256 threads, `unroll` (1, 2, 4 or 8) loads in flight per
// thread per iteration.  sink: one device uint32 (written only in the
// unlikely case described in the kernel).  Returns 0, or -1 for bad
// arguments, or the HIP error code of the launch.
int spicy_probe_stream_read(const void* p, uint64_t bytes, int32_t blocks, int32_t unroll, uint32_t* sink,
                            void* stream) {
    if (!p || !sink || bytes % 16 != 0 || blocks < 1) return -1;
    const uint64_t n16 = bytes / 16;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4* q = static_cast<const uint4*>(p);
    switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(blocks), dim3(256), 0, s, q, n16, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(blocks), dim3(256), 0, s, q, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, q, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, q, n16, sink); break;
    default: return -1;
    }
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
