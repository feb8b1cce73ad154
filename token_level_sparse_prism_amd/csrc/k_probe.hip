// k_probe.hip -- a plain coalesced read of a device buffer: the read-stream ceiling that the
// HBM-bound kernels are compared with.  1024 workgroups of 256 threads; workgroup w reads the
// w-th contiguous 1/1024 of the buffer with 16-byte streaming loads, eight in flight per lane,
// and each wave stores the XOR of what it read to sink[4 w + wave] (so no load is dead).
#include "prism_device.hpp"
#include "prism_prof.hpp"

namespace prism {

constexpr int kProbeWgs = 1024;

__global__ __launch_bounds__(kThreads) void k_read_probe(const uint4* __restrict__ src, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    constexpr int U = 8;
    const size_t per = (n16 + kProbeWgs - 1) / kProbeWgs;
    const size_t b0 = size_t(blockIdx.x) * per;
    const size_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint32_t x = 0;
    for (size_t i0 = b0 + threadIdx.x; i0 < b1; i0 += size_t(kThreads) * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = i0 + size_t(u) * kThreads;
            v[u] = i < b1 ? load16_stream(src + i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x ^= uint32_t(__shfl_xor(int(x), o));
    if (lane_id() == 0) sink[blockIdx.x * (kThreads / 64) + wave_id()] = x;
}

// sink: kProbeWgs * 4 words
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
    launch_k("k_read_probe", k_read_probe, dim3(kProbeWgs), dim3(kThreads), st, static_cast<const uint4*>(src),
             bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace prism
