// k_quant.hip -- key-cache compression for proposal scoring (Prism Attention page, Sec. 4.2
// Quantized Proposal Construction: int8 per-token absmax, and a 2-bit per-token format for the
// INT2 cache the page names) and the workspace zero-fill kernel.
#include "prism_device.hpp"
#include "prism_prof.hpp"

namespace prism {

// One row (token) of D values is handled by D/EPL lanes, each holding 16 bytes.  amax is a
// lane-group max; scale = amax/127 and 127/amax are correctly rounded fp32 divisions; codes are
// rint(x * inv) (one fp32 product, round half to even) clamped to [-127, 127].
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_quantize_keys(const T* __restrict__ K, int8_t* __restrict__ Kq,
                                                            float* __restrict__ scales, Dims d) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / EPL;        // lanes per row
    constexpr int RPW = 64 / LPR;       // rows per wave
    const int lane = lane_id();
    const int sub = lane % LPR;
    const int64_t total_rows = int64_t(d.B) * d.Hkv * d.T_max;
    const int64_t stride = int64_t(gridDim.x) * (kThreads / 64) * RPW;
    for (int64_t row = (int64_t(blockIdx.x) * (kThreads / 64) + wave_id()) * RPW + lane / LPR;
         row < total_rows; row += stride) {
        const int64_t unit = row / d.T_max;
        const int64_t t = row - unit * d.T_max;
        const int b = int(unit / d.Hkv);
        if (t >= seq_len_of(d, b)) continue;  // uniform across the row's lanes
        float x[EPL];
        unpack16<T>(load16(K + row * D + sub * EPL), x);
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float scale = amax / 127.0f;
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        uint32_t packed[EPL / 4];
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) {
            uint32_t w = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float r = __builtin_rintf(x[4 * i + k] * inv);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                w |= (uint32_t(int32_t(r)) & 0xFFu) << (8 * k);
            }
            packed[i] = w;
        }
        int8_t* dst = Kq + row * D + sub * EPL;
        if constexpr (EPL == 8) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
        } else {
            *reinterpret_cast<uint32_t*>(dst) = packed[0];
        }
        if (sub == 0) scales[row] = scale;
    }
}

template <typename T>
static hipError_t quantize_dispatch(const void* K, const Dims& d, int8_t* Kq, float* scales, hipStream_t st) {
    const int64_t rows = int64_t(d.B) * d.Hkv * d.T_max;
    const int64_t rows_per_block = (kThreads / 64) * (64 / (d.D / Elem<T>::kPerLane));
    int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    const T* k = static_cast<const T*>(K);
    switch (d.D) {
        case 64: launch_k("k_quantize_keys", (k_quantize_keys<T, 64>), dim3(blocks), dim3(kThreads), st, k, Kq, scales, d); break;
        case 128: launch_k("k_quantize_keys", (k_quantize_keys<T, 128>), dim3(blocks), dim3(kThreads), st, k, Kq, scales, d); break;
        case 256: launch_k("k_quantize_keys", (k_quantize_keys<T, 256>), dim3(blocks), dim3(kThreads), st, k, Kq, scales, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_keys(const void* K, int bf16, const Dims& d, int8_t* Kq, float* scales, hipStream_t st) {
    return bf16 ? quantize_dispatch<uint16_t>(K, d, Kq, scales, st) : quantize_dispatch<float>(K, d, Kq, scales, st);
}

// INT2 proposal keys.  Per token, [-amax, amax] is cut into four equal cells and a value is
// coded by its cell's centre: scale = amax / 4 (exact), u = x * (2 / amax) (one fp32 product,
// correctly rounded reciprocal), level c = clamp(2 floor(u) + 1, -3, 3) stored as the 2-bit code
// (c + 3) / 2.  A row is D/4 bytes; the 32-bit word w of a row holds dims 16w .. 16w + 15 with
// dim 16w + 4j + i in bits 8i + 2j .. 8i + 2j + 1, so (word >> 2j) & 0x03030303 lines up byte i
// with dim 16w + 4j + i: four consecutive dims, one byte-wise dot product.  One lane per word.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void k_quantize_keys_int2(const T* __restrict__ K, uint32_t* __restrict__ Kq2,
                                                                 float* __restrict__ scales, Dims d) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / 16;  // lanes per row, 16 dims each
    constexpr int RPW = 64 / LPR;
    const int lane = lane_id();
    const int sub = lane % LPR;
    const int64_t total_rows = int64_t(d.B) * d.Hkv * d.T_max;
    const int64_t stride = int64_t(gridDim.x) * (kThreads / 64) * RPW;
    for (int64_t row = (int64_t(blockIdx.x) * (kThreads / 64) + wave_id()) * RPW + lane / LPR;
         row < total_rows; row += stride) {
        const int64_t unit = row / d.T_max;
        const int64_t t = row - unit * d.T_max;
        const int b = int(unit / d.Hkv);
        if (t >= seq_len_of(d, b)) continue;  // uniform across the row's lanes
        float x[16];
#pragma unroll
        for (int p = 0; p < 16 / EPL; ++p) unpack16<T>(load16(K + row * D + sub * 16 + p * EPL), x + p * EPL);
        float amax = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
        for (int o = LPR / 2; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float inv = amax > 0.0f ? 2.0f / amax : 0.0f;
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float c = 2.0f * floorf(x[4 * j + i] * inv) + 1.0f;
                c = fminf(fmaxf(c, -3.0f), 3.0f);
                const uint32_t code = uint32_t(int32_t(c) + 3) >> 1;
                w |= code << (8 * i + 2 * j);
            }
        }
        Kq2[row * (D / 16) + sub] = w;
        if (sub == 0) scales[row] = amax * 0.25f;
    }
}

template <typename T>
static hipError_t quantize_int2_dispatch(const void* K, const Dims& d, uint32_t* Kq2, float* scales, hipStream_t st) {
    const int64_t rows = int64_t(d.B) * d.Hkv * d.T_max;
    const int64_t rows_per_block = (kThreads / 64) * (64 / (d.D / 16));
    int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    const T* k = static_cast<const T*>(K);
    switch (d.D) {
        case 64: launch_k("k_quantize_keys_int2", (k_quantize_keys_int2<T, 64>), dim3(blocks), dim3(kThreads), st, k, Kq2, scales, d); break;
        case 128: launch_k("k_quantize_keys_int2", (k_quantize_keys_int2<T, 128>), dim3(blocks), dim3(kThreads), st, k, Kq2, scales, d); break;
        case 256: launch_k("k_quantize_keys_int2", (k_quantize_keys_int2<T, 256>), dim3(blocks), dim3(kThreads), st, k, Kq2, scales, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_keys_int2(const void* K, int bf16, const Dims& d, uint8_t* Kq2, float* scales, hipStream_t st) {
    uint32_t* w = reinterpret_cast<uint32_t*>(Kq2);
    return bf16 ? quantize_int2_dispatch<uint16_t>(K, d, w, scales, st) : quantize_int2_dispatch<float>(K, d, w, scales, st);
}

__global__ __launch_bounds__(kThreads) void k_zero(uint4* __restrict__ p, size_t n16, uint8_t* __restrict__ tail,
                                                   size_t ntail) {
    const size_t stride = size_t(gridDim.x) * kThreads;
    for (size_t i = size_t(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
    if (bytes == 0) return hipSuccess;
    const size_t n16 = bytes / 16;
    const size_t ntail = bytes - n16 * 16;
    size_t blocks = (n16 + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(kThreads), 0, st, static_cast<uint4*>(p), n16,
                       static_cast<uint8_t*>(p) + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace prism
