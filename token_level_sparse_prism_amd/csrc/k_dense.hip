// k_dense.hip -- dense decode attention over every cached token (the kappa = kp = T_b special
// case of the refined layer; the dense baseline the Prism Attention page compares against in
// Sec. 5.3).  grid (256-token chunks) x units: each workgroup computes its chunk's logits, then a
// softmax(.)V partial; the unit's last workgroup merges the partials.
#include "prism_attend.hpp"
#include "prism_prof.hpp"

namespace prism {

template <typename T, int D, int GP>
__global__ __launch_bounds__(kThreads) void k_dense(DenseArgs a) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / EPL;
    constexpr int RPW = 64 / LPR;
    constexpr int RPR = RPW * (kThreads / 64);
    constexpr int ROUNDS = kDenseChunk / RPR;
    constexpr int U = ROUNDS < 8 ? ROUNDS : 8;
    static_assert(ROUNDS % U == 0, "chunk must hold whole unrolled rounds");

    __shared__ int32_t s_t[kDenseChunk];
    __shared__ float s_y[kDenseChunk][GP];
    __shared__ float s_stat[2 * GP];
    __shared__ float s_red[(kThreads / 64) * GP];
    __shared__ float s_acc[GP * D];
    __shared__ uint32_t s_flag;

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int chunk = ui.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t c0 = int64_t(chunk) * kDenseChunk;
    const int n = int(Tb - c0 < 0 ? 0 : (Tb - c0 > kDenseChunk ? kDenseChunk : Tb - c0));
    const int sub = lane % LPR;
    const int nc = int(gridDim.x);
    float* part_ml = a.part_ml + int64_t(unit) * nc * GP * 2;
    float* part_acc = a.part_acc + int64_t(unit) * nc * GP * D;

    if (n > 0) {
        QRegs<T, D, GP> q;
        q.load(static_cast<const T*>(a.q) + (int64_t(b) * d.Hq + int64_t(g) * G) * D, G, sub);
        const T* Ku = static_cast<const T*>(a.K) + (int64_t(unit) * d.T_max + c0) * D;
        const int rl = wave * RPW + lane / LPR;
        for (int r0 = 0; r0 < ROUNDS; r0 += U) {
            uint4 raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = (r0 + u) * RPR + rl;
                raw[u] = row < n ? load16(Ku + int64_t(row) * D + sub * EPL) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = (r0 + u) * RPR + rl;
                float x[EPL];
                unpack16<T>(raw[u], x);
                float l[GP];
                row_logits<T, D, GP>(q, x, l);
                if (sub == 0 && row < n) {
                    s_t[row] = int32_t(c0 + row);
#pragma unroll
                    for (int h = 0; h < GP; ++h) s_y[row][h] = h < G ? l[h] * a.y_scale : 0.0f;
                }
            }
        }
        __syncthreads();
        const T* Vu = static_cast<const T*>(a.V) + int64_t(unit) * d.T_max * D;
        softmax_v_partial<T, D, GP, kDenseChunk>(Vu, s_t, s_y, n, G, s_stat, s_red, s_acc,
                                                  part_acc + int64_t(chunk) * GP * D,
                                                  part_ml + int64_t(chunk) * GP * 2);
    }

    if (!arrive_last(&a.done[int64_t(unit) * kCtrStride], gridDim.x, &s_flag)) return;

    const int np = int((Tb + kDenseChunk - 1) / kDenseChunk);
    const int64_t hq0 = int64_t(b) * d.Hq + int64_t(g) * G;
    merge_partials<T, D, GP>(part_ml, part_acc, np, G, static_cast<T*>(a.out) + hq0 * D,
                             a.lse ? a.lse + hq0 : nullptr);
    if (tid == 0) a.done[int64_t(unit) * kCtrStride] = 0u;
}

template <typename T, int D>
static hipError_t dense_g(const DenseArgs& a, hipStream_t st) {
    const int units = a.d.B * a.d.Hkv;
    const dim3 grid(int((a.d.T_max + kDenseChunk - 1) / kDenseChunk), units);
    switch (padded_g(a.d.G)) {
        case 1: launch_k("k_dense", (k_dense<T, D, 1>), grid, dim3(kThreads), st, a); break;
        case 2: launch_k("k_dense", (k_dense<T, D, 2>), grid, dim3(kThreads), st, a); break;
        case 4: launch_k("k_dense", (k_dense<T, D, 4>), grid, dim3(kThreads), st, a); break;
        case 8: launch_k("k_dense", (k_dense<T, D, 8>), grid, dim3(kThreads), st, a); break;
        case 16: launch_k("k_dense", (k_dense<T, D, 16>), grid, dim3(kThreads), st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
static hipError_t dense_d(const DenseArgs& a, hipStream_t st) {
    switch (a.d.D) {
        case 64: return dense_g<T, 64>(a, st);
        case 128: return dense_g<T, 128>(a, st);
        case 256: return dense_g<T, 256>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dense(const DenseArgs& a, int bf16, hipStream_t st) {
    return bf16 ? dense_d<uint16_t>(a, st) : dense_d<float>(a, st);
}

}  // namespace prism
