// prism_attend.hpp -- shared pieces of sparse and dense decode attention on gfx950: per-row
// logits for the G query heads of a KV head, a workgroup's softmax(.)V partial over up to 256
// rows, and the log-sum-exp merge of the partials (token-level sparse attention, Prism Attention
// page Sec. 1 and Sec. 2.1; split-K over rows with a merge of (max, sum, weighted V)).
#pragma once

#include "prism_device.hpp"

namespace prism {

// Query registers: lane `sub` of a row group holds dims [sub*EPL, sub*EPL + EPL) of each head.
template <typename T, int D, int GP>
struct QRegs {
    static constexpr int EPL = Elem<T>::kPerLane;
    float v[GP][EPL];
    __device__ __forceinline__ void load(const T* qg, int G, int sub) {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            if (h < G) {
                unpack16<T>(load16(qg + int64_t(h) * D + sub * EPL), v[h]);
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) v[h][e] = 0.0f;
            }
        }
    }
};

// Full-row dot products for every head: partial over the lane's EPL dims, then an all-reduce
// over the LPR lanes of the row group (every lane of the group ends with all GP logits).
template <typename T, int D, int GP>
__device__ __forceinline__ void row_logits(const QRegs<T, D, GP>& q, const float* x, float* l) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / EPL;
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(q.v[h][e], x[e], acc);
        l[h] = acc;
    }
#pragma unroll
    for (int h = 0; h < GP; ++h) l[h] = group_sum<LPR>(l[h]);
}

// softmax(y) V partial of one workgroup of NT threads over n <= NROWS rows (NROWS <= NT).
//   s_t[r]      token id of row r (rows of the unit's V)
//   s_y[r][h]   base-2 exponent-domain logits (logit * sm_scale * log2 e); padded heads unused
// Writes g_ml[h] = (max_r y, sum_r 2^(y - max)) and g_acc[h][d] = sum_r 2^(y - max) V[r][d]
// for h < G, at device scope.  The first min(NT, 256) threads gather and accumulate V; every
// thread takes the barriers.  Uses s_stat[2*GP], s_red[(NT/64)*GP] and s_acc[GP*D] as LDS scratch.
template <typename T, int D, int GP, int NROWS, int NT = kThreads>
__device__ __forceinline__ void softmax_v_partial(const T* __restrict__ Vu, const int32_t* s_t, float (*s_y)[GP],
                                                  int n, int G, float* s_stat, float* s_red, float* s_acc,
                                                  float* __restrict__ g_acc, float* __restrict__ g_ml) {
    constexpr int NA = NT < 256 ? NT : 256;
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / EPL;
    constexpr int RPW = 64 / LPR;
    constexpr int RPR = RPW * (NA / 64);
    constexpr int ROUNDS = (NROWS + RPR - 1) / RPR;
    constexpr int U = ROUNDS < 8 ? ROUNDS : 8;
    static_assert(NROWS <= NT, "one row per thread in the softmax statistics");
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();

    // max and sum per head over the rows (row r on thread r)
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        if (h >= G) break;
        float y = tid < n ? s_y[tid][h] : -INFINITY;
        y = wave_max(y);
        if (lane == 0) s_red[wave * GP + h] = y;
    }
    __syncthreads();
    if (tid < GP) {
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, s_red[w * GP + tid]);
        s_stat[tid] = m;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        if (h >= G) break;
        float p = 0.0f;
        if (tid < n) {
            p = exp2f(s_y[tid][h] - s_stat[h]);
            s_y[tid][h] = p;
        }
        p = wave_sum(p);
        if (lane == 0) s_red[wave * GP + h] = p;
    }
    __syncthreads();
    if (tid < GP) {
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w) l += s_red[w * GP + tid];
        s_stat[GP + tid] = l;
    }

    // weighted V accumulation; lane group = one row, lane = EPL consecutive dims
    const int sub = lane % LPR;
    const int rl = wave * RPW + lane / LPR;
    float acc[GP][EPL];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    if (tid < NA) {
        for (int r0 = 0; r0 < ROUNDS; r0 += U) {
            uint4 raw[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = (r0 + u) * RPR + rl;
                raw[u] = (r0 + u < ROUNDS && row < n) ? load16(Vu + int64_t(s_t[row]) * D + sub * EPL)
                                                       : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = (r0 + u) * RPR + rl;
                if (r0 + u < ROUNDS && row < n) {
                    float x[EPL];
                    unpack16<T>(raw[u], x);
#pragma unroll
                    for (int h = 0; h < GP; ++h) {
                        if (h < G) {
                            const float p = s_y[row][h];
#pragma unroll
                            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
                        }
                    }
                }
            }
        }
        // reduce the row groups of a wave
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1)
#pragma unroll
            for (int h = 0; h < GP; ++h)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], o);
    }
    // then the accumulating waves in a fixed order (deterministic)
    for (int w = 0; w < NA / 64; ++w) {
        if (wave == w && lane < LPR) {
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                if (h < G) {
#pragma unroll
                    for (int e = 0; e < EPL; ++e) {
                        float* dst = &s_acc[h * D + sub * EPL + e];
                        *dst = (w == 0) ? acc[h][e] : *dst + acc[h][e];
                    }
                }
            }
        }
        __syncthreads();
    }
    // partials are read by another workgroup of the same kernel: write through to device scope
    for (int i = tid; i < G * D; i += NT) st_dev(&g_acc[i], s_acc[i]);
    if (tid < G) {
        st_dev(&g_ml[2 * tid], s_stat[tid]);
        st_dev(&g_ml[2 * tid + 1], s_stat[GP + tid]);
    }
}

// Log-sum-exp merge of `np` partials (partial s at g_ml + s*GP*2, g_acc + s*GP*D), read at
// device scope, eight partials per batch of independent loads.  Writes out[h][d] (dtype T) and
// lse[h] (natural log) for h < G; np == 0 gives out = 0, lse = -inf.
template <typename T, int D, int GP, int NT = kThreads>
__device__ __forceinline__ void merge_partials(const float* __restrict__ g_ml, const float* __restrict__ g_acc, int np, int G,
                               T* __restrict__ out, float* __restrict__ lse) {
    constexpr float kLn2 = 0.6931471805599453f;
    constexpr int BATCH = 8;
    for (int i = threadIdx.x; i < G * D; i += NT) {
        const int h = i / D, dd = i % D;
        float M = -INFINITY, L = 0.0f, acc = 0.0f;
        for (int s0 = 0; s0 < np; s0 += BATCH) {
            float m[BATCH], l[BATCH], v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int s = s0 + u;
                const bool ok = s < np;
                m[u] = ok ? ld_dev(&g_ml[(s * GP + h) * 2]) : -INFINITY;
                l[u] = ok ? ld_dev(&g_ml[(s * GP + h) * 2 + 1]) : 0.0f;
                v[u] = ok ? ld_dev(&g_acc[(int64_t(s) * GP + h) * D + dd]) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                if (s0 + u < np) {
                    const float Mn = fmaxf(M, m[u]);
                    const float c_old = exp2f(M - Mn);
                    const float c_new = exp2f(m[u] - Mn);
                    L = L * c_old + l[u] * c_new;
                    acc = acc * c_old + v[u] * c_new;
                    M = Mn;
                }
            }
        }
        const bool empty = np == 0;
        store_elem<T>(&out[int64_t(h) * D + dd], empty ? 0.0f : acc / L);
        if (dd == 0 && lse) lse[h] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
    }
}

// Log-sum-exp merge of `np` partials with the per-partial statistics staged in LDS.  The first
// batch of partial sums is requested before the statistics, so both arrive in one round trip.
// s_tab must hold 3*np*GP + 2*GP floats (fits_lds_merge).  Deterministic: partials are summed in
// index order.
__host__ __device__ constexpr int merge_lds_floats(int np, int GP) { return 3 * np * GP + 2 * GP; }

template <typename T, int D, int GP, int NT = kThreads>
__device__ __forceinline__ void merge_partials_lds(const float* __restrict__ g_ml, const float* __restrict__ g_acc, int np, int G,
                                   T* __restrict__ out, float* __restrict__ lse, float* s_tab) {
    constexpr float kLn2 = 0.6931471805599453f;
    constexpr int OPT = (GP * D + NT - 1) / NT;  // outputs per thread
    constexpr int BATCH = (64 / OPT) < 4 ? 4 : ((64 / OPT) > 32 ? 32 : 64 / OPT);
    const int tid = threadIdx.x;
    float* sm = s_tab;
    float* sl = sm + np * GP;
    float* sw = sl + np * GP;
    float* sM = sw + np * GP;
    float* sL = sM + GP;

    float accv[OPT][BATCH];
    auto load_batch = [&](int s0) {
#pragma unroll
        for (int q = 0; q < OPT; ++q) {
            const int o = tid + q * NT;
            const int h = o / D, dd = o % D;
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int s = s0 + u;
                accv[q][u] = (o < G * D && s < np) ? ld_dev(&g_acc[(int64_t(s) * GP + h) * D + dd]) : 0.0f;
            }
        }
    };
    load_batch(0);
    for (int i = tid; i < np * GP; i += NT) {
        const int h = i % GP;
        sm[i] = h < G ? ld_dev(&g_ml[2 * i]) : -INFINITY;
        sl[i] = h < G ? ld_dev(&g_ml[2 * i + 1]) : 0.0f;
    }
    __syncthreads();
    if (tid < GP) {
        float M = -INFINITY;
        for (int s = 0; s < np; ++s) M = fmaxf(M, sm[s * GP + tid]);
        sM[tid] = M;
    }
    __syncthreads();
    for (int i = tid; i < np * GP; i += NT) {
        const int h = i % GP;
        sw[i] = h < G ? exp2f(sm[i] - sM[h]) : 0.0f;
    }
    __syncthreads();
    if (tid < GP) {
        float L = 0.0f;
        for (int s = 0; s < np; ++s) L = fmaf(sw[s * GP + tid], sl[s * GP + tid], L);
        sL[tid] = L;
    }
    __syncthreads();
    float res[OPT];
#pragma unroll
    for (int q = 0; q < OPT; ++q) res[q] = 0.0f;
    for (int s0 = 0; s0 < np; s0 += BATCH) {
        if (s0 > 0) load_batch(s0);
#pragma unroll
        for (int q = 0; q < OPT; ++q) {
            const int o = tid + q * NT;
            const int h = (o / D) < GP ? o / D : 0;
#pragma unroll
            for (int u = 0; u < BATCH; ++u)
                if (s0 + u < np) res[q] = fmaf(sw[(s0 + u) * GP + h], accv[q][u], res[q]);
        }
    }
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int o = tid + q * NT;
        if (o < G * D) {
            const int h = o / D, dd = o % D;
            const bool empty = np == 0;
            store_elem<T>(&out[o], empty ? 0.0f : res[q] / sL[h]);
            if (dd == 0 && lse) lse[h] = empty ? -INFINITY : (sM[h] + log2f(sL[h])) * kLn2;
        }
    }
}

}  // namespace prism
