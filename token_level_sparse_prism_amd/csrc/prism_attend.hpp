// prism_attend.hpp -- shared pieces of sparse and dense decode attention on gfx950: per-row
// logits for the G query heads of a KV head, a workgroup's softmax(.)V partial over up to 256
// rows, and the log-sum-exp merge of the partials (token-level sparse attention, Prism Attention
// page Sec. 1 and Sec. 2.1; split-K over rows with a merge of (max, sum, weighted V)).
#pragma once

#include "prism_device.hpp"
#include "prism_prof.hpp"

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

// ---- sparse partial with one V row per wave instruction ----------------------------------
// Lane l of a wave holds dims [l*NE, l*NE + NE) of a row, NE = D/64, so a row is one coalesced
// 64-lane load of D*e bytes and no lane ever holds a partial of another lane's dims.
template <typename T, int NE> struct LaneRow;
template <> struct LaneRow<uint16_t, 1> {
    using R = uint32_t;
    static __device__ __forceinline__ R load(const uint16_t* p) { return uint32_t(*p); }
    static __device__ __forceinline__ void unpack(R r, float* x) { x[0] = bf16_bits_to_f32(r); }
};
template <> struct LaneRow<uint16_t, 2> {
    using R = uint32_t;
    static __device__ __forceinline__ R load(const uint16_t* p) { return *reinterpret_cast<const uint32_t*>(p); }
    static __device__ __forceinline__ void unpack(R r, float* x) {
        x[0] = bf16_bits_to_f32(r & 0xFFFFu);
        x[1] = bf16_bits_to_f32(r >> 16);
    }
};
template <> struct LaneRow<uint16_t, 4> {
    using R = uint2;
    static __device__ __forceinline__ R load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    static __device__ __forceinline__ void unpack(R r, float* x) {
        x[0] = bf16_bits_to_f32(r.x & 0xFFFFu);
        x[1] = bf16_bits_to_f32(r.x >> 16);
        x[2] = bf16_bits_to_f32(r.y & 0xFFFFu);
        x[3] = bf16_bits_to_f32(r.y >> 16);
    }
};
template <> struct LaneRow<float, 1> {
    using R = float;
    static __device__ __forceinline__ R load(const float* p) { return *p; }
    static __device__ __forceinline__ void unpack(R r, float* x) { x[0] = r; }
};
template <> struct LaneRow<float, 2> {
    using R = float2;
    static __device__ __forceinline__ R load(const float* p) { return *reinterpret_cast<const float2*>(p); }
    static __device__ __forceinline__ void unpack(R r, float* x) {
        x[0] = r.x;
        x[1] = r.y;
    }
};
template <> struct LaneRow<float, 4> {
    using R = float4;
    static __device__ __forceinline__ R load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    static __device__ __forceinline__ void unpack(R r, float* x) {
        x[0] = r.x;
        x[1] = r.y;
        x[2] = r.z;
        x[3] = r.w;
    }
};

constexpr int kRowsAccFloats = 8192;  // LDS floats for the waves' V partials (one round of heads)

// softmax(y) V partial over the n (1 <= n <= NR) selected rows of one workgroup of NT threads.
//   vrow(t)              the V row of token t (contiguous or paged cache)
//   s_slot[r], s_tok[r]  pool slot and token id of row r
//   logits               the unit's [kp][LS] fp32 logits per pool slot; y = logit * y_scale is
//                        the base-2 exponent-domain logit (heads >= G unused)
// Wave w owns rows [w*RPW, w*RPW + RPW): lane i < RPW loads row i's logits, and the wave issues
// its rows' V loads (branch-free, rows >= n read row 0 and get weight 0) before the statistics,
// so both arrive in one round trip.  One barrier exchanges the per-wave maxima; a row's weights
// go through the wave's own rows of s_p (NR*GP floats, 16-byte aligned).  The waves' partials
// are summed in LDS in wave order, HB heads per round.  Writes g_ml[h] = (max_r y,
// sum_r 2^(y - max)) and g_acc[h * AS + d] = sum_r 2^(y - max) V[r][d] for h < G at device scope
// (AS: the partial's row stride, D unless the rows are a column range of wider rows).
// LDS: s_red 2*(NT/64)*GP floats, s_wacc kRowsAccFloats floats.
template <typename T, int D, int GP, int NR, int NT, typename VRow, int AS = D>
__device__ __forceinline__ void softmax_v_rows(VRow vrow, const float* __restrict__ logits, int LS,
                                               float y_scale, const int32_t* s_slot, const int32_t* s_tok, int n,
                                               int G, float* s_p, float* s_red, float* s_wacc,
                                               float* __restrict__ g_acc, float* __restrict__ g_ml) {
    constexpr int NW = NT / 64;
    constexpr int NE = D / 64;
    using LR = LaneRow<T, NE>;
    using R = typename LR::R;
    constexpr int WORDS = int(sizeof(R)) / 4 > 0 ? int(sizeof(R)) / 4 : 1;
    constexpr int RPW = NR / NW;  // rows per wave
    constexpr int UB = RPW < 32 / WORDS ? RPW : 32 / WORDS;
    constexpr int HB = kRowsAccFloats / (NW * D) < GP ? kRowsAccFloats / (NW * D) : GP;  // heads per LDS round
    static_assert(NR % NW == 0 && RPW <= 64 && RPW % UB == 0, "rows must split evenly over the waves' lanes");
    static_assert(HB >= 1 && GP % HB == 0, "head rounds");
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int row0 = wave * RPW;
    float* s_max = s_red;
    float* s_sum = s_red + NW * GP;
    PRISM_TL(kTlRows, 0);

    // this lane's row: its logits (the lane's load is issued first)
    const bool my_valid = lane < RPW && row0 + lane < n;
    float4 lraw[GP < 4 ? 1 : GP / 4];
    {
        const int64_t j = s_slot[my_valid ? row0 + lane : 0];
#pragma unroll
        for (int h4 = 0; h4 < (GP < 4 ? 1 : GP / 4); ++h4)
            lraw[h4] = reinterpret_cast<const float4*>(logits + j * LS)[h4];
    }
    // the wave's V rows, first batch
    R raw[UB];
#pragma unroll
    for (int u = 0; u < UB; ++u) {
        const int r = row0 + u;
        raw[u] = LR::load(vrow(s_tok[r < n ? r : 0]) + lane * NE);
    }

    // statistics, per wave: the wave's own maximum per head (-inf for a wave without rows), so
    // no barrier stands between a wave's logits and its V accumulation; the cross-wave sum below
    // rescales each wave's partial to the workgroup maximum
    float y[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        const float4 v = lraw[h / 4];
        const float c = (h % 4 == 0) ? v.x : (h % 4 == 1) ? v.y : (h % 4 == 2) ? v.z : v.w;
        y[h] = (my_valid && h < G) ? c * y_scale : -INFINITY;
    }
    static_assert(NW == 16, "the wave maxima fill one DPP row per head");
    float p[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        if (h >= G) {
            p[h] = 0.0f;
            continue;
        }
        const float m = wave_max(y[h]);
        p[h] = my_valid ? exp2_le0(y[h] - m) : 0.0f;  // m is finite where a lane holds a row
        const float l = wave_sum(p[h]);
        if (lane == 0) {
            s_max[wave * GP + h] = m;
            s_sum[wave * GP + h] = l;
        }
    }
    PRISM_TL(kTlRows, 1);
    PRISM_TL(kTlRows, 2);
    PRISM_TL(kTlAttend, 2);
    if (lane < RPW) {  // the wave's rows' weights; read back below by the same wave only
#pragma unroll
        for (int h = 0; h < GP; ++h) s_p[(row0 + lane) * GP + h] = p[h];
    }

    // weighted V accumulation (rows beyond n carry weight 0)
    float acc[GP][NE];
#pragma unroll
    for (int h = 0; h < GP; ++h)
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[h][e] = 0.0f;
#pragma unroll
    for (int i0 = 0; i0 < RPW; i0 += UB) {
        if (i0 > 0) {
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int r = row0 + i0 + u;
                raw[u] = LR::load(vrow(s_tok[r < n ? r : 0]) + lane * NE);
            }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            float x[NE];
            LR::unpack(raw[u], x);
            const float* pw = s_p + (row0 + i0 + u) * GP;
#pragma unroll
            for (int h = 0; h < GP; ++h) {
                if (h < G) {
                    const float w = pw[h];
#pragma unroll
                    for (int e = 0; e < NE; ++e) acc[h][e] = fmaf(w, x[e], acc[h][e]);
                }
            }
        }
    }

    PRISM_TL(kTlRows, 3);
    // sum of the waves' partials in wave order, each scaled by 2^(wave max - workgroup max), HB
    // heads per round; partials are read by another workgroup of the same kernel, so they are
    // written through to device scope
#pragma unroll
    for (int hb = 0; hb < GP; hb += HB) {
        if (hb >= G) break;
        if (hb > 0) __syncthreads();  // the previous round's sums have read s_wacc
#pragma unroll
        for (int h = 0; h < HB; ++h) {
            if (hb + h < G) {
#pragma unroll
                for (int e = 0; e < NE; ++e) s_wacc[(wave * HB + h) * D + lane * NE + e] = acc[hb + h][e];
            }
        }
        __syncthreads();
        const int nb = (G - hb < HB ? G - hb : HB) * D;
        for (int i = tid; i < nb; i += NT) {
            const int h = i / D, dd = i % D;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, s_max[w * GP + hb + h]);  // finite: n >= 1
            float sacc = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w)
                sacc = fmaf(s_wacc[(w * HB + h) * D + dd], exp2_le0(s_max[w * GP + hb + h] - M), sacc);
            st_dev(&g_acc[(hb + h) * AS + dd], sacc);
        }
    }
    if (wave == 0) {
#pragma unroll
        for (int hb = 0; hb < GP; hb += 4) {
            const int hq = hb + (lane >> 4);
            const float mw = hq < G ? s_max[(lane & 15) * GP + hq] : -INFINITY;
            const float M = group_max<16>(mw);
            const float l = group_sum<16>(hq < G ? s_sum[(lane & 15) * GP + hq] * exp2_le0(mw - M) : 0.0f);
            if ((lane & 15) == 0 && hq < G) {
                st_dev(&g_ml[2 * hq], M);
                st_dev(&g_ml[2 * hq + 1], l);
            }
        }
    }
}

// Log-sum-exp merge of `np` partials (partial s at g_ml + s*GP*2, g_acc + s*GP*AS; rows of AS), read at
// device scope, sixteen partials per batch of independent loads: the batch's maximum first, then
// every partial's weight on its own.  Writes out[h][d] (dtype T) and lse[h] (natural log) for
// h < G; np == 0 gives out = 0, lse = -inf.  With kToPartial it writes instead one partial of the
// same form (o_ml, o_acc, at device scope): the merge of the np partials, m = -inf for np == 0.
template <typename T, int D, int GP, int NT = kThreads, bool kToPartial = false, int AS = D>
__device__ __forceinline__ void merge_partials(const float* __restrict__ g_ml, const float* __restrict__ g_acc, int np, int G,
                               T* __restrict__ out, float* __restrict__ lse, float* __restrict__ o_ml = nullptr,
                               float* __restrict__ o_acc = nullptr) {
    constexpr float kLn2 = 0.6931471805599453f;
    constexpr int BATCH = 16;
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
                v[u] = ok ? ld_dev(&g_acc[(int64_t(s) * GP + h) * AS + dd]) : 0.0f;
            }
            float Mn = M;
#pragma unroll
            for (int u = 0; u < BATCH; ++u) Mn = fmaxf(Mn, m[u]);  // finite: the batch holds a partial
            const float c_old = exp2_le0(M - Mn);
            L *= c_old;
            acc *= c_old;
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const float c = exp2_le0(m[u] - Mn);  // 0 for the batch's unused entries
                L = fmaf(l[u], c, L);
                acc = fmaf(v[u], c, acc);
            }
            M = Mn;
        }
        if constexpr (kToPartial) {
            st_dev(&o_acc[h * AS + dd], acc);
            if (dd == 0) {
                st_dev(&o_ml[2 * h], M);
                st_dev(&o_ml[2 * h + 1], L);
            }
        } else {
            const bool empty = np == 0;
            store_elem<T>(&out[int64_t(h) * AS + dd], empty ? 0.0f : acc / L);
            if (dd == 0 && lse) lse[h] = empty ? -INFINITY : (M + log2f(L)) * kLn2;
        }
    }
}

}  // namespace prism
