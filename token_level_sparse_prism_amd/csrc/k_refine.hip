// k_refine.hip -- refined layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4.1: the
// refined layer re-selects its own top-kappa inside the inherited pool; Sec. 5.3: refinement
// touches only the pool, so its cost does not grow with the context).
//
// Two launches per call:
//   k_rscore  grid (pool slices) x units.  Gathers the pool's K rows, computes the G heads'
//             logits (fp32) and the group score S, stores the logits and an order key of S per
//             slot (0 for an empty slot), and adds the slice's histogram of the keys' top 12 bits
//             into the unit's histogram.
//   k_attend  grid (64 selected rows) x units.  Every workgroup loads the unit's keys into LDS and
//             derives the exact top-kappa itself (radix digits 12/12/8, ties to the lower slot),
//             ranks the selected slots in slot order with wave ballots, writes idx for its 64
//             ranks, gathers their V rows and forms a softmax(.)V partial from the stored logits.
//             The unit's last workgroup merges the partials (log-sum-exp) into out and lse and
//             clears the histogram for the next call.
#include "prism_attend.hpp"
#include "prism_prof.hpp"

namespace prism {

template <typename T, int D, int GP, bool kMax>
__global__ __launch_bounds__(kThreads) void k_rscore(RefineArgs a) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / EPL;
    constexpr int RPW = 64 / LPR;
    constexpr int RPR = RPW * (kThreads / 64);
    constexpr int ROUNDS = (kScoreSlice + RPR - 1) / RPR;
    constexpr int U = ROUNDS < 16 ? ROUNDS : 16;
    constexpr int LS = GP < 4 ? 4 : GP;
    static_assert(ROUNDS % U == 0, "slice must hold whole unrolled rounds");

    __shared__ uint32_t s_hist[kHistBins];

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int unit = blockIdx.y;
    const int slice = blockIdx.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp = a.kp;
    const int sub = lane % LPR;

    for (int i = tid; i < kHistBins; i += kThreads) s_hist[i] = 0u;

    QRegs<T, D, GP> q;
    q.load(static_cast<const T*>(a.q) + (int64_t(b) * d.Hq + int64_t(g) * G) * D, G, sub);
    const T* Ku = static_cast<const T*>(a.K) + int64_t(unit) * d.T_max * D;
    const int32_t* pool = a.pool + int64_t(unit) * kp;
    uint32_t* skey = a.skey + int64_t(unit) * a.kstride;
    float* logits = a.logits + int64_t(unit) * kp * LS;
    const int64_t j0 = int64_t(slice) * kScoreSlice;
    const int rl = wave * RPW + lane / LPR;
    __syncthreads();

    for (int r0 = 0; r0 < ROUNDS; r0 += U) {
        int32_t t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = j0 + (r0 + u) * RPR + rl;
            t[u] = (j < kp && (r0 + u) * RPR + rl < kScoreSlice) ? pool[j] : -1;
        }
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            raw[u] = (t[u] >= 0 && t[u] < Tb) ? load16(Ku + int64_t(t[u]) * D + sub * EPL) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = j0 + (r0 + u) * RPR + rl;
            const bool valid = t[u] >= 0 && t[u] < Tb;
            float x[EPL];
            unpack16<T>(raw[u], x);
            float l[GP];
            row_logits<T, D, GP>(q, x, l);
            float S = l[0];
#pragma unroll
            for (int h = 1; h < GP; ++h) {
                if (h < G) S = kMax ? fmaxf(S, l[h]) : S + l[h];
            }
            if (sub == 0 && j < kp && (r0 + u) * RPR + rl < kScoreSlice) {
                const uint32_t key = valid ? order_key(S) : 0u;
                skey[j] = key;
#pragma unroll
                for (int h4 = 0; h4 < LS; h4 += 4) {
                    float4 v;
                    v.x = h4 + 0 < GP ? l[h4 + 0] : 0.0f;
                    v.y = h4 + 1 < GP ? l[h4 + 1] : 0.0f;
                    v.z = h4 + 2 < GP ? l[h4 + 2] : 0.0f;
                    v.w = h4 + 3 < GP ? l[h4 + 3] : 0.0f;
                    *reinterpret_cast<float4*>(&logits[j * LS + h4]) = v;
                }
                if (valid) atomicAdd(&s_hist[key >> kKeyShift], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t* gh = a.ghist + int64_t(unit) * kHistBins;
    for (int i = tid; i < kHistBins; i += kThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// Keys of the unit's pool slots, from LDS (kp <= kLdsKeys) or straight from global memory.
struct KeySrc {
    const uint32_t* lds;
    const uint32_t* glob;
    __device__ __forceinline__ uint32_t operator()(int64_t j) const { return lds ? lds[j] : glob[j]; }
};

template <typename T, int D, int GP>
__global__ __launch_bounds__(kThreads) void k_attend(RefineArgs a) {
    constexpr int LS = GP < 4 ? 4 : GP;
    extern __shared__ uint32_t s_keys[];  // kp words when the keys fit in LDS
    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_tmp[kThreads / 64];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_w[2][kThreads / 64];
    __shared__ int32_t s_slot[kAttendSlice];
    __shared__ int32_t s_t[kAttendSlice];
    __shared__ float s_y[kAttendSlice][GP];
    __shared__ float s_stat[2 * GP];
    __shared__ float s_red[(kThreads / 64) * GP];
    __shared__ float s_acc[GP * D];
    __shared__ uint32_t s_flag;

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int unit = blockIdx.y;
    const int slice = blockIdx.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t kp = a.kp;
    const int64_t Tb = seq_len_of(d, b);
    const int r0 = slice * kAttendSlice;
    const uint32_t* gkeys = a.skey + int64_t(unit) * a.kstride;
    uint32_t* gh = a.ghist + int64_t(unit) * kHistBins;

    // ---- loads: the unit's histogram (16 bins per thread) and its keys into LDS ----
    uint32_t h[16];
    load_hist_desc(gh, h);
    const bool lds_keys = kp <= kLdsKeys;
    if (lds_keys) {
        const int64_t kp4 = kp & ~int64_t(3);
#pragma unroll 4
        for (int64_t j = int64_t(tid) * 4; j < kp4; j += int64_t(kThreads) * 4)
            *reinterpret_cast<uint4*>(&s_keys[j]) = *reinterpret_cast<const uint4*>(&gkeys[j]);
        for (int64_t j = kp4 + tid; j < kp; j += kThreads) s_keys[j] = gkeys[j];
    }
    const KeySrc key{lds_keys ? s_keys : nullptr, gkeys};

    // ---- exact top-kappa threshold: tau and the number of keys equal to tau to take ----
    uint32_t nv = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) nv += (kHistBins - 1 - (tid * 16 + k)) > 0 ? h[k] : 0u;  // bin 0 = empty slots
    const uint32_t n_valid = block_sum_u32(nv, s_tmp);  // its barriers also publish s_keys
    const uint32_t kappa_eff = n_valid < uint32_t(a.kappa) ? n_valid : uint32_t(a.kappa);
    uint32_t tau = 1u, need = 0xFFFFFFFFu;  // kappa_eff == n_valid: every valid key (>= 1) is taken
    if (kappa_eff > 0 && kappa_eff < n_valid) {
        find_crossing_regs<16>(h, kHistBins, kappa_eff, s_tmp, s_res);
        const uint32_t bin = s_res[0], above = s_res[1];
        for (int i = tid; i < kHistBins; i += kThreads) s_hist[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < kp; j += kThreads) {
            const uint32_t k = key(j);
            if ((k >> kKeyShift) == bin) atomicAdd(&s_hist[(k >> 8) & 0xFFFu], 1u);
        }
        __syncthreads();
        find_crossing<kHistBins>(s_hist, kappa_eff - above, s_tmp, s_res);
        const uint32_t da = s_res[0], above_a = s_res[1];
        const uint32_t pre = (bin << 12) | da;
        s_hist[tid] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < kp; j += kThreads) {
            const uint32_t k = key(j);
            if ((k >> 8) == pre) atomicAdd(&s_hist[k & 0xFFu], 1u);
        }
        __syncthreads();
        find_crossing<256>(s_hist, kappa_eff - above - above_a, s_tmp, s_res);
        tau = (pre << 8) | s_res[0];
        need = kappa_eff - above - above_a - s_res[1];
    }

    // ---- ranks of the selected slots in slot order (wave w scans a contiguous quarter) ----
    const int n = int(kappa_eff) - r0 < 0 ? 0 : (int(kappa_eff) - r0 > kAttendSlice ? kAttendSlice : int(kappa_eff) - r0);
    if (n > 0) {
        const int64_t Q = ((kp + 4 * 64 - 1) / (4 * 64)) * 64;
        const int64_t w0 = int64_t(wave) * Q, w1 = (w0 + Q < kp) ? w0 + Q : kp;
        uint32_t eq_w = 0;
        for (int64_t j = w0 + lane; j - lane < w1; j += 64) {
            const uint32_t k = j < w1 ? key(j) : 0u;
            eq_w += __popcll(ballot64(k == tau && k != 0u));
        }
        if (lane == 0) s_w[0][wave] = eq_w;
        __syncthreads();
        uint32_t eq_run = 0;
        for (int w = 0; w < wave; ++w) eq_run += s_w[0][w];
        uint32_t sel_w = 0;
        for (int64_t j = w0 + lane; j - lane < w1; j += 64) {
            const uint32_t k = j < w1 ? key(j) : 0u;
            const bool eq = k == tau && k != 0u;
            const uint64_t me = ballot64(eq);
            const bool take = k > tau || (eq && eq_run + lanes_below(me) < need);
            eq_run += __popcll(me);
            sel_w += __popcll(ballot64(take));
        }
        if (lane == 0) s_w[1][wave] = sel_w;
        __syncthreads();
        uint32_t rank = 0;
        eq_run = 0;
        for (int w = 0; w < wave; ++w) {
            rank += s_w[1][w];
            eq_run += s_w[0][w];
        }
        for (int64_t j = w0 + lane; j - lane < w1 && rank < uint32_t(r0 + n); j += 64) {
            const uint32_t k = j < w1 ? key(j) : 0u;
            const bool eq = k == tau && k != 0u;
            const uint64_t me = ballot64(eq);
            const bool take = k > tau || (eq && eq_run + lanes_below(me) < need);
            eq_run += __popcll(me);
            const uint64_t mt = ballot64(take);
            const uint32_t r = rank + lanes_below(mt);
            if (take && r >= uint32_t(r0) && r < uint32_t(r0 + n)) s_slot[r - r0] = int32_t(j);
            rank += __popcll(mt);
        }
    }
    __syncthreads();

    // ---- idx and the slice's rows ----
    const int32_t* pool = a.pool + int64_t(unit) * kp;
    if (tid < kAttendSlice && r0 + tid < a.kappa) {
        int32_t t = -1;
        if (tid < n) {
            int32_t j = s_slot[tid];
            j = (j >= 0 && j < kp) ? j : 0;  // every rank of the slice was filled; keep reads in bounds
            t = pool[j];
            t = (t >= 0 && t < Tb) ? t : 0;
            s_t[tid] = t;
            const float4* lg = reinterpret_cast<const float4*>(a.logits + (int64_t(unit) * kp + j) * LS);
#pragma unroll
            for (int h4 = 0; h4 < LS; h4 += 4) {
                const float4 v = lg[h4 / 4];
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (h4 + e < GP) s_y[tid][h4 + e] = h4 + e < G ? vv[e] * a.y_scale : 0.0f;
            }
        }
        a.idx[int64_t(unit) * a.kappa + r0 + tid] = t;
    }
    __syncthreads();

    const int nsa = int(gridDim.x);
    float* part_ml = a.part_ml + int64_t(unit) * nsa * GP * 2;
    float* part_acc = a.part_acc + int64_t(unit) * nsa * GP * D;
    if (n > 0) {
        const T* Vu = static_cast<const T*>(a.V) + int64_t(unit) * d.T_max * D;
        softmax_v_partial<T, D, GP, kAttendSlice>(Vu, s_t, s_y, n, G, s_stat, s_red, s_acc,
                                                   part_acc + int64_t(slice) * GP * D,
                                                   part_ml + int64_t(slice) * GP * 2);
    }

    if (!arrive_last(&a.done_a[int64_t(unit) * kCtrStride], gridDim.x, &s_flag)) return;

    const int np = int((kappa_eff + kAttendSlice - 1) / kAttendSlice);
    const int64_t hq0 = int64_t(b) * d.Hq + int64_t(g) * G;
    merge_partials<T, D, GP>(part_ml, part_acc, np, G, static_cast<T*>(a.out) + hq0 * D,
                             a.lse ? a.lse + hq0 : nullptr);
    for (int i = tid; i < kHistBins; i += kThreads) gh[i] = 0u;  // every workgroup has read it
    if (tid == 0) a.done_a[int64_t(unit) * kCtrStride] = 0u;
}

template <typename T, int D, int GP>
static hipError_t launch_refine_t(const RefineArgs& a, int agg_max, hipStream_t st) {
    const int units = a.d.B * a.d.Hkv;
    const dim3 gs((a.kp + kScoreSlice - 1) / kScoreSlice, units);
    const dim3 ga((a.kappa + kAttendSlice - 1) / kAttendSlice, units);
    {
        ProfScope prof("k_rscore", st);
        if (agg_max) hipLaunchKernelGGL((k_rscore<T, D, GP, true>), gs, dim3(kThreads), 0, st, a);
        else hipLaunchKernelGGL((k_rscore<T, D, GP, false>), gs, dim3(kThreads), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        const size_t dyn = a.kp <= kLdsKeys ? size_t(a.kp) * 4 : 0;
        ProfScope prof("k_attend", st);
        hipLaunchKernelGGL((k_attend<T, D, GP>), ga, dim3(kThreads), dyn, st, a);
    }
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t refine_g(const RefineArgs& a, int agg_max, hipStream_t st) {
    switch (padded_g(a.d.G)) {
        case 1: return launch_refine_t<T, D, 1>(a, agg_max, st);
        case 2: return launch_refine_t<T, D, 2>(a, agg_max, st);
        case 4: return launch_refine_t<T, D, 4>(a, agg_max, st);
        case 8: return launch_refine_t<T, D, 8>(a, agg_max, st);
        case 16: return launch_refine_t<T, D, 16>(a, agg_max, st);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t refine_d(const RefineArgs& a, int agg_max, hipStream_t st) {
    switch (a.d.D) {
        case 64: return refine_g<T, 64>(a, agg_max, st);
        case 128: return refine_g<T, 128>(a, agg_max, st);
        case 256: return refine_g<T, 256>(a, agg_max, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_refine(const RefineArgs& a, int bf16, int agg_max, hipStream_t st) {
    return bf16 ? refine_d<uint16_t>(a, agg_max, st) : refine_d<float>(a, agg_max, st);
}

}  // namespace prism
