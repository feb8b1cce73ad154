// k_refine.hip -- refined layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4.1: the
// refined layer re-selects its own top-kappa inside the inherited pool; Sec. 5.3: refinement
// touches only the pool, so its cost does not grow with the context).
//
// Two launches per call:
//   k_rscore  grid (pool slices of 256 slots) x units.  Gathers the pool's K rows, computes the
//             G heads' logits (fp32) and the group score S, stores the logits and an order key of
//             S, and histograms the keys' top 12 bits.  The unit's last workgroup selects the
//             top-kappa slots exactly (radix digits 12/12/8 over the keys, ties to the lower
//             slot) and lists them in slot order.
//   k_attend  grid (64 selected rows) x units.  Writes idx, gathers the selected V rows and
//             forms a softmax(.)V partial from the stored logits; the unit's last workgroup
//             merges the partials (log-sum-exp) into out and lse.
#include "prism_attend.hpp"
#include "prism_prof.hpp"

namespace prism {

enum { kRModeEmpty = 0, kRModeAll = 1, kRModeSelect = 2 };

template <typename T, int D, int GP, bool kMax>
__global__ __launch_bounds__(kThreads) void k_rscore(RefineArgs a) {
    constexpr int EPL = Elem<T>::kPerLane;
    constexpr int LPR = D / EPL;
    constexpr int RPW = 64 / LPR;
    constexpr int RPR = RPW * (kThreads / 64);
    constexpr int ROUNDS = kScoreSlice / RPR;
    constexpr int U = ROUNDS < 8 ? ROUNDS : 8;
    constexpr int LS = GP < 4 ? 4 : GP;
    static_assert(ROUNDS % U == 0, "slice must hold whole unrolled rounds");

    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_tmp[kThreads / 64];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_flag;

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
    uint32_t* skey = a.skey + int64_t(unit) * kp;
    float* logits = a.logits + int64_t(unit) * kp * LS;
    const int j0 = slice * kScoreSlice;
    const int rl = wave * RPW + lane / LPR;
    __syncthreads();

    for (int r0 = 0; r0 < ROUNDS; r0 += U) {
        uint4 raw[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = j0 + (r0 + u) * RPR + rl;
            const int32_t t = j < kp ? pool[j] : -1;
            valid[u] = t >= 0 && t < Tb;
            raw[u] = valid[u] ? load16(Ku + int64_t(t) * D + sub * EPL) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t j = j0 + (r0 + u) * RPR + rl;
            float x[EPL];
            unpack16<T>(raw[u], x);
            float l[GP];
            row_logits<T, D, GP>(q, x, l);
            float S = l[0];
#pragma unroll
            for (int h = 1; h < GP; ++h) {
                if (h < G) S = kMax ? fmaxf(S, l[h]) : S + l[h];
            }
            if (sub == 0 && j < kp) {
                const uint32_t key = valid[u] ? order_key(S) : 0u;
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
                if (valid[u]) atomicAdd(&s_hist[key >> kKeyShift], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t* gh = a.ghist + int64_t(unit) * kHistBins;
    for (int i = tid; i < kHistBins; i += kThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }

    if (!arrive_last(&a.done_s[unit], gridDim.x, &s_flag)) return;

    // ---- last workgroup: exact top-kappa of the unit's pool slots ----
    for (int i = tid; i < kHistBins; i += kThreads) s_hist[i] = gh[i];
    __syncthreads();
    uint32_t nv = 0;
    for (int i = tid; i < kHistBins; i += kThreads) nv += i > 0 ? s_hist[i] : 0u;  // key 0 = empty slot
    const uint32_t n_valid = block_sum_u32(nv, s_tmp);
    const uint32_t kappa_eff = n_valid < uint32_t(a.kappa) ? n_valid : uint32_t(a.kappa);
    uint32_t* st = a.state + int64_t(unit) * 8;
    int32_t* sel = a.sel + int64_t(unit) * a.kappa;
    const uint32_t mode = kappa_eff == 0 ? kRModeEmpty : (kappa_eff == n_valid ? kRModeAll : kRModeSelect);

    uint32_t tau = 1u, need = 0xFFFFFFFFu;  // kRModeAll: every valid key (>= 1) is selected
    if (mode == kRModeSelect) {
        find_crossing<kHistBins>(s_hist, kappa_eff, s_tmp, s_res);
        const uint32_t bin = s_res[0], above = s_res[1];
        for (int i = tid; i < kHistBins; i += kThreads) s_hist[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < kp; j += kThreads) {
            const uint32_t k = skey[j];
            if ((k >> kKeyShift) == bin) atomicAdd(&s_hist[(k >> 8) & 0xFFFu], 1u);
        }
        __syncthreads();
        find_crossing<kHistBins>(s_hist, kappa_eff - above, s_tmp, s_res);
        const uint32_t da = s_res[0], above_a = s_res[1];
        const uint32_t pre = (bin << 12) | da;
        for (int i = tid; i < 256; i += kThreads) s_hist[i] = 0u;
        __syncthreads();
        for (int64_t j = tid; j < kp; j += kThreads) {
            const uint32_t k = skey[j];
            if ((k >> 8) == pre) atomicAdd(&s_hist[k & 0xFFu], 1u);
        }
        __syncthreads();
        find_crossing<256>(s_hist, kappa_eff - above - above_a, s_tmp, s_res);
        tau = (pre << 8) | s_res[0];
        need = kappa_eff - above - above_a - s_res[1];
    }
    if (mode != kRModeEmpty) {
        // ordered compaction over slots: 8 consecutive slots per thread per tile
        constexpr int IT = 8;
        uint32_t out_base = 0, eq_base = 0;
        for (int64_t t0 = 0; t0 < kp; t0 += int64_t(kThreads) * IT) {
            uint32_t k[IT];
            uint32_t neq = 0;
#pragma unroll
            for (int i = 0; i < IT; ++i) {
                const int64_t j = t0 + int64_t(tid) * IT + i;
                k[i] = j < kp ? skey[j] : 0u;
                neq += (k[i] == tau && k[i] != 0u) ? 1u : 0u;
            }
            uint32_t eq_tot;
            uint32_t eqr = eq_base + block_excl_scan(neq, s_tmp, &eq_tot);
            bool take[IT];
            uint32_t ns = 0;
#pragma unroll
            for (int i = 0; i < IT; ++i) {
                bool s = false;
                if (k[i] != 0u) {
                    if (k[i] > tau) s = true;
                    else if (k[i] == tau) { s = eqr < need; ++eqr; }
                }
                take[i] = s;
                ns += s ? 1u : 0u;
            }
            uint32_t s_tot;
            uint32_t pos = out_base + block_excl_scan(ns, s_tmp, &s_tot);
#pragma unroll
            for (int i = 0; i < IT; ++i) {
                if (take[i] && pos < uint32_t(a.kappa)) sel[pos] = int32_t(t0 + int64_t(tid) * IT + i);
                pos += take[i] ? 1u : 0u;
            }
            out_base += s_tot;
            eq_base += eq_tot;
        }
    }
    for (int i = tid; i < kHistBins; i += kThreads) gh[i] = 0u;
    if (tid == 0) {
        st[0] = mode;
        st[1] = kappa_eff;
        a.done_s[unit] = 0u;
    }
}

template <typename T, int D, int GP>
__global__ __launch_bounds__(kThreads) void k_attend(RefineArgs a) {
    constexpr int LS = GP < 4 ? 4 : GP;
    __shared__ int32_t s_t[kAttendSlice];
    __shared__ float s_y[kAttendSlice][GP];
    __shared__ float s_stat[2 * GP];
    __shared__ float s_red[(kThreads / 64) * GP];
    __shared__ float s_acc[GP * D];
    __shared__ uint32_t s_flag;

    const Dims& d = a.d;
    const int tid = threadIdx.x;
    const int unit = blockIdx.y;
    const int slice = blockIdx.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t kp = a.kp;
    const uint32_t* st = a.state + int64_t(unit) * 8;
    const int kappa_eff = int(st[1]);
    const int r0 = slice * kAttendSlice;
    const int32_t* pool = a.pool + int64_t(unit) * kp;
    const int32_t* sel = a.sel + int64_t(unit) * a.kappa;
    const int nsa = int(gridDim.x);
    float* part_ml = a.part_ml + int64_t(unit) * nsa * GP * 2;
    float* part_acc = a.part_acc + int64_t(unit) * nsa * GP * D;

    const int n = kappa_eff - r0 < 0 ? 0 : (kappa_eff - r0 > kAttendSlice ? kAttendSlice : kappa_eff - r0);
    if (tid < kAttendSlice && r0 + tid < a.kappa) {
        int32_t t = -1;
        if (tid < n) {
            int32_t j = sel[r0 + tid];
            j = (j >= 0 && j < kp) ? j : 0;  // selected slots are in range; keep reads in bounds regardless
            t = pool[j];
            t = (t >= 0 && t < seq_len_of(d, b)) ? t : 0;
            s_t[tid] = t;
            const float* lg = a.logits + (int64_t(unit) * kp + j) * LS;
#pragma unroll
            for (int h = 0; h < GP; ++h) s_y[tid][h] = h < G ? lg[h] * a.y_scale : 0.0f;
        }
        a.idx[int64_t(unit) * a.kappa + r0 + tid] = t;
    }
    __syncthreads();
    if (n > 0) {
        const T* Vu = static_cast<const T*>(a.V) + int64_t(unit) * d.T_max * D;
        softmax_v_partial<T, D, GP, kAttendSlice>(Vu, s_t, s_y, n, G, s_stat, s_red, s_acc,
                                                   part_acc + int64_t(slice) * GP * D,
                                                   part_ml + int64_t(slice) * GP * 2);
    }

    if (!arrive_last(&a.done_a[unit], gridDim.x, &s_flag)) return;

    const int np = (kappa_eff + kAttendSlice - 1) / kAttendSlice;
    const int64_t hq0 = int64_t(b) * d.Hq + int64_t(g) * G;
    merge_partials<T, D, GP>(part_ml, part_acc, np, G, static_cast<T*>(a.out) + hq0 * D,
                             a.lse ? a.lse + hq0 : nullptr);
    if (tid == 0) a.done_a[unit] = 0u;
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
        ProfScope prof("k_attend", st);
        hipLaunchKernelGGL((k_attend<T, D, GP>), ga, dim3(kThreads), 0, st, a);
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
