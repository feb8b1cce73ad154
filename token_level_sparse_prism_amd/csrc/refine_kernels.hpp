// refine_kernels.hpp -- refined layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4.1: the
// refined layer re-selects its own top-kappa inside the inherited pool; Sec. 5.3: refinement
// touches only the pool, so its cost does not grow with the context).
//
// Two launches per call:
//   k_rscore  grid (pool slices of 64 slots) x units.  Gathers the pool's K rows, computes the G
//             heads' logits (fp32) and the group score S, and stores the logits and {order key
//             of S, id} per slot (key 0 for an empty slot; id = the token, or with paged caches
//             its row in the KV head's pool).  Plain (cached) stores: k_attend reads them next.
//   k_attend  grid (128 or 256 selected ranks) x units, 1024 threads.  Every workgroup derives the
//             exact top-kappa of its unit from the keys, ranks the selected
//             slots in slot order (ties to the lower slot), writes idx for its ranks, gathers
//             their V rows and forms a softmax(.)V partial from the stored logits.  The unit's
//             last workgroup merges the partials (log-sum-exp) into out and lse.
// The kernels and their launch templates; k_refine.hip (bf16) and k_refine_f32.hip (fp32)
// instantiate them, one dtype per translation unit.
#pragma once

#include "prism_attend.hpp"
#include "prism_prof.hpp"
#include "prism_select.hpp"

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

    const Dims& d = a.d;
    const int lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int slice = ui.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp = a.kp;
    const int sub = lane % LPR;

    QRegs<T, D, GP> q;
    q.load(static_cast<const T*>(a.q) + (int64_t(b) * d.Hq + int64_t(g) * G) * D, G, sub);
    const T* Kb = static_cast<const T*>(a.K);
    const int32_t* pool = a.pool + int64_t(unit) * kp;
    uint2* skey = a.skey + int64_t(unit) * a.kstride;
    float* logits = a.logits + int64_t(unit) * kp * LS;
    const int64_t j0 = int64_t(slice) * kScoreSlice;
    const int rl = wave * RPW + lane / LPR;

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
            raw[u] = (t[u] >= 0 && t[u] < Tb) ? load16(Kb + cache_row(d, b, g, t[u]) * D + sub * EPL) : make_uint4(0, 0, 0, 0);
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
                const uint32_t id = d.pg.table ? uint32_t(cache_row(d, b, g, t[u]) - cache_row0(d, b, g)) : uint32_t(t[u]);
                skey[j] = make_uint2(key, valid ? id : 0xFFFFFFFFu);
#pragma unroll
                for (int h4 = 0; h4 < LS; h4 += 4) {
                    float4 v;
                    v.x = h4 + 0 < GP ? l[h4 + 0] : 0.0f;
                    v.y = h4 + 1 < GP ? l[h4 + 1] : 0.0f;
                    v.z = h4 + 2 < GP ? l[h4 + 2] : 0.0f;
                    v.w = h4 + 3 < GP ? l[h4 + 3] : 0.0f;
                    *reinterpret_cast<float4*>(&logits[j * LS + h4]) = v;
                }
            }
        }
    }
}

// Matrix-core variant for bf16 (dense contraction of the G query heads with the gathered K rows).
// v_mfma_f32_16x16x32_bf16 per 32 dims: A = the unit's queries (16 rows, heads >= G zero), B = 16
// pool rows; lane l carries row / column l % 16 and dims 8 (l / 16) .. + 7 of the step, so a B
// operand is one 16-byte piece of a K row.  A wave scores 16 slots; lane group l / 16 ends with
// heads 4 (l / 16) .. + 3 of slot l % 16.
template <int D, int GP, bool kMax>
__global__ __launch_bounds__(kThreads) void k_rscore_mfma(RefineArgs a) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int STEPS = D / 32;
    constexpr int LS = GP < 4 ? 4 : GP;
    constexpr int SLOTS = 16 * (kThreads / 64);
    static_assert(SLOTS == kScoreSlice, "one slice of slots per workgroup");
    const Dims& d = a.d;
    const int lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp = a.kp;
    const int n = lane & 15, kg = lane >> 4;
    const int64_t j = int64_t(ui.x) * SLOTS + wave * 16 + n;

    // The slot, the query pieces and then the whole K row are each loaded unconditionally (clamped
    // addresses) and fenced from the matrix products: otherwise the compiler waits for the slot
    // together with the queries and issues the row's pieces between the products, one memory
    // round trip each.
    int32_t t = a.pool[int64_t(unit) * kp + (j < kp ? j : kp - 1)];
    const int nq = n < G ? n : G - 1;
    const uint16_t* qh = static_cast<const uint16_t*>(a.q) + (int64_t(b) * d.Hq + int64_t(g) * G + nq) * D + 8 * kg;
    uint4 qraw[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) qraw[s] = load16(qh + 32 * s);
    __builtin_amdgcn_sched_barrier(0);
    if (j >= kp) t = -1;
    const bool valid = t >= 0 && t < Tb;
    const int64_t krow = valid ? cache_row(d, b, g, t) : cache_row0(d, b, g);
    const uint16_t* kr = static_cast<const uint16_t*>(a.K) + krow * D + 8 * kg;
    uint4 kb[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) kb[s] = load16(kr + 32 * s);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 qa[STEPS];  // rows of heads >= G are zero
#pragma unroll
    for (int s = 0; s < STEPS; ++s) qa[s] = __builtin_bit_cast(bf16x8, n < G ? qraw[s] : make_uint4(0u, 0u, 0u, 0u));
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8, kb[s]), acc, 0, 0, 0);

    // group score over the heads this lane holds, then over the lane groups holding heads
    const float l4[4] = {acc[0], acc[1], acc[2], acc[3]};
    float S = kMax ? -INFINITY : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (4 * kg + i < G) S = kMax ? fmaxf(S, l4[i]) : S + l4[i];
    }
    if constexpr (GP > 4) {
        const float o = __shfl_xor(S, 16);
        S = kMax ? fmaxf(S, o) : S + o;
    }
    if constexpr (GP > 8) {
        const float o = __shfl_xor(S, 32);
        S = kMax ? fmaxf(S, o) : S + o;
    }
    if (j < kp) {
        if (4 * kg < LS) {
            float4 v;
            v.x = 4 * kg + 0 < GP ? l4[0] : 0.0f;
            v.y = 4 * kg + 1 < GP ? l4[1] : 0.0f;
            v.z = 4 * kg + 2 < GP ? l4[2] : 0.0f;
            v.w = 4 * kg + 3 < GP ? l4[3] : 0.0f;
            *reinterpret_cast<float4*>(a.logits + (int64_t(unit) * kp + j) * LS + 4 * kg) = v;
        }
        if (kg == 0) {
            const uint32_t key = valid ? order_key(S) : 0u;
            const uint32_t id = d.pg.table ? uint32_t(krow - cache_row0(d, b, g)) : uint32_t(t);
            a.skey[int64_t(unit) * a.kstride + j] = make_uint2(key, valid ? id : 0xFFFFFFFFu);
        }
    }
}

template <typename T, int D, int GP, int NR>
__global__ __launch_bounds__(kAttendThreads) void k_attend(RefineArgs a) {
    constexpr int NT = kAttendThreads;
    constexpr int NW = NT / 64;
    constexpr int LS = GP < 4 ? 4 : GP;
    static_assert(kHistPadded <= kRowsAccFloats && kSelHistWords <= kRowsAccFloats, "LDS buffer too small");
    __shared__ __align__(16) uint32_t s_big[kRowsAccFloats];  // selection histograms, then the waves' V partials
    __shared__ __align__(16) uint32_t s_cand[kSelCandTotal];
    __shared__ uint32_t s_ccount[NW];
    __shared__ uint32_t s_tmp[sel_tmp_words<NT>()];
    __shared__ uint32_t s_res[16];
    __shared__ int32_t s_slot[NR];
    __shared__ int32_t s_tok[NR];
    __shared__ __align__(16) float s_p[NR * GP];
    __shared__ float s_red[2 * NW * GP];
    __shared__ uint32_t s_flag;

    const Dims& d = a.d;
    const int tid = threadIdx.x;
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int slice = ui.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t kp = a.kp;
    const int r0 = slice * NR;

    const SelResult sr = select_ranks<NT>(a.skey + int64_t(unit) * a.kstride, kp, uint32_t(a.kappa), r0, NR, s_big,
                                          s_tmp, s_res, s_cand, s_ccount, s_slot, s_tok);
    const int n = sr.n;

    // ---- the slice's softmax(.)V partial, then idx.  s_tok holds the selected slots' record ids:
    // token ids, or with paged caches the row inside the KV head's pool (pool scoring found it) ----
    const bool paged = d.pg.table != nullptr;
    const int nsa = int(gridDim.x);
    float* part_ml = a.part_ml + int64_t(unit) * nsa * GP * 2;
    float* part_acc = a.part_acc + int64_t(unit) * nsa * GP * D;
    if (n > 0) {
        const T* Vb = static_cast<const T*>(a.V) + cache_row0(d, b, g) * D;
        auto vrow = [&](int32_t id) -> const T* { return Vb + int64_t(uint32_t(id)) * D; };
        softmax_v_rows<T, D, GP, NR, NT>(vrow, a.logits + int64_t(unit) * kp * LS, LS, a.y_scale, s_slot, s_tok, n, G,
                                         s_p, s_red, reinterpret_cast<float*>(s_big), part_acc + int64_t(slice) * GP * D,
                                         part_ml + int64_t(slice) * GP * 2);
    }
    if (tid < NR && r0 + tid < a.kappa) {
        int32_t t = -1;
        if (tid < n) t = paged ? a.pool[int64_t(unit) * kp + s_slot[tid]] : s_tok[tid];
        a.idx[int64_t(unit) * a.kappa + r0 + tid] = t;
    }

    const int np = int((sr.kappa_eff + NR - 1) / NR);  // slices that wrote a partial
    const int64_t hq0 = int64_t(b) * d.Hq + int64_t(g) * G;
    T* out = static_cast<T*>(a.out) + hq0 * D;
    float* lse = a.lse ? a.lse + hq0 : nullptr;
    if (nsa <= kMergeGroup) {  // one level: the last slice merges every partial
        if (!arrive_last(&a.done_a[int64_t(unit) * kCtrStride], nsa, &s_flag)) return;
        merge_partials<T, D, GP, NT>(part_ml, part_acc, np, G, out, lse);
        if (tid == 0) a.done_a[int64_t(unit) * kCtrStride] = 0u;
        return;
    }
    // two levels: the last slice of each group of kMergeGroup merges the group's partials into a
    // group partial; the last group to finish merges the group partials
    const int ngrp = (nsa + kMergeGroup - 1) / kMergeGroup;
    const int grp = slice / kMergeGroup;
    const int gsz = nsa - grp * kMergeGroup < kMergeGroup ? nsa - grp * kMergeGroup : kMergeGroup;
    uint32_t* cg = a.done_g + (int64_t(unit) * ngrp + grp) * kCtrStride;
    if (!arrive_last(cg, gsz, &s_flag)) return;
    const int gnp = np - grp * kMergeGroup <= 0 ? 0 : (np - grp * kMergeGroup < kMergeGroup ? np - grp * kMergeGroup : kMergeGroup);
    float* g2_ml = a.part2_ml + int64_t(unit) * ngrp * GP * 2;
    float* g2_acc = a.part2_acc + int64_t(unit) * ngrp * GP * D;
    merge_partials<T, D, GP, NT, true>(part_ml + int64_t(grp) * kMergeGroup * GP * 2,
                                       part_acc + int64_t(grp) * kMergeGroup * GP * D, gnp, G, nullptr, nullptr,
                                       g2_ml + int64_t(grp) * GP * 2, g2_acc + int64_t(grp) * GP * D);
    if (tid == 0) *cg = 0u;
    if (!arrive_last(&a.done_a[int64_t(unit) * kCtrStride], ngrp, &s_flag)) return;
    merge_partials<T, D, GP, NT>(g2_ml, g2_acc, (np + kMergeGroup - 1) / kMergeGroup, G, out, lse);
    if (tid == 0) a.done_a[int64_t(unit) * kCtrStride] = 0u;
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

template <typename T, int D, int GP>
static hipError_t launch_refine_t(const RefineArgs& a, int agg_max, hipStream_t st) {
    const int units = a.d.B * a.d.Hkv;
    const dim3 gs((a.kp + kScoreSlice - 1) / kScoreSlice, units);
    // one attention workgroup fits a CU: when 128 ranks per workgroup would need more workgroups
    // than there are CUs, take 256 ranks each (half the workgroups, twice the rows each)
    const int64_t n128 = int64_t(units) * ((a.kappa + kAttendRanks - 1) / kAttendRanks);
    const bool wide = n128 > device_cus();
    const int nr = wide ? 2 * kAttendRanks : kAttendRanks;
    const dim3 ga((a.kappa + nr - 1) / nr, units);
    if constexpr (sizeof(T) == 2) {
        if (agg_max) launch_k("k_rscore", (k_rscore_mfma<D, GP, true>), gs, dim3(kThreads), st, a);
        else launch_k("k_rscore", (k_rscore_mfma<D, GP, false>), gs, dim3(kThreads), st, a);
    } else {
        if (agg_max) launch_k("k_rscore", (k_rscore<T, D, GP, true>), gs, dim3(kThreads), st, a);
        else launch_k("k_rscore", (k_rscore<T, D, GP, false>), gs, dim3(kThreads), st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        if (wide) launch_k("k_attend", (k_attend<T, D, GP, 2 * kAttendRanks>), ga, dim3(kAttendThreads), st, a);
        else launch_k("k_attend", (k_attend<T, D, GP, kAttendRanks>), ga, dim3(kAttendThreads), st, a);
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

}  // namespace prism
