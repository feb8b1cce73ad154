// refine_kernels.hpp -- refined layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4.1: the
// refined layer re-selects its own top-kappa inside the inherited pool; Sec. 5.3: refinement
// touches only the pool, so its cost does not grow with the context).
//
// Two launches per call:
//   k_rscore  grid (pool slices of 64 slots) x units.  Gathers the pool's K rows, computes the G
//             heads' logits (fp32) and the group score S, and stores the logits and {order key
//             of S, id} per slot (key 0 for an empty slot; id = the token, or with paged caches
//             its row in the KV head's pool).  Plain (cached) stores: k_attend reads them next.
//   k_attend  grid (slices of 128, 256 or 512 selected ranks; on small grids 2 or 4 workgroups
//             per slice, each for a range of the V columns) x units, 1024 threads.  Every workgroup derives the
//             exact top-kappa of its unit from the keys, ranks the selected
//             slots in slot order (ties to the lower slot), writes idx for its ranks, gathers
//             their V rows and forms a softmax(.)V partial from the stored logits.  The unit's
//             last workgroup merges the partials (log-sum-exp) into out and lse.
//   k_attend_d  in place of k_attend for kappa <= 2048, G <= 8 and small grids: grid (16- or 8-byte
//             pieces of a V row) x units.  Every workgroup takes the whole selection and writes
//             its columns of out directly (no partials, no merge).
// The kernels and their launch templates; k_refine.hip (bf16) and k_refine_f32.hip (fp32)
// instantiate them, one dtype per translation unit.
#pragma once

#include "prism_attend.hpp"
#include "prism_prof.hpp"
#include "prism_select.hpp"

#ifndef PRISM_ATTEND_D8
#define PRISM_ATTEND_D8 1  // the head-dimension split takes 8-byte pieces where twice the grid fits
#endif
#ifndef PRISM_ATTEND_COLSPLIT
#define PRISM_ATTEND_COLSPLIT 1  // split the rank-split attention's columns in two on small grids
#endif

namespace prism {

// The attention kernel's arrival counters are zeroed by the first pool-scoring workgroup (the
// launch boundary orders these stores before every arrival), so a call never depends on what an
// earlier call left in the workspace.
__device__ __forceinline__ void zero_ctrl(const RefineArgs& a, int nthreads) {
    if (blockIdx.x == 0 && blockIdx.y == 0)
        for (int i = threadIdx.x; i < a.ctrl_words; i += nthreads) a.ctrl[i] = 0u;
}

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
    zero_ctrl(a, kThreads);
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
__global__ __launch_bounds__(kRscoreThreads) void k_rscore_mfma(RefineArgs a) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int STEPS = D / 32;
    constexpr int LS = GP < 4 ? 4 : GP;
    constexpr int SLOTS = 16 * (kRscoreThreads / 64);
    const Dims& d = a.d;
    const int lane = lane_id(), wave = wave_id();
    PRISM_TL(kTlRscore, 0);
    zero_ctrl(a, kRscoreThreads);
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
    PRISM_TL(kTlRscore, 1);
}

template <typename T, int D, int GP, int NR, int DS = 1>
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
    const int slice = ui.x / DS;  // DS workgroups per slice of ranks, each for D / DS of the columns
    const int half = ui.x % DS;   // this workgroup's column range
    constexpr int DH = D / DS;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t kp = a.kp;
    const int r0 = slice * NR;
    PRISM_TL(kTlAttend, 0);

    const SelResult sr = select_ranks<NT>(a.skey + int64_t(unit) * a.kstride, kp, uint32_t(a.kappa), r0, NR, s_big,
                                          s_tmp, s_res, s_cand, s_ccount, s_slot, s_tok);
    const int n = sr.n;
    PRISM_TL(kTlAttend, 1);

    // ---- the slice's softmax(.)V partial, then idx.  s_tok holds the selected slots' record ids:
    // token ids, or with paged caches the row inside the KV head's pool (pool scoring found it) ----
    const bool paged = d.pg.table != nullptr;
    const int nsa = int(gridDim.x) / DS;
    float* part_ml = a.part_ml + int64_t(unit) * nsa * GP * 2;
    float* part_acc = a.part_acc + int64_t(unit) * nsa * GP * D;
    if (n > 0) {  // the DS workgroups of a slice write the same (m, l), each its columns of acc
        const T* Vb = static_cast<const T*>(a.V) + cache_row0(d, b, g) * D + half * DH;
        auto vrow = [&](int32_t id) -> const T* { return Vb + int64_t(uint32_t(id)) * D; };
        softmax_v_rows<T, DH, GP, NR, NT, decltype(vrow), D>(
            vrow, a.logits + int64_t(unit) * kp * LS, LS, a.y_scale, s_slot, s_tok, n, G, s_p, s_red,
            reinterpret_cast<float*>(s_big), part_acc + int64_t(slice) * GP * D + half * DH, part_ml + int64_t(slice) * GP * 2);
    }
    if (half == 0 && tid < NR && r0 + tid < a.kappa) {
        int32_t t = -1;
        if (tid < n) t = paged ? a.pool[int64_t(unit) * kp + s_slot[tid]] : s_tok[tid];
        a.idx[int64_t(unit) * a.kappa + r0 + tid] = t;
    }
    PRISM_TL(kTlAttend, 3);

    const int np = int((sr.kappa_eff + NR - 1) / NR);  // slices that wrote a partial
    const int64_t hq0 = int64_t(b) * d.Hq + int64_t(g) * G;
    T* out = static_cast<T*>(a.out) + hq0 * D + half * DH;
    float* lse = a.lse && half == 0 ? a.lse + hq0 : nullptr;
    uint32_t* done = &a.done_a[int64_t(unit) * kCtrStride + half];  // one counter per column range
    if (nsa <= kMergeGroup) {  // one level: the last slice merges every partial
        if (!arrive_last(done, nsa, &s_flag)) return;
        PRISM_TL(kTlAttend, 4);
        merge_partials<T, DH, GP, NT, false, D>(part_ml, part_acc + half * DH, np, G, out, lse);
        if (tid == 0) *done = 0u;
        PRISM_TL(kTlAttend, 5);
        return;
    }
    // two levels: the last slice of each group of kMergeGroup merges the group's partials into a
    // group partial; the last group to finish merges the group partials
    const int ngrp = (nsa + kMergeGroup - 1) / kMergeGroup;
    const int grp = slice / kMergeGroup;
    const int gsz = nsa - grp * kMergeGroup < kMergeGroup ? nsa - grp * kMergeGroup : kMergeGroup;
    uint32_t* cg = a.done_g + (int64_t(unit) * ngrp + grp) * kCtrStride + half;
    if (!arrive_last(cg, gsz, &s_flag)) return;
    const int gnp = np - grp * kMergeGroup <= 0 ? 0 : (np - grp * kMergeGroup < kMergeGroup ? np - grp * kMergeGroup : kMergeGroup);
    float* g2_ml = a.part2_ml + int64_t(unit) * ngrp * GP * 2;
    float* g2_acc = a.part2_acc + int64_t(unit) * ngrp * GP * D;
    merge_partials<T, DH, GP, NT, true, D>(part_ml + int64_t(grp) * kMergeGroup * GP * 2,
                                           part_acc + int64_t(grp) * kMergeGroup * GP * D + half * DH, gnp, G, nullptr,
                                           nullptr, g2_ml + int64_t(grp) * GP * 2, g2_acc + int64_t(grp) * GP * D + half * DH);
    if (tid == 0) *cg = 0u;
    if (!arrive_last(done, ngrp, &s_flag)) return;
    merge_partials<T, DH, GP, NT, false, D>(g2_ml, g2_acc + half * DH, (np + kMergeGroup - 1) / kMergeGroup, G, out, lse);
    if (tid == 0) *done = 0u;
}

// `hi` on the lanes of the banks ((lane / 4) % 4) in BANKM, `lo` elsewhere: a DPP move with an
// identity pattern and a write mask.
template <int BANKM>
__device__ __forceinline__ float bank_pick(float lo, float hi) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(lo), __float_as_int(hi), 0xE4, 0xF, BANKM, false));
}

// One step of recursive halving over lane bit B (5 to 2): afterwards v[i], i < HALF, holds on a
// lane with bit B clear the sum over the lane pair (lane, lane ^ 2^B) of v[i], and on a lane with
// the bit set that of v[i + HALF].  Bits 5 and 4 exchange halves with the gfx950 half-wave and
// row swaps (the swap hands each lane its partner's copy of the half it keeps); bits 3 and 2
// with row rotations under bank write masks (row_ror:n hands lane l the value of lane l - n mod 16).
template <int B, int HALF, int NV>
__device__ __forceinline__ void halve_step(float (&v)[NV]) {
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
        const uint32_t lo = __float_as_uint(v[i]), hi = __float_as_uint(v[i + HALF]);
        if constexpr (B == 5 || B == 4) {
            const auto r = B == 5 ? __builtin_amdgcn_permlane32_swap(lo, hi, false, false)
                                  : __builtin_amdgcn_permlane16_swap(lo, hi, false, false);
            v[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        } else if constexpr (B == 3) {
            int recv = __builtin_amdgcn_update_dpp(int(lo), int(lo), 0x128, 0xF, 0x3, false);  // banks 0, 1: lane + 8
            recv = __builtin_amdgcn_update_dpp(recv, int(hi), 0x128, 0xF, 0xC, false);          // banks 2, 3: lane - 8
            v[i] = bank_pick<0xC>(v[i], v[i + HALF]) + __int_as_float(recv);
        } else {
            int recv = __builtin_amdgcn_update_dpp(int(lo), int(lo), 0x12C, 0xF, 0x5, false);  // banks 0, 2: lane + 4
            recv = __builtin_amdgcn_update_dpp(recv, int(hi), 0x124, 0xF, 0xA, false);          // banks 1, 3: lane - 4
            v[i] = bank_pick<0xA>(v[i], v[i + HALF]) + __int_as_float(recv);
        }
    }
}

// Sum over the 64 lanes of a wave of NV values per lane (NV a power of two, 4 to 64): recursive
// halving over lane bits 5..2 (S = min(log2 NV, 4) steps), then an all-reduce over aligned groups
// of 64 >> S lanes.  Afterwards the first lane of each group holds the wave's sums of values
// [(lane >> (6 - S)) * R, +R) in v[0, R), R = NV >> S.
template <int NV>
__device__ __forceinline__ void wave_reduce_scatter(float (&v)[NV]) {
    static_assert(NV >= 4 && NV <= 64 && (NV & (NV - 1)) == 0, "power of two, 4 to 64");
    constexpr int S = NV >= 16 ? 4 : NV == 8 ? 3 : 2;
    constexpr int R = NV >> S;
    halve_step<5, NV / 2>(v);
    halve_step<4, NV / 4>(v);
    if constexpr (S >= 3) halve_step<3, NV / 8>(v);
    if constexpr (S >= 4) halve_step<2, NV / 16>(v);
#pragma unroll
    for (int j = 0; j < R; ++j) v[j] = group_sum<(64 >> S)>(v[j]);
}

// Refined attention split over the head dimension, for kappa <= KM <= kAttendDRanks and GP <= 8:
// grid (D / DS column pieces) x units, 1024 threads, DS = PB bytes (16 or 8) of a V row.  Every workgroup
// derives the unit's whole selection (the same exact top-kappa and slot-order ranks as k_attend)
// and the softmax statistics over all selected rows, so it writes its DS columns of out and lse
// directly: no partials and no merge.  When units is a multiple of 8 the unit's workgroups share
// one XCD (unit_major), so a V row is fetched into that XCD's L2 once and each workgroup reads its
// piece from there.  8-byte pieces halve each workgroup's multiply-adds and lane reductions (the
// part of the work that is not repeated per workgroup) where twice the workgroups still fit the CUs.
// Thread t takes ranks t, t + 1024, ...; each wave weights its rows by its own maximum and the
// waves' sums are rescaled to the workgroup maximum and combined in LDS in wave order.
template <typename T, int D, int GP, int KM, int PB>
__global__ __launch_bounds__(kAttendThreads) void k_attend_d(RefineArgs a) {
    constexpr int NT = kAttendThreads;
    constexpr int NW = NT / 64;
    constexpr int DS = PB / int(sizeof(T));
    using VR = std::conditional_t<PB == 16, uint4, uint2>;
    constexpr int NS = D / DS;
    constexpr int RPT = KM / NT;
    constexpr int NV = GP * DS;
    constexpr int LS = GP < 4 ? 4 : GP;  // logit stride
    constexpr int L4 = LS / 4;           // 16-byte logit pieces per slot
    static_assert((PB == 16 || PB == 8) && GP <= 8 && NV >= 4 && NV <= 64 && KM % NT == 0 && KM <= kAttendDRanks &&
                  NS >= 2, "head-dimension split shape");
    static_assert(kHistPadded <= kRowsAccFloats && kSelHistWords <= kRowsAccFloats, "LDS buffer too small");
    __shared__ __align__(16) uint32_t s_big[kRowsAccFloats];  // selection histograms
    __shared__ __align__(16) uint32_t s_cand[kSelCandTotal];
    __shared__ uint32_t s_ccount[NW];
    __shared__ uint32_t s_tmp[sel_tmp_words<NT>()];
    __shared__ uint32_t s_res[16];
    __shared__ int32_t s_slot[KM];
    __shared__ int32_t s_tok[KM];
    __shared__ float s_max[NW * GP];
    __shared__ float s_sum[NW * GP];
    __shared__ float s_part[NW * NV];

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int piece = ui.x;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t kp = a.kp;

    PRISM_TL(kTlAttendD, 0);
    const SelResult sr = select_ranks<NT>(a.skey + int64_t(unit) * a.kstride, kp, uint32_t(a.kappa), 0, KM, s_big,
                                          s_tmp, s_res, s_cand, s_ccount, s_slot, s_tok);
    const int n = sr.n;
    const bool paged = d.pg.table != nullptr;
    PRISM_TL(kTlAttendD, 1);

    // idx: piece p writes ranks [p * per, (p + 1) * per); ranks at or beyond n hold -1
    {
        const int per = (a.kappa + NS - 1) / NS;
        const int r = piece * per + tid;
        if (tid < per && r < a.kappa) {
            int32_t t = -1;
            if (r < n) t = paged ? a.pool[int64_t(unit) * kp + s_slot[r]] : s_tok[r];
            a.idx[int64_t(unit) * a.kappa + r] = t;
        }
    }
    const int64_t hq0 = int64_t(b) * d.Hq + int64_t(g) * G;
    T* out = static_cast<T*>(a.out) + hq0 * D + piece * DS;
    float* lse = a.lse ? a.lse + hq0 : nullptr;
    if (n == 0) {  // no valid slot: out = 0, lse = -inf
        if (tid < G * DS) store_elem<T>(&out[(tid / DS) * D + tid % DS], 0.0f);
        if (piece == 0 && lse && tid < G) lse[tid] = -INFINITY;
        return;
    }

    // this thread's rows: logits of the GP heads and the piece of the V row (clamped, unconditional
    // loads; rows at or beyond n carry weight 0)
    const float* lg = a.logits + int64_t(unit) * kp * LS;
    const T* Vb = static_cast<const T*>(a.V) + cache_row0(d, b, g) * D + piece * DS;
    float4 lraw[RPT][L4];
    VR vraw[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = tid + i * NT;
        const int rr = r < n ? r : 0;
#pragma unroll
        for (int j = 0; j < L4; ++j) lraw[i][j] = reinterpret_cast<const float4*>(lg + int64_t(s_slot[rr]) * LS)[j];
        vraw[i] = *reinterpret_cast<const VR*>(Vb + int64_t(uint32_t(s_tok[rr])) * D);
    }
    float y[RPT][GP];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const bool valid = tid + i * NT < n;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
            const float4 v = lraw[i][h / 4];
            const float c = h % 4 == 0 ? v.x : h % 4 == 1 ? v.y : h % 4 == 2 ? v.z : v.w;
            y[i][h] = (valid && h < G) ? c * a.y_scale : -INFINITY;
        }
    }
    // each wave weights its rows by its own maximum per head (a wave without rows holds -inf and
    // weight 0); the cross-wave sum below rescales to the workgroup maximum, so no barrier stands
    // between a wave's loads and its accumulation
    float M[GP];
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        float m = y[0][h];
#pragma unroll
        for (int i = 1; i < RPT; ++i) m = fmaxf(m, y[i][h]);
        M[h] = wave_max(m);
        if (lane == 0) s_max[wave * GP + h] = M[h];
    }
    PRISM_TL(kTlAttendD, 2);
    static_assert(NW == 16, "one wave maximum per DPP lane");
    float acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = 0.0f;
#pragma unroll
    for (int h = 0; h < GP; ++h) {
        float l = 0.0f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float p = (tid + i * NT < n && h < G) ? exp2_le0(y[i][h] - M[h]) : 0.0f;  // M finite there
            l += p;
            float x[Elem<T>::kPerLane];
            if constexpr (PB == 16) unpack16<T>(vraw[i], x);
            else unpack16<T>(make_uint4(vraw[i].x, vraw[i].y, 0u, 0u), x);  // the first DS values
#pragma unroll
            for (int e = 0; e < DS; ++e) acc[h * DS + e] = fmaf(p, x[e], acc[h * DS + e]);
        }
        l = wave_sum(l);
        if (lane == 0) s_sum[wave * GP + h] = l;
    }
    PRISM_TL(kTlAttendD, 3);
    wave_reduce_scatter<NV>(acc);
    {
        constexpr int S = NV >= 16 ? 4 : NV == 8 ? 3 : 2;
        constexpr int R = NV >> S;
        if ((lane & ((64 >> S) - 1)) == 0) {
#pragma unroll
            for (int j = 0; j < R; ++j) s_part[wave * NV + (lane >> (6 - S)) * R + j] = acc[j];
        }
    }
    PRISM_TL(kTlAttendD, 4);
    __syncthreads();
    PRISM_TL(kTlAttendD, 5);
    // the waves' sums: output o = h DS + e takes one row of 16 lanes, lane w holding wave w's
    // maximum, rescaled sum and weight sum; DPP reductions inside the row
    static_assert(NW == 16 && NV * NW <= NT, "one DPP row of 16 lanes per output");
    if (tid < NV * NW) {
        const int o = tid / NW, w = tid % NW;
        const int h = o / DS, e = o % DS;
        const float mw = h < G ? s_max[w * GP + h] : 0.0f;
        const float Mh = group_max<16>(mw);  // finite where h < G: n >= 1
        const float c = h < G ? exp2_le0(mw - Mh) : 0.0f;  // 0 for a wave without rows
        const float sacc = group_sum<16>(s_part[w * NV + o] * c);
        const float L = group_sum<16>(s_sum[w * GP + h] * c);
        if (w == 0 && h < G) {
            store_elem<T>(&out[int64_t(h) * D + e], sacc / L);
            if (e == 0 && piece == 0 && lse) {
                constexpr float kLn2 = 0.6931471805599453f;
                lse[h] = (Mh + log2f(L)) * kLn2;
            }
        }
    }
    PRISM_TL(kTlAttendD, 6);
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
    const dim3 gsm((a.kp + 16 * (kRscoreThreads / 64) - 1) / (16 * (kRscoreThreads / 64)), units);
    // one attention workgroup fits a CU: when 128 ranks per workgroup would need more workgroups
    // than there are CUs, take 256 ranks each (half the workgroups, twice the rows each), and
    // 512 when 256 would still need more than one round
    const int64_t cus = device_cus();
    const int64_t n128 = int64_t(units) * ((a.kappa + kAttendRanks - 1) / kAttendRanks);
    const int64_t n256 = int64_t(units) * ((a.kappa + 2 * kAttendRanks - 1) / (2 * kAttendRanks));
    const int nr = n128 <= cus ? kAttendRanks : (n256 <= cus ? 2 * kAttendRanks : 4 * kAttendRanks);
    const dim3 ga((a.kappa + nr - 1) / nr, units);
    if constexpr (sizeof(T) == 2) {
        if (agg_max) launch_k("k_rscore", (k_rscore_mfma<D, GP, true>), gsm, dim3(kRscoreThreads), st, a);
        else launch_k("k_rscore", (k_rscore_mfma<D, GP, false>), gsm, dim3(kRscoreThreads), st, a);
    } else {
        if (agg_max) launch_k("k_rscore", (k_rscore<T, D, GP, true>), gs, dim3(kThreads), st, a);
        else launch_k("k_rscore", (k_rscore<T, D, GP, false>), gs, dim3(kThreads), st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (PRISM_ATTEND_DSPLIT && GP <= 8) {
        // head-dimension split while its grid (D / 16-byte pieces per unit) fits one workgroup per
        // CU: every workgroup gathers all kappa rows, so on fuller grids the rank split is faster
        constexpr int ns = D / Elem<T>::kPerLane;  // 16-byte pieces
        constexpr bool half_ok = PRISM_ATTEND_D8 && GP * Elem<T>::kPerLane / 2 >= 4;
        if (a.kappa <= kAttendDRanks && int64_t(units) * ns <= int64_t(device_cus())) {
            const bool small = a.kappa <= kAttendDRanks / 2;
            if constexpr (half_ok) {
                if (int64_t(units) * 2 * ns <= int64_t(device_cus())) {
                    const dim3 gd(2 * ns, units);
                    if (small) launch_k("k_attend", (k_attend_d<T, D, GP, kAttendDRanks / 2, 8>), gd, dim3(kAttendThreads), st, a);
                    else launch_k("k_attend", (k_attend_d<T, D, GP, kAttendDRanks, 8>), gd, dim3(kAttendThreads), st, a);
                    return hipGetLastError();
                }
            }
            const dim3 gd(ns, units);
            if (small) launch_k("k_attend", (k_attend_d<T, D, GP, kAttendDRanks / 2, 16>), gd, dim3(kAttendThreads), st, a);
            else launch_k("k_attend", (k_attend_d<T, D, GP, kAttendDRanks, 16>), gd, dim3(kAttendThreads), st, a);
            return hipGetLastError();
        }
    }
    if (nr == 4 * kAttendRanks) launch_k("k_attend", (k_attend<T, D, GP, 4 * kAttendRanks>), ga, dim3(kAttendThreads), st, a);
    else if (nr == 2 * kAttendRanks) launch_k("k_attend", (k_attend<T, D, GP, 2 * kAttendRanks>), ga, dim3(kAttendThreads), st, a);
    else {
        // at most a quarter (a half) of the CUs busy at 128 ranks: four (two) workgroups per
        // slice, each for that share of the columns of V (that share of the rows' bytes; the
        // merges run per column range)
        if constexpr (PRISM_ATTEND_COLSPLIT && D / 4 >= 64) {
            if (4 * n128 <= cus) {
                launch_k("k_attend", (k_attend<T, D, GP, kAttendRanks, 4>), dim3(4 * ga.x, ga.y), dim3(kAttendThreads), st,
                         a);
                return hipGetLastError();
            }
        }
        if constexpr (PRISM_ATTEND_COLSPLIT && D / 2 >= 64) {
            if (2 * n128 <= cus) {
                launch_k("k_attend", (k_attend<T, D, GP, kAttendRanks, 2>), dim3(2 * ga.x, ga.y), dim3(kAttendThreads), st,
                         a);
                return hipGetLastError();
            }
        }
        launch_k("k_attend", (k_attend<T, D, GP, kAttendRanks>), ga, dim3(kAttendThreads), st, a);
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
