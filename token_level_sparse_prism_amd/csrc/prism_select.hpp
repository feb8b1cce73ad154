// prism_select.hpp -- exact top-kappa selection of one unit's pool slots inside one workgroup
// (the refined layer's re-selection within the inherited pool, Prism Attention page Sec. 4.1).
//
// Input per pool slot: {order key of the group score S (0 = empty slot), token id}.
//   1. The keys' top 12 bits are counted in an LDS histogram; a workgroup scan over it in
//      descending bin order finds the bin that holds the kappa-th largest key.
//   2. The keys of that bin are compacted into per-wave LDS lists with wave ballots.
//   3. The candidates' next 8 bits (19..12) are counted in a 256-bin LDS histogram and one wave
//      finds the sub-bin of the threshold; the few keys of that sub-bin give the exact threshold
//      key tau, how many keys equal to tau are taken and how many there are, by direct counting.
//      When a wave's list overflows, two radix digits (12 + 8 bits) over every key are used.
//   4. Selected slots are ranked in slot order, ties at tau going to the lower slot, with
//      workgroup scans; ranks [r0, r0 + n) land in LDS with their token ids.
// Keys are read in tiles of 8192 slots, two slots per thread and row (one 16-byte load).
// Pools of one tile take select_ranks_lean (below), which builds the level-2 histogram straight
// from the registers and ranks with one packed scan; the general path above serves larger pools
// and thresholds with heavy ties.
#pragma once

#include "prism_device.hpp"
#include "prism_prof.hpp"

#ifndef PRISM_SELECT_LEAN
#define PRISM_SELECT_LEAN 1  // single-tile pools take the lean selection path
#endif

namespace prism {

constexpr int64_t kSelTile = 8192;
template <int NT> constexpr int sel_rows() { return int(kSelTile / (2 * NT)); }
// LDS words of the selection's scan scratch (s_tmp)
template <int NT> constexpr int sel_tmp_words() { return (NT / 64) * (sel_rows<NT>() > 2 ? sel_rows<NT>() : 2); }
constexpr int kSelCandTotal = 2048;  // LDS list of the threshold bin's keys, split over the waves
template <int NT> constexpr int sel_cand_per_wave() { return kSelCandTotal / (NT / 64); }

struct SelResult {
    uint32_t kappa_eff;  // min(kappa, number of valid slots)
    int n;               // ranks [r0, r0 + n) written to s_slot / s_tok
};

// s_res words
enum : int {
    kResValid = 0, kResKappa, kResBin, kResAbove, kResCount, kResTau, kResNeed, kResEq,
    kResOvf, kResBin2, kResAbove2, kResC2, kResScratch
};

template <int NT>
__device__ __forceinline__ void sel_load_tile(const uint2* __restrict__ gk, int64_t kp, int64_t t0, uint4* kv) {
#pragma unroll
    for (int r = 0; r < sel_rows<NT>(); ++r) {
        const int64_t j = t0 + int64_t(r) * 2 * NT + int64_t(threadIdx.x) * 2;
        if (j + 2 <= kp) {
            kv[r] = *reinterpret_cast<const uint4*>(gk + j);
        } else {
            const uint2 v = j < kp ? gk[j] : make_uint2(0u, 0xFFFFFFFFu);
            kv[r] = make_uint4(v.x, v.y, 0u, 0xFFFFFFFFu);
        }
    }
}

// LDS: the 4096-bin level-1 histogram, then the 256-bin level-2 histogram.
constexpr int kHist1Words = kHistBins;
constexpr int kSelHistWords = kHist1Words + 256;

// Level-2 crossing, run by one wave over the 256-bin histogram of bits 19..12 of the threshold
// bin's keys: lane l holds bins 255 - 4 l - k (k < 4).  Requires 1 <= R <= the histogram total.
__device__ __forceinline__ void sel_sub_crossing(const uint32_t* s_h2, uint32_t R, uint32_t* s_res) {
    const int lane = lane_id();
    const uint4 x = reinterpret_cast<const uint4*>(s_h2)[63 - lane];  // bins 252 - 4 l .. 255 - 4 l
    const uint32_t c[4] = {x.w, x.z, x.y, x.x};
    const uint32_t sum = (c[0] + c[1]) + (c[2] + c[3]);
    const uint32_t incl = wave_incl_scan(sum);
    uint32_t acc = incl - sum;
    if (acc < R && R <= incl) {
        bool f = false;
        uint32_t bin = 0, above = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool hit = !f && acc + c[k] >= R;
            bin = hit ? uint32_t(255 - 4 * lane - k) : bin;
            above = hit ? acc : above;
            f = f || hit;
            acc += f ? 0u : c[k];
        }
        s_res[kResBin2] = bin;
        s_res[kResAbove2] = above;
    }
}

// Histogram of the digit (k >> shift) & mask over the keys whose bits from pre_shift up equal
// `pre`, from the per-wave lists when none overflowed, else from every key again.
template <int NT>
__device__ __forceinline__ void sel_digit_hist(const uint2* __restrict__ gk, int64_t kp, int ntiles, uint4* kv,
                                               const uint32_t* s_cand, const uint32_t* s_ccount, bool from_list,
                                               uint32_t pre, int pre_shift, int shift, uint32_t mask, bool padded,
                                               uint32_t* s_hist) {
    const int tid = threadIdx.x;
    if (from_list) {
        for (int w = 0; w < NT / 64; ++w) {
            const int c = int(s_ccount[w]);
            for (int i = tid; i < c; i += NT) {
                const uint32_t k = s_cand[w * sel_cand_per_wave<NT>() + i];
                if ((k >> pre_shift) == pre) {
                    const int bin = int((k >> shift) & mask);
                    atomicAdd(&s_hist[padded ? hpad(bin) : bin], 1u);
                }
            }
        }
    } else {
        for (int t = 0; t < ntiles; ++t) {
            if (ntiles > 1) sel_load_tile<NT>(gk, kp, int64_t(t) * kSelTile, kv);
#pragma unroll
            for (int r = 0; r < sel_rows<NT>(); ++r) {
                const uint32_t k2[2] = {kv[r].x, kv[r].z};
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    if ((k2[e] >> pre_shift) == pre && k2[e]) {
                        const int bin = int((k2[e] >> shift) & mask);
                        atomicAdd(&s_hist[padded ? hpad(bin) : bin], 1u);
                    }
                }
            }
        }
    }
}

// Exclusive prefix sum over the workgroup in thread order with one barrier: s_w (NT/64 words)
// must not be touched by other code between the caller's previous barrier and its next one.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan1(uint32_t v, uint32_t* s_w, uint32_t* total) {
    const uint32_t x = wave_incl_scan(v);
    if (lane_id() == 63) s_w[wave_id()] = x;
    __syncthreads();
    uint32_t before, tot;
    wave_totals_prefix<NT / 64>(s_w, &before, &tot);
    *total = tot;
    return before + x - v;
}

constexpr int kLeanShort = 256;  // keys sharing the threshold's top 20 bits that the lean path ranks directly

// N exclusive prefix sums over the workgroup in thread order with one barrier (s_w: N * NT/64
// words, not touched by other code between the caller's previous barrier and its next one).
template <int N, int NT>
__device__ __forceinline__ void block_excl_scan1_n(const uint32_t* v, uint32_t* pre, uint32_t* tot, uint32_t* s_w) {
    constexpr int NW = NT / 64;
    uint32_t x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = wave_incl_scan(v[i]);
    if (lane_id() == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i) s_w[i * NW + wave_id()] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t before;
        wave_totals_prefix<NW>(s_w + i * NW, &before, &tot[i]);
        pre[i] = before + x[i] - v[i];
    }
}

// Ranks in slot order of one tile's selected slots when every key at or above tau is taken:
// thread t holds slots slot0 + 2 NT r + 2 t + e in kv[r] (keys .x/.z, ids .y/.w).  Per row, two
// wave ballots give every slot's rank among the wave's slots; the waves' counts per row are
// exchanged once (one barrier) and prefixed with a 16-lane DPP scan.  Slots of ranks
// [r0, r0 + n) land in s_slot / s_tok.  Returns base plus the tile's selected count; ends with a
// barrier (s_tmp, ROWS * NT/64 words, is free again).
template <int NT>
__device__ __forceinline__ uint32_t sel_rank_ge_tile(const uint4* kv, uint32_t tau, int32_t slot_t0, uint32_t base,
                                                     int r0, int n, uint32_t* s_tmp, int32_t* s_slot,
                                                     int32_t* s_tok) {
    constexpr int NW = NT / 64;
    constexpr int ROWS = sel_rows<NT>();
    static_assert(NW <= 16 && ROWS * NW <= sel_tmp_words<NT>(), "wave counts fit s_tmp");
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    uint64_t m0[ROWS], m1[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        m0[r] = ballot64(kv[r].x >= tau);
        m1[r] = ballot64(kv[r].z >= tau);
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < ROWS; ++r) s_tmp[r * NW + wave] = uint32_t(__popcll(m0[r]) + __popcll(m1[r]));
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        uint32_t x = lane < NW ? s_tmp[r * NW + lane] : 0u;
        x += dpp_u32<0x111>(x);
        x += dpp_u32<0x112>(x);
        x += dpp_u32<0x114>(x);
        x += dpp_u32<0x118>(x);
        const uint32_t before = wu > 0 ? readlane_u32(x, wu - 1) : 0u;
        const uint32_t rank0 = base + before + lanes_below(m0[r]) + lanes_below(m1[r]);
        const bool s0 = kv[r].x >= tau, s1 = kv[r].z >= tau;
        const int32_t slot0 = slot_t0 + r * 2 * NT + tid * 2;
        const uint32_t off0 = rank0 - uint32_t(r0);  // wraps for ranks below r0
        const uint32_t off1 = off0 + (s0 ? 1u : 0u);
        if (s0 && off0 < uint32_t(n)) {
            s_slot[off0] = slot0;
            s_tok[off0] = int32_t(kv[r].y);
        }
        if (s1 && off1 < uint32_t(n)) {
            s_slot[off1] = slot0 + 1;
            s_tok[off1] = int32_t(kv[r].w);
        }
        base += readlane_u32(x, NW - 1);
    }
    __syncthreads();  // s_tmp is free again, s_slot / s_tok complete
    return base;
}

// Single-tile selection (kp <= kSelTile, NT * 8 == kSelTile).  Thread t holds slots
// 2 NT r + 2 t + e (rows r < 4, e < 2) in registers for the whole selection, loaded as one
// coalesced 16-byte {key, id} pair per row.
//   1. level-1 histogram of the keys' top 12 bits (LDS atomics), a one-barrier workgroup scan in
//      descending bin order: the bin of the kappa-th largest key;
//   2. level-2 histogram of bits 19..12 over that bin's keys, straight from the registers, and
//      one wave's crossing over its 256 bins;
//   3. the keys sharing those top 20 bits (typically a few) go to a short LDS list, where each
//      finds its rank among them by direct counting: the exact threshold tau, how many keys equal
//      to tau are taken and how many there are;
//   4. one workgroup scan of the per-row counts (keys taken, and keys equal to tau when only some
//      are taken), packed two rows to a word, gives every selected slot its rank in slot order,
//      ties at tau to the lower slot.
// Returns false, after a barrier and with nothing written but LDS scratch, when more than
// kLeanShort keys share the threshold's top 20 bits (heavy ties); select_ranks then takes its
// general path.
template <int NT>
__device__ __forceinline__ bool select_ranks_lean(const uint2* __restrict__ gk, int64_t kp, uint32_t kappa, int r0,
                                                  int nmax, uint32_t* s_hist, uint32_t* s_tmp, uint32_t* s_res,
                                                  uint32_t* s_short, int32_t* s_slot, int32_t* s_tok,
                                                  SelResult* out) {
    constexpr int ROWS = sel_rows<NT>();
    static_assert(ROWS == 4 && NT * 4 == kHistBins, "4 rows of 2 slots and 4 level-1 bins per thread");
    static_assert(4 * (NT / 64) <= sel_tmp_words<NT>(), "the rank scan's words fit s_tmp");
    const int tid = threadIdx.x, wave = wave_id();
    PRISM_TL(kTlSelect, 0);
    uint4 kv[ROWS];
    sel_load_tile<NT>(gk, kp, 0, kv);
    for (int i = tid; i < kSelHistWords / 4; i += NT) reinterpret_cast<uint4*>(s_hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        if (kv[r].x) atomicAdd(&s_hist[kv[r].x >> kKeyShift], 1u);
        if (kv[r].z) atomicAdd(&s_hist[kv[r].z >> kKeyShift], 1u);
    }
    __syncthreads();
    PRISM_TL(kTlSelect, 1);

    // level-1 crossing: thread t holds bins 4095 - 4t - k (k < 4)
    uint32_t kap;
    {
        const uint4 x = *reinterpret_cast<const uint4*>(s_hist + (kHistBins - 4 * (tid + 1)));
        const uint32_t c[4] = {x.w, x.z, x.y, x.x};
        const uint32_t sum = (c[0] + c[1]) + (c[2] + c[3]);
        uint32_t total;
        uint32_t acc = block_excl_scan1<NT>(sum, s_tmp, &total);
        kap = kappa < total ? kappa : total;
        if (tid == 0) {
            s_res[kResValid] = total;
            s_res[kResC2] = 0u;
        }
        if (kap > 0u && kap < total && acc < kap && kap <= acc + sum) {  // exactly one thread
            bool f = false;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool hit = !f && acc + c[k] >= kap;
                if (hit) {
                    s_res[kResBin] = uint32_t(kHistBins - 1 - 4 * tid - k);
                    s_res[kResAbove] = acc;
                }
                f = f || hit;
                acc += f ? 0u : c[k];
            }
        }
    }
    __syncthreads();
    PRISM_TL(kTlSelect, 2);
    const uint32_t n_valid = s_res[kResValid];
    out->kappa_eff = kap;
    out->n = 0;
    if (kap == 0) return true;

    uint32_t tau = 1u, need = 0xFFFFFFFFu, eq_total = 0u;  // default: every valid key is taken
    if (kap < n_valid) {
        const uint32_t bin = s_res[kResBin];
        const uint32_t R = kap - s_res[kResAbove];  // rank of tau inside the bin: 1 <= R <= its count
        uint32_t* s_h2 = s_hist + kHist1Words;      // zeroed with the level-1 histogram
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            if (kv[r].x && (kv[r].x >> kKeyShift) == bin) atomicAdd(&s_h2[(kv[r].x >> 12) & 0xFFu], 1u);
            if (kv[r].z && (kv[r].z >> kKeyShift) == bin) atomicAdd(&s_h2[(kv[r].z >> 12) & 0xFFu], 1u);
        }
        __syncthreads();
        if (wave == 0) sel_sub_crossing(s_h2, R, s_res);
        __syncthreads();
        PRISM_TL(kTlSelect, 3);
        const uint32_t bin2 = s_res[kResBin2];
        const uint32_t c2 = s_h2[bin2];
        if (c2 > uint32_t(kLeanShort)) {  // the same for every thread
            __syncthreads();              // every thread has read the LDS above before it is reused
            return false;
        }
        const uint32_t pre = (bin << 8) | bin2;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            if (kv[r].x && (kv[r].x >> 12) == pre) s_short[atomicAdd(&s_res[kResC2], 1u)] = kv[r].x;
            if (kv[r].z && (kv[r].z >> 12) == pre) s_short[atomicAdd(&s_res[kResC2], 1u)] = kv[r].z;
        }
        __syncthreads();
        const uint32_t R2 = R - s_res[kResAbove2];
        if (uint32_t(tid) < c2) {
            const uint32_t k = s_short[tid];
            uint32_t gt = 0, ge = 0;
            for (uint32_t j = 0; j < c2; ++j) {
                const uint32_t x = s_short[j];
                gt += x > k ? 1u : 0u;
                ge += x >= k ? 1u : 0u;
            }
            if (gt < R2 && R2 <= ge) {  // every holder of tau writes the same three words
                s_res[kResTau] = k;
                s_res[kResNeed] = R2 - gt;
                s_res[kResEq] = ge - gt;
            }
        }
        __syncthreads();
        tau = s_res[kResTau];
        need = s_res[kResNeed];
        eq_total = s_res[kResEq];
    }
    PRISM_TL(kTlSelect, 4);

    const bool take_all_eq = need >= eq_total;
    const int n = int(kap) - r0 <= 0 ? 0 : (int(kap) - r0 > nmax ? nmax : int(kap) - r0);
    if (take_all_eq) {  // every key at or above tau is taken: ballot ranks
        sel_rank_ge_tile<NT>(kv, tau, 0, 0u, r0, n, s_tmp, s_slot, s_tok);
        PRISM_TL(kTlSelect, 5);
        out->n = n;
        return true;
    }
    // some keys equal to tau are left out: ranks in slot order (row-major over the tile) from the
    // per-thread and per-row counts of keys above tau and keys equal to tau, two rows per
    // 16-bit-packed word, one workgroup scan
    uint32_t v[4], pre[4], tot[4];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        uint32_t sel = 0, eq = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint4 k = kv[2 * p + h];
            const uint32_t gt = (k.x > tau ? 1u : 0u) + (k.z > tau ? 1u : 0u);
            const uint32_t e = (k.x == tau ? 1u : 0u) + (k.z == tau ? 1u : 0u);
            sel += gt << (16 * h);
            eq += e << (16 * h);
        }
        v[p] = sel;
        v[2 + p] = eq;
    }
    // s_tmp's words from the crossing scan were last read before the barriers above
    block_excl_scan1_n<4, NT>(v, pre, tot, s_tmp);
    uint32_t rows_sel = 0, rows_eq = 0;  // taken keys and ties of the rows before
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int p = r / 2, sh = 16 * (r % 2);
        const uint32_t sel_before = rows_sel + ((pre[p] >> sh) & 0xFFFFu);
        uint32_t eqi = rows_eq + ((pre[2 + p] >> sh) & 0xFFFFu);  // ties before this row's slots
        uint32_t rank = sel_before + (eqi < need ? eqi : need);
        const uint32_t k2[2] = {kv[r].x, kv[r].z};
        const int32_t t2[2] = {int32_t(kv[r].y), int32_t(kv[r].w)};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const bool eqk = k2[e] == tau;
            const bool take = k2[e] > tau || (eqk && eqi < need);
            eqi += eqk ? 1u : 0u;
            const uint32_t off = rank - uint32_t(r0);  // wraps for ranks below r0
            if (take && off < uint32_t(n)) {
                s_slot[off] = r * 2 * NT + tid * 2 + e;
                s_tok[off] = t2[e];
            }
            rank += take ? 1u : 0u;
        }
        rows_sel += (tot[p] >> sh) & 0xFFFFu;
        rows_eq += (tot[2 + p] >> sh) & 0xFFFFu;
    }
    __syncthreads();
    PRISM_TL(kTlSelect, 5);
    out->n = n;
    return true;
}

// gk: the unit's [kp] {key, id} slots (16-byte aligned); ids pass through to s_tok.
// LDS: s_hist kSelHistWords words, 16-byte aligned; s_tmp sel_tmp_words<NT>() words; s_res 16 words;
// s_cand kSelCandTotal words (16-byte aligned), s_ccount NT/64 words, s_slot / s_tok nmax each.
// A pool of at most kSelTile slots takes select_ranks_lean unless its threshold has heavy ties.
template <int NT>
__device__ __forceinline__ SelResult select_ranks(const uint2* __restrict__ gk, int64_t kp, uint32_t kappa, int r0, int nmax, uint32_t* s_hist,
                                                  uint32_t* s_tmp, uint32_t* s_res, uint32_t* s_cand,
                                                  uint32_t* s_ccount, int32_t* s_slot, int32_t* s_tok) {
    constexpr int NW = NT / 64;
    constexpr int ROWS = sel_rows<NT>();
    constexpr int CPW = sel_cand_per_wave<NT>();
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const int ntiles = int((kp + kSelTile - 1) / kSelTile);
    if constexpr (NT * 8 == kSelTile && PRISM_SELECT_LEAN) {
        if (kp <= kSelTile) {
            SelResult r;
            if (select_ranks_lean<NT>(gk, kp, kappa, r0, nmax, s_hist, s_tmp, s_res, s_cand, s_slot, s_tok, &r))
                return r;
        }
    }
    uint4 kv[ROWS];

    // ---- level-1 histogram (the LDS is cleared while the first keys are in flight) ----
    PRISM_TL(kTlSelect, 0);
    sel_load_tile<NT>(gk, kp, 0, kv);
    for (int i = tid; i < kSelHistWords / 4; i += NT) reinterpret_cast<uint4*>(s_hist)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        if (t > 0) sel_load_tile<NT>(gk, kp, int64_t(t) * kSelTile, kv);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            if (kv[r].x) atomicAdd(&s_hist[kv[r].x >> kKeyShift], 1u);
            if (kv[r].z) atomicAdd(&s_hist[kv[r].z >> kKeyShift], 1u);
        }
    }
    __syncthreads();
    PRISM_TL(kTlSelect, 1);
    // ---- crossing: thread t holds bins 4095 - 4t - k (k < 4), one 16-byte LDS read ----
    {
        static_assert(NT * 4 == kHistBins, "four bins per thread");
        const uint4 x = *reinterpret_cast<const uint4*>(s_hist + (kHistBins - 4 * (tid + 1)));
        const uint32_t c[4] = {x.w, x.z, x.y, x.x};
        const uint32_t sum = (c[0] + c[1]) + (c[2] + c[3]);
        uint32_t total;
        uint32_t acc = block_excl_scan<NT>(sum, s_tmp, &total);
        const uint32_t kap = kappa < total ? kappa : total;
        if (tid == 0) {
            s_res[kResValid] = total;
            s_res[kResKappa] = kap;
            s_res[kResOvf] = 0u;
            s_res[kResC2] = 0u;
        }
        if (kap > 0u && kap < total && acc < kap && kap <= acc + sum) {  // exactly one thread
            bool f = false;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool hit = !f && acc + c[k] >= kap;
                if (hit) {
                    s_res[kResBin] = uint32_t(kHistBins - 1 - 4 * tid - k);
                    s_res[kResAbove] = acc;
                    s_res[kResCount] = c[k];
                }
                f = f || hit;
                acc += f ? 0u : c[k];
            }
        }
    }
    if (ntiles > 1) sel_load_tile<NT>(gk, kp, 0, kv);
    __syncthreads();
    PRISM_TL(kTlSelect, 2);
    const uint32_t n_valid = s_res[kResValid];
    const uint32_t kappa_eff = s_res[kResKappa];
    SelResult res{kappa_eff, 0};
    if (kappa_eff == 0) return res;

    // ---- threshold tau, the number of keys equal to tau to take, and how many there are ----
    uint32_t tau = 1u, need = 0xFFFFFFFFu, eq_total = 0u;  // default: every valid key is taken
    if (kappa_eff < n_valid) {
        const uint32_t bin = s_res[kResBin], above = s_res[kResAbove];
        uint32_t cnt = 0;
        for (int t = 0; t < ntiles; ++t) {
            if (t > 0) sel_load_tile<NT>(gk, kp, int64_t(t) * kSelTile, kv);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const uint32_t k2[2] = {kv[r].x, kv[r].z};
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const bool f = (k2[e] >> kKeyShift) == bin && k2[e] != 0u;
                    const uint64_t m = ballot64(f);
                    const uint32_t pos = cnt + lanes_below(m);
                    if (f && pos < uint32_t(CPW)) s_cand[wave * CPW + pos] = k2[e];
                    cnt += uint32_t(__popcll(m));
                }
            }
        }
        if (lane == 0) s_ccount[wave] = cnt;
        if (lane == 0 && cnt > uint32_t(CPW)) s_res[kResOvf] = 1u;
        __syncthreads();
        PRISM_TL(kTlSelect, 3);
        const bool overflow = s_res[kResOvf] != 0u;
        const uint32_t R = kappa_eff - above;  // rank of tau inside the bin, 1 <= R <= count of the bin
        if (!overflow) {
            // level 2: bits 19..12 of the wave's own list
            uint32_t* s_h2 = s_hist + kHist1Words;
            const uint32_t k0 = uint32_t(lane) < cnt ? s_cand[wave * CPW + lane] : 0u;
            const uint32_t k1 = uint32_t(lane) + 64 < cnt ? s_cand[wave * CPW + 64 + lane] : 0u;
            if (k0) atomicAdd(&s_h2[(k0 >> 12) & 0xFFu], 1u);
            if (k1) atomicAdd(&s_h2[(k1 >> 12) & 0xFFu], 1u);
            __syncthreads();
            if (wave == 0) sel_sub_crossing(s_h2, R, s_res);
            __syncthreads();
            // the sub-bin's keys into one short list (any order), in the dead level-1 buffer
            const uint32_t pre = (bin << 8) | s_res[kResBin2];
            const uint32_t R2 = R - s_res[kResAbove2];
            const bool f0 = k0 != 0u && (k0 >> 12) == pre;
            const bool f1 = k1 != 0u && (k1 >> 12) == pre;
            const uint64_t m0 = ballot64(f0), m1 = ballot64(f1);
            const uint32_t nf = uint32_t(__popcll(m0) + __popcll(m1));
            if (nf) {
                uint32_t base = 0;
                if (lane == 0) base = atomicAdd(&s_res[kResC2], nf);
                base = readlane_u32(base, 0);
                if (f0) s_hist[base + lanes_below(m0)] = k0;
                if (f1) s_hist[base + uint32_t(__popcll(m0)) + lanes_below(m1)] = k1;
            }
            __syncthreads();
            const uint32_t c2 = s_res[kResC2];
            for (uint32_t i = tid; i < c2; i += NT) {
                const uint32_t k = s_hist[i];
                uint32_t gt = 0, ge = 0;
                for (uint32_t j = 0; j < c2; ++j) {
                    const uint32_t x = s_hist[j];
                    gt += x > k ? 1u : 0u;
                    ge += x >= k ? 1u : 0u;
                }
                if (gt < R2 && R2 <= ge) {
                    s_res[kResTau] = k;
                    s_res[kResNeed] = R2 - gt;
                    s_res[kResEq] = ge - gt;
                }
            }
            __syncthreads();
        } else {
            // radix digits 2 (bits 19..8) and 3 (bits 7..0) of the keys in the bin
            uint32_t* s_r2 = s_res + kResScratch;
            for (int i = tid; i < kHistPadded; i += NT) s_hist[i] = 0u;
            __syncthreads();
            sel_digit_hist<NT>(gk, kp, ntiles, kv, s_cand, s_ccount, !overflow, bin, kKeyShift, 8, 0xFFFu, true,
                               s_hist);
            __syncthreads();
            find_crossing<kHistBins, NT>(s_hist, R, s_tmp, s_r2);
            const uint32_t pre = (bin << 12) | s_r2[0];
            const uint32_t above_a = s_r2[1];
            __syncthreads();
            if (tid < 256) s_hist[tid] = 0u;
            __syncthreads();
            sel_digit_hist<NT>(gk, kp, ntiles, kv, s_cand, s_ccount, !overflow, pre, 8, 0, 0xFFu, false, s_hist);
            __syncthreads();
            find_crossing<256, NT>(s_hist, R - above_a, s_tmp, s_r2);
            if (tid == 0) {
                s_res[kResTau] = (pre << 8) | s_r2[0];
                s_res[kResNeed] = R - above_a - s_r2[1];
                s_res[kResEq] = s_r2[2];
            }
            __syncthreads();
        }
        PRISM_TL(kTlSelect, 4);
        tau = s_res[kResTau];
        need = s_res[kResNeed];
        eq_total = s_res[kResEq];
        if (ntiles > 1) sel_load_tile<NT>(gk, kp, 0, kv);  // the rank pass starts from the first tile
    }

    const int n = int(kappa_eff) - r0 <= 0 ? 0 : (int(kappa_eff) - r0 > nmax ? nmax : int(kappa_eff) - r0);
    res.n = n;
    if (n == 0) return res;

    // ---- ranks in slot order; ranks [r0, r0 + n) land in s_slot / s_tok ----
    const bool take_all_eq = need >= eq_total;  // every key equal to tau is taken: select key >= tau
    if (take_all_eq) {
        uint32_t base = 0;
        for (int t = 0; t < ntiles && base < uint32_t(r0 + n); ++t) {
            if (t > 0) sel_load_tile<NT>(gk, kp, int64_t(t) * kSelTile, kv);
            base = sel_rank_ge_tile<NT>(kv, tau, int32_t(int64_t(t) * kSelTile), base, r0, n, s_tmp, s_slot, s_tok);
        }
        PRISM_TL(kTlSelect, 5);
        return res;
    }
    // per-row counts of one thread are at most 2, two rows share a 32-bit word (16 bits each)
    constexpr int NP = ROWS / 2 > 0 ? ROWS / 2 : 1;
    uint32_t eq_base = 0, rank_base = 0;
    for (int t = 0; t < ntiles && rank_base < uint32_t(r0 + n); ++t) {
        if (t > 0) sel_load_tile<NT>(gk, kp, int64_t(t) * kSelTile, kv);
        uint32_t eqc[NP], eqp[NP], eqt[NP], selc[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            eqc[p] = 0;
            selc[p] = 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                if (2 * p + half >= ROWS) continue;
                const uint4 v = kv[2 * p + half];
                const uint32_t ge = (v.x >= tau ? 1u : 0u) + (v.z >= tau ? 1u : 0u);
                const uint32_t eq = (v.x == tau ? 1u : 0u) + (v.z == tau ? 1u : 0u);
                eqc[p] += eq << (16 * half);
                selc[p] += (take_all_eq ? ge : ge - eq) << (16 * half);  // keys above tau, or >= tau
            }
        }
        if (!take_all_eq) {
            block_excl_scan_n<NP, NT>(eqc, eqp, eqt, s_tmp);
            uint32_t run = eq_base;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const uint32_t ec = (eqc[p] >> (16 * half)) & 0xFFFFu;
                    const uint32_t eqb = run + ((eqp[p] >> (16 * half)) & 0xFFFFu);
                    const uint32_t take = eqb >= need ? 0u : (ec < need - eqb ? ec : need - eqb);
                    selc[p] += take << (16 * half);
                    run += (eqt[p] >> (16 * half)) & 0xFFFFu;
                }
            }
        }
        uint32_t selp[NP], selt[NP];
        block_excl_scan_n<NP, NT>(selc, selp, selt, s_tmp);
        uint32_t rrun = rank_base;
        uint32_t run = eq_base;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int p = r / 2, sh = 16 * (r % 2);
            uint32_t rank = rrun + ((selp[p] >> sh) & 0xFFFFu);
            uint32_t eqr = run + (take_all_eq ? 0u : ((eqp[p] >> sh) & 0xFFFFu));
            const uint4 v = kv[r];
            const uint32_t k2[2] = {v.x, v.z};
            const int32_t t2[2] = {int32_t(v.y), int32_t(v.w)};
            const int32_t slot0 = int32_t(int64_t(t) * kSelTile + int64_t(r) * 2 * NT + tid * 2);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const bool eq = k2[e] == tau;
                const bool take = k2[e] > tau || (eq && (take_all_eq || eqr < need));
                eqr += eq ? 1u : 0u;
                const uint32_t off = rank - uint32_t(r0);  // wraps for ranks below r0
                if (take && off < uint32_t(n)) {
                    s_slot[off] = slot0 + e;
                    s_tok[off] = t2[e];
                }
                rank += take ? 1u : 0u;
            }
            rrun += (selt[p] >> sh) & 0xFFFFu;
            if (!take_all_eq) run += (eqt[p] >> sh) & 0xFFFFu;
        }
        eq_base = run;
        rank_base = rrun;
    }
    __syncthreads();
    return res;
}

}  // namespace prism
