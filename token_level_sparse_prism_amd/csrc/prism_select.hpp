// prism_select.hpp -- exact top-kappa selection of one unit's pool slots inside one workgroup
// (the refined layer's re-selection within the inherited pool, Prism Attention page Sec. 4.1).
//
// Keys are 32-bit order keys of the group scores, one per pool slot (0 = empty slot).  They are
// read from global memory in rows of 1024 (four consecutive slots per thread, one 16-byte load),
// up to eight rows per tile held in registers.  The threshold comes from three radix digits
// (12/12/8 bits): the first histogram covers every key; the keys of the threshold bin are then
// compacted into a short LDS list (wave ballots) and the two lower digits are histogrammed over
// that list.  Selected slots are ranked in slot order (ties at the threshold go to the lower
// slot) with two multi-row workgroup scans.  The per-key work is branch-free.
#pragma once

#include "prism_device.hpp"

namespace prism {

// A tile is 8192 keys: NT threads x sel_rows<NT>() rows of four keys.
constexpr int64_t kSelTile = 8192;
template <int NT> constexpr int sel_rows() { return int(kSelTile / (4 * NT)); }
// LDS list of the threshold bin's keys: 2048 entries split over the waves
template <int NT> constexpr int sel_cand_per_wave() { return 2048 / (NT / 64); }
constexpr int kSelCandTotal = 2048;

struct SelResult {
    uint32_t kappa_eff;  // min(kappa, number of valid slots)
    int n;               // ranks [r0, r0 + n) written to s_slot
};

template <int NT>
__device__ __forceinline__ void sel_load_tile(const uint32_t* __restrict__ gkeys, int64_t kp, int64_t t0,
                                              uint4* kv) {
#pragma unroll
    for (int r = 0; r < sel_rows<NT>(); ++r) {
        const int64_t j = t0 + int64_t(r) * 4 * NT + int64_t(threadIdx.x) * 4;
        if (j + 4 <= kp) {
            kv[r] = *reinterpret_cast<const uint4*>(gkeys + j);
        } else {
            kv[r].x = j < kp ? gkeys[j] : 0u;
            kv[r].y = j + 1 < kp ? gkeys[j + 1] : 0u;
            kv[r].z = j + 2 < kp ? gkeys[j + 2] : 0u;
            kv[r].w = j + 3 < kp ? gkeys[j + 3] : 0u;
        }
    }
}

__device__ __forceinline__ void unpack4(const uint4& v, uint32_t* k) {
    k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
}

// Histogram of the digit (k >> shift) & mask over the keys whose bits from pre_shift up equal
// `pre`.  Reads the compacted per-wave lists when none overflowed, else every key again.
template <int NT>
__device__ __forceinline__ void sel_digit_hist(const uint32_t* __restrict__ gkeys, int64_t kp, int ntiles, uint4* kv,
                                               const uint32_t* s_cand, const uint32_t* s_ccount, bool from_list,
                                               uint32_t pre, int pre_shift, int shift, uint32_t mask,
                                               bool padded, uint32_t* s_hist) {
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
            if (ntiles > 1) sel_load_tile<NT>(gkeys, kp, int64_t(t) * kSelTile, kv);
#pragma unroll
            for (int r = 0; r < sel_rows<NT>(); ++r) {
                uint32_t k[4];
                unpack4(kv[r], k);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if ((k[e] >> pre_shift) == pre && k[e]) {
                        const int bin = int((k[e] >> shift) & mask);
                        atomicAdd(&s_hist[padded ? hpad(bin) : bin], 1u);
                    }
                }
            }
        }
    }
}

// s_hist: kHistPadded words; s_tmp: (NT/64) * max(1, sel_rows/2) words; s_cand: kSelCandTotal
// words; s_ccount: NT/64 words; s_slot: nmax slots.
template <int NT>
__device__ __forceinline__ SelResult select_slice(const uint32_t* __restrict__ gkeys, int64_t kp, uint32_t kappa,
                                                  int r0, int nmax, uint32_t* s_hist, uint32_t* s_tmp,
                                                  uint32_t* s_res, uint32_t* s_cand, uint32_t* s_ccount,
                                                  int32_t* s_slot) {
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    constexpr int ROWS = sel_rows<NT>();
    constexpr int CPW = sel_cand_per_wave<NT>();
    const int ntiles = int((kp + kSelTile - 1) / kSelTile);
    uint4 kv[ROWS];

    // ---- digit 1: top 12 bits of every key (empty and padding slots land in bin 0) ----
    for (int i = tid; i < kHistPadded; i += NT) s_hist[i] = 0u;
    __syncthreads();
    uint32_t nv = 0;
    for (int t = 0; t < ntiles; ++t) {
        sel_load_tile<NT>(gkeys, kp, int64_t(t) * kSelTile, kv);
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            uint32_t k[4];
            unpack4(kv[r], k);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                nv += k[e] != 0u ? 1u : 0u;
                atomicAdd(&s_hist[hpad(int(k[e] >> kKeyShift))], 1u);
            }
        }
    }
    const uint32_t n_valid = block_sum_u32<NT>(nv, s_tmp);
    const uint32_t kappa_eff = n_valid < kappa ? n_valid : kappa;
    SelResult res{kappa_eff, 0};
    if (kappa_eff == 0) return res;
    if (tid == 0) s_hist[hpad(0)] = 0u;  // bin 0 holds no valid key
    __syncthreads();

    // ---- threshold tau and the number of keys equal to it to take ----
    uint32_t tau = 1u, need = 0xFFFFFFFFu;  // every valid key is taken
    if (kappa_eff < n_valid) {
        find_crossing<kHistBins, NT>(s_hist, kappa_eff, s_tmp, s_res);
        const uint32_t bin = s_res[0], above = s_res[1];
        // compact the threshold bin's keys, per wave, into LDS
        uint32_t cnt = 0;
        for (int t = 0; t < ntiles; ++t) {
            if (ntiles > 1) sel_load_tile<NT>(gkeys, kp, int64_t(t) * kSelTile, kv);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                uint32_t k[4];
                unpack4(kv[r], k);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool f = (k[e] >> kKeyShift) == bin && k[e] != 0u;
                    const uint64_t m = ballot64(f);
                    const uint32_t pos = cnt + lanes_below(m);
                    if (f && pos < uint32_t(CPW)) s_cand[wave * CPW + pos] = k[e];
                    cnt += uint32_t(__popcll(m));
                }
            }
        }
        if (lane == 0) s_ccount[wave] = cnt;
        for (int i = tid; i < kHistPadded; i += NT) s_hist[i] = 0u;
        __syncthreads();
        bool from_list = true;
        for (int w = 0; w < NT / 64; ++w) from_list = from_list && s_ccount[w] <= uint32_t(CPW);
        sel_digit_hist<NT>(gkeys, kp, ntiles, kv, s_cand, s_ccount, from_list, bin, kKeyShift, 8, 0xFFFu, true, s_hist);
        __syncthreads();
        find_crossing<kHistBins, NT>(s_hist, kappa_eff - above, s_tmp, s_res);
        const uint32_t pre = (bin << 12) | s_res[0];
        const uint32_t above_a = s_res[1];
        if (tid < 256) s_hist[tid] = 0u;
        __syncthreads();
        sel_digit_hist<NT>(gkeys, kp, ntiles, kv, s_cand, s_ccount, from_list, pre, 8, 0, 0xFFu, false, s_hist);
        __syncthreads();
        find_crossing<256, NT>(s_hist, kappa_eff - above - above_a, s_tmp, s_res);
        tau = (pre << 8) | s_res[0];
        need = kappa_eff - above - above_a - s_res[1];
    }
    if (ntiles > 1) sel_load_tile<NT>(gkeys, kp, 0, kv);  // the rank pass starts from the first tile

    const int n = int(kappa_eff) - r0 <= 0 ? 0 : (int(kappa_eff) - r0 > nmax ? nmax : int(kappa_eff) - r0);
    res.n = n;
    if (n == 0) return res;

    // ---- ranks in slot order; ranks [r0, r0 + n) land in s_slot ----
    uint32_t eq_base = 0, rank_base = 0;
    for (int t = 0; t < ntiles && rank_base < uint32_t(r0 + n); ++t) {
        if (ntiles > 1 && t > 0) sel_load_tile<NT>(gkeys, kp, int64_t(t) * kSelTile, kv);
        // per-row counts, two rows per 32-bit word (a row holds at most 1024 keys)
        constexpr int NP = ROWS / 2 > 0 ? ROWS / 2 : 1;
        uint32_t eqc[NP], gtc[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            eqc[p] = gtc[p] = 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                uint32_t k[4];
                if (2 * p + half >= ROWS) continue;
                unpack4(kv[2 * p + half], k);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    eqc[p] += ((k[e] == tau && k[e] != 0u) ? 1u : 0u) << (16 * half);
                    gtc[p] += (k[e] > tau ? 1u : 0u) << (16 * half);
                }
            }
        }
        uint32_t eqp[NP], eqt[NP];
        block_excl_scan_n<NP, NT>(eqc, eqp, eqt, s_tmp);
        uint32_t selc[NP];
        uint32_t run = eq_base;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            selc[p] = 0;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const uint32_t ec = (eqc[p] >> (16 * half)) & 0xFFFFu;
                const uint32_t eqb = run + ((eqp[p] >> (16 * half)) & 0xFFFFu);
                const uint32_t take = eqb >= need ? 0u : (ec < need - eqb ? ec : need - eqb);
                selc[p] += (((gtc[p] >> (16 * half)) & 0xFFFFu) + take) << (16 * half);
                run += (eqt[p] >> (16 * half)) & 0xFFFFu;
            }
        }
        uint32_t selp[NP], selt[NP];
        block_excl_scan_n<NP, NT>(selc, selp, selt, s_tmp);
        uint32_t rrun = rank_base;
        run = eq_base;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const int p = r / 2, sh = 16 * (r % 2);
            uint32_t rank = rrun + ((selp[p] >> sh) & 0xFFFFu);
            uint32_t eqr = run + ((eqp[p] >> sh) & 0xFFFFu);
            uint32_t k[4];
            unpack4(kv[r], k);
            const int32_t slot0 = int32_t(int64_t(t) * kSelTile + int64_t(r) * 4 * NT + tid * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool eq = k[e] == tau && k[e] != 0u;
                const bool take = k[e] > tau || (eq && eqr < need);
                eqr += eq ? 1u : 0u;
                const uint32_t off = rank - uint32_t(r0);  // wraps for ranks below r0
                if (take && off < uint32_t(n)) s_slot[off] = slot0 + e;
                rank += take ? 1u : 0u;
            }
            rrun += (selt[p] >> sh) & 0xFFFFu;
            run += (eqt[p] >> sh) & 0xFFFFu;
        }
        eq_base = run;
        rank_base = rrun;
    }
    __syncthreads();
    return res;
}

}  // namespace prism
