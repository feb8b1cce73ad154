// scan_kernel.hpp -- the proposal layer's full-context scan on gfx950 (Prism Attention page,
// Sec. 4.2: the anchor layer scores every token with the compressed key cache).  The scan streams
// the int8 or 2-bit keys once, writes a 32-bit order key per token and adds each workgroup's
// histogram of the keys' top 12 bits into the unit's histogram.  Two kernels share that work:
// k_scan_w (one 1024-thread workgroup per CU, waves claiming batches) where the grid fills the
// chip, k_scan (256-thread workgroups, fixed chunks) elsewhere.  k_scan8.hip and k_scan2.hip
// instantiate them, one key format per translation unit.
#pragma once

#include "prism_device.hpp"
#include "prism_prof.hpp"

#ifndef PRISM_SCAN_NIBBLE
#define PRISM_SCAN_NIBBLE 1  // 2-bit keys, SUM: the wide scan's dot products on 4-bit digits (v_dot8_i32_i4)
#endif
#ifndef PRISM_SCAN_Q_FIRST
#define PRISM_SCAN_Q_FIRST 0  // 1: SUM wide scan requests its first rows only after the query has arrived
#endif

namespace prism {

template <int CH>
__device__ __forceinline__ int scan_chunk_tokens(int64_t Tb, int64_t c0) {
    return int(Tb - c0 < 0 ? 0 : (Tb - c0 > CH ? CH : Tb - c0));
}

// ---------------------------------------------------------------------------------------------
// k_scan.  NQ int8 query vectors are dotted with each key row:
//   agg SUM, G == 1: NQ = 1, the head's codes;
//   agg SUM, G  > 1: NQ = 2, the group's code sums split as qsum = 16*hi + lo with lo in
//                    [-8, 7] and |hi| <= 127, so A = 16*(hi.K) + lo.K exactly in int32;
//   agg MAX:         NQ = GP (G rounded up to a power of two), one vector per head.
// A lane covers DPL dims of a key row (D/DPL lanes per token) and loads them as one piece per
// row: 16 bytes of int8 codes (DPL = 16, a wave reads 1 KiB of consecutive rows per load), or
// for 2-bit codes 16 bytes (DPL = 64, when at most two query vectors hold registers) or one
// 32-bit word (DPL = 16, agg MAX).  A 2-bit code b stands for the level c = 2b - 3, so a lane's
// share of q.c is 2 (q.b) - 3 (sum of its q codes), exact in int32; q.b over one 32-bit word is
// four byte-wise dot products of its bit pairs.  Workgroup x of unit y handles chunks
// x, x + gridDim.x, ...
template <int KB, int DPL> struct ScanRow;
#ifndef PRISM_SCAN_LOADS8
#define PRISM_SCAN_LOADS8 8
#endif
#ifndef PRISM_SCAN_LOADS2
#define PRISM_SCAN_LOADS2 4
#endif
template <> struct ScanRow<8, 16> {
    using R = uint4;
    static constexpr int kLoads = PRISM_SCAN_LOADS8;  // loads in flight per lane
    static __device__ __forceinline__ R load(const int8_t* p) { return load16_stream(p); }
    static __device__ __forceinline__ R zero() { return make_uint4(0u, 0u, 0u, 0u); }
};
template <> struct ScanRow<2, 64> {
    using R = uint4;
    static constexpr int kLoads = PRISM_SCAN_LOADS2;  // the q words take the registers of the other four
    static __device__ __forceinline__ R load(const int8_t* p) { return load16_stream(p); }
    static __device__ __forceinline__ R zero() { return make_uint4(0u, 0u, 0u, 0u); }
};
template <> struct ScanRow<2, 16> {
    using R = uint32_t;
    static constexpr int kLoads = 32;
    static __device__ __forceinline__ R load(const int8_t* p) {
        return uint32_t(__builtin_nontemporal_load(reinterpret_cast<const int*>(p)));
    }
    static __device__ __forceinline__ R zero() { return 0u; }
};

// The lane's contribution to q_n . key for one row: qw = the lane's q words of vector n (four
// per 16 dims), c3 = -3 * (sum of the lane's q codes) for 2-bit keys.
__device__ __forceinline__ int dot_2bit_word(const int* qw, uint32_t w, int acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_sdot4(qw[j], int((w >> (2 * j)) & 0x03030303u), acc, false);
    return acc;
}
template <int KB>
__device__ __forceinline__ int lane_dot(const int* qw, uint4 k, int c3) {
    if constexpr (KB == 8) {
        int acc = 0;
        acc = __builtin_amdgcn_sdot4(qw[0], int(k.x), acc, false);
        acc = __builtin_amdgcn_sdot4(qw[1], int(k.y), acc, false);
        acc = __builtin_amdgcn_sdot4(qw[2], int(k.z), acc, false);
        acc = __builtin_amdgcn_sdot4(qw[3], int(k.w), acc, false);
        return acc;
    } else {
        int acc = dot_2bit_word(qw, k.x, 0);
        acc = dot_2bit_word(qw + 4, k.y, acc);
        acc = dot_2bit_word(qw + 8, k.z, acc);
        acc = dot_2bit_word(qw + 12, k.w, acc);
        return 2 * acc + c3;
    }
}
template <int KB>
__device__ __forceinline__ int lane_dot(const int* qw, uint32_t w, int c3) {
    return 2 * dot_2bit_word(qw, w, 0) + c3;
}

// 2-bit keys against three signed base-16 digit vectors of the summed query codes (8 nibble words
// each): a 32-bit key word gives two nibble words under the masks 0x33333333 and
// (w >> 2) & 0x33333333 (codes 0..3, non-negative as signed 4-bit values), and each meets one
// v_dot8_i32_i4 per digit.  sum_d qs_d b_d = 256 S2 + 16 S1 + S0 exactly in int32.
__device__ __forceinline__ int lane_dot_nib(const int (*qn)[8], uint4 k, int c3) {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
    int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int lo = int(w[m] & 0x33333333u), hi = int((w[m] >> 2) & 0x33333333u);
        s0 = __builtin_amdgcn_sdot8(qn[0][2 * m], lo, s0, false);
        s1 = __builtin_amdgcn_sdot8(qn[1][2 * m], lo, s1, false);
        s2 = __builtin_amdgcn_sdot8(qn[2][2 * m], lo, s2, false);
        s0 = __builtin_amdgcn_sdot8(qn[0][2 * m + 1], hi, s0, false);
        s1 = __builtin_amdgcn_sdot8(qn[1][2 * m + 1], hi, s1, false);
        s2 = __builtin_amdgcn_sdot8(qn[2][2 * m + 1], hi, s2, false);
    }
    return 2 * (256 * s2 + 16 * s1 + s0) + c3;
}

// The query quantizer: clamp(rint(x * inv), -127, 127) with inv = 127 / absmax (one fp32 product,
// round half to even), as for the keys.
__device__ __forceinline__ int scan_qcode(float x, float inv) {
    const float r = __builtin_rintf(x * inv);
    return int(fminf(fmaxf(r, -127.0f), 127.0f));
}

// kPg: 0 contiguous caches; 1 paged, a page id per row; 2 paged with pages of at least TPR tokens,
// so the TPR tokens of a round share one page and its base is a scalar.
// CH: tokens per workgroup work item (1024, or 256 for small grids; see launch_scan_kb).
template <int D, int NQ, bool kMax, int KB, int kPg, int CH>
__global__ __launch_bounds__(kThreads) void k_scan(ProposeArgs a) {
    constexpr bool paged = kPg != 0;       // rows through the page table (d.pg.table != nullptr)
    constexpr int DPL = (KB == 2 && NQ <= 2) ? 64 : 16;  // dims per lane
    using SR = ScanRow<KB, DPL>;
    constexpr int QW = DPL / 4;            // q words per vector and lane
    constexpr int LPT = D / DPL;           // lanes per token
    constexpr int TPW = 64 / LPT;          // tokens per wave per load
    constexpr int TPR = TPW * (kThreads / 64);
    constexpr int ROUNDS = CH / TPR;
    // loads in flight per lane: fewer 2-bit row words when many query vectors hold registers
    constexpr int UW = KB == 8 ? SR::kLoads : (NQ <= 2 ? SR::kLoads : (NQ <= 8 ? SR::kLoads / 2 : SR::kLoads / 4));
    constexpr int U = UW < ROUNDS ? UW : ROUNDS;
    constexpr int RB = D * KB / 8;         // bytes per key row
    static_assert(ROUNDS % U == 0, "chunk must hold whole unrolled rounds");

    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_key[CH];  // the chunk's aggregated int32 dot products
    __shared__ __attribute__((aligned(16))) int8_t s_q[NQ][D];
    __shared__ float s_red[kThreads / 64];
    __shared__ int32_t s_pg[paged ? CH : 1];  // paged: the physical pages of the chunk's tokens

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);
    const int nch = int((d.T_max + CH - 1) / CH);  // work items of CH tokens per unit
    const int sub = lane % LPT;
    const int tok_lane = wave * TPW + lane / LPT;

    // Every global load below is unconditional, at a clamped in-bounds address, and loads past
    // the chunk's tokens are simply not used: a load under a branch makes the compiler merge its
    // wait counts with the path that skips it, and the merged counts wait for loads that are still
    // streaming.  For the same reason the per-call zeroing goes before the first load.
    if (ui.x == 0) {  // per-call state of the later kernels
        uint32_t* h2 = a.hist2 + int64_t(unit) * kHistBins;
        for (int i = tid; i < kHistBins; i += kThreads) h2[i] = 0u;
        if (tid < kCandLists) a.cand_cnt[(int64_t(unit) * kCandLists + tid) * kCtrStride] = 0u;
    }

    // ---- query quantization: one absmax over the group's G*D values (s_hist holds q meanwhile).
    // Loads complete in issue order, so the small query and scale loads go out before the first
    // chunk's key rows, which then stream in while the codes are computed.  The scales stay in
    // registers until the chunk's keys are formed after the streaming loop, so the prologue
    // waits for the query alone.
    float* s_qf = reinterpret_cast<float*>(s_hist);
    const int64_t qoff = (int64_t(b) * d.Hq + int64_t(g) * G) * D;
    const int qe = a.q_bf16 ? 8 : 4;  // values per 16-byte piece
    constexpr int QP = (kMaxG * 256 / 4 + kThreads - 1) / kThreads;  // 16-byte query pieces per thread, max
    uint4 qraw[QP];
    const int npieces = G * D / qe;
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int p = min(tid + i * kThreads, npieces - 1);
        qraw[i] = load16(static_cast<const uint8_t*>(a.q) + (qoff * (a.q_bf16 ? 2 : 4)) + p * 16);
    }
    int chunk = ui.x;  // < nch: the grid has at most nch workgroups per unit
    int64_t c0 = int64_t(chunk) * CH;
    int nvalid = scan_chunk_tokens<CH>(Tb, c0);
    int last = nvalid > 0 ? nvalid - 1 : 0;  // clamp for loads (token c0 + 0 exists: c0 < T_max)
    // paged: the chunk's page ids go to LDS once (clamped into the pool; page 0 for an empty
    // chunk), and a row of the chunk is found there; lp = log2 of the page size
    const int lp = d.pg.log2p;
    const int64_t npool = d.pg.slots >> lp;
    auto fill_pages = [&]() {
        const int64_t p0 = c0 >> lp;
        const int npg = int(((c0 + last) >> lp) - p0 + 1);
        for (int i = tid; i < npg; i += kThreads) {
            int64_t pg = nvalid > 0 ? d.pg.table[int64_t(b) * d.pg.max_pages + p0 + i] : 0;
            s_pg[i] = int32_t(pg < 0 ? 0 : (pg >= npool ? npool - 1 : pg));
        }
    };
    // the row of token t of the current chunk inside KV head g's pool (< 2^23, so 32-bit offsets)
    auto paged_slot = [&](int64_t t) -> uint32_t {
        return (uint32_t(s_pg[(t >> lp) - (c0 >> lp)]) << lp) + uint32_t(t & ((int64_t(1) << lp) - 1));
    };
    const int8_t* kq_head = a.Kq + int64_t(g) * d.pg.slots * RB;
    const uint32_t lane_off = uint32_t(tok_lane * RB + sub * (RB / LPT));  // kPg == 2: a lane's offset in a round
    const float* sc_head = a.scales + int64_t(g) * d.pg.slots;
    if constexpr (paged) {
        fill_pages();
        __syncthreads();
    }
    // scl[i]: the scale of token c0 + tid + i * kThreads of the current chunk
    float scl[CH / kThreads];
    auto load_scales = [&]() {
        const float* sc = a.scales + int64_t(unit) * d.T_max + c0;
#pragma unroll
        for (int i = 0; i < CH / kThreads; ++i) {
            const int t = min(tid + i * kThreads, last);
            if constexpr (paged) scl[i] = sc_head[paged_slot(c0 + t)];
            else scl[i] = sc[t];
        }
    };
    // round r of the chunk: tokens c0 + r * TPR + [0, TPR), clamped to the last token (kPg == 2:
    // to the last token's round, which lies in one page)
    auto load_row = [&](int r) -> typename SR::R {
        if constexpr (kPg == 2) {
            const int i0 = min(r * TPR, last & ~(TPR - 1));
            const int64_t t0 = c0 + i0;
            const int64_t pg = __builtin_amdgcn_readfirstlane(s_pg[(t0 >> lp) - (c0 >> lp)]);
            return SR::load(kq_head + ((pg << lp) + (t0 & ((int64_t(1) << lp) - 1))) * RB + lane_off);
        } else if constexpr (paged) {
            const int tok = min(r * TPR + tok_lane, last);
            return SR::load(kq_head + paged_slot(c0 + tok) * uint32_t(RB) + uint32_t(sub * (RB / LPT)));
        } else {
            const int tok = min(r * TPR + tok_lane, last);
            return SR::load(a.Kq + (int64_t(unit) * d.T_max + c0 + tok) * RB + sub * (RB / LPT));
        }
    };
    load_scales();
    // rolling buffer of U rows per lane: a register is refilled with the row U rounds ahead as
    // soon as it has been used, so about U loads stay in flight through the whole chunk
    typename SR::R kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kv[u] = load_row(u);

    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int p = tid + i * kThreads;
        float x[8];
        if (a.q_bf16) unpack16<uint16_t>(qraw[i], x);
        else unpack16<float>(qraw[i], x);
        if (p < npieces) {
            for (int e = 0; e < qe; ++e) {
                s_qf[p * qe + e] = x[e];
                amax = fmaxf(amax, fabsf(x[e]));
            }
        }
    }
    amax = wave_max(amax);
    if (lane == 0) s_red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    auto code = [&](float x) -> int {
        float r = __builtin_rintf(x * inv);
        return int(fminf(fmaxf(r, -127.0f), 127.0f));
    };
    for (int dd = tid; dd < D; dd += kThreads) {
        if constexpr (kMax) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) s_q[h][dd] = int8_t(h < G ? code(s_qf[h * D + dd]) : 0);
        } else if constexpr (NQ == 1) {
            s_q[0][dd] = int8_t(code(s_qf[dd]));
        } else {
            int qs = 0;
            for (int h = 0; h < G; ++h) qs += code(s_qf[h * D + dd]);
            const int lo = ((qs + 8) & 15) - 8;
            const int hi = (qs - lo) >> 4;
            s_q[0][dd] = int8_t(hi);
            s_q[1][dd] = int8_t(lo);
        }
    }
    __syncthreads();
    int qv[NQ][QW];
    int c3[NQ];  // 2-bit keys: -3 * (sum of the lane's q codes) per vector
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        int qs = 0;
#pragma unroll
        for (int m = 0; m < QW / 4; ++m) {
            const uint4 w = *reinterpret_cast<const uint4*>(&s_q[n][sub * DPL + 16 * m]);
            qv[n][4 * m] = int(w.x); qv[n][4 * m + 1] = int(w.y); qv[n][4 * m + 2] = int(w.z); qv[n][4 * m + 3] = int(w.w);
        }
#pragma unroll
        for (int i = 0; i < QW; ++i) qs = __builtin_amdgcn_sdot4(qv[n][i], 0x01010101, qs, false);
        c3[n] = -3 * qs;
    }
    for (int i = tid; i < kHistBins; i += kThreads) s_hist[i] = 0u;  // q is in registers now
    __syncthreads();

    // round r's row is in kv[u]: aggregate it into s_key
    auto consume = [&](int r, int u) {
        const int tok = r * TPR + tok_lane;
        int A;
        if constexpr (kMax) {
            int best = 0;
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                const int acc = group_sum_i<LPT>(lane_dot<KB>(qv[h], kv[u], c3[h]));
                if (h < G) best = (h == 0 || acc > best) ? acc : best;
            }
            A = best;
        } else {
            int acc0 = lane_dot<KB>(qv[0], kv[u], c3[0]);
            if constexpr (NQ == 2) acc0 = acc0 * 16 + lane_dot<KB>(qv[1], kv[u], c3[1]);
            A = group_sum_i<LPT>(acc0);
        }
        if (sub == 0 && tok < nvalid) s_key[tok] = uint32_t(A);
    };
    for (;;) {  // chunks of this workgroup; the current chunk's first U rounds are in flight
        if (nvalid == 0) break;  // later chunks of this workgroup are past T_b too
#pragma unroll 1
        for (int r0 = 0; r0 < ROUNDS - U; r0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                consume(r0 + u, u);
                kv[u] = load_row(r0 + U + u);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) consume(ROUNDS - U + u, u);
        __syncthreads();

        // ---- scores and keys out (coalesced), top-digit histogram ----
        uint32_t* kout = a.keys + int64_t(unit) * a.kstride + c0;
        float* sout = a.scores ? a.scores + int64_t(unit) * d.T_max + c0 : nullptr;
#pragma unroll
        for (int i = 0; i < CH / kThreads; ++i) {
            const int t = tid + i * kThreads;
            if (t < nvalid) {
                const float score = float(int(s_key[t])) * scl[i];  // one fp32 product
                const uint32_t k = order_key(score);
                atomicAdd(&s_hist[k >> kKeyShift], 1u);
                kout[t] = k;
                if (sout) sout[t] = key_to_float(k);
            }
        }
        __syncthreads();

        chunk += gridDim.x;
        if (chunk >= nch) break;
        c0 = int64_t(chunk) * CH;
        nvalid = scan_chunk_tokens<CH>(Tb, c0);
        if (nvalid == 0) break;
        last = nvalid - 1;
        if constexpr (paged) {
            fill_pages();
            __syncthreads();
        }
        load_scales();
#pragma unroll
        for (int u = 0; u < U; ++u) kv[u] = load_row(u);
    }
    uint32_t* gh = a.hist1 + (int64_t(unit) * a.hist_rep + ui.x % a.hist_rep) * kHistBins;
    for (int i = tid; i < kHistBins; i += kThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// ---------------------------------------------------------------------------------------------
// k_scan_w: the same scan for grids that give every CU a workgroup, one 1024-thread workgroup per
// CU.  A work item of CHW tokens is cut into batches of U wave-loads (U * TPW consecutive tokens);
// wave w starts on batch w and then takes the next unclaimed batch from an LDS counter.  The
// waves that a CU serves first take more batches, so its waves finish together instead of the
// CU's last-dispatched waves setting the end.  A wave turns each batch it has used into keys at
// once.  Paging needs pages of at least TPW tokens (a wave-load then lies in one page, whose base
// is a scalar).
constexpr int kScanWideThreads = 1024;
constexpr int kScanWideChunk = 4096;

template <int D, int NQ, bool kMax, int KB, int kPg, int CHW>
__global__ __launch_bounds__(kScanWideThreads) void k_scan_w(ProposeArgs a) {
    constexpr int NT = kScanWideThreads;
    constexpr int NW = NT / 64;
    constexpr bool paged = kPg != 0;
    static_assert(kPg != 1, "pages smaller than a wave-load use k_scan");
    // NQ == 3 (2-bit keys, SUM): the group's summed query codes as three signed base-16 digits,
    // each dotted with the keys' 2-bit codes eight dims at a time (v_dot8_i32_i4)
    constexpr bool kNib = KB == 2 && NQ == 3 && !kMax;
    constexpr int DPL = (KB == 2 && (NQ <= 2 || kNib)) ? 64 : 16;
    using SR = ScanRow<KB, DPL>;
    constexpr int QW = DPL / 4;
    constexpr int LPT = D / DPL;
    constexpr int TPW = 64 / LPT;          // tokens per wave-load
    constexpr int U0 = KB == 8 ? SR::kLoads : ((NQ <= 2 || kNib) ? SR::kLoads : (NQ <= 8 ? SR::kLoads / 2 : SR::kLoads / 4));
    constexpr int U = U0 * TPW * NW <= CHW ? U0 : CHW / (TPW * NW);  // a batch per wave to start on
    constexpr int BT = U * TPW;            // tokens per batch
    constexpr int SPL = (BT + 63) / 64;    // a batch's scales (and keys) per lane
    static_assert(CHW % BT == 0 && CHW / BT >= NW, "every wave starts on a batch of its own");
    constexpr int RB = D * KB / 8;

    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_key[CHW];  // aggregated int32 dot products, each batch's by its wave
    // the query's code vectors (MAX: one per head; SUM: the summed codes or their digits)
    __shared__ __attribute__((aligned(16))) int8_t s_q[NQ][D];
    __shared__ float s_red[NW];
    __shared__ float s_qs[kMax ? 1 : kMaxG * 256];  // SUM: the group's query (fp32)
    __shared__ __attribute__((aligned(16))) uint32_t s_qn[kNib ? (D / DPL) * 24 : 4];
    __shared__ int32_t s_pg[paged ? CHW / TPW + 2 : 1];
    __shared__ uint32_t s_next;

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);
    const int nch = int((d.T_max + CHW - 1) / CHW);
    const int sub = lane % LPT;
    const int tl = lane / LPT;             // the lane's token inside a wave-load
    PRISM_TL(kTlScan, 0);

    // Every global load below is unconditional, at a clamped in-bounds address, and loads past
    // the work item's tokens are simply not used: a load under a branch makes the compiler merge
    // its wait counts with the path that skips it, and the merged counts wait for loads that are
    // still streaming.  For the same reason the per-call zeroing goes before the first load.
    if (ui.x == 0) {  // per-call state of the later kernels
        uint32_t* h2 = a.hist2 + int64_t(unit) * kHistBins;
        for (int i = tid; i < kHistBins; i += NT) h2[i] = 0u;
        if (tid < kCandLists) a.cand_cnt[(int64_t(unit) * kCandLists + tid) * kCtrStride] = 0u;
    }
    float* s_qf = kMax ? reinterpret_cast<float*>(s_hist) : s_qs;
    const int64_t qoff = (int64_t(b) * d.Hq + int64_t(g) * G) * D;
    const int qe = a.q_bf16 ? 8 : 4;
    constexpr int QP = (kMaxG * 256 / 4 + NT - 1) / NT;
    uint4 qraw[QP];
    const int npieces = G * D / qe;
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int p = min(tid + i * NT, npieces - 1);
        qraw[i] = load16(static_cast<const uint8_t*>(a.q) + (qoff * (a.q_bf16 ? 2 : 4)) + p * 16);
    }
    int chunk = ui.x;  // < nch: the grid has at most nch workgroups per unit
    int64_t c0 = int64_t(chunk) * CHW;
    int nvalid = scan_chunk_tokens<CHW>(Tb, c0);
    int last = nvalid > 0 ? nvalid - 1 : 0;  // clamp for loads (token c0 + 0 exists: c0 < T_max)
    const int lp = d.pg.log2p;
    const int64_t npool = d.pg.slots >> lp;
    auto fill_pages = [&]() {  // the work item's pages, clamped into the pool (page 0 if none)
        const int64_t p0 = c0 >> lp;
        const int npg = int(((c0 + last) >> lp) - p0 + 1);
        for (int i = tid; i < npg; i += NT) {
            int64_t pg = nvalid > 0 ? d.pg.table[int64_t(b) * d.pg.max_pages + p0 + i] : 0;
            s_pg[i] = int32_t(pg < 0 ? 0 : (pg >= npool ? npool - 1 : pg));
        }
    };
    const int8_t* kq_head = a.Kq + int64_t(g) * d.pg.slots * RB;
    const float* sc_head = a.scales + int64_t(g) * d.pg.slots;
    const uint32_t lane_off = uint32_t(tl * RB + sub * (RB / LPT));
    if constexpr (paged) {
        fill_pages();
        __syncthreads();
    }
    // scales of batch b: lane l holds those of its tokens b * BT + l + 64 i (clamped to the last)
    auto load_scales = [&](int bb, float* sc) {
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const int t = min(bb * BT + lane + 64 * i, last);
            if constexpr (paged) {
                const int64_t tt = c0 + t;
                sc[i] = sc_head[(int64_t(s_pg[(tt >> lp) - (c0 >> lp)]) << lp) + (tt & ((int64_t(1) << lp) - 1))];
            } else {
                sc[i] = a.scales[int64_t(unit) * d.T_max + c0 + t];
            }
        }
    };
    // wave-load `it` of the work item: tokens c0 + it * TPW + [0, TPW), clamped to the last token
    // (paged: to the last token's wave-load, which lies in one page)
    auto load_item = [&](int it) -> typename SR::R {
        if constexpr (paged) {
            const int i0 = min(it * TPW, last & ~(TPW - 1));
            const int64_t t0 = c0 + i0;
            const int64_t pg = __builtin_amdgcn_readfirstlane(s_pg[(t0 >> lp) - (c0 >> lp)]);
            return SR::load(kq_head + ((pg << lp) + (t0 & ((int64_t(1) << lp) - 1))) * RB + lane_off);
        } else {
            const int tok = min(it * TPW + tl, last);
            return SR::load(a.Kq + (int64_t(unit) * d.T_max + c0 + tok) * RB + sub * (RB / LPT));
        }
    };
    int nb = (nvalid + BT - 1) / BT;  // batches holding tokens
    int bcur = wave;                  // wave w starts on batch w
    float sc_cur[SPL], sc_nxt[SPL];   // scales of batch bcur and of the batch being loaded
    typename SR::R kv[U];
    auto load_first = [&]() {
        load_scales(bcur, sc_cur);    // before the rows: loads complete in issue order
#pragma unroll
        for (int u = 0; u < U; ++u) kv[u] = load_item(bcur * U + u);
    };
    if constexpr (kMax || !PRISM_SCAN_Q_FIRST) load_first();
    if (tid == 0) s_next = NW;

    constexpr int QV = kNib ? 8 : QW;      // q words per vector and lane (nibble words: 8 per digit)
    int qv[NQ][QV];
    int c3[NQ];
    if constexpr (kMax) {
        // MAX: one code vector per head, quantized once by the workgroup
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < QP; ++i) {
            const int p = tid + i * NT;
            float x[8];
            if (a.q_bf16) unpack16<uint16_t>(qraw[i], x);
            else unpack16<float>(qraw[i], x);
            if (p < npieces) {
                for (int e = 0; e < qe; ++e) {
                    s_qf[p * qe + e] = x[e];
                    amax = fmaxf(amax, fabsf(x[e]));
                }
            }
        }
        amax = wave_max(amax);
        if (lane == 0) s_red[wave] = amax;
        __syncthreads();
        amax = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) amax = fmaxf(amax, s_red[w]);
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        for (int dd = tid; dd < D; dd += NT) {
#pragma unroll
            for (int h = 0; h < NQ; ++h) s_q[h][dd] = int8_t(h < G ? scan_qcode(s_qf[h * D + dd], inv) : 0);
        }
        __syncthreads();
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
#pragma unroll
            for (int m = 0; m < QW / 4; ++m) {
                const uint4 w = *reinterpret_cast<const uint4*>(&s_q[n][sub * DPL + 16 * m]);
                qv[n][4 * m] = int(w.x); qv[n][4 * m + 1] = int(w.y); qv[n][4 * m + 2] = int(w.z); qv[n][4 * m + 3] = int(w.w);
            }
        }
        for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
        __syncthreads();
    } else {
        // SUM: the group's query goes to LDS as fp32 with each wave's absmax, and the histogram
        // is cleared; after the barrier, thread dd < D forms dim dd's summed code (and its
        // digits), so the quantization is done once per workgroup rather than once per wave
        // (16 waves repeating it cost more VALU issue time than the barriers it saved)
        float amax = 0.0f;
        const int wu = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
        for (int i = 0; i < QP; ++i) {
            // a wave without pieces skips the wait for its (clamped, unused) query load, which
            // sits behind the other waves' row loads
            if (i * NT + wu * 64 >= npieces) continue;
            const int p = tid + i * NT;
            float x[8];
            if (a.q_bf16) unpack16<uint16_t>(qraw[i], x);
            else unpack16<float>(qraw[i], x);
            if (p < npieces) {
                for (int e = 0; e < qe; ++e) {
                    s_qf[p * qe + e] = x[e];
                    amax = fmaxf(amax, fabsf(x[e]));
                }
            }
        }
        amax = wave_max(amax);
        if (lane == 0) s_red[wave] = amax;
        // the work item's first rows are requested once the query is in: issued at the kernel's
        // start they flood the memory system, and the query's few loads wait behind the flood
        PRISM_TL(kTlScan, 1);
        if constexpr (PRISM_SCAN_Q_FIRST) {
            __builtin_amdgcn_sched_barrier(0);  // keep the row loads behind the query's use
            load_first();
        }
        for (int i = tid; i < kHistBins; i += NT) s_hist[i] = 0u;
        __syncthreads();
        PRISM_TL(kTlScan, 2);
        amax = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) amax = fmaxf(amax, s_red[w]);
        const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
        if (tid < D) {
            const int dd = tid;
            if constexpr (NQ == 1) {
                s_q[0][dd] = int8_t(scan_qcode(s_qf[dd], inv));
            } else {
                int qs = 0;
                for (int h = 0; h < G; ++h) qs += scan_qcode(s_qf[h * D + dd], inv);
                const int d0 = ((qs + 8) & 15) - 8;
                if constexpr (kNib) {
                    // qs = 256 d2 + 16 d1 + d0 with every digit in [-8, 7] (|qs| <= 15 * 127)
                    const int r1 = (qs - d0) >> 4;
                    const int d1 = ((r1 + 8) & 15) - 8;
                    s_q[0][dd] = int8_t(d0);
                    s_q[1][dd] = int8_t(d1);
                    s_q[2][dd] = int8_t((r1 - d1) >> 4);
                } else {  // qs = 16 hi + lo
                    s_q[0][dd] = int8_t((qs - d0) >> 4);
                    s_q[1][dd] = int8_t(d0);
                }
            }
        }
        __syncthreads();
        if constexpr (kNib) {
            // nibble k of word 2m holds the digit of dim 16m + 8 (k & 1) + (k >> 1), of word 2m + 1
            // that of dim 16m + 4 + 8 (k & 1) + (k >> 1): the order in which the 2-bit codes of one
            // 32-bit key word land in nibbles under the masks 0x33333333 and 0x33333333 << 2.
            // Thread l < LPT * 24 packs word l once; then every lane reads the 24 words of its dims.
            constexpr int NWD = LPT * 24;
            static_assert(NWD <= NT, "one thread per packed word");
            if (tid < NWD) {
                const int l = tid;
                const int sb = l / 24, n = (l % 24) / 8, m = (l % 8) / 2, hf = l % 2;
                const uint32_t* src = reinterpret_cast<const uint32_t*>(&s_q[n][sb * DPL + 16 * m]);
                s_qn[l] = (src[hf] & 0x0F0F0F0Fu) | ((src[2 + hf] & 0x0F0F0F0Fu) << 4);
            }
            __syncthreads();
#pragma unroll
            for (int n = 0; n < 3; ++n) {
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const uint4 w = *reinterpret_cast<const uint4*>(&s_qn[sub * 24 + 8 * n + 4 * m]);
                    qv[n][4 * m] = int(w.x); qv[n][4 * m + 1] = int(w.y); qv[n][4 * m + 2] = int(w.z); qv[n][4 * m + 3] = int(w.w);
                }
            }
        } else {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
#pragma unroll
                for (int m = 0; m < QW / 4; ++m) {
                    const uint4 w = *reinterpret_cast<const uint4*>(&s_q[n][sub * DPL + 16 * m]);
                    qv[n][4 * m] = int(w.x); qv[n][4 * m + 1] = int(w.y); qv[n][4 * m + 2] = int(w.z); qv[n][4 * m + 3] = int(w.w);
                }
            }
        }
    }
    if constexpr (kNib) {  // -3 * (the sum of the lane's summed query codes), from the digits
        int sd[3];
#pragma unroll
        for (int n = 0; n < 3; ++n) {
            sd[n] = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) sd[n] = __builtin_amdgcn_sdot8(qv[n][i], 0x11111111, sd[n], false);
        }
        c3[0] = -3 * (256 * sd[2] + 16 * sd[1] + sd[0]);
    } else {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            int qs = 0;
#pragma unroll
            for (int i = 0; i < QW; ++i) qs = __builtin_amdgcn_sdot4(qv[n][i], 0x01010101, qs, false);
            c3[n] = -3 * qs;
        }
    }

    auto claim = [&]() -> int {
        uint32_t v = 0u;
        if (lane == 0) v = atomicAdd(&s_next, 1u);
        return __builtin_amdgcn_readfirstlane(int(v));
    };
    // the wave's rows of batch bcur are in kv: aggregate them into s_key
    auto consume = [&](int u) {
        const int tok = (bcur * U + u) * TPW + tl;
        int A;
        if constexpr (kMax) {
            int best = 0;
#pragma unroll
            for (int h = 0; h < NQ; ++h) {
                const int acc = group_sum_i<LPT>(lane_dot<KB>(qv[h], kv[u], c3[h]));
                if (h < G) best = (h == 0 || acc > best) ? acc : best;
            }
            A = best;
        } else {
            if constexpr (kNib) {
                A = group_sum_i<LPT>(lane_dot_nib(qv, kv[u], c3[0]));
            } else {
                int acc0 = lane_dot<KB>(qv[0], kv[u], c3[0]);
                if constexpr (NQ == 2) acc0 = acc0 * 16 + lane_dot<KB>(qv[1], kv[u], c3[1]);
                A = group_sum_i<LPT>(acc0);
            }
        }
        if (sub == 0 && tok < nvalid) s_key[tok] = uint32_t(A);
    };
    // the wave's products of batch bb are in s_key (written by this wave, so in order): scores,
    // keys out (coalesced) and the top-digit histogram
    uint32_t* kout = a.keys + int64_t(unit) * a.kstride;
    float* sout = a.scores ? a.scores + int64_t(unit) * d.T_max : nullptr;
    auto keys_out = [&](int bb, const float* sc) {
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const int t = bb * BT + lane + 64 * i;
            if ((BT % 64 == 0 || lane + 64 * i < BT) && t < nvalid) {
                const float score = float(int(s_key[t])) * sc[i];  // one fp32 product
                const uint32_t k = order_key(score);
                atomicAdd(&s_hist[k >> kKeyShift], 1u);
                kout[c0 + t] = k;
                if (sout) sout[c0 + t] = key_to_float(k);
            }
        }
    };
    PRISM_TL(kTlScan, 3);
    for (;;) {  // work items of this workgroup; the rows of its first batch per wave are in flight
        if (nvalid == 0) break;  // later work items are past T_b too
        nb = __builtin_amdgcn_readfirstlane(nb);
        int bnext = claim();
        while (bnext < nb) {
            const int bfut = claim();  // the batch after, claimed one batch ahead
            load_scales(bnext, sc_nxt);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                consume(u);
                kv[u] = load_item(bnext * U + u);
            }
            keys_out(bcur, sc_cur);
#pragma unroll
            for (int i = 0; i < SPL; ++i) sc_cur[i] = sc_nxt[i];
            bcur = bnext;
            bnext = bfut;
        }
        if (bcur < nb) {
#pragma unroll
            for (int u = 0; u < U; ++u) consume(u);
            keys_out(bcur, sc_cur);
        }
        __syncthreads();  // every wave is done claiming from s_next and adding to s_hist

        chunk += gridDim.x;
        if (chunk >= nch) break;
        c0 = int64_t(chunk) * CHW;
        nvalid = scan_chunk_tokens<CHW>(Tb, c0);
        if (nvalid == 0) break;
        last = nvalid - 1;
        if (tid == 0) s_next = NW;
        if constexpr (paged) fill_pages();
        __syncthreads();  // the reset counter (and the pages) before the work item's claims
        nb = (nvalid + BT - 1) / BT;
        bcur = wave;
        load_scales(bcur, sc_cur);
#pragma unroll
        for (int u = 0; u < U; ++u) kv[u] = load_item(bcur * U + u);
    }
    PRISM_TL(kTlScan, 4);
    uint32_t* gh = a.hist1 + (int64_t(unit) * a.hist_rep + ui.x % a.hist_rep) * kHistBins;
    for (int i = tid; i < kHistBins; i += NT) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
    PRISM_TL(kTlScan, 5);
}

// ---------------------------------------------------------------------------------------------
template <int D, int KB, int P, int CH>
static hipError_t launch_scan_p(const ProposeArgs& a, int agg_max, dim3 grid, hipStream_t st) {
    const int G = a.d.G;
    if (!agg_max) {
        if (G == 1) launch_k("k_scan", (k_scan<D, 1, false, KB, P, CH>), grid, dim3(kThreads), st, a);
        else launch_k("k_scan", (k_scan<D, 2, false, KB, P, CH>), grid, dim3(kThreads), st, a);
    } else {
        switch (padded_g(G)) {
            case 1: launch_k("k_scan", (k_scan<D, 1, true, KB, P, CH>), grid, dim3(kThreads), st, a); break;
            case 2: launch_k("k_scan", (k_scan<D, 2, true, KB, P, CH>), grid, dim3(kThreads), st, a); break;
            case 4: launch_k("k_scan", (k_scan<D, 4, true, KB, P, CH>), grid, dim3(kThreads), st, a); break;
            case 8: launch_k("k_scan", (k_scan<D, 8, true, KB, P, CH>), grid, dim3(kThreads), st, a); break;
            case 16: launch_k("k_scan", (k_scan<D, 16, true, KB, P, CH>), grid, dim3(kThreads), st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int D, int KB, int CH>
static hipError_t launch_scan_ch(const ProposeArgs& a, int agg_max, dim3 grid, hipStream_t st) {
    if (!a.d.pg.table) return launch_scan_p<D, KB, 0, CH>(a, agg_max, grid, st);
    // tokens per scan round: 256 threads over D/DPL lanes per token (see k_scan)
    const int dpl = (KB == 2 && (agg_max ? padded_g(a.d.G) : (a.d.G == 1 ? 1 : 2)) <= 2) ? 64 : 16;
    const int tpr = kThreads * dpl / D;
    if ((1 << a.d.pg.log2p) >= tpr && tpr <= CH) return launch_scan_p<D, KB, 2, CH>(a, agg_max, grid, st);
    return launch_scan_p<D, KB, 1, CH>(a, agg_max, grid, st);
}

template <int D, int KB, int P>
static hipError_t launch_scan_w_p(const ProposeArgs& a, int agg_max, dim3 grid, hipStream_t st) {
    constexpr int C = kScanWideChunk;
    const dim3 blk(kScanWideThreads);
    const int G = a.d.G;
    if (!agg_max) {
        // 2-bit keys with at most 15 heads per group: the summed codes fit three base-16 digits
        if constexpr (KB == 2 && PRISM_SCAN_NIBBLE) {
            if (G <= 15) {
                launch_k("k_scan", (k_scan_w<D, 3, false, KB, P, C>), grid, blk, st, a);
                return hipGetLastError();
            }
        }
        if (G == 1) launch_k("k_scan", (k_scan_w<D, 1, false, KB, P, C>), grid, blk, st, a);
        else launch_k("k_scan", (k_scan_w<D, 2, false, KB, P, C>), grid, blk, st, a);
    } else {
        switch (padded_g(G)) {
            case 1: launch_k("k_scan", (k_scan_w<D, 1, true, KB, P, C>), grid, blk, st, a); break;
            case 2: launch_k("k_scan", (k_scan_w<D, 2, true, KB, P, C>), grid, blk, st, a); break;
            case 4: launch_k("k_scan", (k_scan_w<D, 4, true, KB, P, C>), grid, blk, st, a); break;
            default: return hipErrorInvalidValue;  // launch_scan_wide leaves G > 4 to k_scan
        }
    }
    return hipGetLastError();
}

// The wide scan when its work items give at least one workgroup per CU (kScanWgs / 4 of them)
// and any pages hold a whole wave-load; returns false when the caller should use k_scan.
template <int KB>
static bool launch_scan_wide(const ProposeArgs& a, int agg_max, hipStream_t st, hipError_t* err) {
#if PRISM_SCAN_WIDE
    const int units = a.d.B * a.d.Hkv;
    const int64_t nchw = (a.d.T_max + kScanWideChunk - 1) / kScanWideChunk;
    constexpr int wgs = kScanWgs / 4;
    if (int64_t(units) * nchw < wgs) return false;
    const int nq = agg_max ? padded_g(a.d.G) : (a.d.G == 1 ? 1 : 2);
    if (nq > 4) return false;  // more query vectors than 128 registers per lane hold
    const int dpl = (KB == 2 && nq <= 2) ? 64 : 16;
    const int tpw = 64 * dpl / a.d.D;  // tokens per wave-load
    if (a.d.pg.table && (1 << a.d.pg.log2p) < tpw) return false;
    int per_unit = (wgs + units - 1) / units;
    per_unit = per_unit < 1 ? 1 : (per_unit > nchw ? int(nchw) : per_unit);
    const dim3 grid(per_unit, units);
    const bool pg = a.d.pg.table != nullptr;
    switch (a.d.D) {
        case 64: *err = pg ? launch_scan_w_p<64, KB, 2>(a, agg_max, grid, st) : launch_scan_w_p<64, KB, 0>(a, agg_max, grid, st); break;
        case 128: *err = pg ? launch_scan_w_p<128, KB, 2>(a, agg_max, grid, st) : launch_scan_w_p<128, KB, 0>(a, agg_max, grid, st); break;
        case 256: *err = pg ? launch_scan_w_p<256, KB, 2>(a, agg_max, grid, st) : launch_scan_w_p<256, KB, 0>(a, agg_max, grid, st); break;
        default: *err = hipErrorInvalidValue;
    }
    return true;
#else
    (void)a; (void)agg_max; (void)st; (void)err;
    return false;
#endif
}

// The scan's launch: the wide scan where it applies, else k_scan on the grid of scan_plan (the
// caller sets a.hist_rep from the same plan; a smaller grid only leaves copies unused).
template <int KB>
hipError_t launch_scan_kb(const ProposeArgs& a, int agg_max, hipStream_t st) {
    hipError_t err = hipSuccess;
    if (launch_scan_wide<KB>(a, agg_max, st, &err)) return err;
    const int units = a.d.B * a.d.Hkv;
    const ScanPlan pl = scan_plan(units, a.d.T_max, a.nchunks);
    const bool small = pl.ch != kChunk;
    const dim3 grid(pl.per_unit, units);
    switch (a.d.D) {
        case 64: return small ? launch_scan_ch<64, KB, 256>(a, agg_max, grid, st) : launch_scan_ch<64, KB, kChunk>(a, agg_max, grid, st);
        case 128: return small ? launch_scan_ch<128, KB, 256>(a, agg_max, grid, st) : launch_scan_ch<128, KB, kChunk>(a, agg_max, grid, st);
        case 256: return small ? launch_scan_ch<256, KB, 256>(a, agg_max, grid, st) : launch_scan_ch<256, KB, kChunk>(a, agg_max, grid, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace prism
