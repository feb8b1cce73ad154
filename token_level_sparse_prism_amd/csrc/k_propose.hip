// k_propose.hip -- proposal layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4
// Overview and Sec. 4.1: the anchor layer scores the whole context and emits an expanded pool;
// Sec. 4.2: the scoring uses the compressed key cache; Sec. 5.1: pool size n = rho * kappa).
//
// Three launches per call, none of which waits on another workgroup:
//   k_scan     streams the compressed keys once (the HBM-bound pass: int8 codes, or the 2-bit
//              INT2 codes), writes a 32-bit order key per token and adds each workgroup's
//              histogram of the keys' top 12 bits into the unit's histogram (hist1).
//   k_cand     (per 1024-token chunk) finds from hist1 the bin that holds the kp-th largest key,
//              counts the chunk's keys above that bin, appends the keys inside it to the unit's
//              candidate list and histograms their bits 19..8 (hist2).
//   k_compact  (per chunk) finishes the exact threshold from hist2 and the candidate list, derives
//              the chunk's output offset from the counts of the chunks before it, and writes the
//              pool in ascending token order: every key above the threshold and the lowest-index
//              keys equal to it.
// The selection is exact integer work, so the pool is bit-identical to a full sort by
// (score desc, token asc).
#include "prism_device.hpp"
#include "prism_prof.hpp"

namespace prism {

enum { kStBin = 0, kStAbove = 1, kStKpEff = 2 };
constexpr int kFewCand = 256;  // LDS list of the candidates that share tau's top 24 bits

__device__ __forceinline__ int chunk_tokens(int64_t Tb, int64_t c0) {
    return int(Tb - c0 < 0 ? 0 : (Tb - c0 > kChunk ? kChunk : Tb - c0));
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
template <> struct ScanRow<8, 16> {
    using R = uint4;
    static constexpr int kLoads = 8;  // loads in flight per lane
    static __device__ __forceinline__ R load(const int8_t* p) { return load16_stream(p); }
    static __device__ __forceinline__ R zero() { return make_uint4(0u, 0u, 0u, 0u); }
};
template <> struct ScanRow<2, 64> {
    using R = uint4;
    static constexpr int kLoads = 4;  // the q words take the registers of the other four
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

// kPg: 0 contiguous caches; 1 paged, a page id per row; 2 paged with pages of at least TPR tokens,
// so the TPR tokens of a round share one page and its base is a scalar.
template <int D, int NQ, bool kMax, int KB, int kPg>
__global__ __launch_bounds__(kThreads) void k_scan(ProposeArgs a) {
    constexpr bool kPaged = kPg != 0;
    constexpr int DPL = (KB == 2 && NQ <= 2) ? 64 : 16;  // dims per lane
    using SR = ScanRow<KB, DPL>;
    constexpr int QW = DPL / 4;            // q words per vector and lane
    constexpr int LPT = D / DPL;           // lanes per token
    constexpr int TPW = 64 / LPT;          // tokens per wave per load
    constexpr int TPR = TPW * (kThreads / 64);
    constexpr int ROUNDS = kChunk / TPR;
    // loads in flight per lane: fewer 2-bit row words when many query vectors hold registers
    constexpr int UW = KB == 8 ? SR::kLoads : (NQ <= 2 ? SR::kLoads : (NQ <= 8 ? SR::kLoads / 2 : SR::kLoads / 4));
    constexpr int U = UW < ROUNDS ? UW : ROUNDS;
    constexpr int RB = D * KB / 8;         // bytes per key row
    static_assert(ROUNDS % U == 0, "chunk must hold whole unrolled rounds");

    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_key[kChunk];
    __shared__ float s_scale[kChunk];
    __shared__ __attribute__((aligned(16))) int8_t s_q[NQ][D];
    __shared__ float s_red[kThreads / 64];
    __shared__ int32_t s_pg[kPaged ? kChunk : 1];  // paged: the physical pages of the chunk's tokens

    const Dims& d = a.d;
    const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int b = unit / d.Hkv, g = unit % d.Hkv;
    const int G = d.G;
    const int64_t Tb = seq_len_of(d, b);

    if (ui.x == 0) {  // per-call state of the later kernels
        uint32_t* h2 = a.hist2 + int64_t(unit) * kHistBins;
        for (int i = tid; i < kHistBins; i += kThreads) h2[i] = 0u;
        if (tid < kCandLists) a.cand_cnt[(int64_t(unit) * kCandLists + tid) * kCtrStride] = 0u;
    }
    const int sub = lane % LPT;
    const int tok_lane = wave * TPW + lane / LPT;

    // ---- query quantization: one absmax over the group's G*D values (s_hist holds q meanwhile).
    // Loads complete in issue order, so the small query and scale loads go out before the first
    // chunk's key rows, which then stream in while the codes are computed.
    float* s_qf = reinterpret_cast<float*>(s_hist);
    const int64_t qoff = (int64_t(b) * d.Hq + int64_t(g) * G) * D;
    const int qe = a.q_bf16 ? 8 : 4;  // values per 16-byte piece
    constexpr int QP = (kMaxG * 256 / 4 + kThreads - 1) / kThreads;  // 16-byte query pieces per thread, max
    uint4 qraw[QP];
    const int npieces = G * D / qe;
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int p = tid + i * kThreads;
        qraw[i] = p < npieces ? load16(static_cast<const uint8_t*>(a.q) + (qoff * (a.q_bf16 ? 2 : 4)) + p * 16)
                              : make_uint4(0, 0, 0, 0);
    }
    int chunk = ui.x;
    int64_t c0 = int64_t(chunk) * kChunk;
    int nvalid = chunk < a.nchunks ? chunk_tokens(Tb, c0) : 0;
    constexpr bool paged = kPaged;  // rows through the page table (d.pg.table != nullptr)
    // paged: the chunk's page ids go to LDS once (clamped into the pool), and a row of the chunk is
    // found there; pg0 = the chunk's first page, lp = log2 of the page size
    const int lp = d.pg.log2p;
    const int64_t npool = d.pg.slots >> lp;
    auto fill_pages = [&](int64_t cc0, int nv) {
        const int64_t p0 = cc0 >> lp;
        const int npg = nv > 0 ? int(((cc0 + nv - 1) >> lp) - p0 + 1) : 0;
        for (int i = tid; i < npg; i += kThreads) {
            int64_t pg = d.pg.table[int64_t(b) * d.pg.max_pages + p0 + i];
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
        fill_pages(c0, nvalid);
        __syncthreads();
    }
    float scl_pre[kChunk / kThreads];
    {
        const float* scl = a.scales + int64_t(unit) * d.T_max + c0;
#pragma unroll
        for (int i = 0; i < kChunk / kThreads; ++i) {
            const int t = tid + i * kThreads;
            if constexpr (paged) scl_pre[i] = t < nvalid ? sc_head[paged_slot(c0 + t)] : 0.0f;
            else scl_pre[i] = t < nvalid ? scl[t] : 0.0f;
        }
    }
    // rolling buffer of U rows per lane: a register is refilled with the row U rounds ahead as
    // soon as it has been used, so about U loads stay in flight through the whole chunk
    typename SR::R kv[U];
    const int8_t* krow = a.Kq + (int64_t(unit) * d.T_max + c0 + tok_lane) * RB + sub * (RB / LPT);  // this lane's first row
    auto load_row = [&](int r) -> typename SR::R {
        if (r * TPR + tok_lane >= nvalid) return SR::zero();
        if constexpr (kPg == 2) {
            const int64_t t0 = c0 + int64_t(r) * TPR;  // the round's first token, page-aligned run
            const int64_t pg = __builtin_amdgcn_readfirstlane(s_pg[(t0 >> lp) - (c0 >> lp)]);
            return SR::load(kq_head + ((pg << lp) + (t0 & ((int64_t(1) << lp) - 1))) * RB + lane_off);
        } else if constexpr (paged) {
            return SR::load(kq_head + paged_slot(c0 + r * TPR + tok_lane) * uint32_t(RB) + uint32_t(sub * (RB / LPT)));
        } else {
            return SR::load(krow + r * (TPR * RB));
        }
    };
#pragma unroll
    for (int u = 0; u < U; ++u) kv[u] = load_row(u);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int p = tid + i * kThreads;
        if (p < npieces) {
            float x[8];
            if (a.q_bf16) unpack16<uint16_t>(qraw[i], x);
            else unpack16<float>(qraw[i], x);
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
#pragma unroll
    for (int i = 0; i < kChunk / kThreads; ++i) s_scale[tid + i * kThreads] = scl_pre[i];
    __syncthreads();

    bool first = true;
    for (; chunk < a.nchunks; chunk += gridDim.x) {
        if (!first) {
            c0 = int64_t(chunk) * kChunk;
            nvalid = chunk_tokens(Tb, c0);
            krow = a.Kq + (int64_t(unit) * d.T_max + c0 + tok_lane) * RB + sub * (RB / LPT);
        }
        if (nvalid == 0) break;  // later chunks of this workgroup are past T_b too
        if (!first) {
            if constexpr (paged) {
                fill_pages(c0, nvalid);
                __syncthreads();
            }
            const float* scl = a.scales + int64_t(unit) * d.T_max + c0;
#pragma unroll 4
            for (int i = tid; i < nvalid; i += kThreads) {
                if constexpr (paged) s_scale[i] = sc_head[paged_slot(c0 + i)];
                else s_scale[i] = scl[i];
            }
            __syncthreads();
        }

        // ---- streaming int8 scan ----
        if (!first) {
#pragma unroll
            for (int u = 0; u < U; ++u) kv[u] = load_row(u);
        }
#pragma unroll 1
        for (int r0 = 0; r0 < ROUNDS; r0 += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tok = (r0 + u) * TPR + tok_lane;
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
                if (sub == 0 && tok < nvalid) {
                    const float score = float(A) * s_scale[tok];  // one fp32 product
                    s_key[tok] = order_key(score);
                }
                if (r0 + U < ROUNDS) kv[u] = load_row(r0 + U + u);
            }
        }
        first = false;
        __syncthreads();

        // ---- keys out (coalesced), top-digit histogram ----
        uint32_t* kout = a.keys + int64_t(unit) * a.kstride + c0;
        float* sout = a.scores ? a.scores + int64_t(unit) * d.T_max + c0 : nullptr;
        for (int i = tid; i < nvalid; i += kThreads) {
            const uint32_t k = s_key[i];
            atomicAdd(&s_hist[k >> kKeyShift], 1u);
            kout[i] = k;
            if (sout) sout[i] = key_to_float(k);
        }
        __syncthreads();
    }
    uint32_t* gh = a.hist1 + int64_t(unit) * kHistBins;
    for (int i = tid; i < kHistBins; i += kThreads) {
        const uint32_t c = s_hist[i];
        if (c) atomicAdd(&gh[i], c);
    }
}

// ---------------------------------------------------------------------------------------------
// k_cand: grid (chunks, units).
__global__ __launch_bounds__(kThreads) void k_cand(ProposeArgs a) {
    __shared__ uint32_t s_tmp[kThreads / 64 * 2];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_base;

    const Dims& d = a.d;
    const int tid = threadIdx.x;
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int chunk = ui.x;
    const int b = unit / d.Hkv;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp_eff = Tb < a.kp ? Tb : a.kp;
    if (Tb == 0 || kp_eff == Tb) return;  // empty sequence / take-all: nothing to select
    const int64_t c0 = int64_t(chunk) * kChunk;
    const int nvalid = chunk_tokens(Tb, c0);

    // keys of the chunk (4 consecutive tokens per thread) and the unit's top-digit histogram
    const uint32_t* keys = a.keys + int64_t(unit) * a.kstride + c0;
    uint32_t k[4];
    if (tid * 4 + 3 < nvalid) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + tid * 4);
        k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = tid * 4 + i < nvalid ? keys[tid * 4 + i] : 0u;
    }
    uint32_t h[16];
    load_hist_desc(a.hist1 + int64_t(unit) * kHistBins, h);
    find_crossing_regs<16>(h, kHistBins, uint32_t(kp_eff), s_tmp, s_res);
    const uint32_t bin = s_res[0];
    if (chunk == 0 && tid == 0) {
        uint32_t* st = a.state + int64_t(unit) * 8;
        st[kStBin] = bin;
        st[kStAbove] = s_res[1];
        st[kStKpEff] = uint32_t(kp_eff);
    }

    uint32_t ngt = 0, ncand = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (tid * 4 + i < nvalid) {
            const uint32_t kb = k[i] >> kKeyShift;
            ngt += kb > bin ? 1u : 0u;
            ncand += kb == bin ? 1u : 0u;
        }
    }
    uint32_t v2[2] = {ngt, ncand}, p2[2], t2[2];
    block_excl_scan_n<2>(v2, p2, t2, s_tmp);
    uint32_t cpre = p2[1];
    if (tid == 0) {
        a.cnt_gt[int64_t(unit) * a.nchunks + chunk] = t2[0];
        s_base = t2[1] ? atomicAdd(&a.cand_cnt[(int64_t(unit) * kCandLists + chunk % kCandLists) * kCtrStride], t2[1])
                       : 0u;
    }
    __syncthreads();
    if (ncand) {
        uint2* cand = a.cand + (int64_t(unit) * kCandLists + chunk % kCandLists) * a.cand_cap;
        uint32_t* h2 = a.hist2 + int64_t(unit) * kHistBins;
        const uint32_t base = s_base;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tid * 4 + i < nvalid && (k[i] >> kKeyShift) == bin) {
                const uint32_t pos = base + cpre++;
                if (pos < uint64_t(a.cand_cap)) cand[pos] = make_uint2(k[i], uint32_t(c0 + tid * 4 + i));
                atomicAdd(&h2[(k[i] >> 8) & 0xFFFu], 1u);
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------
// k_compact: grid (chunks, units).  Chunk 0 also writes the -1 padding and clears hist1.
__global__ __launch_bounds__(kThreads) void k_compact(ProposeArgs a) {
    __shared__ uint32_t s_tmp[kThreads / 64 * 5];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_hist[256];
    __shared__ uint2 s_few[kFewCand];  // candidates sharing tau's top 24 bits
    __shared__ uint32_t s_nfew;

    const Dims& d = a.d;
    const int tid = threadIdx.x;
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int chunk = ui.x;
    const int b = unit / d.Hkv;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp_eff = Tb < a.kp ? Tb : a.kp;
    const int64_t c0 = int64_t(chunk) * kChunk;
    const int nvalid = chunk_tokens(Tb, c0);
    int32_t* pool = a.pool + int64_t(unit) * a.kp;

    if (chunk == 0) {
        for (int64_t j = kp_eff + tid; j < a.kp; j += kThreads) pool[j] = -1;
        uint32_t* h1 = a.hist1 + int64_t(unit) * kHistBins;
        for (int i = tid; i < kHistBins; i += kThreads) h1[i] = 0u;  // zero for the next call
    }
    if (Tb == 0 || nvalid == 0) return;
    if (kp_eff == Tb) {  // take all
        for (int i = tid; i < nvalid; i += kThreads) pool[c0 + i] = int32_t(c0 + i);
        return;
    }

    // loads: state, hist2 (descending layout), candidate count, counts of the earlier chunks, keys
    const uint32_t* st = a.state + int64_t(unit) * 8;
    const uint32_t bin = st[kStBin];
    const uint32_t above = st[kStAbove];
    // candidate sub-list l is read by threads 32 l .. 32 l + 31
    static_assert(kCandLists * 32 == kThreads, "32 threads per candidate sub-list");
    const int cl_id = tid >> 5, cl_lane = tid & 31;
    const uint2* cand = a.cand + (int64_t(unit) * kCandLists + cl_id) * a.cand_cap;
    uint32_t cn = a.cand_cnt[(int64_t(unit) * kCandLists + cl_id) * kCtrStride];
    cn = cn < uint64_t(a.cand_cap) ? cn : uint32_t(a.cand_cap);
    uint32_t h[16];
    load_hist_desc(a.hist2 + int64_t(unit) * kHistBins, h);
    uint32_t gt_before = 0;
    const uint32_t* cg = a.cnt_gt + int64_t(unit) * a.nchunks;
#pragma unroll 4
    for (int i = tid; i < chunk; i += kThreads) gt_before += cg[i];
    const uint32_t* keys = a.keys + int64_t(unit) * a.kstride + c0;
    uint32_t k[4];
    if (tid * 4 + 3 < nvalid) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + tid * 4);
        k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = tid * 4 + i < nvalid ? keys[tid * 4 + i] : 0u;
    }

    // digit A (bits 19..8) of the threshold
    const uint32_t need_bin = uint32_t(kp_eff) - above;
    find_crossing_regs<16>(h, kHistBins, need_bin, s_tmp, s_res);
    const uint32_t da = s_res[0], above_a = s_res[1];
    const uint32_t pre = (bin << 12) | da;
    // one pass over the candidates: the earlier chunks' candidates above pre (all of them above
    // tau), and the last-byte histogram and list of those sharing pre
    s_hist[tid] = 0u;
    if (tid == 0) s_nfew = 0u;
    __syncthreads();
    uint32_t cgt = 0;
    constexpr int CB = 16;  // candidate loads in flight per thread
    for (uint32_t i0 = 0; i0 < cn; i0 += CB * 32) {
        uint2 e[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const uint32_t i = i0 + u * 32 + cl_lane;
            e[u] = i < cn ? cand[i] : make_uint2(0u, 0xFFFFFFFFu);
        }
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const uint32_t hi = e[u].x >> 8;
            if (e[u].y != 0xFFFFFFFFu) {
                if (hi == pre) {
                    atomicAdd(&s_hist[e[u].x & 0xFFu], 1u);
                    const uint32_t q = atomicAdd(&s_nfew, 1u);
                    if (q < uint32_t(kFewCand)) s_few[q] = e[u];
                } else if (hi > pre && e[u].y < uint32_t(c0)) {
                    ++cgt;
                }
            }
        }
    }
    __syncthreads();
    find_crossing<256>(s_hist, need_bin - above_a, s_tmp, s_res);
    const uint32_t tau = (pre << 8) | s_res[0];
    const uint32_t need = need_bin - above_a - s_res[1];  // keys equal to tau to take, >= 1

    // the earlier chunks' candidates sharing pre: above tau, or equal to it
    uint32_t ceq = 0;
    const uint32_t nfew = s_nfew;
    if (nfew <= uint32_t(kFewCand)) {
        for (uint32_t i = tid; i < nfew; i += kThreads) {
            const uint2 e = s_few[i];
            if (e.y < uint32_t(c0)) {
                cgt += e.x > tau ? 1u : 0u;
                ceq += e.x == tau ? 1u : 0u;
            }
        }
    } else {  // more than kFewCand keys share tau's top 24 bits: scan the lists again
        for (uint32_t i = cl_lane; i < cn; i += 32) {
            const uint2 e = cand[i];
            if ((e.x >> 8) == pre && e.y < uint32_t(c0)) {
                cgt += e.x > tau ? 1u : 0u;
                ceq += e.x == tau ? 1u : 0u;
            }
        }
    }
    // one workgroup scan gives the chunk's output offset and every thread's first output slot:
    // the keys above tau before it plus the ties taken before it (ties go to the lowest tokens)
    uint32_t ngt_t = 0, neq_t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (tid * 4 + i < nvalid) {
            ngt_t += k[i] > tau ? 1u : 0u;
            neq_t += k[i] == tau ? 1u : 0u;
        }
    }
    uint32_t v5[5] = {gt_before, cgt, ceq, ngt_t, neq_t}, p5[5], t5[5];
    block_excl_scan_n<5>(v5, p5, t5, s_tmp);
    const uint32_t eq_before = t5[2];                                  // ties in earlier chunks
    const uint32_t eq_left = need > eq_before ? need - eq_before : 0u;  // ties still to take
    uint32_t pos = t5[0] + t5[1] + min(eq_before, need) + p5[3] + min(p5[4], eq_left);
    uint32_t eqr = p5[4];  // ties of this chunk before this thread's keys
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bool sel = false;
        if (tid * 4 + i < nvalid) {
            if (k[i] > tau) sel = true;
            else if (k[i] == tau) { sel = eqr < eq_left; ++eqr; }
        }
        if (sel && pos < uint32_t(a.kp)) pool[pos] = int32_t(c0 + tid * 4 + i);
        pos += sel ? 1u : 0u;
    }
}

// ---------------------------------------------------------------------------------------------
template <int D, int KB, int P>
static hipError_t launch_scan_p(const ProposeArgs& a, int agg_max, dim3 grid, hipStream_t st) {
    const int G = a.d.G;
    if (!agg_max) {
        if (G == 1) launch_k("k_scan", (k_scan<D, 1, false, KB, P>), grid, dim3(kThreads), st, a);
        else launch_k("k_scan", (k_scan<D, 2, false, KB, P>), grid, dim3(kThreads), st, a);
    } else {
        switch (padded_g(G)) {
            case 1: launch_k("k_scan", (k_scan<D, 1, true, KB, P>), grid, dim3(kThreads), st, a); break;
            case 2: launch_k("k_scan", (k_scan<D, 2, true, KB, P>), grid, dim3(kThreads), st, a); break;
            case 4: launch_k("k_scan", (k_scan<D, 4, true, KB, P>), grid, dim3(kThreads), st, a); break;
            case 8: launch_k("k_scan", (k_scan<D, 8, true, KB, P>), grid, dim3(kThreads), st, a); break;
            case 16: launch_k("k_scan", (k_scan<D, 16, true, KB, P>), grid, dim3(kThreads), st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

template <int D, int KB>
static hipError_t launch_scan(const ProposeArgs& a, int agg_max, dim3 grid, hipStream_t st) {
    if (!a.d.pg.table) return launch_scan_p<D, KB, 0>(a, agg_max, grid, st);
    // tokens per scan round: 256 threads over D/DPL lanes per token (see k_scan)
    const int dpl = (KB == 2 && (agg_max ? padded_g(a.d.G) : (a.d.G == 1 ? 1 : 2)) <= 2) ? 64 : 16;
    const int tpr = kThreads * dpl / D;
    if ((1 << a.d.pg.log2p) >= tpr) return launch_scan_p<D, KB, 2>(a, agg_max, grid, st);
    return launch_scan_p<D, KB, 1>(a, agg_max, grid, st);
}

hipError_t launch_propose(const ProposeArgs& a, int agg_max, hipStream_t st) {
    const int units = a.d.B * a.d.Hkv;
    const dim3 grid(a.nchunks, units);
    int per_unit = (kScanWgs + units - 1) / units;
    per_unit = per_unit < 1 ? 1 : (per_unit > a.nchunks ? a.nchunks : per_unit);
    const dim3 sgrid(per_unit, units);
    hipError_t e;
    const bool two = a.key_bits == 2;
    switch (a.d.D) {
        case 64: e = two ? launch_scan<64, 2>(a, agg_max, sgrid, st) : launch_scan<64, 8>(a, agg_max, sgrid, st); break;
        case 128: e = two ? launch_scan<128, 2>(a, agg_max, sgrid, st) : launch_scan<128, 8>(a, agg_max, sgrid, st); break;
        case 256: e = two ? launch_scan<256, 2>(a, agg_max, sgrid, st) : launch_scan<256, 8>(a, agg_max, sgrid, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    {
        launch_k("k_cand", k_cand, grid, dim3(kThreads), st, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    {
        launch_k("k_compact", k_compact, grid, dim3(kThreads), st, a);
    }
    return hipGetLastError();
}

}  // namespace prism
