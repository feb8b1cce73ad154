// k_propose.hip -- proposal layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4
// Overview and Sec. 4.1: the anchor layer scores the whole context and emits an expanded pool;
// Sec. 4.2: the scoring uses the compressed key cache; Sec. 5.1: pool size n = rho * kappa).
//
// Three launches per call, none of which waits on another workgroup:
//   k_scan     streams the int8 keys once (the HBM-bound pass), writes a 32-bit order key per
//              token and adds each workgroup's histogram of the keys' top 12 bits into the unit's
//              histogram (hist1).
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
// A lane holds 16 bytes of a key row (D/16 lanes per token); a wave reads 1 KiB of
// consecutive rows per load.  Workgroup x of unit y handles chunks x, x + gridDim.x, ...
template <int D, int NQ, bool kMax>
__global__ __launch_bounds__(kThreads) void k_scan(ProposeArgs a) {
    constexpr int LPT = D / 16;            // lanes per token
    constexpr int TPW = 64 / LPT;          // tokens per wave per load
    constexpr int TPR = TPW * (kThreads / 64);
    constexpr int ROUNDS = kChunk / TPR;
    constexpr int U = 8;                   // loads in flight per lane
    static_assert(ROUNDS % U == 0, "chunk must hold whole unrolled rounds");

    __shared__ uint32_t s_hist[kHistBins];
    __shared__ uint32_t s_key[kChunk];
    __shared__ float s_scale[kChunk];
    __shared__ __attribute__((aligned(16))) int8_t s_q[NQ][D];
    __shared__ float s_red[kThreads / 64];

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
    float scl_pre[kChunk / kThreads];
    {
        const float* scl = a.scales + int64_t(unit) * d.T_max + c0;
#pragma unroll
        for (int i = 0; i < kChunk / kThreads; ++i) {
            const int t = tid + i * kThreads;
            scl_pre[i] = t < nvalid ? scl[t] : 0.0f;
        }
    }
    // rolling buffer of U rows per lane: a register is refilled with the row U rounds ahead as
    // soon as it has been used, so about U loads stay in flight through the whole chunk
    uint4 kv[U];
    const int8_t* krow = a.Kq + (int64_t(unit) * d.T_max + c0 + tok_lane) * D + sub * 16;  // this lane's first row
    auto load_row = [&](int r) -> uint4 {
        return r * TPR + tok_lane < nvalid ? load16_stream(krow + r * (TPR * D)) : make_uint4(0, 0, 0, 0);
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
    int qv[NQ][4];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const uint4 w = *reinterpret_cast<const uint4*>(&s_q[n][sub * 16]);
        qv[n][0] = int(w.x); qv[n][1] = int(w.y); qv[n][2] = int(w.z); qv[n][3] = int(w.w);
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
            krow = a.Kq + (int64_t(unit) * d.T_max + c0 + tok_lane) * D + sub * 16;
        }
        if (nvalid == 0) break;  // later chunks of this workgroup are past T_b too
        if (!first) {
            const float* scl = a.scales + int64_t(unit) * d.T_max + c0;
#pragma unroll 4
            for (int i = tid; i < nvalid; i += kThreads) s_scale[i] = scl[i];
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
                const int k4[4] = {int(kv[u].x), int(kv[u].y), int(kv[u].z), int(kv[u].w)};
                int A;
                if constexpr (kMax) {
                    int best = 0;
#pragma unroll
                    for (int h = 0; h < NQ; ++h) {
                        int acc = 0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_sdot4(qv[h][i], k4[i], acc, false);
                        acc = group_sum_i<LPT>(acc);
                        if (h < G) best = (h == 0 || acc > best) ? acc : best;
                    }
                    A = best;
                } else {
                    int acc0 = 0;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc0 = __builtin_amdgcn_sdot4(qv[0][i], k4[i], acc0, false);
                    if constexpr (NQ == 2) {
                        int acc1 = 0;
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc1 = __builtin_amdgcn_sdot4(qv[1][i], k4[i], acc1, false);
                        acc0 = acc0 * 16 + acc1;
                    }
                    acc0 = group_sum_i<LPT>(acc0);
                    A = acc0;
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
template <int D>
static hipError_t launch_scan(const ProposeArgs& a, int agg_max, dim3 grid, hipStream_t st) {
    const int G = a.d.G;
    if (!agg_max) {
        if (G == 1) launch_k("k_scan", (k_scan<D, 1, false>), grid, dim3(kThreads), st, a);
        else launch_k("k_scan", (k_scan<D, 2, false>), grid, dim3(kThreads), st, a);
    } else {
        switch (padded_g(G)) {
            case 1: launch_k("k_scan", (k_scan<D, 1, true>), grid, dim3(kThreads), st, a); break;
            case 2: launch_k("k_scan", (k_scan<D, 2, true>), grid, dim3(kThreads), st, a); break;
            case 4: launch_k("k_scan", (k_scan<D, 4, true>), grid, dim3(kThreads), st, a); break;
            case 8: launch_k("k_scan", (k_scan<D, 8, true>), grid, dim3(kThreads), st, a); break;
            case 16: launch_k("k_scan", (k_scan<D, 16, true>), grid, dim3(kThreads), st, a); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

hipError_t launch_propose(const ProposeArgs& a, int agg_max, hipStream_t st) {
    const int units = a.d.B * a.d.Hkv;
    const dim3 grid(a.nchunks, units);
    int per_unit = (kScanWgs + units - 1) / units;
    per_unit = per_unit < 1 ? 1 : (per_unit > a.nchunks ? a.nchunks : per_unit);
    const dim3 sgrid(per_unit, units);
    hipError_t e;
    switch (a.d.D) {
        case 64: e = launch_scan<64>(a, agg_max, sgrid, st); break;
        case 128: e = launch_scan<128>(a, agg_max, sgrid, st); break;
        case 256: e = launch_scan<256>(a, agg_max, sgrid, st); break;
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
