// k_propose.hip -- proposal layer of Prism Attention on gfx950 (Prism Attention page, Sec. 4
// Overview and Sec. 4.1: the anchor layer scores the whole context and emits an expanded pool;
// Sec. 4.2: the scoring uses the compressed key cache; Sec. 5.1: pool size n = rho * kappa).
//
// Three launches per call, none of which waits on another workgroup:
//   k_scan     (scan_kernel.hpp, instantiated in k_scan8.hip and k_scan2.hip) streams the
//              compressed keys once (the HBM-bound pass: int8 codes, or the 2-bit INT2 codes),
//              writes a 32-bit order key per token and adds each workgroup's histogram of the
//              keys' top 12 bits into the unit's histogram (hist1).
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

// The chunk's keys, 4 consecutive tokens per thread (0 past nvalid).  One unconditional 16-byte
// load at a clamped offset inside the unit's kstride (c0 + 4 <= kstride, both multiples of 4):
// a load under a branch would make the compiler wait for it before the loads after it.
__device__ __forceinline__ void chunk_keys(const ProposeArgs& a, int unit, int64_t c0, int nvalid, uint32_t* k) {
    const int tid = threadIdx.x;
    const int64_t lim = a.kstride - c0 - 4;
    const int64_t off = int64_t(tid) * 4 < lim ? int64_t(tid) * 4 : lim;
    const uint4 v = *reinterpret_cast<const uint4*>(a.keys + int64_t(unit) * a.kstride + c0 + off);
    k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (tid * 4 + i >= nvalid) k[i] = 0u;
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
    uint32_t k[4];
    chunk_keys(a, unit, c0, nvalid, k);
    uint32_t h[16];
    load_hist_desc(a.hist1 + int64_t(unit) * a.hist_rep * kHistBins, h);
    for (int r = 1; r < a.hist_rep; ++r) {  // the scan spread the histogram over hist_rep copies
        uint32_t hr[16];
        load_hist_desc(a.hist1 + (int64_t(unit) * a.hist_rep + r) * kHistBins, hr);
#pragma unroll
        for (int k = 0; k < 16; ++k) h[k] += hr[k];
    }
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
// k_compact: grid (chunks, units).  Chunk 0 also writes the -1 padding; every chunk clears its
// slice of hist1.
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
    }
    {  // the unit's histogram copies are zeroed for the next call, a slice per chunk
        const int words = kHistBins * a.hist_rep;
        const int per = (words + a.nchunks - 1) / a.nchunks;
        uint32_t* h1 = a.hist1 + int64_t(unit) * words;
        const int w1 = (chunk + 1) * per < words ? (chunk + 1) * per : words;
        for (int i = chunk * per + tid; i < w1; i += kThreads) h1[i] = 0u;
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
    const uint32_t* cg = a.cnt_gt + int64_t(unit) * a.nchunks;
    const uint32_t g0 = cg[tid < chunk ? tid : 0];  // unconditional (see chunk_keys)
    uint32_t gt_before = tid < chunk ? g0 : 0u;
    for (int i = tid + kThreads; i < chunk; i += kThreads) gt_before += cg[i];
    uint32_t k[4];
    chunk_keys(a, unit, c0, nvalid, k);

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

hipError_t launch_scan8(const ProposeArgs& a, int agg_max, hipStream_t st);
hipError_t launch_scan2(const ProposeArgs& a, int agg_max, hipStream_t st);

hipError_t launch_propose(const ProposeArgs& args, int agg_max, hipStream_t st) {
    ProposeArgs a = args;
    const int units = a.d.B * a.d.Hkv;
    a.hist_rep = scan_plan(units, a.d.T_max, a.nchunks).rep;
    const dim3 grid(a.nchunks, units);
    hipError_t e = a.key_bits == 2 ? launch_scan2(a, agg_max, st) : launch_scan8(a, agg_max, st);
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
