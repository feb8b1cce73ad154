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

// Chunk c of a workgroup that takes chunks c0 .. c0 + M - 1: its first token, its valid tokens
// (0 for chunks past nchunks or past T_b) and the chunk whose keys are loaded (clamped into the
// row, so that no load leaves the unit's key row).
struct ChunkRef {
    int64_t c0;
    int nvalid;
    int64_t load_c0;
};
__device__ __forceinline__ ChunkRef chunk_ref(const ProposeArgs& a, int64_t Tb, int c) {
    ChunkRef r;
    r.c0 = int64_t(c) * kChunk;
    r.nvalid = c < a.nchunks ? chunk_tokens(Tb, r.c0) : 0;
    r.load_c0 = int64_t(c < a.nchunks ? c : a.nchunks - 1) * kChunk;
    return r;
}

// ---------------------------------------------------------------------------------------------
// k_cand: grid (chunk groups of M, units).  The group shares one read of the unit's histogram and
// one threshold-bin search; each chunk then counts its keys above the bin and appends those inside
// it to its candidate sub-list (chunk mod kCandLists).
template <int M>
__global__ __launch_bounds__(kThreads) void k_cand(ProposeArgs a) {
    __shared__ uint32_t s_tmp[kThreads / 64 * (M > 2 ? M : 2)];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_base[M];

    const Dims& d = a.d;
    const int tid = threadIdx.x;
    PRISM_TL(kTlCand, 0);
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int cfirst = ui.x * M;
    const int b = unit / d.Hkv;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp_eff = Tb < a.kp ? Tb : a.kp;
    if (Tb == 0 || kp_eff == Tb) return;  // empty sequence / take-all: nothing to select

    // keys of the M chunks (4 consecutive tokens per thread and chunk) and the unit's top-digit
    // histogram
    uint32_t k[M][4];
    ChunkRef cr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        cr[m] = chunk_ref(a, Tb, cfirst + m);
        chunk_keys(a, unit, cr[m].load_c0, cr[m].nvalid, k[m]);
    }
    uint32_t h[16];
    load_hist_desc(a.hist1 + int64_t(unit) * a.hist_rep * kHistBins, h);
    for (int r = 1; r < a.hist_rep; ++r) {  // the scan spread the histogram over hist_rep copies
        uint32_t hr[16];
        load_hist_desc(a.hist1 + (int64_t(unit) * a.hist_rep + r) * kHistBins, hr);
#pragma unroll
        for (int j = 0; j < 16; ++j) h[j] += hr[j];
    }
    find_crossing_regs<16>(h, kHistBins, uint32_t(kp_eff), s_tmp, s_res);
    PRISM_TL(kTlCand, 1);
    const uint32_t bin = s_res[0];
    if (cfirst == 0 && tid == 0) {
        uint32_t* st = a.state + int64_t(unit) * 8;
        st[kStBin] = bin;
        st[kStAbove] = s_res[1];
        st[kStKpEff] = uint32_t(kp_eff);
    }

    // per chunk: keys above the bin (low 16 bits) and inside it (high 16 bits); at most 4 each per
    // thread and 1024 per chunk
    uint32_t v[M], pre[M], tot[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        uint32_t ngt = 0, ncand = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tid * 4 + i < cr[m].nvalid) {
                const uint32_t kb = k[m][i] >> kKeyShift;
                ngt += kb > bin ? 1u : 0u;
                ncand += kb == bin ? 1u : 0u;
            }
        }
        v[m] = ngt | (ncand << 16);
    }
    block_excl_scan_n<M>(v, pre, tot, s_tmp);
    if (tid < M) {  // thread m publishes chunk m's counts and reserves its candidate slots
        uint32_t t = tot[0];
#pragma unroll
        for (int m = 1; m < M; ++m) t = tid == m ? tot[m] : t;
        const int c = cfirst + tid;
        if (c < a.nchunks) {
            a.cnt_gt[int64_t(unit) * a.nchunks + c] = t & 0xFFFFu;
            const uint32_t nc = t >> 16;
            s_base[tid] = nc ? atomicAdd(&a.cand_cnt[(int64_t(unit) * kCandLists + c % kCandLists) * kCtrStride], nc)
                             : 0u;
        }
    }
    __syncthreads();
    uint32_t* h2 = a.hist2 + int64_t(unit) * kHistBins;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if ((v[m] >> 16) == 0) continue;
        const int c = cfirst + m;
        uint2* cand = a.cand + (int64_t(unit) * kCandLists + c % kCandLists) * a.cand_cap;
        uint32_t pos = s_base[m] + (pre[m] >> 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tid * 4 + i < cr[m].nvalid && (k[m][i] >> kKeyShift) == bin) {
                if (pos < uint64_t(a.cand_cap)) cand[pos] = make_uint2(k[m][i], uint32_t(cr[m].c0 + tid * 4 + i));
                ++pos;
                atomicAdd(&h2[(k[m][i] >> 8) & 0xFFFu], 1u);
            }
        }
    }
    PRISM_TL(kTlCand, 2);
}

// ---------------------------------------------------------------------------------------------
// k_compact: grid (chunk groups of M, units).  The group shares the exact threshold (one read of
// the level-2 histogram and one pass over the candidate lists); each chunk then writes its
// selected tokens at its own offset.  Chunk 0 also writes the -1 padding; every chunk clears its
// slice of hist1.
template <int M>
__global__ __launch_bounds__(kThreads) void k_compact(ProposeArgs a) {
    __shared__ uint32_t s_tmp[kThreads / 64 * (3 + M)];
    __shared__ uint32_t s_res[4];
    __shared__ uint32_t s_hist[256];
    __shared__ uint2 s_few[kFewCand];  // candidates sharing tau's top 24 bits
    __shared__ uint32_t s_nfew;

    const Dims& d = a.d;
    const int tid = threadIdx.x;
    PRISM_TL(kTlCompact, 0);
    const UnitIdx ui = unit_major();
    const int unit = ui.unit;
    const int cfirst = ui.x * M;
    const int b = unit / d.Hkv;
    const int64_t Tb = seq_len_of(d, b);
    const int64_t kp_eff = Tb < a.kp ? Tb : a.kp;
    const int64_t c0 = int64_t(cfirst) * kChunk;  // the group's first token
    int32_t* pool = a.pool + int64_t(unit) * a.kp;

    if (cfirst == 0) {
        for (int64_t j = kp_eff + tid; j < a.kp; j += kThreads) pool[j] = -1;
    }
    {  // the unit's histogram copies are zeroed for the next call, a slice per chunk
        const int words = kHistBins * a.hist_rep;
        const int per = (words + a.nchunks - 1) / a.nchunks;
        uint32_t* h1 = a.hist1 + int64_t(unit) * words;
        const int cend = cfirst + M < a.nchunks ? cfirst + M : a.nchunks;
        const int w0 = cfirst * per < words ? cfirst * per : words;
        const int w1 = cend * per < words ? cend * per : words;
        for (int i = w0 + tid; i < w1; i += kThreads) h1[i] = 0u;
    }
    ChunkRef cr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) cr[m] = chunk_ref(a, Tb, cfirst + m);
    if (Tb == 0 || cr[0].nvalid == 0) return;  // later chunks are past T_b too
    if (kp_eff == Tb) {  // take all
#pragma unroll
        for (int m = 0; m < M; ++m)
            for (int i = tid; i < cr[m].nvalid; i += kThreads) pool[cr[m].c0 + i] = int32_t(cr[m].c0 + i);
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
    const uint32_t g0 = cg[tid < cfirst ? tid : 0];  // unconditional (see chunk_keys)
    uint32_t gt_before = tid < cfirst ? g0 : 0u;
    for (int i = tid + kThreads; i < cfirst; i += kThreads) gt_before += cg[i];
    uint32_t k[M][4];
#pragma unroll
    for (int m = 0; m < M; ++m) chunk_keys(a, unit, cr[m].load_c0, cr[m].nvalid, k[m]);

    // digit A (bits 19..8) of the threshold
    const uint32_t need_bin = uint32_t(kp_eff) - above;
    find_crossing_regs<16>(h, kHistBins, need_bin, s_tmp, s_res);
    PRISM_TL(kTlCompact, 1);
    const uint32_t da = s_res[0], above_a = s_res[1];
    const uint32_t pre = (bin << 12) | da;
    // one pass over the candidates: the candidates of chunks before the group above pre (all of
    // them above tau), and the last-byte histogram and list of those sharing pre
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
    PRISM_TL(kTlCompact, 2);
    find_crossing<256>(s_hist, need_bin - above_a, s_tmp, s_res);
    PRISM_TL(kTlCompact, 3);
    const uint32_t tau = (pre << 8) | s_res[0];
    const uint32_t need = need_bin - above_a - s_res[1];  // keys equal to tau to take, >= 1

    // the candidates before the group sharing pre: above tau, or equal to it
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
    // one workgroup scan: the keys above tau and the ties before the group, and per chunk the
    // thread's keys above tau (low 16 bits) and equal to it (high 16 bits)
    uint32_t v[3 + M], p[3 + M], t[3 + M];
    v[0] = gt_before;
    v[1] = cgt;
    v[2] = ceq;
#pragma unroll
    for (int m = 0; m < M; ++m) {
        uint32_t ngt_t = 0, neq_t = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tid * 4 + i < cr[m].nvalid) {
                ngt_t += k[m][i] > tau ? 1u : 0u;
                neq_t += k[m][i] == tau ? 1u : 0u;
            }
        }
        v[3 + m] = ngt_t | (neq_t << 16);
    }
    block_excl_scan_n<3 + M>(v, p, t, s_tmp);
    // chunk m: keys above tau before it = those before the group plus the group's earlier chunks';
    // ties before it likewise; ties go to the lowest tokens
    uint32_t gt_run = t[0] + t[1], eq_run = t[2];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const uint32_t eq_left = need > eq_run ? need - eq_run : 0u;  // ties still to take
        uint32_t pos = gt_run + min(eq_run, need) + (p[3 + m] & 0xFFFFu) + min(p[3 + m] >> 16, eq_left);
        uint32_t eqr = p[3 + m] >> 16;  // ties of this chunk before this thread's keys
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bool sel = false;
            if (tid * 4 + i < cr[m].nvalid) {
                if (k[m][i] > tau) sel = true;
                else if (k[m][i] == tau) { sel = eqr < eq_left; ++eqr; }
            }
            if (sel && pos < uint32_t(a.kp)) pool[pos] = int32_t(cr[m].c0 + tid * 4 + i);
            pos += sel ? 1u : 0u;
        }
        gt_run += t[3 + m] & 0xFFFFu;
        eq_run += t[3 + m] >> 16;
    }
    PRISM_TL(kTlCompact, 4);
}

hipError_t launch_scan8(const ProposeArgs& a, int agg_max, hipStream_t st);
hipError_t launch_scan2(const ProposeArgs& a, int agg_max, hipStream_t st);

hipError_t launch_propose(const ProposeArgs& args, int agg_max, hipStream_t st) {
    ProposeArgs a = args;
    const int units = a.d.B * a.d.Hkv;
    a.hist_rep = scan_plan(units, a.d.T_max, a.nchunks).rep;
    hipError_t e = a.key_bits == 2 ? launch_scan2(a, agg_max, st) : launch_scan8(a, agg_max, st);
    if (e != hipSuccess) return e;
    // chunks per selection workgroup: one while the grid has at most kSelWgs workgroups, then
    // enough (up to 8) to bring it back there; a group shares the histogram reads and the pass
    // over the candidate lists, which every workgroup repeats
#ifndef PRISM_SEL_WGS
#define PRISM_SEL_WGS 512
#endif
    constexpr int64_t kSelWgs = PRISM_SEL_WGS;
    int M = 1;
    while (M < 8 && int64_t(units) * a.nchunks > kSelWgs * M) M *= 2;
    const dim3 grid((a.nchunks + M - 1) / M, units);
    switch (M) {
        case 1: launch_k("k_cand", k_cand<1>, grid, dim3(kThreads), st, a); break;
        case 2: launch_k("k_cand", k_cand<2>, grid, dim3(kThreads), st, a); break;
        case 4: launch_k("k_cand", k_cand<4>, grid, dim3(kThreads), st, a); break;
        default: launch_k("k_cand", k_cand<8>, grid, dim3(kThreads), st, a); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    switch (M) {
        case 1: launch_k("k_compact", k_compact<1>, grid, dim3(kThreads), st, a); break;
        case 2: launch_k("k_compact", k_compact<2>, grid, dim3(kThreads), st, a); break;
        case 4: launch_k("k_compact", k_compact<4>, grid, dim3(kThreads), st, a); break;
        default: launch_k("k_compact", k_compact<8>, grid, dim3(kThreads), st, a); break;
    }
    return hipGetLastError();
}

}  // namespace prism
