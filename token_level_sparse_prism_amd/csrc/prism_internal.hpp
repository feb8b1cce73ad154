// prism_internal.hpp -- constants, workspace layout and kernel argument blocks shared by the
// host API (prism_api.hip) and the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prism {

// ---- tiling constants --------------------------------------------------------------------
#ifndef PRISM_HIST_WGS
#define PRISM_HIST_WGS 256             // scan workgroups per copy of a unit's key histogram
#endif
#ifndef PRISM_SCAN_WIDE
#define PRISM_SCAN_WIDE 1              // one 1024-thread scan workgroup per CU on large grids
#endif
#ifndef PRISM_SCAN_WGS
#define PRISM_SCAN_WGS 1024            // target scan workgroups over all units
#endif
#ifndef PRISM_ATTEND_DSPLIT
#define PRISM_ATTEND_DSPLIT 1          // head-dimension split of the refined attention (no merge)
#endif
#ifndef PRISM_SCORE_SLICE
#define PRISM_SCORE_SLICE 64
#endif
constexpr int kThreads = 256;          // every kernel runs 4 waves of 64 lanes
constexpr int kChunk = 1024;           // tokens per chunk in the proposal kernels
constexpr int kScanWgs = PRISM_SCAN_WGS;
constexpr int kScoreSlice = PRISM_SCORE_SLICE;  // pool slots per workgroup in pool scoring
#ifndef PRISM_RSCORE_THREADS
#define PRISM_RSCORE_THREADS 256
#endif
constexpr int kRscoreThreads = PRISM_RSCORE_THREADS;  // matrix-core pool scoring: 16 slots per wave
constexpr int kAttendRanks = 128;      // selected rows per workgroup in sparse attention
constexpr int kHistRep = 8;            // most copies of a unit's key histogram (see ScanPlan)
constexpr int kMergeGroup = 16;        // partials merged by one workgroup (two levels above it)
constexpr int kAttendDRanks = 2048;   // most selected rows of the head-dimension split attention
constexpr int kAttendThreads = 1024;   // 16 waves: the selection's latency is shared by 4 waves per SIMD
constexpr int kDenseChunk = 256;       // tokens per workgroup in dense attention
constexpr int kCtrStride = 16;         // counters sit 64 bytes apart (no shared cache line)
constexpr int kCandLists = 8;          // candidate sub-lists per unit (chunk % kCandLists), one counter each
constexpr int kHistBits = 12;          // first radix digit: top 12 bits of the order key
constexpr int kHistBins = 1 << kHistBits;
constexpr int kKeyShift = 32 - kHistBits;
constexpr int64_t kMaxT = int64_t(1) << 23;
constexpr int kMaxChunks = int(kMaxT / kChunk);
constexpr int kMaxG = 16;

// ---- workspace layout ----------------------------------------------------------------------
// The first `ctrl_bytes` of a workspace hold counters and histograms that must be zero when a
// call starts; the call's last workgroups put them back to zero.
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
// per-unit rows of 32-bit keys are padded to whole 16-byte vectors
inline int64_t key_stride(int64_t n) { return (n + 3) & ~int64_t(3); }
// capacity of one candidate sub-list: every token of the chunks that feed it
inline int64_t cand_list_cap(int64_t T_max) {
    const int64_t nch = (T_max + kChunk - 1) / kChunk;
    return (nch + kCandLists - 1) / kCandLists * kChunk;
}

// The proposal scan's grid: about kScanWgs workgroups over all units, each taking work items of
// `ch` tokens (1024, or 256 when 1024-token items would give fewer than kScanWgs workgroups), and
// the unit's key histogram spread over `rep` copies, one per 256 of its workgroups, so that at
// most about 256 workgroups add into one copy's busiest bins.
struct ScanPlan {
    int ch, per_unit, rep;
};
inline ScanPlan scan_plan(int units, int64_t T_max, int nchunks) {
    ScanPlan p;
    p.ch = int64_t(units) * nchunks < kScanWgs ? 256 : kChunk;
    const int nch = int((T_max + p.ch - 1) / p.ch);
    int per_unit = (kScanWgs + units - 1) / units;
    p.per_unit = per_unit < 1 ? 1 : (per_unit > nch ? nch : per_unit);
    p.rep = (p.per_unit + PRISM_HIST_WGS - 1) / PRISM_HIST_WGS;
    p.rep = p.rep < 1 ? 1 : (p.rep > kHistRep ? kHistRep : p.rep);
    return p;
}

struct ProposeWs {
    size_t hist1, ctrl_bytes;
    size_t hist2, cand_cnt, state, cnt_gt, keys, cand, total;
};

// hist1 must be zero when a call starts (the call's compaction kernel zeroes it again);
// hist2 and cand_cnt are zeroed by the call's own scan kernel.
inline ProposeWs propose_ws(int64_t units, int64_t T_max) {
    ProposeWs w{};
    const int64_t nch = (T_max + kChunk - 1) / kChunk;
    size_t o = 0;
    w.hist1 = o;     o = align256(o + size_t(units) * scan_plan(int(units), T_max, int((T_max + kChunk - 1) / kChunk)).rep * kHistBins * 4);
    w.ctrl_bytes = o;
    w.hist2 = o;     o = align256(o + size_t(units) * kHistBins * 4);
    w.cand_cnt = o;  o = align256(o + size_t(units) * kCandLists * kCtrStride * 4);
    w.state = o;     o = align256(o + size_t(units) * 8 * 4);
    w.cnt_gt = o;    o = align256(o + size_t(units) * nch * 4);
    w.keys = o;      o = align256(o + size_t(units) * key_stride(T_max) * 4);
    w.cand = o;      o = align256(o + size_t(units) * kCandLists * cand_list_cap(T_max) * 8);
    w.total = o;
    return w;
}

struct RefineWs {
    size_t done_a, done_g, ctrl_bytes;
    size_t skey, logits, part_ml, part_acc, part2_ml, part2_acc, total;
};

inline int padded_g(int G) {
    int gp = 1;
    while (gp < G) gp <<= 1;
    return gp;
}
inline int logit_stride(int GP) { return GP < 4 ? 4 : GP; }

// The refine and dense layouts put their data after the proposal's zero-on-entry region of the
// same (units, T_max), so a proposal, refine and dense calls of one shape can share a workspace:
// none of them leaves anything but zeros in the others' control words.
inline RefineWs refine_ws(int64_t units, int64_t T_max, int64_t kp, int64_t kappa, int GP, int D,
                          bool after_propose_ctrl = true) {
    RefineWs w{};
    const int64_t nsa = (kappa + kAttendRanks - 1) / kAttendRanks;
    size_t o = 0;
    const int64_t ngrp = (nsa + kMergeGroup - 1) / kMergeGroup;
    w.done_a = o;   o = align256(o + size_t(units) * kCtrStride * 4);
    w.done_g = o;   o = align256(o + size_t(units) * ngrp * kCtrStride * 4);
    w.ctrl_bytes = o;
    const size_t pc = after_propose_ctrl ? propose_ws(units, T_max).ctrl_bytes : 0;
    o = o > pc ? o : pc;
    w.skey = o;     o = align256(o + size_t(units) * key_stride(kp) * 8);
    w.logits = o;   o = align256(o + size_t(units) * kp * logit_stride(GP) * 4);
    w.part_ml = o;  o = align256(o + size_t(units) * nsa * GP * 2 * 4);
    w.part_acc = o; o = align256(o + size_t(units) * nsa * GP * D * 4);
    w.part2_ml = o; o = align256(o + size_t(units) * ngrp * GP * 2 * 4);
    w.part2_acc = o; o = align256(o + size_t(units) * ngrp * GP * D * 4);
    w.total = o;
    return w;
}

struct DenseWs {
    size_t done, ctrl_bytes, part_ml, part_acc, total;
};

inline DenseWs dense_ws(int64_t units, int64_t T_max, int GP, int D) {
    DenseWs w{};
    const int64_t nc = (T_max + kDenseChunk - 1) / kDenseChunk;
    size_t o = 0;
    w.done = o;     o = align256(o + size_t(units) * kCtrStride * 4);
    w.ctrl_bytes = o;
    const size_t pc = propose_ws(units, T_max).ctrl_bytes;
    o = o > pc ? o : pc;
    w.part_ml = o;  o = align256(o + size_t(units) * nc * GP * 2 * 4);
    w.part_acc = o; o = align256(o + size_t(units) * nc * GP * D * 4);
    w.total = o;
    return w;
}

// ---- kernel argument blocks ---------------------------------------------------------------
// Where a KV head's cache rows live.  Contiguous (table == nullptr): unit (b, g) owns rows
// [unit * T_max, (unit + 1) * T_max).  Paged: KV head g owns a pool of `slots` rows, and token t
// of sequence b is in row g * slots + page * P + (t mod P), page = table[b][t / P], P = 2^log2p.
struct Paging {
    const int32_t* table;  // [B][max_pages] device, or nullptr
    int32_t max_pages;
    int32_t log2p;
    int64_t slots;
};

struct Dims {
    int B, Hq, Hkv, G, D;
    int64_t T_max;
    const int32_t* seq_lens;
    Paging pg;             // table == nullptr: contiguous [B][Hkv][T_max] caches
};

struct ProposeArgs {
    Dims d;
    const void* q;
    int q_bf16;
    const int8_t* Kq;       // int8 codes [U][T_max][D], or 2-bit codes [U][T_max][D/4] bytes
    int key_bits;           // 8 or 2
    const float* scales;
    int32_t kp;
    int nchunks;
    int64_t kstride;        // key_stride(T_max)
    int32_t* pool;
    float* scores;          // optional
    uint32_t* hist1;        // [U][hist_rep][kHistBins]  top 12 bits of every key
    int hist_rep;           // copies of hist1 the scan spreads its workgroups over (1 .. kHistRep)
    uint32_t* hist2;        // [U][kHistBins]  bits 19..8 of the keys in the threshold bin
    uint32_t* cand_cnt;     // [U][kCandLists][kCtrStride]
    int64_t cand_cap;       // cand_list_cap(T_max)
    uint32_t* state;        // [U][8]: bin, above, kp_eff
    uint32_t* cnt_gt;       // [U][nchunks] keys above the threshold bin per chunk
    uint32_t* keys;         // [U][kstride]
    uint2* cand;            // [U][kCandLists][cand_cap]: (key, token) of the threshold bin
};

struct RefineArgs {
    Dims d;
    const void* q;
    const void* K;
    const void* V;
    const int32_t* pool;
    int32_t kp, kappa;
    int64_t kstride;        // key_stride(kp)
    float y_scale;          // sm_scale * log2(e): logits -> base-2 exponent domain
    void* out;
    int32_t* idx;
    float* lse;
    uint32_t* done_a;       // [U][kCtrStride]
    uint32_t* done_g;       // [U][ngrp][kCtrStride]: per group of kMergeGroup slices (two-level merge)
    uint32_t* ctrl;         // the arrival counters above, ctrl_words words from done_a: pool scoring
    int ctrl_words;         // zeroes them, so a call needs no zeroed workspace
    uint2* skey;            // [U][kstride] {order key of S (0 = empty slot), id} per pool slot: id = the
                            // token, or with paged caches its row in the KV head's pool
    float* logits;          // [U][kp][LS]
    float* part_ml;         // [U][nsa][GP][2]
    float* part_acc;        // [U][nsa][GP][D]
    float* part2_ml;        // [U][ngrp][GP][2]: group partials of the two-level merge
    float* part2_acc;       // [U][ngrp][GP][D]
};

struct DenseArgs {
    Dims d;
    const void* q;
    const void* K;
    const void* V;
    float y_scale;
    void* out;
    float* lse;
    uint32_t* done;         // [U][kCtrStride]
    float* part_ml;         // [U][nc][GP][2]
    float* part_acc;        // [U][nc][GP][D]
};

// ---- launchers (defined in the kernel files) ----------------------------------------------
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_quantize_keys_int2(const void* K, int bf16, const Dims& d, uint8_t* Kq2, float* scales,
                                     hipStream_t st);
hipError_t launch_quantize_keys(const void* K, int bf16, const Dims& d, int8_t* Kq, float* scales,
                                hipStream_t st);
hipError_t launch_propose(const ProposeArgs& a, int agg_max, hipStream_t st);
hipError_t launch_refine(const RefineArgs& a, int bf16, int agg_max, hipStream_t st);
hipError_t launch_dense(const DenseArgs& a, int bf16, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace prism
