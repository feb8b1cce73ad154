// prism_internal.hpp -- constants, workspace layout and kernel argument blocks shared by the
// host API (prism_api.hip) and the gfx950 kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace prism {

// ---- tiling constants --------------------------------------------------------------------
constexpr int kThreads = 256;          // every kernel runs 4 waves of 64 lanes
constexpr int kChunk = 1024;           // tokens per workgroup in the proposal kernels
constexpr int kScoreSlice = 256;       // pool slots per workgroup in pool scoring
constexpr int kAttendSlice = 64;       // selected rows per workgroup in sparse attention
constexpr int kDenseChunk = 256;       // tokens per workgroup in dense attention
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

struct ProposeWs {
    size_t ghist, done_scan, done_cand, cand_cnt, ctrl_bytes;
    size_t state, cnt_gt, offs, keys, cand, total;
};

inline ProposeWs propose_ws(int64_t units, int64_t T_max) {
    ProposeWs w{};
    const int64_t nch = (T_max + kChunk - 1) / kChunk;
    size_t o = 0;
    w.ghist = o;     o = align256(o + size_t(units) * kHistBins * 4);
    w.done_scan = o; o = align256(o + size_t(units) * 4);
    w.done_cand = o; o = align256(o + size_t(units) * 4);
    w.cand_cnt = o;  o = align256(o + size_t(units) * 4);
    w.ctrl_bytes = o;
    w.state = o;     o = align256(o + size_t(units) * 8 * 4);
    w.cnt_gt = o;    o = align256(o + size_t(units) * nch * 4);
    w.offs = o;      o = align256(o + size_t(units) * nch * 8);
    w.keys = o;      o = align256(o + size_t(units) * T_max * 4);
    w.cand = o;      o = align256(o + size_t(units) * T_max * 8);
    w.total = o;
    return w;
}

struct RefineWs {
    size_t ghist, done_s, done_a, ctrl_bytes;
    size_t state, skey, logits, sel, part_ml, part_acc, total;
};

inline int padded_g(int G) {
    int gp = 1;
    while (gp < G) gp <<= 1;
    return gp;
}
inline int logit_stride(int GP) { return GP < 4 ? 4 : GP; }

inline RefineWs refine_ws(int64_t units, int64_t kp, int64_t kappa, int GP, int D) {
    RefineWs w{};
    const int64_t nsa = (kappa + kAttendSlice - 1) / kAttendSlice;
    size_t o = 0;
    w.ghist = o;    o = align256(o + size_t(units) * kHistBins * 4);
    w.done_s = o;   o = align256(o + size_t(units) * 4);
    w.done_a = o;   o = align256(o + size_t(units) * 4);
    w.ctrl_bytes = o;
    w.state = o;    o = align256(o + size_t(units) * 8 * 4);
    w.skey = o;     o = align256(o + size_t(units) * kp * 4);
    w.logits = o;   o = align256(o + size_t(units) * kp * logit_stride(GP) * 4);
    w.sel = o;      o = align256(o + size_t(units) * kappa * 4);
    w.part_ml = o;  o = align256(o + size_t(units) * nsa * GP * 2 * 4);
    w.part_acc = o; o = align256(o + size_t(units) * nsa * GP * D * 4);
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
    w.done = o;     o = align256(o + size_t(units) * 4);
    w.ctrl_bytes = o;
    w.part_ml = o;  o = align256(o + size_t(units) * nc * GP * 2 * 4);
    w.part_acc = o; o = align256(o + size_t(units) * nc * GP * D * 4);
    w.total = o;
    return w;
}

// ---- kernel argument blocks ---------------------------------------------------------------
struct Dims {
    int B, Hq, Hkv, G, D;
    int64_t T_max;
    const int32_t* seq_lens;
};

struct ProposeArgs {
    Dims d;
    const void* q;
    int q_bf16;
    const int8_t* Kq;
    const float* scales;
    int32_t kp;
    int nchunks;
    int32_t* pool;
    float* scores;          // optional
    uint32_t* ghist;        // [U][kHistBins]
    uint32_t* done_scan;    // [U]
    uint32_t* done_cand;    // [U]
    uint32_t* cand_cnt;     // [U]
    uint32_t* state;        // [U][8]: mode, bin, above, hbin, tau, need, kp_eff
    uint32_t* cnt_gt;       // [U][nchunks]
    uint2* offs;            // [U][nchunks]: (output offset, equal-key rank base)
    uint32_t* keys;         // [U][T_max]
    uint2* cand;            // [U][T_max]: (key, token)
};

struct RefineArgs {
    Dims d;
    const void* q;
    const void* K;
    const void* V;
    const int32_t* pool;
    int32_t kp, kappa;
    float y_scale;          // sm_scale * log2(e): logits -> base-2 exponent domain
    void* out;
    int32_t* idx;
    float* lse;
    uint32_t* ghist;        // [U][kHistBins]
    uint32_t* done_s;       // [U]
    uint32_t* done_a;       // [U]
    uint32_t* state;        // [U][8]: mode, kappa_eff
    uint32_t* skey;         // [U][kp]
    float* logits;          // [U][kp][LS]
    int32_t* sel;           // [U][kappa] selected pool slots
    float* part_ml;         // [U][nsa][GP][2]
    float* part_acc;        // [U][nsa][GP][D]
};

struct DenseArgs {
    Dims d;
    const void* q;
    const void* K;
    const void* V;
    float y_scale;
    void* out;
    float* lse;
    uint32_t* done;         // [U]
    float* part_ml;         // [U][nc][GP][2]
    float* part_acc;        // [U][nc][GP][D]
};

// ---- launchers (defined in the kernel files) ----------------------------------------------
hipError_t launch_quantize_keys(const void* K, int bf16, const Dims& d, int8_t* Kq, float* scales,
                                hipStream_t st);
hipError_t launch_propose(const ProposeArgs& a, int agg_max, hipStream_t st);
hipError_t launch_refine(const RefineArgs& a, int bf16, int agg_max, hipStream_t st);
hipError_t launch_dense(const DenseArgs& a, int bf16, hipStream_t st);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace prism
