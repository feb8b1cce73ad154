// prism_api.hip -- the C ABI declared in include/prism.h: argument validation, workspace carving
// and kernel launches.  Validation touches no HIP API, so invalid calls return before any device
// work (and can be exercised on a host without a GPU).
#include <math.h>

#include <mutex>

#include "../../include/prism.h"
#include "prism_internal.hpp"
#include "prism_prof.hpp"

using namespace prism;

// Scratch of prism_refine_attend_static: one copy per GPU, held until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device array: its device address is taken
// once per device with hipGetSymbolAddress (static_scratch below) and only that address is used.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`, looked up on the first call on
// that device (with the device current) and kept.
prism_status static_scratch(void** out);

thread_local int g_last_hip_error = 0;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

prism_status check_shape(const prism_shape* s) {
    if (!s) return PRISM_ERR_INVALID_ARG;
    if (s->B < 1 || s->Hq < 1 || s->Hkv < 1 || s->T_max < 1) return PRISM_ERR_INVALID_ARG;
    if (s->Hq % s->Hkv != 0) return PRISM_ERR_INVALID_ARG;
    if (s->Hq / s->Hkv > kMaxG) return PRISM_ERR_UNSUPPORTED;
    if (s->D != 64 && s->D != 128 && s->D != 256) return PRISM_ERR_UNSUPPORTED;
    if (s->T_max > kMaxT) return PRISM_ERR_UNSUPPORTED;
    if (int64_t(s->B) * s->Hkv > 65535) return PRISM_ERR_UNSUPPORTED;  // grid.y bound
    if (s->seq_lens && !aligned(s->seq_lens, 4)) return PRISM_ERR_INVALID_ARG;
    return PRISM_OK;
}

bool valid_dtype(int dt) { return dt == PRISM_F32 || dt == PRISM_BF16; }
bool valid_agg(int ag) { return ag == PRISM_AGG_SUM || ag == PRISM_AGG_MAX; }

Dims dims_of(const prism_shape* s) {
    Dims d;
    d.B = s->B;
    d.Hq = s->Hq;
    d.Hkv = s->Hkv;
    d.G = s->Hq / s->Hkv;
    d.D = s->D;
    d.T_max = s->T_max;
    d.seq_lens = s->seq_lens;
    d.pg = Paging{nullptr, 0, 0, 0};
    return d;
}

prism_status hip_status(hipError_t e) {
    if (e == hipSuccess) return PRISM_OK;
    g_last_hip_error = int(e);
    return PRISM_ERR_HIP;
}

uint8_t* carve(void* ws, size_t off) { return static_cast<uint8_t*>(ws) + off; }

prism_status static_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return PRISM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (!p) return PRISM_ERR_HIP;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return PRISM_OK;
}

}  // namespace

extern "C" {

size_t prism_workspace_bytes(int op, const prism_shape* s, int32_t kp, int32_t kappa) {
    if (check_shape(s) != PRISM_OK) return 0;
    const int64_t units = int64_t(s->B) * s->Hkv;
    const int GP = padded_g(s->Hq / s->Hkv);
    switch (op) {
        case PRISM_OP_PROPOSE:
            if (kp < 1) return 0;
            return propose_ws(units, s->T_max).total;
        case PRISM_OP_REFINE:
            if (kp < 1 || kappa < 1 || kappa > kp) return 0;
            return refine_ws(units, s->T_max, kp, kappa, GP, s->D).total;
        case PRISM_OP_DENSE:
            return dense_ws(units, s->T_max, GP, s->D).total;
        default:
            return 0;
    }
}

prism_status prism_workspace_init(void* ws, size_t ws_bytes, void* stream) {
    if (!ws || !aligned(ws, 256)) return PRISM_ERR_INVALID_ARG;
    return hip_status(launch_zero(ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

prism_status prism_quantize_keys(const void* K, prism_dtype dt, const prism_shape* s, int8_t* Kq,
                                 float* scales, void* stream) {
    prism_status st = check_shape(s);
    if (st != PRISM_OK) return st;
    if (!valid_dtype(dt)) return PRISM_ERR_INVALID_ARG;
    if (!K || !Kq || !scales) return PRISM_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Kq, 16) || !aligned(scales, 4)) return PRISM_ERR_INVALID_ARG;
    const Dims d = dims_of(s);
    return hip_status(launch_quantize_keys(K, dt == PRISM_BF16, d, Kq, scales, static_cast<hipStream_t>(stream)));
}

// A page descriptor: page_size a power of two up to 2^20, a table of max_pages >= 1 columns that
// covers T_max logical tokens, a pool of num_slots rows (a multiple of page_size) per KV head.
static prism_status paging_of(const prism_paging* p, const prism_shape* s, Paging* out) {
    if (!p || !p->page_table || !aligned(p->page_table, 4)) return PRISM_ERR_INVALID_ARG;
    if (p->page_size < 1 || p->page_size > (1 << 20) || (p->page_size & (p->page_size - 1))) return PRISM_ERR_INVALID_ARG;
    if (p->max_pages < 1 || p->num_slots < p->page_size || p->num_slots % p->page_size) return PRISM_ERR_INVALID_ARG;
    if (int64_t(p->max_pages) * p->page_size < s->T_max) return PRISM_ERR_INVALID_ARG;
    if (p->num_slots > kMaxT) return PRISM_ERR_UNSUPPORTED;  // 2^23 rows per head: 32-bit row offsets
    int lg = 0;
    while ((1 << lg) < p->page_size) ++lg;
    *out = Paging{p->page_table, p->max_pages, lg, p->num_slots};
    return PRISM_OK;
}

static prism_status propose_impl(const void* q, prism_dtype qdt, const void* Kq, int key_bits, const float* scales,
                                 const prism_shape* s, const prism_paging* paging, int32_t kp, prism_agg agg,
                                 int32_t* pool, float* scores, void* ws, size_t ws_bytes, void* stream) {
    prism_status st = check_shape(s);
    if (st != PRISM_OK) return st;
    if (!valid_dtype(qdt) || !valid_agg(agg) || kp < 1) return PRISM_ERR_INVALID_ARG;
    if (!q || !Kq || !scales || !pool || !ws) return PRISM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(Kq, 16) || !aligned(scales, 4) || !aligned(pool, 4) ||
        (scores && !aligned(scores, 4)) || !aligned(ws, 256))
        return PRISM_ERR_INVALID_ARG;
    const int64_t units = int64_t(s->B) * s->Hkv;
    const ProposeWs L = propose_ws(units, s->T_max);
    if (ws_bytes < L.total) return PRISM_ERR_WORKSPACE;

    ProposeArgs a{};
    a.d = dims_of(s);
    if (paging && (st = paging_of(paging, s, &a.d.pg)) != PRISM_OK) return st;
    a.q = q;
    a.q_bf16 = qdt == PRISM_BF16;
    a.Kq = static_cast<const int8_t*>(Kq);
    a.key_bits = key_bits;
    a.scales = scales;
    a.kp = kp;
    a.nchunks = int((s->T_max + kChunk - 1) / kChunk);
    a.kstride = key_stride(s->T_max);
    a.pool = pool;
    a.scores = scores;
    a.hist1 = reinterpret_cast<uint32_t*>(carve(ws, L.hist1));
    a.hist2 = reinterpret_cast<uint32_t*>(carve(ws, L.hist2));
    a.cand_cnt = reinterpret_cast<uint32_t*>(carve(ws, L.cand_cnt));
    a.state = reinterpret_cast<uint32_t*>(carve(ws, L.state));
    a.cnt_gt = reinterpret_cast<uint32_t*>(carve(ws, L.cnt_gt));
    a.keys = reinterpret_cast<uint32_t*>(carve(ws, L.keys));
    a.cand = reinterpret_cast<uint2*>(carve(ws, L.cand));
    a.cand_cap = cand_list_cap(s->T_max);
    return hip_status(launch_propose(a, agg == PRISM_AGG_MAX, static_cast<hipStream_t>(stream)));
}

prism_status prism_propose(const void* q, prism_dtype qdt, const int8_t* Kq, const float* scales,
                           const prism_shape* s, int32_t kp, prism_agg agg, int32_t* pool, float* scores,
                           void* ws, size_t ws_bytes, void* stream) {
    return propose_impl(q, qdt, Kq, 8, scales, s, nullptr, kp, agg, pool, scores, ws, ws_bytes, stream);
}

prism_status prism_quantize_keys_int2(const void* K, prism_dtype dt, const prism_shape* s, uint8_t* Kq2,
                                      float* scales, void* stream) {
    prism_status st = check_shape(s);
    if (st != PRISM_OK) return st;
    if (!valid_dtype(dt)) return PRISM_ERR_INVALID_ARG;
    if (!K || !Kq2 || !scales) return PRISM_ERR_INVALID_ARG;
    if (!aligned(K, 16) || !aligned(Kq2, 16) || !aligned(scales, 4)) return PRISM_ERR_INVALID_ARG;
    const Dims d = dims_of(s);
    return hip_status(launch_quantize_keys_int2(K, dt == PRISM_BF16, d, Kq2, scales, static_cast<hipStream_t>(stream)));
}

prism_status prism_propose_int2(const void* q, prism_dtype qdt, const uint8_t* Kq2, const float* scales,
                                const prism_shape* s, int32_t kp, prism_agg agg, int32_t* pool, float* scores,
                                void* ws, size_t ws_bytes, void* stream) {
    return propose_impl(q, qdt, Kq2, 2, scales, s, nullptr, kp, agg, pool, scores, ws, ws_bytes, stream);
}

prism_status prism_propose_paged(const void* q, prism_dtype qdt, const void* Kq_pool, int32_t key_bits,
                                 const float* scales_pool, const prism_shape* s, const prism_paging* paging,
                                 int32_t kp, prism_agg agg, int32_t* pool, float* scores, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (!paging || (key_bits != 8 && key_bits != 2)) return PRISM_ERR_INVALID_ARG;
    return propose_impl(q, qdt, Kq_pool, key_bits, scales_pool, s, paging, kp, agg, pool, scores, ws, ws_bytes, stream);
}

static prism_status refine_impl(const void* q, const void* K, const void* V, prism_dtype dt,
                                const prism_shape* s, const prism_paging* paging, const int32_t* pool, int32_t kp,
                                int32_t kappa, prism_agg agg, float sm_scale, void* out, int32_t* idx, float* lse,
                                void* ws, size_t ws_bytes, void* stream, bool use_static = false) {
    prism_status st = check_shape(s);
    if (st != PRISM_OK) return st;
    if (!valid_dtype(dt) || !valid_agg(agg)) return PRISM_ERR_INVALID_ARG;
    if (kp < 1 || kappa < 1 || kappa > kp || !(sm_scale >= 0.0f) || isinf(sm_scale)) return PRISM_ERR_INVALID_ARG;
    if (!q || !K || !V || !pool || !out || !idx || (!ws && !use_static)) return PRISM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16) || !aligned(pool, 4) ||
        !aligned(idx, 4) || (lse && !aligned(lse, 4)) || (!use_static && !aligned(ws, 256)))
        return PRISM_ERR_INVALID_ARG;
    const int64_t units = int64_t(s->B) * s->Hkv;
    const int GP = padded_g(s->Hq / s->Hkv);
    const RefineWs L = refine_ws(units, s->T_max, kp, kappa, GP, s->D, !use_static);
    if (use_static) {
        if (L.total > kStaticScratchBytes) return PRISM_ERR_WORKSPACE;
    } else if (ws_bytes < L.total) {
        return PRISM_ERR_WORKSPACE;
    }
    if ((int64_t(kp) + kScoreSlice - 1) / kScoreSlice > 65535) return PRISM_ERR_UNSUPPORTED;

    RefineArgs a{};
    a.d = dims_of(s);
    if (paging && (st = paging_of(paging, s, &a.d.pg)) != PRISM_OK) return st;
    if (use_static && (st = static_scratch(&ws)) != PRISM_OK) return st;
    a.q = q;
    a.K = K;
    a.V = V;
    a.pool = pool;
    a.kp = kp;
    a.kappa = kappa;
    a.kstride = key_stride(kp);
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf(float(s->D));
    a.y_scale = scale * 1.4426950408889634f;
    a.out = out;
    a.idx = idx;
    a.lse = lse;
    a.done_a = reinterpret_cast<uint32_t*>(carve(ws, L.done_a));
    a.done_g = reinterpret_cast<uint32_t*>(carve(ws, L.done_g));
    a.ctrl = a.done_a;
    a.ctrl_words = int(L.ctrl_bytes / 4);
    a.part2_ml = reinterpret_cast<float*>(carve(ws, L.part2_ml));
    a.part2_acc = reinterpret_cast<float*>(carve(ws, L.part2_acc));
    a.skey = reinterpret_cast<uint2*>(carve(ws, L.skey));
    a.logits = reinterpret_cast<float*>(carve(ws, L.logits));
    a.part_ml = reinterpret_cast<float*>(carve(ws, L.part_ml));
    a.part_acc = reinterpret_cast<float*>(carve(ws, L.part_acc));
    if (use_static) prof_suppress(true);
    const hipError_t e = launch_refine(a, dt == PRISM_BF16, agg == PRISM_AGG_MAX, static_cast<hipStream_t>(stream));
    if (use_static) prof_suppress(false);
    return hip_status(e);
}

prism_status prism_refine_attend(const void* q, const void* K, const void* V, prism_dtype dt,
                                 const prism_shape* s, const int32_t* pool, int32_t kp, int32_t kappa,
                                 prism_agg agg, float sm_scale, void* out, int32_t* idx, float* lse,
                                 void* ws, size_t ws_bytes, void* stream) {
    return refine_impl(q, K, V, dt, s, nullptr, pool, kp, kappa, agg, sm_scale, out, idx, lse, ws, ws_bytes, stream);
}

prism_status prism_refine_attend_static(const void* q, const void* K, const void* V, prism_dtype dt,
                                        const prism_shape* s, const int32_t* pool, int32_t kp, int32_t kappa,
                                        prism_agg agg, float sm_scale, void* out, int32_t* idx, float* lse,
                                        void* stream) {
    return refine_impl(q, K, V, dt, s, nullptr, pool, kp, kappa, agg, sm_scale, out, idx, lse, nullptr, 0, stream,
                       true);
}

prism_status prism_refine_attend_paged(const void* q, const void* K_pool, const void* V_pool, prism_dtype dt,
                                       const prism_shape* s, const prism_paging* paging, const int32_t* pool,
                                       int32_t kp, int32_t kappa, prism_agg agg, float sm_scale, void* out,
                                       int32_t* idx, float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (!paging) return PRISM_ERR_INVALID_ARG;
    return refine_impl(q, K_pool, V_pool, dt, s, paging, pool, kp, kappa, agg, sm_scale, out, idx, lse, ws, ws_bytes,
                       stream);
}

prism_status prism_dense_ref(const void* q, const void* K, const void* V, prism_dtype dt, const prism_shape* s,
                             float sm_scale, void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
    prism_status st = check_shape(s);
    if (st != PRISM_OK) return st;
    if (!valid_dtype(dt) || !(sm_scale >= 0.0f) || isinf(sm_scale)) return PRISM_ERR_INVALID_ARG;
    if (!q || !K || !V || !out || !ws) return PRISM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(out, 16) || (lse && !aligned(lse, 4)) ||
        !aligned(ws, 256))
        return PRISM_ERR_INVALID_ARG;
    const int64_t units = int64_t(s->B) * s->Hkv;
    const int GP = padded_g(s->Hq / s->Hkv);
    const DenseWs L = dense_ws(units, s->T_max, GP, s->D);
    if (ws_bytes < L.total) return PRISM_ERR_WORKSPACE;

    DenseArgs a{};
    a.d = dims_of(s);
    a.q = q;
    a.K = K;
    a.V = V;
    const float scale = sm_scale > 0.0f ? sm_scale : 1.0f / sqrtf(float(s->D));
    a.y_scale = scale * 1.4426950408889634f;
    a.out = out;
    a.lse = lse;
    a.done = reinterpret_cast<uint32_t*>(carve(ws, L.done));
    a.part_ml = reinterpret_cast<float*>(carve(ws, L.part_ml));
    a.part_acc = reinterpret_cast<float*>(carve(ws, L.part_acc));
    return hip_status(launch_dense(a, dt == PRISM_BF16, static_cast<hipStream_t>(stream)));
}

prism_status prism_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes < 16 || bytes % 16 || !aligned(src, 16) || !aligned(sink, 4))
        return PRISM_ERR_INVALID_ARG;
    return hip_status(launch_read_probe(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int prism_last_hip_error(void) { return g_last_hip_error; }

const char* prism_status_str(prism_status st) {
    switch (st) {
        case PRISM_OK: return "PRISM_OK";
        case PRISM_ERR_INVALID_ARG: return "PRISM_ERR_INVALID_ARG";
        case PRISM_ERR_UNSUPPORTED: return "PRISM_ERR_UNSUPPORTED";
        case PRISM_ERR_WORKSPACE: return "PRISM_ERR_WORKSPACE";
        case PRISM_ERR_HIP: return "PRISM_ERR_HIP";
        default: return "PRISM_ERR_UNKNOWN";
    }
}

}  // extern "C"
