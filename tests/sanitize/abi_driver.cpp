// abi_driver.cpp -- the C ABI's host side (csrc/prism_api.hip and csrc/prism_prof.hip, compiled for
// the host only) with every kernel launcher replaced by a stub.  The stubs count launches and check
// that every region the API carved out of the caller's workspace lies inside it.  Invalid calls
// must return their status before any launch; valid calls must launch once with regions in bounds.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py; no GPU
// is touched.  Test infrastructure only.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/prism.h"
#include "../../token_level_sparse_prism_amd/csrc/prism_internal.hpp"

namespace prism {
static int g_launches = 0;
static const uint8_t* g_ws = nullptr;
static size_t g_ws_bytes = 0;
static int g_bad = 0;

static void in_ws(const void* p, size_t bytes, const char* what) {
    const uint8_t* b = static_cast<const uint8_t*>(p);
    if (b < g_ws || b + bytes > g_ws + g_ws_bytes) {
        fprintf(stderr, "region %s [%p, +%zu) outside the workspace [%p, +%zu)\n", what, p, bytes, (const void*)g_ws,
                g_ws_bytes);
        ++g_bad;
    }
}

hipError_t launch_read_probe(const void*, size_t, uint32_t*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_quantize_keys_int2(const void*, int, const Dims&, uint8_t*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_quantize_keys(const void*, int, const Dims&, int8_t*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_zero(void*, size_t, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_propose(const ProposeArgs& a, int, hipStream_t) {
    ++g_launches;
    const int64_t U = int64_t(a.d.B) * a.d.Hkv;
    const int rep = scan_plan(int(U), a.d.T_max, a.nchunks).rep;
    in_ws(a.hist1, size_t(U) * rep * kHistBins * 4, "hist1");
    in_ws(a.hist2, size_t(U) * kHistBins * 4, "hist2");
    in_ws(a.cand_cnt, size_t(U) * kCandLists * kCtrStride * 4, "cand_cnt");
    in_ws(a.state, size_t(U) * 8 * 4, "state");
    in_ws(a.cnt_gt, size_t(U) * a.nchunks * 4, "cnt_gt");
    in_ws(a.keys, size_t(U) * a.kstride * 4, "keys");
    in_ws(a.cand, size_t(U) * kCandLists * a.cand_cap * 8, "cand");
    return hipSuccess;
}
hipError_t launch_refine(const RefineArgs& a, int, int, hipStream_t) {
    ++g_launches;
    const int64_t U = int64_t(a.d.B) * a.d.Hkv;
    const int GP = padded_g(a.d.G);
    const int64_t nsa = (a.kappa + kAttendRanks - 1) / kAttendRanks;
    const int64_t ngrp = (nsa + kMergeGroup - 1) / kMergeGroup;
    in_ws(a.done_a, size_t(U) * kCtrStride * 4, "done_a");
    in_ws(a.done_g, size_t(U) * ngrp * kCtrStride * 4, "done_g");
    in_ws(a.ctrl, size_t(a.ctrl_words) * 4, "ctrl");
    in_ws(a.skey, size_t(U) * a.kstride * 8, "skey");
    in_ws(a.logits, size_t(U) * a.kp * logit_stride(GP) * 4, "logits");
    in_ws(a.part_ml, size_t(U) * nsa * GP * 2 * 4, "part_ml");
    in_ws(a.part_acc, size_t(U) * nsa * GP * a.d.D * 4, "part_acc");
    in_ws(a.part2_ml, size_t(U) * ngrp * GP * 2 * 4, "part2_ml");
    in_ws(a.part2_acc, size_t(U) * ngrp * GP * a.d.D * 4, "part2_acc");
    return hipSuccess;
}
hipError_t launch_dense(const DenseArgs& a, int, hipStream_t) {
    ++g_launches;
    const int64_t U = int64_t(a.d.B) * a.d.Hkv;
    const int GP = padded_g(a.d.G);
    const int64_t nc = (a.d.T_max + kDenseChunk - 1) / kDenseChunk;
    in_ws(a.done, size_t(U) * kCtrStride * 4, "done");
    in_ws(a.part_ml, size_t(U) * nc * GP * 2 * 4, "dense part_ml");
    in_ws(a.part_acc, size_t(U) * nc * GP * a.d.D * 4, "dense part_acc");
    return hipSuccess;
}
}  // namespace prism

using prism::g_bad;
using prism::g_launches;

static int g_fail = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            fprintf(stderr, "line %d: expectation failed: %s\n", __LINE__, #cond); \
            ++g_fail;                                                       \
        }                                                                   \
    } while (0)

// A 256-byte aligned host buffer standing in for a device allocation (never dereferenced).
static void* buf(size_t bytes) {
    void* p = nullptr;
    if (posix_memalign(&p, 256, bytes ? bytes : 256) != 0) abort();
    return p;
}

static void set_ws(void* ws, size_t bytes) {
    prism::g_ws = static_cast<const uint8_t*>(ws);
    prism::g_ws_bytes = bytes;
}

int main() {
    for (int cfg = 0; cfg < 3; ++cfg) {
        const int B = cfg == 2 ? 8 : 2, Hq = cfg == 1 ? 16 : 32, Hkv = 8, D = cfg == 1 ? 256 : 128;
        const int64_t T = cfg == 0 ? 131072 : 5000;
        const int32_t kp = cfg == 0 ? 8192 : 1500, kappa = cfg == 0 ? 2048 : 700;
        prism_shape s = {B, Hq, Hkv, D, T, nullptr};
        void* q = buf(size_t(B) * Hq * D * 4);
        void* K = buf(64);
        void* pool = buf(size_t(B) * Hkv * kp * 4);
        void* idx = buf(size_t(B) * Hkv * kappa * 4);
        void* out = buf(size_t(B) * Hq * D * 4);
        void* lse = buf(size_t(B) * Hq * 4);
        // proposal: exact workspace, then one byte short
        const size_t wp = prism_workspace_bytes(PRISM_OP_PROPOSE, &s, kp, 0);
        EXPECT(wp > 0);
        void* ws = buf(wp);
        set_ws(ws, wp);
        int before = g_launches;
        EXPECT(prism_propose(q, PRISM_BF16, (const int8_t*)K, (const float*)K, &s, kp, PRISM_AGG_SUM, (int32_t*)pool,
                             nullptr, ws, wp, nullptr) == PRISM_OK);
        EXPECT(g_launches == before + 1);
        EXPECT(prism_propose(q, PRISM_BF16, (const int8_t*)K, (const float*)K, &s, kp, PRISM_AGG_SUM, (int32_t*)pool,
                             nullptr, ws, wp - 1, nullptr) == PRISM_ERR_WORKSPACE);
        EXPECT(prism_propose_int2(q, PRISM_BF16, (const uint8_t*)K, (const float*)K, &s, kp, PRISM_AGG_MAX,
                                  (int32_t*)pool, nullptr, ws, wp, nullptr) == PRISM_OK);
        free(ws);
        // refine and dense
        const size_t wr = prism_workspace_bytes(PRISM_OP_REFINE, &s, kp, kappa);
        ws = buf(wr);
        set_ws(ws, wr);
        before = g_launches;
        EXPECT(prism_refine_attend(q, K, K, PRISM_BF16, &s, (const int32_t*)pool, kp, kappa, PRISM_AGG_SUM, 0.0f, out,
                                   (int32_t*)idx, (float*)lse, ws, wr, nullptr) == PRISM_OK);
        EXPECT(g_launches == before + 1);
        EXPECT(prism_refine_attend(q, K, K, PRISM_BF16, &s, (const int32_t*)pool, kp, kp + 1, PRISM_AGG_SUM, 0.0f, out,
                                   (int32_t*)idx, (float*)lse, ws, wr, nullptr) == PRISM_ERR_INVALID_ARG);
        free(ws);
        const size_t wd = prism_workspace_bytes(PRISM_OP_DENSE, &s, 0, 0);
        ws = buf(wd);
        set_ws(ws, wd);
        EXPECT(prism_dense_ref(q, K, K, PRISM_F32, &s, 0.0f, out, (float*)lse, ws, wd, nullptr) == PRISM_OK);
        free(ws);
        // paged calls
        const int32_t P = 64;
        const int32_t max_pages = int32_t((T + P - 1) / P);
        void* table = buf(size_t(B) * max_pages * 4);
        prism_paging pg = {(const int32_t*)table, max_pages, P, int64_t(B) * max_pages * P};
        ws = buf(wp);
        set_ws(ws, wp);
        EXPECT(prism_propose_paged(q, PRISM_BF16, K, 8, (const float*)K, &s, &pg, kp, PRISM_AGG_SUM, (int32_t*)pool,
                                   nullptr, ws, wp, nullptr) == PRISM_OK);
        prism_paging bad = pg;
        bad.page_size = 48;
        before = g_launches;
        EXPECT(prism_propose_paged(q, PRISM_BF16, K, 8, (const float*)K, &s, &bad, kp, PRISM_AGG_SUM, (int32_t*)pool,
                                   nullptr, ws, wp, nullptr) == PRISM_ERR_INVALID_ARG);
        EXPECT(g_launches == before);
        free(ws);
        ws = buf(wr);
        set_ws(ws, wr);
        EXPECT(prism_refine_attend_paged(q, K, K, PRISM_BF16, &s, &pg, (const int32_t*)pool, kp, kappa, PRISM_AGG_SUM,
                                         0.0f, out, (int32_t*)idx, (float*)lse, ws, wr, nullptr) == PRISM_OK);
        free(ws);
        free(table);
        free(q); free(K); free(pool); free(idx); free(out); free(lse);
    }
    // invalid arguments: nothing launched
    prism_shape s = {1, 32, 8, 128, 4096, nullptr};
    void* p = buf(4096);
    const int before = g_launches;
    EXPECT(prism_propose(p, PRISM_BF16, (const int8_t*)p, (const float*)p, &s, 0, PRISM_AGG_SUM, (int32_t*)p, nullptr,
                         p, 1 << 30, nullptr) == PRISM_ERR_INVALID_ARG);
    prism_shape big = {1, 32, 8, 128, (int64_t(1) << 23) + 1, nullptr};
    EXPECT(prism_propose(p, PRISM_BF16, (const int8_t*)p, (const float*)p, &big, 64, PRISM_AGG_SUM, (int32_t*)p,
                         nullptr, p, 1 << 30, nullptr) == PRISM_ERR_UNSUPPORTED);
    EXPECT(prism_refine_attend(p, p, p, PRISM_BF16, &s, (const int32_t*)p, 64, 16, PRISM_AGG_SUM, -1.0f, p,
                               (int32_t*)p, nullptr, p, 1 << 30, nullptr) == PRISM_ERR_INVALID_ARG);
    EXPECT(prism_quantize_keys(nullptr, PRISM_BF16, &s, (int8_t*)p, (float*)p, nullptr) == PRISM_ERR_INVALID_ARG);
    prism_shape huge = {1, 64, 64, 256, int64_t(1) << 20, nullptr};  // needs far more than the static scratch
    EXPECT(prism_refine_attend_static(p, p, p, PRISM_BF16, &huge, (const int32_t*)p, 1 << 20, 2048, PRISM_AGG_SUM,
                                      0.0f, p, (int32_t*)p, nullptr, nullptr) == PRISM_ERR_WORKSPACE);
    EXPECT(g_launches == before);
    EXPECT(strcmp(prism_status_str(PRISM_ERR_HIP), "PRISM_ERR_HIP") == 0);
    free(p);
    if (g_bad || g_fail) {
        fprintf(stderr, "%d regions out of bounds, %d failed expectations\n", g_bad, g_fail);
        return 1;
    }
    printf("abi driver ok: %d launches checked\n", g_launches);
    return 0;
}
