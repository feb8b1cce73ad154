/*
 * prism.h -- C ABI of the MI355X (gfx950) decode hot path of Prism Attention.
 *
 * Method: "Prism Attention: Proposal-Refined Index Sharing Mechanism for
 * Efficient LLMs Inference" (paperpeel page of arXiv 2610.22985).  An anchor
 * (proposal) layer scores the whole context with a compressed key cache and
 * emits an expanded candidate pool of n = rho*kappa tokens (Sec. 4 Overview,
 * Sec. 4.1, Sec. 4.2, Sec. 5.1 Implementation Details); each following
 * refined layer computes exact scores over that pool only, keeps its own
 * top-kappa and attends to them (Sec. 4.1; Sec. 5.3 notes the refinement
 * cost does not depend on the context length).
 *
 * Conventions shared by every entry point
 *  - Shapes.  B sequences, Hq query heads, Hkv KV heads, G = Hq / Hkv query
 *    heads per KV head (1 <= G <= 16), head dim D in {64, 128, 256},
 *    capacity T_max tokens (1 <= T_max <= 2^23).  Query head h belongs to KV
 *    head h / G.  A "unit" is one (b, g) pair: one pool and one index set
 *    per KV head, shared by its G query heads.
 *  - Layouts (row-major, contiguous, all on the device):
 *      q          [B][Hq][D]            dtype (fp32 or bf16)
 *      K, V       [B][Hkv][T_max][D]    dtype
 *      Kq         [B][Hkv][T_max][D]    int8
 *      Kq2        [B][Hkv][T_max][D/4]  uint8 (four 2-bit codes per byte)
 *      scales     [B][Hkv][T_max]       fp32
 *      pool       [B][Hkv][kp]          int32
 *      idx        [B][Hkv][kappa]       int32
 *      out        [B][Hq][D]            dtype
 *      lse        [B][Hq]               fp32
 *      seq_lens   [B]                   int32 (device) or NULL = all T_max;
 *                 values are clamped to [0, T_max] on the device.
 *  - Alignment: q, K, V, Kq and out 16-byte aligned; every other pointer
 *    4-byte aligned; the workspace 256-byte aligned.
 *  - Ownership: the caller owns every buffer.  The library allocates no
 *    memory and keeps no state between calls.
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream).  Argument and launch errors are returned at once;
 *    device faults surface at the next synchronisation.
 *  - Errors: a call that fails validation writes nothing and launches
 *    nothing.
 *  - Workspace: query its size with prism_workspace_bytes.  It must be
 *    zero-filled before its first use (prism_workspace_init does that).
 *    The proposal calls need their histogram words zero on entry and leave
 *    them zero on completion; refine calls zero their own arrival counters
 *    (their first kernel does), and the refine and dense layouts keep their
 *    data clear of the proposal's zero-on-entry words of the same B*Hkv and
 *    T_max.  So one zero-filled workspace, large enough for each call, serves
 *    any sequence of completed calls in which every proposal call has the
 *    same B*Hkv and T_max; a proposal call with a different B*Hkv or T_max
 *    than the previous one on that workspace needs prism_workspace_init
 *    first (its histogram may then overlap words the previous call left
 *    non-zero, which would give wrong pools without an error).  Calls that
 *    run at the same time must use different workspaces.
 *  - Determinism: pools and index sets are bit-identical from run to run;
 *    attention outputs are too (fixed split and merge order).
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum prism_status {
    PRISM_OK = 0,
    PRISM_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape, kappa > kp, ... */
    PRISM_ERR_UNSUPPORTED = 2, /* D not in {64,128,256}, G > 16, T_max > 2^23, ... */
    PRISM_ERR_WORKSPACE = 3,   /* workspace smaller than prism_workspace_bytes() */
    PRISM_ERR_HIP = 4          /* a HIP launch failed; see prism_last_hip_error() */
} prism_status;

typedef enum prism_dtype { PRISM_F32 = 0, PRISM_BF16 = 1 } prism_dtype;

/* How the G query heads of a KV head combine into one selection score. */
typedef enum prism_agg { PRISM_AGG_SUM = 0, PRISM_AGG_MAX = 1 } prism_agg;

typedef enum prism_op { PRISM_OP_PROPOSE = 0, PRISM_OP_REFINE = 1, PRISM_OP_DENSE = 2 } prism_op;

typedef struct prism_shape {
    int32_t B, Hq, Hkv, D;
    int64_t T_max;
    const int32_t* seq_lens; /* device [B] or NULL */
} prism_shape;

/* Workspace bytes needed by `op` for this shape (kp, kappa ignored where
 * unused).  Returns 0 when the arguments are invalid. */
size_t prism_workspace_bytes(int op, const prism_shape* s, int32_t kp, int32_t kappa);

/* Zero-fills a workspace with a kernel on `stream` (safe to record in a
 * HIP graph).  ws must be 256-byte aligned. */
prism_status prism_workspace_init(void* ws, size_t ws_bytes, void* stream);

/*
 * Key-cache compression for proposal scoring (Sec. 4.2 "Quantized Proposal
 * Construction"; the page names INT2: this int8 format is the library's main
 * one, prism_quantize_keys_int2 below gives a 2-bit format).  For every
 * (b, g, t < T_b): amax = max_d |K|; scale = amax / 127 (fp32, correctly
 * rounded); codes = clamp(rint(K * (127 / amax)), -127, 127) with one fp32
 * product and round-half-to-even; an all-zero row gives scale 0 and codes 0.
 * Rows t >= T_b are not written.  In: K (dtype).  Out: Kq, scales.
 */
prism_status prism_quantize_keys(const void* K, prism_dtype dt, const prism_shape* s,
                                 int8_t* Kq, float* scales, void* stream);

/*
 * Proposal layer (Sec. 4 Overview, Sec. 4.1 candidate pool C_t^F,
 * Sec. 4.2; pool size n = rho*kappa, Sec. 5.1).  Per unit:
 *   qi = int8 codes of the unit's G query heads under ONE shared absmax
 *        (same quantizer as prism_quantize_keys);
 *   A[t] = sum over heads (agg SUM) or max over heads (agg MAX) of the int32
 *        dot products qi[h] . Kq[t];
 *   score[t] = float(A[t]) * scales[t] (one fp32 product), -0 -> +0;
 *   pool = the first min(kp, T_b) tokens under (score desc, t asc), written
 *        in ascending t order, the rest of the kp slots = -1.
 * In: q (qdt), Kq, scales.  Out: pool [B][Hkv][kp]; scores [B][Hkv][T_max]
 * fp32 (optional, NULL to skip; entries t >= T_b untouched).
 * Workspace: prism_workspace_bytes(PRISM_OP_PROPOSE, s, kp, 0).
 */
prism_status prism_propose(const void* q, prism_dtype qdt, const int8_t* Kq, const float* scales,
                           const prism_shape* s, int32_t kp, prism_agg agg, int32_t* pool,
                           float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * INT2 key cache for proposal scoring (Sec. 4.2 compresses the proposal
 * layer's key cache to INT2 and prints no scheme; this is the library's
 * reading).  For every (b, g, t < T_b): amax = max_d |K|; scale = amax / 4
 * (exact); u = K * (2 / amax) (one fp32 product, the reciprocal correctly
 * rounded); level c = clamp(2 * floor(u) + 1, -3, 3) in {-3, -1, +1, +3}, so
 * [-amax, amax] is cut into four equal cells coded by their centres and K is
 * reconstructed as scale * c.  A value on a cell edge takes the upper cell;
 * an all-zero row gives scale 0 and c = +1.  Storage: 2-bit codes
 * b = (c + 3) / 2, D/4 bytes per row; 32-bit word w of a row (little endian)
 * holds dims 16w .. 16w + 15, dim 16w + 4j + i in bits 8i + 2j .. 8i + 2j + 1.
 * Rows t >= T_b are not written.  In: K (dtype).  Out: Kq2
 * [B][Hkv][T_max][D/4] bytes (16-byte aligned), scales [B][Hkv][T_max] fp32.
 */
prism_status prism_quantize_keys_int2(const void* K, prism_dtype dt, const prism_shape* s,
                                      uint8_t* Kq2, float* scales, void* stream);

/*
 * Proposal layer over the INT2 key cache: prism_propose with the levels c of
 * prism_quantize_keys_int2 in place of the int8 codes, i.e.
 * A[t] = sum (SUM) or max (MAX) over heads of the int32 dot products
 * qi[h] . c[t], score[t] = float(A[t]) * scales[t], and the same pool rule.
 * Same arguments, outputs, workspace and errors as prism_propose.
 */
prism_status prism_propose_int2(const void* q, prism_dtype qdt, const uint8_t* Kq2, const float* scales,
                                const prism_shape* s, int32_t kp, prism_agg agg, int32_t* pool,
                                float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Refined layer (Sec. 4.1: the refined layer re-selects its own top-kappa
 * within the inherited pool; token-level sparse attention of Sec. 1 and
 * Sec. 2.1).  Per unit, over the valid pool slots j (0 <= pool[j] < T_b):
 *   l[h, j] = q[h] . K[pool[j]]  (fp32 accumulation of exact products);
 *   S[j] = sum over the G heads (SUM) or max (MAX);
 *   idx = the first min(kappa, #valid) slots under (S desc, slot asc) --
 *        slot order is token order because pools are ascending -- written
 *        as token ids in ascending order, -1 padded to kappa;
 *   for each head h: out[h] = softmax(l[h, idx] * sm_scale) . V[idx],
 *        lse[h] = natural-log sum-exp of the scaled logits;
 *   no valid slot: out = 0, lse = -inf.
 * sm_scale = 0 selects 1/sqrt(D).  pool must be ascending (as written by
 * prism_propose); its entries are not otherwise checked -- out-of-range ones
 * are skipped.  Out: out (dtype, rounded to nearest even), idx, lse
 * (optional).  Workspace: prism_workspace_bytes(PRISM_OP_REFINE, s, kp, kappa).
 */
prism_status prism_refine_attend(const void* q, const void* K, const void* V, prism_dtype dt,
                                 const prism_shape* s, const int32_t* pool, int32_t kp,
                                 int32_t kappa, prism_agg agg, float sm_scale, void* out,
                                 int32_t* idx, float* lse, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * Paged caches (a serving layout: sequences of different lengths share one
 * pool of fixed-size pages).  Each KV head g owns a pool of num_slots rows;
 * token t of sequence b is stored in row
 *     g * num_slots + page_table[b * max_pages + t / page_size] * page_size
 *       + t % page_size
 * of every per-row cache (K, V, int8 or 2-bit keys, scales), i.e. the pools
 * are [Hkv][num_slots][D] (K, V: dtype; Kq: int8; Kq2: D/4 bytes) and
 * [Hkv][num_slots] (scales).  page_size is a power of two (1 .. 2^20, 1 is
 * a per-token map); max_pages * page_size >= T_max; num_slots is a multiple
 * of page_size (at most 2^23, else PRISM_ERR_UNSUPPORTED).  Page ids outside [0, num_slots/page_size)
 * are clamped into the pool (a wrong row is read, nothing outside the pool).
 * The key quantizers are per row, so a pool is compressed by
 * prism_quantize_keys[_int2] with shape {B = 1, Hkv, T_max = num_slots}.
 * Pools, index sets, scores and outputs keep logical token ids and the
 * layouts above; seq_lens works as before.  Results equal those of the same
 * call on contiguous caches holding the same rows, bit for bit.
 */
typedef struct prism_paging {
    const int32_t* page_table; /* device [B][max_pages], physical page ids */
    int32_t max_pages;
    int32_t page_size;
    int64_t num_slots;
} prism_paging;

/* prism_propose (key_bits 8) or prism_propose_int2 (key_bits 2) over paged
 * key pools.  Same outputs, workspace and errors; an invalid paging
 * descriptor or key_bits gives PRISM_ERR_INVALID_ARG. */
prism_status prism_propose_paged(const void* q, prism_dtype qdt, const void* Kq_pool, int32_t key_bits,
                                 const float* scales_pool, const prism_shape* s, const prism_paging* paging,
                                 int32_t kp, prism_agg agg, int32_t* pool, float* scores, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * prism_refine_attend without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same computation, arguments, outputs
 * and errors as prism_refine_attend minus ws / ws_bytes.  Its scratch is a
 * static device array of the library, 32 MiB (33554432 bytes) on each GPU
 * it runs on, held until the process ends; the call allocates nothing.  It
 * needs the refine layout's bytes for this shape, kp and kappa without the
 * proposal-sharing gap: units * (8 * ceil4(kp) + 4 * kp * max(4, Gp))
 * plus the split partials, about 24 MiB at B*Hkv = 64, kp = 8192,
 * kappa = 2048, G = 8, D = 128; a call that needs more than 32 MiB returns
 * PRISM_ERR_WORKSPACE before any device work.  Every call on one GPU uses
 * that GPU's one array: calls that overlap in time on one GPU (two streams,
 * two host threads) race and give wrong results; calls ordered on one stream
 * are safe (the call zeroes the counters it needs itself).  The first call
 * on a device looks the array's address up once (hipGetSymbolAddress).
 */
prism_status prism_refine_attend_static(const void* q, const void* K, const void* V, prism_dtype dt,
                                        const prism_shape* s, const int32_t* pool, int32_t kp,
                                        int32_t kappa, prism_agg agg, float sm_scale, void* out,
                                        int32_t* idx, float* lse, void* stream);

/* prism_refine_attend over paged K and V pools (same outputs, workspace and
 * errors). */
prism_status prism_refine_attend_paged(const void* q, const void* K_pool, const void* V_pool, prism_dtype dt,
                                       const prism_shape* s, const prism_paging* paging, const int32_t* pool,
                                       int32_t kp, int32_t kappa, prism_agg agg, float sm_scale, void* out,
                                       int32_t* idx, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Dense decode attention over every t < T_b (the kappa = kp = T_b special
 * case of the refined layer): out[h] = softmax(q[h] . K[0..T_b) * sm_scale)
 * . V[0..T_b), lse as above.  This is the full attention that the Prism
 * page's efficiency comparison (Sec. 5.3, end-to-end latency against
 * FlashAttention at 16K-128K contexts) measures the sparse path against:
 * here a reference and a baseline, not part of the sparse path.
 * Workspace: prism_workspace_bytes(PRISM_OP_DENSE, s, 0, 0).
 */
prism_status prism_dense_ref(const void* q, const void* K, const void* V, prism_dtype dt,
                             const prism_shape* s, float sm_scale, void* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * Diagnostics: per-kernel timing with HIP events.  While enabled, every kernel launch made by
 * the calls above is bracketed by two events recorded on its stream (this adds event packets
 * between kernels, so it is for measurement passes, not for production steps).
 * prism_profile_query synchronises the recorded events and returns, for one kernel name
 * ("k_quantize_keys", "k_quantize_keys_int2", "k_scan", "k_cand", "k_compact", "k_rscore",
 * "k_attend", "k_dense", "k_read_probe"), the
 * number of launches and their summed duration in milliseconds since the last reset.
 */
prism_status prism_profile_enable(int on);
prism_status prism_profile_query(const char* name, int* launches, double* total_ms);
void prism_profile_reset(void);

/*
 * Diagnostics: the read-stream ceiling.  One plain coalesced read of `bytes` (a multiple of 16,
 * src 16-byte aligned) with 16-byte streaming loads over 1024 workgroups, each reading one
 * contiguous 1/1024 of the buffer; the XOR of what each wave read goes to sink (4096 words).
 * Timed like the other kernels ("k_read_probe" in prism_profile_query), it gives the HBM read
 * rate that the scan kernel is compared with.
 */
prism_status prism_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Diagnostics: per-workgroup phase timeline, present only in the timeline build of the library
 * (lib/libprism_tl.so, compiled with PRISM_TIMELINE=1; the normal build returns
 * PRISM_ERR_UNSUPPORTED).  Thread 0 of every workgroup of the proposal and refine kernels
 * stores the GPU's 100 MHz real-time counter at the kernel's phase points; each launch
 * overwrites its workgroups' entries.  prism_timeline_read synchronises the device and copies
 * kernel `kernel`'s (0 k_scan, 1 k_cand, 2 k_compact, 3 k_rscore, 4 k_attend, 7 k_attend_d; 5
 * and 6 are the selection inside either attention kernel and the rows phase of k_attend) stamps of
 * workgroups [0, max_wgs) (linear workgroup id, at most 8192) into out[max_wgs][8]; 0 marks a
 * phase a workgroup did not reach.  prism_timeline_clear zeroes every stamp.
 */
prism_status prism_timeline_read(int kernel, unsigned long long* out, int64_t max_wgs);
prism_status prism_timeline_clear(void);

/* The hipError_t of the last failed HIP call on this thread (0 if none). */
int prism_last_hip_error(void);

/* Static string naming a status code. */
const char* prism_status_str(prism_status st);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */
