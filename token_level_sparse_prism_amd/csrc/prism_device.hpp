// prism_device.hpp -- device helpers for the gfx950 kernels: element loads, order keys, wave and
// workgroup reductions/scans, radix-digit crossing search and the last-workgroup handshake.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prism_internal.hpp"

namespace prism {

typedef int v4i __attribute__((ext_vector_type(4)));

// ---- element access ------------------------------------------------------------------------
// Rows are read 16 bytes per lane: 8 bf16 values (stored as their uint16 bit patterns) or 4 fp32.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int kPerLane = 8; };
template <> struct Elem<float> { static constexpr int kPerLane = 4; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint4 load16_stream(const void* p) {
    v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
    return make_uint4(uint32_t(v.x), uint32_t(v.y), uint32_t(v.z), uint32_t(v.w));
}

template <typename T>
__device__ __forceinline__ void unpack16(const uint4& r, float* x);

template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& r, float* x) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void unpack16<float>(const uint4& r, float* x) {
    x[0] = __uint_as_float(r.x);
    x[1] = __uint_as_float(r.y);
    x[2] = __uint_as_float(r.z);
    x[3] = __uint_as_float(r.w);
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_bits_to_f32(*p); }
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float v);
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float v) { *p = v; }

// ---- order keys ----------------------------------------------------------------------------
// Monotone map float -> uint32: a > b  <=>  key(a) > key(b) for non-NaN values, with -0 first
// mapped to +0 so equal values get equal keys.  Finite values never map to key 0, which marks an
// empty slot.
__device__ __forceinline__ float canon_zero(float f) { return f == 0.0f ? 0.0f : f; }

__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(canon_zero(f));
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ---- wave / workgroup primitives -----------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Data-parallel-primitive (DPP) lane moves: VALU operand swizzles, no LDS round trip.
// Controls used: quad_perm [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140, row_shr:n = 0x110 + n.  Lanes whose source lies outside their row of 16
// read 0 (bound_ctrl).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
    return uint32_t(__builtin_amdgcn_readlane(int(v), l));
}
__device__ __forceinline__ float readlane_f32(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// All-reduce over aligned groups of N lanes (N in {1, 2, 4, 8, 16, 32, 64}); every lane of a
// group ends with the group's result.  Groups of up to 16 lanes stay inside a DPP row.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp_f32<0xB1>(v);
    if constexpr (N >= 4) v += dpp_f32<0x4E>(v);
    if constexpr (N >= 8) v += dpp_f32<0x141>(v);
    if constexpr (N >= 16) v += dpp_f32<0x140>(v);
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 64) v += __shfl_xor(v, 32);
    return v;
}
template <int N>
__device__ __forceinline__ int group_sum_i(int v) {
    if constexpr (N >= 2) v += int(dpp_u32<0xB1>(uint32_t(v)));
    if constexpr (N >= 4) v += int(dpp_u32<0x4E>(uint32_t(v)));
    if constexpr (N >= 8) v += int(dpp_u32<0x141>(uint32_t(v)));
    if constexpr (N >= 16) v += int(dpp_u32<0x140>(uint32_t(v)));
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 64) v += __shfl_xor(v, 32);
    return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
    static_assert(N >= 1 && N <= 16, "groups inside a DPP row");
    if constexpr (N >= 2) v = fmaxf(v, dpp_f32<0xB1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_f32<0x4E>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_f32<0x141>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
    return v;
}

// 2^x by the hardware instruction (no range reduction): for x <= 0, where the result is in
// [0, 1] and tiny results may flush to zero.
__device__ __forceinline__ float exp2_le0(float x) { return __builtin_amdgcn_exp2f(x); }

// Whole-wave reductions, result uniform across the wave.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xB1>(v));
    v = fmaxf(v, dpp_f32<0x4E>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)), fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<16>(v);
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

// Inclusive prefix sum over the wave: row_shr steps inside rows of 16, then the row totals.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    x += dpp_u32<0x111>(x);
    x += dpp_u32<0x112>(x);
    x += dpp_u32<0x114>(x);
    x += dpp_u32<0x118>(x);
    const uint32_t r0 = readlane_u32(x, 15), r1 = readlane_u32(x, 31), r2 = readlane_u32(x, 47);
    const int row = lane_id() >> 4;
    return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Prefix over the NW (<= 16) per-wave totals in s_tot[0..NW): lane i of every wave reads total i
// and a row-0 DPP scan forms the prefix; the wave's exclusive prefix and the grand total are
// taken with readlane.
template <int NW>
__device__ __forceinline__ void wave_totals_prefix(const uint32_t* s_tot, uint32_t* before, uint32_t* total) {
    static_assert(NW >= 1 && NW <= 16, "one DPP row holds the wave totals");
    const int lane = lane_id();
    uint32_t x = lane < NW ? s_tot[lane] : 0u;
    if constexpr (NW > 1) x += dpp_u32<0x111>(x);
    if constexpr (NW > 2) x += dpp_u32<0x112>(x);
    if constexpr (NW > 4) x += dpp_u32<0x114>(x);
    if constexpr (NW > 8) x += dpp_u32<0x118>(x);
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    *before = w > 0 ? readlane_u32(x, w - 1) : 0u;
    *total = readlane_u32(x, NW - 1);
}

// Exclusive prefix sum over the workgroup (NT lanes, thread order).  s_tmp holds NT/64 words.  Returns the thread's exclusive prefix; *total gets the workgroup sum.
template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_tmp, uint32_t* total) {
    const int lane = lane_id(), w = wave_id();
    const uint32_t x = wave_incl_scan(v);
    if (lane == 63) s_tmp[w] = x;
    __syncthreads();
    uint32_t before, tot;
    wave_totals_prefix<NT / 64>(s_tmp, &before, &tot);
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// N independent exclusive prefix sums over the workgroup at once (thread order), one barrier pair.
// s_tmp holds (NT/64) * N words.  pre[i] = sum of v[i] over lower threads; tot[i] = total.
template <int N, int NT = kThreads>
__device__ __forceinline__ void block_excl_scan_n(const uint32_t* v, uint32_t* pre, uint32_t* tot, uint32_t* s_tmp) {
    constexpr int NW = NT / 64;
    const int lane = lane_id(), w = wave_id();
    uint32_t x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = wave_incl_scan(v[i]);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i) s_tmp[i * NW + w] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t before;
        wave_totals_prefix<NW>(s_tmp + i * NW, &before, &tot[i]);
        pre[i] = before + x[i] - v[i];
    }
    __syncthreads();
}

template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, uint32_t* s_tmp) {
    uint32_t tot;
    block_excl_scan<NT>(v, s_tmp, &tot);
    return tot;
}

// Radix-digit crossing search over NB bins spread BPT per thread in DESCENDING bin order:
// thread i holds c[k] = count of bin (NB - 1 - (i*BPT + k)).  Finds the bin b with
// above(b) < target <= above(b) + count(b), above(b) = count of the bins above b; requires
// 1 <= target <= total.  Result in s_res[0..2] = (b, above(b), count(b)), visible to all threads
// on return.
template <int BPT, int NT = kThreads>
__device__ __forceinline__ void find_crossing_regs(const uint32_t* c, int NB, uint32_t target, uint32_t* s_tmp,
                                                   uint32_t* s_res) {
    const int tid = threadIdx.x;
    uint32_t sum = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) sum += c[k];
    uint32_t tot;
    uint32_t acc = block_excl_scan<NT>(sum, s_tmp, &tot);
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        const int bin = NB - 1 - (tid * BPT + k);
        if (bin >= 0 && acc < target && acc + c[k] >= target) {
            s_res[0] = uint32_t(bin);
            s_res[1] = acc;
            s_res[2] = c[k];
        }
        acc += c[k];
    }
    __syncthreads();
}

// LDS histograms of kHistBins bins keep one pad word per 16 bins, so that the 16 consecutive bins
// a thread reads in find_crossing start on different banks across the wave.
constexpr int kHistPadded = kHistBins + kHistBins / 16;
__device__ __forceinline__ int hpad(int bin) { return bin + (bin >> 4); }

// Same search over a histogram in LDS (padded layout when NB == kHistBins).
template <int NB, int NT = kThreads>
__device__ __forceinline__ void find_crossing(const uint32_t* s_hist, uint32_t target, uint32_t* s_tmp,
                                              uint32_t* s_res) {
    constexpr int BPT = NB >= NT ? NB / NT : 1;  // with fewer bins than threads the top threads hold none
    uint32_t c[BPT];
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
        const int bin = NB - 1 - (int(threadIdx.x) * BPT + k);
        c[k] = bin >= 0 ? s_hist[NB == kHistBins ? hpad(bin) : bin] : 0u;
    }
    find_crossing_regs<BPT, NT>(c, NB, target, s_tmp, s_res);
}

// Loads a 4096-bin global histogram 16 bins per thread in the descending layout above.
__device__ __forceinline__ void load_hist_desc(const uint32_t* __restrict__ h, uint32_t* c) {
    const int base = kHistBins - 16 * (int(threadIdx.x) + 1);  // ascending bins base .. base+15
    const uint4* p = reinterpret_cast<const uint4*>(h + base);
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = p[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[15 - 4 * i] = v[i].x;
        c[14 - 4 * i] = v[i].y;
        c[13 - 4 * i] = v[i].z;
        c[12 - 4 * i] = v[i].w;
    }
}

// ---- device-scope data hand-off inside one kernel ----------------------------------------
// Values another workgroup reads in the same kernel are written through to device scope and read
// at device scope; the handshake waits for this workgroup's stores to complete and counts
// arrivals with one relaxed atomic on a per-unit counter (no cache write-back fence).
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint2* p, uint2 v) {
    const uint64_t x = uint64_t(v.x) | (uint64_t(v.y) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint2 ld_dev(const uint2* p) {
    const uint64_t x = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint2(uint32_t(x), uint32_t(x >> 32));
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t total, uint32_t* s_flag) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's device-scope stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = (prev == total - 1) ? 1u : 0u;
    }
    __syncthreads();
    return *s_flag != 0u;
}

// ---- wave ballots --------------------------------------------------------------------------
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

// Workgroup (x, unit) of an (nx, units) grid, taken from the linear workgroup id so that the
// workgroups of a unit share one XCD when units is a multiple of 8 (workgroups are dealt to the
// eight XCDs round-robin by linear id).  A unit's scratch then stays in one XCD's L2 from one
// kernel to the next.  Any other placement gives the same results.
struct UnitIdx {
    int unit, x;
};
__device__ __forceinline__ UnitIdx unit_major() {
    const int L = int(blockIdx.x + blockIdx.y * gridDim.x);
    return {L % int(gridDim.y), L / int(gridDim.y)};
}

__device__ __forceinline__ int64_t seq_len_of(const Dims& d, int b) {
    if (!d.seq_lens) return d.T_max;
    int64_t t = d.seq_lens[b];
    return t < 0 ? 0 : (t > d.T_max ? d.T_max : t);
}

// Cache row (K, V, compressed keys, scales) of token t of sequence b at KV head g.  Page ids are
// clamped into the pool, so a bad table entry reads a wrong row of the pool, never memory
// outside it.
__device__ __forceinline__ int64_t cache_row(const Dims& d, int b, int g, int64_t t) {
    if (d.pg.table == nullptr) return (int64_t(b) * d.Hkv + g) * d.T_max + t;
    int64_t page = d.pg.table[int64_t(b) * d.pg.max_pages + (t >> d.pg.log2p)];
    const int64_t npages = d.pg.slots >> d.pg.log2p;
    page = page < 0 ? 0 : (page >= npages ? npages - 1 : page);
    return int64_t(g) * d.pg.slots + (page << d.pg.log2p) + (t & ((int64_t(1) << d.pg.log2p) - 1));
}
// The first cache row of unit (b, g): a safe row for lanes that hold no token.
__device__ __forceinline__ int64_t cache_row0(const Dims& d, int b, int g) {
    return d.pg.table == nullptr ? (int64_t(b) * d.Hkv + g) * d.T_max : int64_t(g) * d.pg.slots;
}

}  // namespace prism
