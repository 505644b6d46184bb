// common.h -- internal helpers shared by the libmoe HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workspace: a header of int32 counters that are zero between calls (each
// user restores them), then the scratch regions.  A counter that many
// workgroups hit sits on a 128-byte line of its own: device-scope atomics on
// one line are served one after another.  Header: 4 KiB for the router's
// token tiles (and the error word), one line per 16-column output tile
// (d_model <= 16,384) for the down kernel's fused combine, then one line per
// (token tile, 32-expert column slice) for the router's column slices.
constexpr int kCntLine = 32;        // int32 counters per 128-byte line
constexpr size_t kCombineCnt = 4096;                       // byte offset of the combine counters
constexpr size_t kRouteSliceCnt = kCombineCnt + (16384 / 16) * 128;   // router slice counters
constexpr int kRouteSliceCntLines = 16 * 32;                          // 16 tiles x 32 slices
constexpr size_t kWsHeader = kRouteSliceCnt + (size_t)kRouteSliceCntLines * 128;
constexpr int kRouteTile = 8;       // tokens per tile of the one-launch router
// the one-launch router's tile tt counts its arrivals at counters[kCntLine * tt]
// (tiles 0..15: bytes 0..2047)
// The error word: sticky bits set by kernels that find a precondition
// violated in their device-side input (zeroed by moe_workspace_init only).
constexpr size_t kWsErrorWord = MOE_WS_ERROR_OFFSET;
constexpr int kErrIdRange = MOE_WS_ERR_ID_RANGE;
constexpr int kErrIdRepeat = MOE_WS_ERR_ID_REPEAT;
static_assert(kWsErrorWord >= 2048 && kWsErrorWord + 4 <= kCombineCnt, "error word inside the router's 4 KiB");

// ------------------------------------------------- cross-workgroup hand-off
// Each XCD has its own L2, so data passed between workgroups is written and
// read at device scope (the sc1 forms, served by the device-coherent level)
// instead of paying an agent-scope fence, which writes back the whole L2.
// Ordering: every thread waits for its own stores to complete, the block
// synchronises, then one thread bumps the arrival counter.
__device__ __forceinline__ void store_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_int(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish_then_count(int32_t *counter, int n_arrivals, int &last_flag) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (old == n_arrivals - 1);
    }
    __syncthreads();
}

struct QMatDev {
    const uint8_t *lo;
    const uint8_t *hi;
    const uint16_t *scale;
    const uint16_t *min;
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, h);
    return static_cast<float>(v);
}

// Packed fp4 (e2m1) -> two bf16/fp16.  A nibble 0b00qq read as e2m1 is q/2,
// so with scale 2 a 2-bit code converts to exactly q.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4_bf16(uint32_t v, float scale) {
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, SEL);
    return __builtin_bit_cast(uint32_t, r);
}

template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4_f16(uint32_t v, float scale) {
    f16x2 r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, scale, SEL);
    return __builtin_bit_cast(uint32_t, r);
}

// B operand (8 values, k = 8g..8g+7 of one 32-block) from the lane's lo dword
// holding blocks (2*half, 2*half+1): HALF selects which 16 bits.  SCALE is 2
// (exact codes) for lo bits; Q3 takes q3_operand below.
template <int HALF, bool F16>
__device__ __forceinline__ u32x4 lo_operand(uint32_t dw) {
    const uint32_t a = dw & 0x33333333u;         // codes 0,1 of every byte
    const uint32_t b = (dw >> 2) & 0x33333333u;  // codes 2,3 of every byte
    u32x4 r;
    if constexpr (F16) {
        r[0] = cvt_fp4_f16<2 * HALF>(a, 2.0f);
        r[1] = cvt_fp4_f16<2 * HALF>(b, 2.0f);
        r[2] = cvt_fp4_f16<2 * HALF + 1>(a, 2.0f);
        r[3] = cvt_fp4_f16<2 * HALF + 1>(b, 2.0f);
    } else {
        r[0] = cvt_fp4_bf16<2 * HALF>(a, 2.0f);
        r[1] = cvt_fp4_bf16<2 * HALF>(b, 2.0f);
        r[2] = cvt_fp4_bf16<2 * HALF + 1>(a, 2.0f);
        r[3] = cvt_fp4_bf16<2 * HALF + 1>(b, 2.0f);
    }
    return r;
}

// Q3 operand holding q - 4 for the 8 codes of block J (lane's lo dword J/2,
// the lane's third-bit word H).  The third bits are stored so that bit
// 4 n + 2 (J/2) of H belongs to the code whose low bits sit in nibble n of
// (lo & 0x33333333) and bit 4 n + 2 (J/2) + 1 to nibble n of
// ((lo >> 2) & 0x33333333).  A low-bits nibble A (0..3) then becomes the
// fp4 (e2m1) code of (q - 4) / 2: A itself when the third bit is set
// (q - 4 = A), 12 - A when it is clear (sign bit and magnitude 4 - A:
// q - 4 = A - 4), so one conversion with scale 2 gives q - 4 exactly.
template <int J, bool F16>
__device__ __forceinline__ u32x4 q3_operand(uint32_t dw, uint32_t H) {
    constexpr int D = J >> 1, HALF = J & 1;
    const uint32_t a = dw & 0x33333333u, b = (dw >> 2) & 0x33333333u;
    const uint32_t ha = (H >> (2 * D)) & 0x11111111u, hb = (H >> (2 * D + 1)) & 0x11111111u;
    const uint32_t ma = (ha << 4) - ha, mb = (hb << 4) - hb;   // 0xF where the third bit is set
    const uint32_t na = (a & ma) | ((0xCCCCCCCCu - a) & ~ma);
    const uint32_t nb = (b & mb) | ((0xCCCCCCCCu - b) & ~mb);
    u32x4 r;
    if constexpr (F16) {
        r[0] = cvt_fp4_f16<2 * HALF>(na, 2.0f);
        r[1] = cvt_fp4_f16<2 * HALF>(nb, 2.0f);
        r[2] = cvt_fp4_f16<2 * HALF + 1>(na, 2.0f);
        r[3] = cvt_fp4_f16<2 * HALF + 1>(nb, 2.0f);
    } else {
        r[0] = cvt_fp4_bf16<2 * HALF>(na, 2.0f);
        r[1] = cvt_fp4_bf16<2 * HALF>(nb, 2.0f);
        r[2] = cvt_fp4_bf16<2 * HALF + 1>(na, 2.0f);
        r[3] = cvt_fp4_bf16<2 * HALF + 1>(nb, 2.0f);
    }
    return r;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// 64 lanes x 16 bytes from global memory straight into LDS [dst, dst + 1 KiB),
// lane l's bytes at dst + 16 l.
__device__ __forceinline__ void copy_to_lds16(const void *src, void *dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt left alone)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier that waits for nothing itself.  __syncthreads() makes the
// compiler drain every outstanding vector-memory operation first (vmcnt(0))
// when global->LDS copies are in flight, which empties a multi-stage copy
// pipeline at each step.  Callers wait for exactly what the other waves must
// see (wait_vm<N>: their own copies into the stage about to be read) and then
// meet here; the memory clobber keeps the compiler from moving LDS or global
// accesses across the barrier.  Each wave's reads of a stage are consumed by
// its own matrix ops before it arrives, so a stage that is refilled after the
// barrier has no reads pending.
__device__ __forceinline__ void wg_barrier() { __asm__ volatile("s_barrier" ::: "memory"); }
// A barrier over LDS only: this wave's LDS accesses complete, then meet.  For
// a block that has global stores (or loads) in flight that no other thread
// reads back, where __syncthreads() would wait for them all first.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    wg_barrier();
}

// Locate the group handled by `slot`: slot 0 = shared expert (rows 0..T-1 in
// token order), slot s >= 1 = the (s-1)-th expert with a non-empty segment.
// Executed by one wave; all lanes get the result.  Returns false if the slot
// has no group.
struct Group {
    int expert;     // -1 = shared
    int row0;       // first row in the expert-sorted pair order (routed) or 0
    int nrows;
    int hrow0;      // first row of this group in the h scratch buffer
};

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int l = __lane_id();
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int t = __shfl_up(v, o, 64);
        if (l >= o) v += t;
    }
    return v;
}

// The n-th (0-based) set bit of a 64-bit mask (wave-uniform), -1 if none.
__device__ __forceinline__ int nth_set_bit(unsigned long long m, int n) {
    int base = 0;
#pragma unroll
    for (int w = 32; w >= 1; w >>= 1) {
        const unsigned long long lo = m & ((1ull << w) - 1ull);
        const int c = __popcll(lo);
        if (n >= c) {
            n -= c;
            m >>= w;
            base += w;
        } else {
            m = lo;
        }
    }
    return (m & 1ull) && n == 0 ? base : -1;
}

// Expert e is non-empty iff offsets[e+1] > offsets[e].  Lane l looks at
// experts l, l+64, ...; all loads are issued before any is used.  One ballot
// per row of 64 experts counts the non-empty ones in index order; the row
// holding the target is kept and its set bit located once at the end.
__device__ inline bool find_group(const int32_t *__restrict__ offsets, int E, int T, int P, int slot,
                                  Group &g) {
    if (slot == 0) {
        g.expert = -1;
        g.row0 = 0;
        g.nrows = T;
        g.hrow0 = P;
        return T > 0;
    }
    const int target = slot - 1;  // index among non-empty experts
    const int l = __lane_id();
    const int per = (E + 63) / 64;  // <= 16
    // One round trip: lane l loads the start and end offsets of experts
    // l + 64 i (unconditional loads at clamped indices: a predicated load
    // would be waited for inside its own branch; past E both read offsets[E],
    // an empty range).  Plain loads: every workgroup of a launch reads the
    // same offsets, so all but the first on each XCD hit its L2.
    int lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = l + 64 * i;
        lo[i] = offsets[e < E ? e : E];
        hi[i] = offsets[e < E ? e + 1 : E];
    }
    int cum = 0, sel_row = -1, sel_n = 0;
    unsigned long long sel_m = 0ull;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i < per) {
            const unsigned long long m = __ballot(hi[i] > lo[i]);
            const int c = __popcll(m);
            const bool hit = sel_row < 0 && target < cum + c;
            sel_m = hit ? m : sel_m;
            sel_n = hit ? target - cum : sel_n;
            sel_row = hit ? i : sel_row;
            cum += c;
        }
    }
    if (sel_row < 0) return false;
    const int bit = nth_set_bit(sel_m, sel_n);
    // start and end of the found expert: lane `bit` of row sel_row holds them
    int a = lo[0], b = hi[0];
#pragma unroll
    for (int i = 1; i < 16; ++i)
        if (i == sel_row) {
            a = lo[i];
            b = hi[i];
        }
    const int row0 = __builtin_amdgcn_readlane(a, bit);
    const int end = __builtin_amdgcn_readlane(b, bit);
    g.expert = 64 * sel_row + bit;
    g.row0 = row0;
    g.nrows = end - row0;
    g.hrow0 = row0;
    return true;
}

// silu(g) * u * 2^-2a in fp32, as (g 2^-a) / (1 + e^-g) * (u 2^-a): the
// power-of-two scalings are exact, so this is silu(g) * u scaled, and it
// stays finite for any g, u whose scaled product fits
__device__ __forceinline__ float swiglu(float g, float u, int a) {
    return ldexpf(g, -a) / (1.0f + __expf(-g)) * ldexpf(u, -a);
}

// ---------------------------------------------------------------- launchers
// (defined in the .hip files; return hipError_t of the launch)
// offsets, sorted_pair, pair_pos (all or none): also list the pairs by expert
// (T <= kRouteTile and k <= 64 only)
hipError_t launch_route_small(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, int k, int32_t *ids, float *w, void *ws,
                              hipStream_t s, int32_t *offsets = nullptr, int32_t *sorted_pair = nullptr,
                              int32_t *pair_pos = nullptr, int tail_from = -1);
hipError_t launch_router_gemm(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, void *ws, hipStream_t s);
size_t router_gemm_ws_bytes(int d, int E);
constexpr int kRouteSmallTMax = 128;   // T above this: router GEMM + top-k kernel
constexpr int kWaveTopkMaxK = 64;      // register top-k (one wave per token) up to this k
static_assert(kRouteSmallTMax / kRouteTile * kCntLine * 4 <= 2048, "tile counters run into the error word");
hipError_t launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w,
                       hipStream_t s);
size_t route_ws_bytes(int d, int E, int T);

// tail_from >= k: every pair; tail_from < k: route tail-skip
hipError_t launch_dispatch(const int32_t *ids, int T, int E, int k, int tail_from, int32_t *offsets,
                           int32_t *sorted_pair, int32_t *pair_pos, void *ws, hipStream_t s);
size_t dispatch_ws_bytes(int E, int T, int k);

// Which experts an FFN launch computes: the routed groups, the shared
// expert, or both.  Without the routed part offsets, sorted_pair and y_pairs
// are not read (they may be null) and k may be 0; without the shared part
// y_shared is not written.
constexpr int kFfnRouted = 1, kFfnShared = 2, kFfnBoth = 3;

// With out given (parts = both), the down kernel also writes moe_combine's
// out from pair_pos and topk_w, bit-identical to a separate combine.
hipError_t launch_ffn_small(const moe_layer &L, const uint16_t *x, int T, int k,
                            const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                            float *y_shared, void *ws, int parts, hipStream_t s,
                            const int32_t *pair_pos = nullptr, const float *topk_w = nullptr,
                            float *out = nullptr);
size_t ffn_small_ws_bytes(int d, int f, int E, int T, int k);
constexpr int kSmallTMax = 16;   // above: the grouped matrix-core path
// moe_expert_ffn_combine fuses the merge into the down kernel up to this
// batch (per layer, measured: T = 1 and 4 gain 0.8 and 0.4 us; T = 8 and 16
// lose, the merge taking longer with more arriving workgroups per tile)
constexpr int kFuseCombineTMax = 4;

hipError_t launch_ffn_prefill(const moe_layer &L, const uint16_t *x, int T, int k,
                              const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                              float *y_shared, void *ws, int parts, hipStream_t s);
size_t ffn_prefill_ws_bytes(int d, int f, int E, int T, int k);
// the same grouped GEMM built for mid-size batches (64-row items, two
// workgroups per compute unit)
hipError_t launch_ffn_prefill_mid(const moe_layer &L, const uint16_t *x, int T, int k,
                                  const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                                  float *y_shared, void *ws, int parts, hipStream_t s);
size_t ffn_prefill_mid_ws_bytes(int d, int f, int E, int T, int k);
constexpr int kPfMidTMax = 2048;   // T above this: the large-chunk build

hipError_t launch_combine(const float *y_pairs, const float *y_shared, const int32_t *pair_pos,
                          const float *w, int T, int k, int d, float *out, hipStream_t s);

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);

}  // namespace moe
