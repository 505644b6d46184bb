// ffn_prefill.hip -- expert FFN for large token batches (prompt chunks).
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 …", section
// "긴 프롬프트와 긴 컨텍스트 처리": prompts are read in chunks of up to 8,192
// tokens; section "Strata의 동작 원리": each token uses 10 of 512 routed experts
// plus the shared expert; [guide] tech.okbari.net "Strata와 Qwen3.8-Flash-Next…",
// section "24GB에 들어가는 원리": a wide batch touches many experts at once.
//
// Grouped GEMM on the matrix cores (v_mfma_f32_32x32x16_f16, fp32 accumulate):
//   gate/up:  [rows of group g] x d  .  (W_gate_g | W_up_g)^T   -> h = silu(g)*u
//   down:     [rows of group g] x f  .  W_down_g^T              -> y (fp32)
//
// Scheduling.  A prepass turns the dispatch offsets into work items (group,
// chunk of up to 192 rows) on the device: groups are ordered by work, largest first
// (the shared expert counts double: it runs two products per weight), and
// dealt round-robin to the eight XCDs, so all chunks of one expert -- which
// share its weights -- and all column tiles of one chunk -- which share its
// activation rows -- land in one XCD's L2.  The GEMM kernels are persistent:
// each workgroup takes (item, column tile) units by atomic ticket from its own
// XCD's queue, largest first, then steals from the other queues once its own
// is empty.  An expert with thousands of rows is just many units; a skewed
// router costs no idle tail beyond one unit.
//
// Operands:
//   A (activations): x converted once to fp16 after an exact power-of-two
//     scaling per token row (x * 2^-a, 2^a <= max|x_row| < 2^(a+1)), so any
//     bf16 row fits fp16's range; or h, stored as h * 2^-2a.  The gate/up
//     epilogue takes the true gate value back (2^a times its accumulator)
//     for the sigmoid, and the down epilogue multiplies y by 2^2a: both
//     exact, so the scaling changes no result beyond fp16's subnormal range.
//     Each 192-row x 128-column stage is copied global -> LDS
//     by the direct-to-LDS loads (no registers), two stages in flight; the
//     16-byte chunks of a row are XOR-swizzled by the row index so the
//     fragment reads are free of bank conflicts.
//   B (weights): never touch LDS.  Two 16-row storage units give each lane the
//     bytes of its 32x32x16 B fragments (two 8-byte code slots per unit pair
//     and step); the lane turns codes into fp16 with the fp4 convert and
//     applies the block scale with one packed fp16 FMA per two weights:
//     fp16(d*q + m) rounded once (Q3: fp16(d*(q-4))).  Dequantisation for the
//     next 16-column k-step overlaps the matrix ops of the current one.
// Precision: routed experts use the fp16-rounded weights and fp16 h; the
// shared expert (weight 1 in every token's output) uses exact weights as fp16
// hi + lo and h as fp16 hi + lo (the product lo*lo, below 2^-22 relative, is
// dropped).  Max |err| / rms(out) stays near 1.1e-3 on these workloads.
#include "common.h"

// The file is built twice.  The default build serves large chunks: 192-row
// work items, one GEMM workgroup per compute unit.  With MOE_PF_MID it serves
// mid-size batches (up to a few thousand tokens, where the matrix work per
// weight byte is small): 64-row items and two workgroups per compute unit,
// so twice the weight loads are in flight.  Each build keeps its kernels in a
// namespace of its own.
#ifdef MOE_PF_MID
#define MOE_PF_ROWS 64
#define MOE_PF_OCC 2
#define MOE_PF_NS pf_mid
#define MOE_PF_LAUNCH launch_ffn_prefill_mid
#define MOE_PF_WS ffn_prefill_mid_ws_bytes
#else
#define MOE_PF_ROWS 192
#define MOE_PF_OCC 1
#define MOE_PF_NS pf_big
#define MOE_PF_LAUNCH launch_ffn_prefill
#define MOE_PF_WS ffn_prefill_ws_bytes
#endif

namespace moe {
namespace MOE_PF_NS {

constexpr int PF_MT = MOE_PF_ROWS;                // rows per work item (multiple of 64, <= 192)
constexpr int PF_KS = 128;                        // K per pipeline stage
constexpr int PF_STAGE = PF_MT * PF_KS * 2;       // bytes of one A stage
constexpr int PF_NSTAGE = 3;                      // A stages in flight
static_assert(PF_MT % 64 == 0 && PF_MT <= 192, "item rows: a multiple of 64, at most 192");
constexpr int PF_NXCD = 8;                        // XCDs (L2 domains) per device
constexpr int PF_SORT = 2048;                     // sort slots, >= E + 1

struct PfItem {
    int32_t expert;  // -1 = shared
    int32_t row0;    // first row (sorted position, or token for the shared expert)
    int32_t nrows;
    int32_t hrow0;   // first row in the h buffer
};

// Scheduling block at the head of the prefill workspace.
struct PfSched {
    int32_t n_items;
    int32_t xq[PF_NXCD + 1];         // items of XCD x: [xq[x], xq[x + 1])
    int32_t ticket[2][PF_NXCD];      // per GEMM launch, per XCD queue
};
static_assert(sizeof(PfSched) <= 256, "PfSched must fit its 256-byte slot");
static_assert(sizeof(PfItem) == 16, "items are read as one 16-byte vector");

// ---------------------------------------------------------------- prepass
// One block of 1024 threads.  Group 0 is the shared expert (T rows), group
// 1 + e the routed expert e.  Sort key: (work desc, group asc), work = rows
// (x2 for the shared expert); bitonic sort in LDS over the next power of two
// >= E + 1 slots (at most PF_SORT).
__device__ __forceinline__ void build_items_block(const int32_t *__restrict__ offsets, int E, int T, int P,
                                                  int parts, PfItem *__restrict__ items,
                                                  PfSched *__restrict__ sched) {
    __shared__ unsigned long long key[PF_SORT];
    __shared__ int start[PF_SORT / PF_NXCD * PF_NXCD];
    __shared__ int xcount[PF_NXCD];
    __shared__ int g_rows[PF_SORT], g_row0[PF_SORT];   // per group, read from offsets once
    const int tid = threadIdx.x, lane = __lane_id(), wv = tid >> 6;
    const int G = E + 1;
    int NS = 128;                 // sort width: a power of two >= G (at least 128)
    while (NS < G) NS <<= 1;
    for (int g = tid; g < PF_SORT; g += 1024) {
        unsigned long long kk = 0;
        int rows = 0, r0 = 0;
        if (g == 0 ? (parts & kFfnShared) != 0 : g < G && (parts & kFfnRouted) != 0) {
            r0 = g == 0 ? 0 : offsets[g - 1];
            rows = g == 0 ? T : offsets[g] - r0;
            const unsigned long long work = g == 0 ? 2ull * rows : (unsigned long long)rows;
            if (rows > 0) kk = (work << 11) | (unsigned long long)(2047 - g);
        }
        key[g] = kk;
        g_rows[g] = rows;
        g_row0[g] = r0;
    }
    __syncthreads();
    // bitonic sort, descending.  With stride <= 64 the pairs of wave w lie in
    // its own keys [128 w, 128 w + 128); between two such stages a wave only
    // orders its own LDS accesses, and a block barrier is needed only where
    // this stage or the next crosses waves (and after the last).
    for (int size = 2; size <= NS; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (tid < NS / 2) {
                const int i = 2 * tid - (tid & (stride - 1));   // lower index of this thread's pair
                const int j = i + stride;
                const bool desc = ((i & size) == 0);
                const unsigned long long a = key[i], b = key[j];
                if ((a < b) == desc) {
                    key[i] = b;
                    key[j] = a;
                }
            }
            const bool cross = stride > 64 || (stride == 1 && (size > 64 || size == NS));
            if (cross)
                __syncthreads();
            else
                __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
    }
    // rank r -> XCD r % 8, position r / 8; per-XCD exclusive scan of chunk counts
    auto nch_of = [&](int r) -> int {
        const unsigned long long kk = key[r];
        if (kk == 0) return 0;
        const int g = 2047 - (int)(kk & 2047);
        return (g_rows[g] + PF_MT - 1) / PF_MT;
    };
    if (wv < PF_NXCD) {
        int carry = 0;
        for (int c = 0; c * 64 * PF_NXCD < NS; ++c) {
            const int r = (c * 64 + lane) * PF_NXCD + wv;
            const int v = r < NS ? nch_of(r) : 0;
            const int incl = wave_incl_scan(v) + carry;
            if (r < NS) start[r] = incl - v;
            carry = __shfl(incl, 63);
        }
        if (lane == 0) xcount[wv] = carry;
    }
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int x = 0; x < PF_NXCD; ++x) {
            sched->xq[x] = acc;
            acc += xcount[x];
        }
        sched->xq[PF_NXCD] = acc;
        sched->n_items = acc;
    }
    if (tid < 2 * PF_NXCD) sched->ticket[tid / PF_NXCD][tid % PF_NXCD] = 0;
    int xbase[PF_NXCD];
    {
        int acc = 0;
#pragma unroll
        for (int x = 0; x < PF_NXCD; ++x) {
            xbase[x] = acc;
            acc += xcount[x];
        }
    }
    for (int r = tid; r < NS; r += 1024) {
        const unsigned long long kk = key[r];
        if (kk == 0) continue;
        const int g = 2047 - (int)(kk & 2047);
        const int rows = g_rows[g];
        const int r0 = g_row0[g];
        const int nch = (rows + PF_MT - 1) / PF_MT;
        const int base = xbase[r % PF_NXCD] + start[r];
        for (int c = 0; c < nch; ++c) {
            const int n = rows - c * PF_MT < PF_MT ? rows - c * PF_MT : PF_MT;
            items[base + c] = g == 0 ? PfItem{-1, c * PF_MT, n, P + c * PF_MT}
                                     : PfItem{g - 1, r0 + c * PF_MT, n, r0 + c * PF_MT};
        }
    }
}

// The two prepasses in one launch: block 0 builds the work items, the other
// blocks convert x to fp16, one wave per token row: a = the exponent of the
// row's largest magnitude (0 for a zero row) goes to xexp[t], and the row is
// stored as fp16(x * 2^-a), so its largest value lies in [1, 2).
__global__ __launch_bounds__(1024) void pf_prep_kernel(const int32_t *__restrict__ offsets, int E, int T,
                                                       int P, int parts, PfItem *__restrict__ items,
                                                       PfSched *__restrict__ sched,
                                                       const uint16_t *__restrict__ x,
                                                       uint16_t *__restrict__ x16, int32_t *__restrict__ xexp,
                                                       int d) {
    if (blockIdx.x == 0) {
        build_items_block(offsets, E, T, P, parts, items, sched);
        return;
    }
    const int wv = threadIdx.x >> 6, lane = __lane_id();
    const int cpr = d / 8;   // 16-byte chunks per row
    for (int t = (blockIdx.x - 1) * 16 + wv; t < T; t += (gridDim.x - 1) * 16) {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (size_t)t * d);
        u32x4 *dst = reinterpret_cast<u32x4 *>(x16 + (size_t)t * d);
        uint32_t mx = 0u;   // largest magnitude, as bf16 bits without the sign
        for (int c = lane; c < cpr; c += 64) {
            const u32x4 v = src[c];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t lo = v[q] & 0x7fffu, hi = (v[q] >> 16) & 0x7fffu;
                mx = lo > mx ? lo : mx;
                mx = hi > mx ? hi : mx;
            }
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t u = (uint32_t)__shfl_xor((int)mx, o, 64);
            mx = u > mx ? u : mx;
        }
        // exponent field of the largest magnitude (0: zero or subnormal)
        const int ef = (int)(mx >> 7);
        const int a = mx == 0u ? 0 : (ef == 0 ? -126 : ef - 127);
        if (lane == 0) xexp[t] = a;
        for (int c = lane; c < cpr; c += 64) {
            const u32x4 v = src[c];   // the row's second read: cached
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = ldexpf(__uint_as_float(v[q] << 16), -a);
                const float hi = ldexpf(__uint_as_float(v[q] & 0xffff0000u), -a);
                const _Float16 hl = static_cast<_Float16>(lo), hh = static_cast<_Float16>(hi);
                o[q] = (uint32_t)__builtin_bit_cast(uint16_t, hl) | ((uint32_t)__builtin_bit_cast(uint16_t, hh) << 16);
            }
            dst[c] = o;
        }
    }
}

// ------------------------------------------------------------ B fragments
// Code bytes of one lane for one storage unit and one 16-column k-step pair:
// a storage unit holds, for lane slot (g, rr), row rr's codes at columns
// 32j + 8g .. +8 of each 32-block j (8 bytes); the sub-block scales/mins of
// row rr; and for Q3 one word of third bits.
template <int FMT>
struct BRaw {
    u32x2 lo;
    uint32_t hi;
    u32x2 sc, mn;
};

__device__ __forceinline__ uint32_t half_pair(const u32x2 &v, int j) {
    const uint32_t h = (v[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    return h | (h << 16);
}

// One packed fp16 FMA, a*b + c rounded once per half.
__device__ __forceinline__ uint32_t pk_fma_f16(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    __asm__("v_pk_fma_f16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// fp16(w) for the 8 weights of block J (rounded once).
template <int FMT, int J>
__device__ __forceinline__ u32x4 bfrag_f16(const BRaw<FMT> &b) {
    const uint32_t d = half_pair(b.sc, J);
    u32x4 r;
    if constexpr (FMT == MOE_FMT_Q2_B32) {
        const u32x4 q = lo_operand<J & 1, true>(b.lo[J >> 1]);   // exact codes 0..3 as fp16
        const uint32_t m = half_pair(b.mn, J);
        r.x = pk_fma_f16(q.x, d, m);
        r.y = pk_fma_f16(q.y, d, m);
        r.z = pk_fma_f16(q.z, d, m);
        r.w = pk_fma_f16(q.w, d, m);
    } else {
        const u32x4 q = q3_operand<J, true>(b.lo[J >> 1], b.hi);   // exact q - 4 as fp16
        r.x = pk_fma_f16(q.x, d, 0u);
        r.y = pk_fma_f16(q.y, d, 0u);
        r.z = pk_fma_f16(q.z, d, 0u);
        r.w = pk_fma_f16(q.w, d, 0u);
    }
    return r;
}

// exact weights split as fp16 hi + lo: w = fp32(d*q + m) (exact), hi = fp16(w),
// lo = fp16(w - hi).  qword holds two fp16 codes (Q3: q - 4, with m = 0).
// Exact weights split into fp16 hi + lo.  hi = fp16(d*q + m) is one packed
// fp16 FMA (one rounding).  lo = fp16(w - hi) with w = d*q + m from a
// mixed-precision FMA on the fp16 inputs, exact in fp32 for block-32 codes
// and fp16 scales; w - hi is exact in fp32 too.  For the second pass of the
// shared down projection lo is zeroed: d and m are scaled by s = 0 (exact) and
// the residual is -hi*s + w*s.
template <int SEL>
__device__ __forceinline__ float fma_mix_f32(uint32_t q2, uint32_t d2, uint32_t m2) {
    float r;
    if constexpr (SEL == 0)
        __asm__("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,1,1]" : "=v"(r) : "v"(q2), "v"(d2), "v"(m2));
    else
        __asm__("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,1,1]" : "=v"(r) : "v"(q2), "v"(d2), "v"(m2));
    return r;
}
// fp16 pair (fp16(w0s - hi.lo * s), fp16(w1s - hi.hi * s))
__device__ __forceinline__ uint32_t residual_pair(uint32_t hi2, float w0s, float w1s, float s) {
    uint32_t r = 0;
    __asm__("v_fma_mixlo_f16 %0, -%1, %2, %3 op_sel_hi:[1,0,0]" : "+v"(r) : "v"(hi2), "v"(s), "v"(w0s));
    __asm__("v_fma_mixhi_f16 %0, -%1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(r) : "v"(hi2), "v"(s), "v"(w1s));
    return r;
}

// exact weights of block J as fp16 hi + lo (lo multiplied by lo_scale, 1 or 0)
template <int FMT, int J>
__device__ __forceinline__ void bfrag_split(const BRaw<FMT> &b, float lo_scale, u32x4 &hi, u32x4 &lo) {
    const uint32_t d = half_pair(b.sc, J);
    u32x4 q;
    uint32_t m;
    if constexpr (FMT == MOE_FMT_Q3_B32) {
        q = q3_operand<J, true>(b.lo[J >> 1], b.hi);   // q - 4: w = d (q - 4)
        m = 0u;
    } else {
        q = lo_operand<J & 1, true>(b.lo[J >> 1]);
        m = half_pair(b.mn, J);
    }
    const uint32_t s2 = lo_scale != 0.f ? 0x3C003C00u : 0u;   // (s, s) in fp16
    const uint32_t ds = pk_fma_f16(d, s2, 0u), ms = pk_fma_f16(m, s2, 0u);
    uint32_t hv[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t qi = i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
        hv[i] = pk_fma_f16(qi, d, m);
        lv[i] = residual_pair(hv[i], fma_mix_f32<0>(qi, ds, ms), fma_mix_f32<1>(qi, ds, ms), lo_scale);
    }
    hi = u32x4{hv[0], hv[1], hv[2], hv[3]};
    lo = u32x4{lv[0], lv[1], lv[2], lv[3]};
}

// Fragment of 32-block J from one code slot: fp16-rounded weights (routed),
// or exact weights as fp16 hi + lo (shared expert; lo scaled by lo_scale).
template <int FMT, bool SPLIT>
__device__ __forceinline__ void frag_j(const BRaw<FMT> &b, int J, float lo_scale, u32x4 &hi, u32x4 &lo) {
    if constexpr (SPLIT) {
        switch (J) {
            case 0: bfrag_split<FMT, 0>(b, lo_scale, hi, lo); break;
            case 1: bfrag_split<FMT, 1>(b, lo_scale, hi, lo); break;
            case 2: bfrag_split<FMT, 2>(b, lo_scale, hi, lo); break;
            default: bfrag_split<FMT, 3>(b, lo_scale, hi, lo); break;
        }
    } else {
        switch (J) {
            case 0: hi = bfrag_f16<FMT, 0>(b); break;
            case 1: hi = bfrag_f16<FMT, 1>(b); break;
            case 2: hi = bfrag_f16<FMT, 2>(b); break;
            default: hi = bfrag_f16<FMT, 3>(b); break;
        }
    }
}

__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

struct PfGemmArgs {
    QMatDev w0, w1;            // routed experts: gate, up (gate/up) or down (down)
    QMatDev s0, s1;            // shared expert, same roles
    const PfItem *items;
    PfSched *sched;
    const int32_t *xexp;       // per token: x row scaled by 2^-xexp, h rows by 2^-2xexp
    const uint16_t *a_hi;      // gate/up: x as fp16 [T][d]; down: h [(P + T)][f]
    const uint16_t *a_lo;      // down: h_lo [T][f] (shared rows)
    const int32_t *sorted_pair;
    uint16_t *h_out;           // [(P + T)][f]
    uint16_t *h_lo_out;        // [T][f]
    float *y_pairs, *y_shared;
    int k, d, f, nt, launch;
};

// Tile geometry.  A unit is PF_MT rows x (4 waves x NTW n-tiles of 32 weight
// rows), all of K; one workgroup per CU (up to 256 + 256 registers per lane)
// with three A stages.  Accumulators: PF_MT / 32 m-tiles x NTW n-tiles x 16.
//   gate/up: a wave owns HCOLS = 16 NTW h columns (NTW/2 gate + NTW/2 up
//   n-tiles); down: OCOLS = 32 NTW outputs.
#ifndef MOE_PF_NTW
#define MOE_PF_NTW 2
#endif
template <int NTW, int NW>
struct PfGeom {
    static constexpr int NI = PF_MT / (4 * NW);     // A copy instructions per wave per stage
    static_assert(NI * 4 * NW == PF_MT, "a stage's rows split evenly over the waves");
    static constexpr int HCOLS = 16 * NTW;          // gate/up: h columns per wave
    static constexpr int OCOLS = 32 * NTW;          // down: output columns per wave
    // epilogue staging per wave (in the A stages); pitches put rows 4 apart
    // (the two half-waves) in different banks
    static constexpr int EP0_PITCH = HCOLS + 8;     // [gate | up][32][EP0_PITCH] floats
    static constexpr int EP0H_PITCH = HCOLS + 8;    // gate/up: [h | h_lo][32][EP0H_PITCH] halves
    static constexpr int EP1_PITCH = OCOLS + 8;     // [32][EP1_PITCH] floats
    static constexpr int EP_WAVE = (2 * 32 * EP0_PITCH > 32 * EP1_PITCH ? 2 * 32 * EP0_PITCH : 32 * EP1_PITCH) * 4;
    static_assert(NW * EP_WAVE <= PF_NSTAGE * PF_STAGE, "epilogue staging must fit in the A stages");
    // sub-steps that issue the next stages' loads: weights in [0, NBS), A
    // copies (two per sub-step) in [NBS, NBS + NI / 2)
    static constexpr int NBS = NTW / 2 > 0 ? NTW / 2 : 1;
    static_assert(NBS + NI / 2 <= 8 && NI % 2 == 0, "loads must fit in the eight sub-steps");
};
constexpr int kPfNtw = MOE_PF_NTW;
// down: waves per workgroup and 32-column n-tiles per wave
#ifndef MOE_PF_DOWN_NW
#if MOE_PF_OCC == 1
#define MOE_PF_DOWN_NW 8
#else
#define MOE_PF_DOWN_NW 4
#endif
#endif
constexpr int kPfDownNw = MOE_PF_DOWN_NW;
constexpr int kPfDownNtw = kPfDownNw == 8 ? 1 : kPfNtw;
// gate/up: eight waves of one n-tile (gate or up rows) or four of two
#ifndef MOE_PF_GU_NW
#if MOE_PF_OCC == 1
#define MOE_PF_GU_NW 8
#else
#define MOE_PF_GU_NW 4
#endif
#endif
constexpr int kPfGuNw = MOE_PF_GU_NW;
constexpr int kPfGuNtw = kPfGuNw == 8 ? 1 : kPfNtw;

// silu(g) * u * 2^-2a from the accumulators g_a = g * 2^-a, u_a = u * 2^-a:
// g_a * sigmoid(g) * u_a, the sigmoid taken at the true g = g_a * 2^a, with
// the hardware reciprocal (about 1 ulp); h is rounded to fp16 right after
__device__ __forceinline__ float swiglu_scaled(float ga, float ua, int a) {
    return ga * __builtin_amdgcn_rcpf(1.0f + __expf(-ldexpf(ga, a))) * ua;
}

// One unit: the rows of one item x one column tile, all of K.
// MODE 0 (gate/up, K = d): wave w owns h columns c0 = tile * 4 HCOLS + w HCOLS
//   .. +HCOLS; n-tiles 0 .. NTW/2 - 1 are those gate rows, the rest the same
//   up rows, so each SwiGLU pair sits in one lane and register.
// MODE 1 (down, K = f): wave w owns outputs tile * 4 OCOLS + w OCOLS .. +OCOLS.
// A wave's columns are all in range or all past the end (d, f are multiples
// of 128); past the end it reads the last valid weights and stores nothing.
// SH (shared expert): exact weights as hi + lo.  For MODE 1 the K loop runs
//   twice: A = h_hi with B hi and lo, then A = h_lo with B hi.
// MT: 32-row m-tiles that hold rows of the item (1..4).
template <int FMT, int MODE, bool SH, int MT, int NTW, int NW>
__device__ __forceinline__ void pf_unit(const PfGemmArgs &a, const PfItem &item, int tile,
                                        uint8_t *As, int *s_row, int *s_exp, const PfItem *pf_items,
                                        int *pf_ticket, int &pf_t, int pf_n, PfItem *pf_dst) {
    using G = PfGeom<NTW, NW>;
    constexpr int PF_NI = G::NI;
    // gate/up with eight waves, one n-tile each: waves 0-3 hold gate rows,
    // waves 4-7 the up rows of the same 32 h columns (pair wv & 3)
    constexpr bool GU8 = MODE == 0 && NW == 8;
    static_assert(!GU8 || NTW == 1, "eight gate/up waves take one n-tile each");
    const int tid = threadIdx.x, l = __lane_id();
    const int wv = wave_uniform(tid >> 6);
    const int h = l >> 5, uu = (l >> 4) & 1, rr = l & 15;
    const int K = MODE == 0 ? a.d : a.f;
    const int KC = K / PF_KS;
    const int NSTEP = (MODE == 1 && SH) ? 2 * KC : KC;
    const int nrows = item.nrows;
    const int e = SH ? 0 : item.expert;

    // B: storage-unit index (at kc = 0) of this lane's unit in n-tile n
    const QMatDev W0 = SH ? a.s0 : a.w0;
    const QMatDev W1 = SH ? a.s1 : a.w1;
    size_t ub[NTW];
    bool cols_valid;
    if constexpr (GU8) {
        const int rpe = a.f / 16;
        const int c0 = tile * 4 * 32 + (wv & 3) * 32;
        cols_valid = c0 < a.f;
        int t16 = c0 / 16 + uu;
        t16 = t16 < rpe ? t16 : rpe - 1;
        ub[0] = ((size_t)e * rpe + t16) * KC;
    } else if constexpr (MODE == 0) {
        const int rpe = a.f / 16;
        const int c0 = tile * NW * G::HCOLS + wv * G::HCOLS;
        cols_valid = c0 < a.f;
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            int t16 = (c0 + 32 * (n % (NTW / 2))) / 16 + uu;
            t16 = t16 < rpe ? t16 : rpe - 1;
            ub[n] = ((size_t)e * rpe + t16) * KC;
        }
    } else {
        const int rpe = a.d / 16;
        const int c0 = tile * NW * G::OCOLS + wv * G::OCOLS;
        cols_valid = c0 < a.d;
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            int t16 = (c0 + 32 * n) / 16 + uu;
            t16 = t16 < rpe ? t16 : rpe - 1;
            ub[n] = ((size_t)e * rpe + t16) * KC;
        }
    }
    // slot 0 = (h, rr) -> columns 32j + 8h; slot 1 = (2 + h, rr) -> 32j + 16 + 8h
    auto load_b_tile = [&](BRaw<FMT> (&br)[NTW][2], int kc, int n) {
        const QMatDev &W = (MODE == 0 && (GU8 ? wv >= 4 : n >= NTW / 2)) ? W1 : W0;
        const size_t u = ub[n] + kc;
        const uint8_t *lo = W.lo + u * 512;
        // a routed expert's weights are mostly read by one item: nontemporal
        // (the shared expert's are re-read by every item: cached)
        auto ld = [&](const auto *p) { return SH ? *p : __builtin_nontemporal_load(p); };
        br[n][0].lo = ld(reinterpret_cast<const u32x2 *>(lo + (h * 16 + rr) * 8));
        br[n][1].lo = ld(reinterpret_cast<const u32x2 *>(lo + ((2 + h) * 16 + rr) * 8));
        if constexpr (FMT == MOE_FMT_Q3_B32) {
            const uint8_t *hp = W.hi + u * 256;
            br[n][0].hi = ld(reinterpret_cast<const uint32_t *>(hp + (h * 16 + rr) * 4));
            br[n][1].hi = ld(reinterpret_cast<const uint32_t *>(hp + ((2 + h) * 16 + rr) * 4));
        }
        const u32x2 sc = ld(reinterpret_cast<const u32x2 *>(W.scale + u * 64 + rr * 4));
        br[n][0].sc = sc;
        br[n][1].sc = sc;
        if constexpr (FMT == MOE_FMT_Q2_B32) {
            const u32x2 mn = ld(reinterpret_cast<const u32x2 *>(W.min + u * 64 + rr * 4));
            br[n][0].mn = mn;
            br[n][1].mn = mn;
        }
    };

    BRaw<FMT> bcur[NTW][2], bnext[NTW][2];
    // source row (token, or h row) of each tile row; rows past the item's
    // end repeat its last row and are never stored.  The first step's
    // weights are loaded right after the pair lookup and before its use, so
    // their latency runs under the lookup, the barrier and the A copies.
    int src = 0, tok = 0;
    if (tid < PF_MT) {
        const int r = tid < nrows ? tid : nrows - 1;
        tok = SH ? item.row0 + r : a.sorted_pair[item.row0 + r] / a.k;
        if constexpr (MODE == 0)
            src = tok;
        else
            src = item.hrow0 + r;
    }
#pragma unroll
    for (int n = 0; n < NTW; ++n) load_b_tile(bcur, 0, n);
    if (tid < PF_MT) s_row[tid] = src;
    // the row's power-of-two exponent, used in the epilogue (loaded now, its
    // latency runs under the K loop)
    const int rexp = tid < PF_MT ? a.xexp[tok] : 0;
    // LDS only: the previous unit's output stores may still be in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    wg_barrier();

    // A copy slots of this lane: instruction i covers tile rows 4 (NI wv + i)
    // .. +4; lane l takes row R = 4 (NI wv + i) + l / 16 and stores physical
    // chunk l % 16, which holds logical chunk (l % 16) ^ (R % 16)
    int arow_i[PF_NI];
    const char *abase = reinterpret_cast<const char *>(a.a_hi);
#pragma unroll
    for (int i = 0; i < PF_NI; ++i) arow_i[i] = s_row[4 * (PF_NI * wv + i) + (l >> 4)];
    auto switch_to_lo = [&]() {
        abase = reinterpret_cast<const char *>(a.a_lo);
#pragma unroll
        for (int i = 0; i < PF_NI; ++i) {
            const int R = 4 * (PF_NI * wv + i) + (l >> 4);
            arow_i[i] = item.row0 + (R < nrows ? R : nrows - 1);
        }
    };
    auto issue_a_part = [&](int kc, int i) {
        const int kk = kc < KC ? kc : kc - KC;
        uint8_t *dst = As + (kc % PF_NSTAGE) * PF_STAGE + wv * PF_NI * 1024;
        const int R = 4 * (PF_NI * wv + i) + (l >> 4);
        const int c = (l & 15) ^ (R & 15);
        copy_to_lds16(abase + (size_t)arow_i[i] * (K * 2) + (kk * (PF_KS * 2) + c * 16), dst + i * 1024);
    };
    auto issue_a = [&](int kc) {
#pragma unroll
        for (int i = 0; i < PF_NI; ++i) issue_a_part(kc, i);
    };

    f32x16 acc[MT][NTW];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

    // the 16-byte fragment chunk 2s + h of tile row m*32 + l%32, swizzled
    const uint8_t *arow_base = As + (l & 31) * (PF_KS * 2);
    auto read_a = [&](int stage, int m, int s) -> u32x4 {
        const int pos = (2 * s + h) ^ (l & 15);
        return *reinterpret_cast<const u32x4 *>(arow_base + stage * PF_STAGE + m * 32 * (PF_KS * 2) +
                                                pos * 16);
    };

    // Loads return in issue order, so one vmcnt wait and one barrier per step
    // cover them (see issue_part).
    issue_a(0);
    if (NSTEP > 1) {
        if (MODE == 1 && SH && KC == 1) switch_to_lo();
        issue_a(1);
        wait_vm<PF_NI>();
    } else {
        wait_vm<0>();
    }
    // a full barrier here (it also drains stage 1): with no copy in flight at
    // loop entry the compiler adds no vector-memory wait before the LDS reads
    // of the steps, so the copy of step kc + 2 stays in flight through the
    // barrier that ends step kc
    __syncthreads();
    // The next unit's ticket (thread 0; pf_ticket is this queue's counter)
    // is taken two k-steps before the end: late enough that no WG holds a
    // ticket for a unit it will not start soon (an early ticket leaves the
    // queue's last units waiting behind long ones while other WGs idle),
    // early enough that the atomic has returned when the loop ends.
    const int kt = NSTEP > 2 ? NSTEP - 2 : 0;
    for (int kc = 0; kc < NSTEP; ++kc) {
        const int st = kc % PF_NSTAGE;
        if (tid == 0 && kc == kt) pf_t = atomicAdd(pf_ticket, 1);
        const bool more1 = kc + 1 < NSTEP, more2 = kc + 2 < NSTEP;
        const int kb = kc + 1 < KC ? kc + 1 : kc + 1 - KC;
        const int ka = kc + 2;     // A stage copied during this step
        const bool amore = more2;
        if (amore && MODE == 1 && SH && ka == KC) switch_to_lo();
        // the next stages' loads are spread over the sub-steps, between the
        // matrix ops: the weights of step kc + 1 first, then the A copy of
        // step kc + 2, so vmcnt(NI) at the end of the step leaves only the
        // latter in flight
        auto issue_part = [&](int s) {
            if (s < G::NBS) {
                if (more1) {
#pragma unroll
                    for (int n = s * NTW / G::NBS; n < (s + 1) * NTW / G::NBS; ++n) load_b_tile(bnext, kb, n);
                }
            } else if (s < G::NBS + PF_NI / 2) {
                if (amore) {
                    issue_a_part(ka, 2 * (s - G::NBS));
                    issue_a_part(ka, 2 * (s - G::NBS) + 1);
                }
            }
        };
        // shared down, second pass (A = h_lo): weight lo fragments are zeroed
        const float lo_scale = (MODE == 1 && SH && kc >= KC) ? 0.f : 1.f;
        {
        // one wave per SIMD: fragments of sub-step s + 1 are read and
        // dequantised while the matrix ops of sub-step s run
        u32x4 af[2][MT], bf[2][NTW], bl[2][NTW];
#pragma unroll
        for (int m = 0; m < MT; ++m) af[0][m] = read_a(st, m, 0);
#pragma unroll
        for (int n = 0; n < NTW; ++n) frag_j<FMT, SH>(bcur[n][0], 0, lo_scale, bf[0][n], bl[0][n]);
        static_for<0, 8>([&](auto s_) {
            constexpr int s = decltype(s_)::value;
            constexpr int cb = s & 1, nb = cb ^ 1;
            issue_part(s);
            if constexpr (s < 7) {
#pragma unroll
                for (int m = 0; m < MT; ++m) af[nb][m] = read_a(st, m, s + 1);
#pragma unroll
                for (int n = 0; n < NTW; ++n)
                    frag_j<FMT, SH>(bcur[n][(s + 1) & 1], (s + 1) >> 1, lo_scale, bf[nb][n], bl[nb][n]);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    acc[m][n] = mfma32(af[cb][m], bf[cb][n], acc[m][n]);
                    if constexpr (SH) acc[m][n] = mfma32(af[cb][m], bl[cb][n], acc[m][n]);
                }
            // keep the next step's reads and dequantisation within this step
            __builtin_amdgcn_sched_barrier(0);
        });
        }
        if (more2)
            wait_vm<PF_NI>();
        else
            wait_vm<0>();
        wg_barrier();
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) bcur[n][sl] = bnext[n][sl];
    }

    // every copy has landed (the last step waited for all); said once more
    // outside the branch so the compiler knows it and does not make each LDS
    // read of the epilogue wait for the stores before it
    wait_vm<0>();
    if (tid < PF_MT) s_exp[tid] = rexp;
    __syncthreads();
    // the next unit's item (thread 0), loaded while the epilogue runs
    // (thread 0: pf_t is the next ticket of this queue, pf_items its items,
    // pf_n its unit count; other threads: pf_t = pf_n)
    u32x4 pfv = {0u, 0u, 0u, 0u};
    const int pt = pf_t;
    const bool pf_on = tid == 0 && pt < pf_n;
    if (pf_on) {
        typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
        pfv = *(global_u32x4 *)(pf_items + pt / a.nt);
    }
    // epilogue, one m-tile at a time through a wave-private LDS region (the A
    // stages are free now): accumulators out as written by the matrix core
    // (D row 8 (r / 4) + 4 h + r % 4, column l % 32), then read back along
    // rows so each lane stores 16 contiguous bytes.
    if constexpr (GU8) {
        // The two waves of a column pair split the m-tiles: the gate wave
        // takes the first MH, the up wave the rest.  Each first hands the
        // other its sums for the other's m-tiles through LDS ([pair][m][r]
        // [lane] floats, 4 KiB per pair and m-tile), then applies SwiGLU to
        // its own m-tiles and stores h as below.
        constexpr int MH = (MT + 1) / 2;
        constexpr int XCH = 4 * (PF_MT / 32) * 16 * 64 * 4;
        constexpr int EPH = 40;                          // h staging pitch (32 columns + 8), halves
        constexpr int EPW = 2 * 32 * EPH * 2;            // h and h_lo, bytes per wave
        static_assert(XCH + 8 * EPW <= PF_NSTAGE * PF_STAGE, "exchange and staging fit in the A stages");
        const int pr = wv & 3;
        const bool upw = wv >= 4;
        float *xch = reinterpret_cast<float *>(As);
        if (cols_valid) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (upw ? m < MH : m >= MH) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) xch[((pr * MT + m) * 16 + r) * 64 + l] = acc[m][0][r];
                }
        }
        lds_barrier();
        if (cols_valid) {
            uint16_t *eh = reinterpret_cast<uint16_t *>(As + XCH + wv * EPW);
            uint16_t *el = eh + 32 * EPH;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (upw ? m < MH : m >= MH) continue;
                int rx[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) rx[r] = s_exp[m * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 8 * (r >> 2) + 4 * h + (r & 3);
                    const float ov = xch[((pr * MT + m) * 16 + r) * 64 + l];
                    const float gv = upw ? ov : acc[m][0][r], uv = upw ? acc[m][0][r] : ov;
                    const float hv = swiglu_scaled(gv, uv, rx[r]);
                    const _Float16 hh = static_cast<_Float16>(hv);
                    eh[row * EPH + (l & 31)] = __builtin_bit_cast(uint16_t, hh);
                    if constexpr (SH)
                        el[row * EPH + (l & 31)] =
                            __builtin_bit_cast(uint16_t, static_cast<_Float16>(hv - static_cast<float>(hh)));
                }
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                // 4 lanes per row, 8 columns each
                const int c0 = tile * 4 * 32 + pr * 32 + (l & 3) * 8;
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const int row = it * 16 + (l >> 2);
                    const int grow = m * 32 + row;
                    const u32x4 hw = *reinterpret_cast<const u32x4 *>(eh + row * EPH + (l & 3) * 8);
                    u32x4 lw;
                    if constexpr (SH) lw = *reinterpret_cast<const u32x4 *>(el + row * EPH + (l & 3) * 8);
                    if (grow < nrows) {
                        *reinterpret_cast<u32x4 *>(a.h_out + (size_t)(item.hrow0 + grow) * a.f + c0) = hw;
                        if constexpr (SH)
                            *reinterpret_cast<u32x4 *>(a.h_lo_out + (size_t)(item.row0 + grow) * a.f + c0) = lw;
                    }
                }
                // the next m-tile overwrites the staging: finish reading it first
                __builtin_amdgcn_s_waitcnt(0xC07F);
            }
        }
    } else if (cols_valid) {
        float *ep = reinterpret_cast<float *>(As + wv * G::EP_WAVE);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if constexpr (MODE == 0) {
                // SwiGLU on the accumulators (a column's gate and up sums sit
                // in the same lane and register), h as fp16 (and its residual
                // for the shared expert) into [32 rows][EP0H_PITCH] halves,
                // read back along rows for 16-byte stores
                uint16_t *eh = reinterpret_cast<uint16_t *>(ep);
                uint16_t *el = eh + 32 * G::EP0H_PITCH;
                int rx[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) rx[r] = s_exp[m * 32 + 8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll
                for (int n = 0; n < NTW / 2; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 8 * (r >> 2) + 4 * h + (r & 3);
                        const float hv = swiglu_scaled(acc[m][n][r], acc[m][n + NTW / 2][r], rx[r]);
                        const _Float16 hh = static_cast<_Float16>(hv);
                        eh[row * G::EP0H_PITCH + n * 32 + (l & 31)] = __builtin_bit_cast(uint16_t, hh);
                        if constexpr (SH)
                            el[row * G::EP0H_PITCH + n * 32 + (l & 31)] =
                                __builtin_bit_cast(uint16_t, static_cast<_Float16>(hv - static_cast<float>(hh)));
                    }
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                constexpr int LPR = G::HCOLS / 8;    // lanes per row (8 columns each)
                const int c0 = tile * NW * G::HCOLS + wv * G::HCOLS + (l % LPR) * 8;
#pragma unroll
                for (int it = 0; it < 32 * LPR / 64; ++it) {
                    const int row = it * (64 / LPR) + l / LPR;
                    const int grow = m * 32 + row;
                    const u32x4 hw = *reinterpret_cast<const u32x4 *>(eh + row * G::EP0H_PITCH + (l % LPR) * 8);
                    u32x4 lw;
                    if constexpr (SH) lw = *reinterpret_cast<const u32x4 *>(el + row * G::EP0H_PITCH + (l % LPR) * 8);
                    if (grow < nrows) {
                        *reinterpret_cast<u32x4 *>(a.h_out + (size_t)(item.hrow0 + grow) * a.f + c0) = hw;
                        if constexpr (SH)
                            *reinterpret_cast<u32x4 *>(a.h_lo_out + (size_t)(item.row0 + grow) * a.f + c0) = lw;
                    }
                }
            } else {
                // [32 rows][EP1_PITCH]: the wave's OCOLS columns
#pragma unroll
                for (int n = 0; n < NTW; ++n)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 8 * (r >> 2) + 4 * h + (r & 3);
                        ep[row * G::EP1_PITCH + n * 32 + (l & 31)] = acc[m][n][r];
                    }
                __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                float *out = SH ? a.y_shared : a.y_pairs;
                constexpr int LPR = G::OCOLS / 4;    // lanes per row (4 columns each)
                const int c0 = tile * NW * G::OCOLS + wv * G::OCOLS + (l % LPR) * 4;
#pragma unroll 2
                for (int it = 0; it < 32 * LPR / 64; ++it) {
                    const int row = it * (64 / LPR) + l / LPR;
                    const int grow = m * 32 + row;
                    f32x4 v = *reinterpret_cast<const f32x4 *>(ep + row * G::EP1_PITCH + (l % LPR) * 4);
                    // y = (h * 2^-2a) . W * 2^2a
                    const int ya = 2 * s_exp[grow];
#pragma unroll
                    for (int c = 0; c < 4; ++c) v[c] = ldexpf(v[c], ya);
                    // y is read once, by the merge: nontemporal stores
                    if (grow < nrows)
                        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(out + (size_t)(item.row0 + grow) * a.d + c0));
                }
            }
            // the next m-tile overwrites the region: finish reading it first
            __builtin_amdgcn_s_waitcnt(0xC07F);
        }
    }
    if (pf_on) *reinterpret_cast<u32x4 *>(pf_dst) = pfv;
    // LDS only: the output stores need not land before the next unit
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    wg_barrier();
}

// Persistent grouped GEMM: workgroups take (item, column tile) units by
// ticket from their XCD's queue, then from the others.
template <int FMT, int MODE, int NTW, int NW>
__global__ __launch_bounds__(64 * NW, MOE_PF_OCC) void pf_gemm_kernel(PfGemmArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t As[PF_NSTAGE * PF_STAGE];
    __shared__ int s_row[PF_MT];
    __shared__ int s_exp[PF_MT];
    __shared__ int s_ticket;
    __shared__ int s_xq[PF_NXCD + 1];   // queue bounds (fixed for the launch)
    __shared__ __attribute__((aligned(16))) PfItem s_next;   // item of ticket s_next_t in queue s_next_x
    __shared__ int s_next_t, s_next_x;
    unsigned xcd;
    __asm__ volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcd));
    xcd &= PF_NXCD - 1;
    // the ticket for the next unit is taken at the start of the current one,
    // and its item is loaded during the current unit's epilogue
    if (threadIdx.x == 0) {
        s_ticket = atomicAdd(&a.sched->ticket[a.launch][xcd], 1);
        s_next_t = -1;
        s_next_x = -1;
    }
    if (threadIdx.x <= PF_NXCD) s_xq[threadIdx.x] = a.sched->xq[threadIdx.x];
    __syncthreads();
    for (int q = 0; q < PF_NXCD;) {
        const int x = (int)((xcd + q) & (PF_NXCD - 1));
        const int t = wave_uniform(s_ticket);
        const int i0 = s_xq[x];
        const int n_units = (s_xq[x + 1] - i0) * a.nt;
        if (t >= n_units) {
            ++q;
            __syncthreads();
            if (threadIdx.x == 0 && q < PF_NXCD)
                s_ticket = atomicAdd(&a.sched->ticket[a.launch][(xcd + q) & (PF_NXCD - 1)], 1);
            __syncthreads();
            continue;
        }
        int nxt = n_units;   // thread 0: the next ticket, taken inside the unit
        int *tk = &a.sched->ticket[a.launch][x];
        const bool have = s_next_t == t && s_next_x == x;   // uniform
        typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
        u32x4 iv;
        if (have)
            iv = *reinterpret_cast<const u32x4 *>(&s_next);
        else
            iv = *(global_u32x4 *)(a.items + i0 + t / a.nt);
        const PfItem item{(int32_t)iv.x, (int32_t)iv.y, (int32_t)iv.z, (int32_t)iv.w};
        const int tile = t % a.nt;
        constexpr int MTX = PF_MT / 32;
        if (item.expert < 0) {
            pf_unit<FMT, MODE, true, MTX, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next);
        } else {
            switch ((item.nrows + 31) >> 5) {
                case 1: pf_unit<FMT, MODE, false, 1, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next); break;
                case 2: pf_unit<FMT, MODE, false, 2, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next); break;
                case 3: pf_unit<FMT, MODE, false, 3, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next); break;
                case 4: pf_unit<FMT, MODE, false, 4 < MTX ? 4 : MTX, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next); break;
                case 5: pf_unit<FMT, MODE, false, 5 < MTX ? 5 : MTX, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next); break;
                default: pf_unit<FMT, MODE, false, MTX, NTW, NW>(a, item, tile, As, s_row, s_exp, a.items + i0, tk, nxt, n_units, &s_next); break;
            }
        }
        // pf_unit ended with a barrier: every thread has read s_ticket
        if (threadIdx.x == 0) {
            s_ticket = nxt;
            s_next_t = nxt < n_units ? nxt : -1;
            s_next_x = x;
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ host
struct PfWs {
    PfSched *sched;
    PfItem *items;
    int32_t *xexp;
    uint16_t *x16;
    uint16_t *h;
    uint16_t *h_lo;
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static size_t pf_max_items(int E, int T, int k) {
    const size_t P = (size_t)T * k;
    return (T + PF_MT - 1) / PF_MT + P / PF_MT + (size_t)(E < (int)P ? E : P) + 1;
}

static PfWs pf_carve(void *ws, int d, int f, int E, int T, int k) {
    char *p = static_cast<char *>(ws) + kWsHeader;
    PfWs w;
    w.sched = reinterpret_cast<PfSched *>(p);
    p += 256;
    w.items = reinterpret_cast<PfItem *>(p);
    p += align256(pf_max_items(E, T, k) * sizeof(PfItem));
    w.xexp = reinterpret_cast<int32_t *>(p);
    p += align256((size_t)T * sizeof(int32_t));
    w.x16 = reinterpret_cast<uint16_t *>(p);
    p += align256((size_t)T * d * 2);
    w.h = reinterpret_cast<uint16_t *>(p);
    p += align256(((size_t)T * k + T) * f * 2);
    w.h_lo = reinterpret_cast<uint16_t *>(p);
    return w;
}

static size_t ws_bytes(int d, int f, int E, int T, int k) {
    return 256 + align256(pf_max_items(E, T, k) * sizeof(PfItem)) + align256((size_t)T * sizeof(int32_t)) +
           align256((size_t)T * d * 2) +
           align256(((size_t)T * k + T) * f * 2) + align256((size_t)T * f * 2);
}

// persistent grid: occ workgroups per compute unit
static int pf_grid(int occ) {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256 * occ;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev] * occ;
}


template <int FMT>
static void pf_launch_fmt(const moe_layer &L, const uint16_t *x, int T, int k, const int32_t *offsets,
                          const int32_t *sorted_pair, float *y_pairs, float *y_shared, const PfWs &w,
                          int parts, hipStream_t s) {
    const int d = L.d_model, f = L.d_ff, E = L.n_experts;
    const int P = T * k;
    // x conversion: one wave per token row, 16 rows per block
    size_t blocks = ((size_t)T + 15) / 16;
    if (blocks > 2048) blocks = 2048;
    hipLaunchKernelGGL(pf_prep_kernel, dim3((unsigned)(1 + blocks)), dim3(1024), 0, s, offsets, E, T, P,
                       parts, w.items, w.sched, x, w.x16, w.xexp, d);
    PfGemmArgs a{};
    a.items = w.items;
    a.sched = w.sched;
    a.xexp = w.xexp;
    a.sorted_pair = sorted_pair;
    a.h_out = w.h;
    a.h_lo_out = w.h_lo;
    a.y_pairs = y_pairs;
    a.y_shared = y_shared;
    a.k = k;
    a.d = d;
    a.f = f;
    using G = PfGeom<kPfNtw, 4>;   // a gate/up unit spans 4 x 32 h columns either way
    using GD = PfGeom<kPfDownNtw, kPfDownNw>;
    const int grid = pf_grid(MOE_PF_OCC);
    // gate/up + SwiGLU
    a.w0 = QMatDev{L.gate.lo, L.gate.hi, L.gate.scale, L.gate.min};
    a.w1 = QMatDev{L.up.lo, L.up.hi, L.up.scale, L.up.min};
    a.s0 = QMatDev{L.sh_gate.lo, L.sh_gate.hi, L.sh_gate.scale, L.sh_gate.min};
    a.s1 = QMatDev{L.sh_up.lo, L.sh_up.hi, L.sh_up.scale, L.sh_up.min};
    a.a_hi = w.x16;
    a.a_lo = nullptr;
    a.nt = (f + 4 * G::HCOLS - 1) / (4 * G::HCOLS);
    a.launch = 0;
    hipLaunchKernelGGL((pf_gemm_kernel<FMT, 0, kPfGuNtw, kPfGuNw>), dim3(grid), dim3(64 * kPfGuNw), 0, s, a);
    // down
    a.w0 = a.w1 = QMatDev{L.down.lo, L.down.hi, L.down.scale, L.down.min};
    a.s0 = a.s1 = QMatDev{L.sh_down.lo, L.sh_down.hi, L.sh_down.scale, L.sh_down.min};
    a.a_hi = w.h;
    a.a_lo = w.h_lo;
    a.nt = (d + kPfDownNw * GD::OCOLS - 1) / (kPfDownNw * GD::OCOLS);
    a.launch = 1;
    hipLaunchKernelGGL((pf_gemm_kernel<FMT, 1, kPfDownNtw, kPfDownNw>), dim3(grid), dim3(64 * kPfDownNw), 0, s, a);
}

static hipError_t launch(const moe_layer &L, const uint16_t *x, int T, int k, const int32_t *offsets,
                         const int32_t *sorted_pair, float *y_pairs, float *y_shared, void *ws, int parts,
                         hipStream_t s) {
    const PfWs w = pf_carve(ws, L.d_model, L.d_ff, L.n_experts, T, k);
    if (L.format == MOE_FMT_Q2_B32)
        pf_launch_fmt<MOE_FMT_Q2_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, w, parts, s);
    else
        pf_launch_fmt<MOE_FMT_Q3_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, w, parts, s);
    return hipGetLastError();
}

}  // namespace MOE_PF_NS

size_t MOE_PF_WS(int d, int f, int E, int T, int k) { return MOE_PF_NS::ws_bytes(d, f, E, T, k); }

hipError_t MOE_PF_LAUNCH(const moe_layer &L, const uint16_t *x, int T, int k, const int32_t *offsets,
                         const int32_t *sorted_pair, float *y_pairs, float *y_shared, void *ws, int parts,
                         hipStream_t s) {
    return MOE_PF_NS::launch(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, ws, parts, s);
}

}  // namespace moe
