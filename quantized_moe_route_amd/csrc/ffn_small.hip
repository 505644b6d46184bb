// ffn_small.hip -- expert FFN when every expert group has few rows (decode,
// MTP verify: T <= 16 tokens).
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 …", section
// "Strata의 동작 원리": 10 routed experts plus the always-resident shared expert
// per token and layer; [video] kangdaejong.com strata summary, section "픽업":
// the selected experts' 2-3-bit weights are decompressed and computed on the
// GPU.
//
// Each expert's weights are read exactly once per layer for all of its rows.
// The work is HBM-bound, so the design minimises ALU work per weight byte:
//   - one wave owns 16 weight rows x a slice of K; the storage order gives
//     every lane one 8-byte piece (4 blocks x 8 codes) per 16x128 unit, so a
//     wave load is 512 contiguous bytes;
//   - 2-bit codes become exact bf16/fp16 integers with the fp4 conversion
//     (two masks + four converts per 16 codes); for Q3 each code's third bit
//     turns its low-bits nibble into the fp4 code of (q - 4) / 2 (a select
//     per nibble), so the same four converts give q - 4 exactly;
//   - the 32-wide K block is exactly one 16x16x32 matrix-core step, so the
//     product codes x activations comes out per block, and the block scale and
//     minimum are applied in fp32: acc += d*P + m*X (Q2, X = sum of the
//     block's activations, a matrix-core step against ones) or d*P (Q3, P
//     over q - 4).
//   Weights are therefore used exactly (no rounding of d*q + m), and all sums
//   are fp32.
//   - gate/up: A = the batch's x rows (bf16, exact; each group row then takes
//     its token's sums); h = silu(g)*u in fp32 is written as fp16 hi + fp16
//     lo (22 significant bits) of h * 2^-2a, where 2^a <= max|x_t| < 2^(a+1)
//     for the row's token t (an exact power-of-two scaling, so h fits fp16's
//     range for any bf16 x); a goes to hx[row] and the down projection
//     multiplies y by 2^2a.
//   - down: A stacks the group's h_hi rows over its h_lo rows in one 16-row
//     tile, so one fp16 matrix-core step covers both halves.
//   - four waves of a workgroup split K; partial sums meet in LDS in a fixed
//     order.
//   - up to 8 (gate/up: 16) tokens the activation rows are staged in LDS once
//     per workgroup instead of being loaded into each wave's registers: fewer
//     registers, more resident waves, and each byte read from L2 once per
//     workgroup.
#include "common.h"

namespace moe {

constexpr uint32_t kOneBf16x2 = 0x3F803F80u;
constexpr uint32_t kOneF16x2 = 0x3C003C00u;

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// Everything one lane needs from one 16 x 128 unit of the gate and up
// matrices, plus its activation pieces.  Loads of a batch of units are all
// issued before the first is used, so a wave pays HBM latency once per batch.
template <int FMT, int MT>
struct GateUpUnit {
    u32x2 lg, lu, sg, su, mg, mu;
    uint32_t hg, hu;
    u32x4 A[MT][4];
};

// The codes of one unit of gate and up (the block scales and minimums come
// through piece_gather below).
template <int FMT, int MT>
__device__ __forceinline__ void gateup_load_codes(GateUpUnit<FMT, MT> &U, const QMatDev &Wg, const QMatDev &Wu,
                                                  size_t unit, int lane) {
    auto ld = [](const auto *p) { return __builtin_nontemporal_load(p); };   // read once
    U.lg = ld(reinterpret_cast<const u32x2 *>(Wg.lo + unit * 512 + lane * 8));
    U.lu = ld(reinterpret_cast<const u32x2 *>(Wu.lo + unit * 512 + lane * 8));
    if constexpr (FMT == MOE_FMT_Q3_B32) {
        U.hg = ld(reinterpret_cast<const uint32_t *>(Wg.hi + unit * 256 + lane * 4));
        U.hu = ld(reinterpret_cast<const uint32_t *>(Wu.hi + unit * 256 + lane * 4));
    }
}

// Block scales (and Q2 minimums) of a wave's batch of units: P pieces of 128
// bytes (a unit's 16 rows x 4 blocks of fp16), gathered with one 16-byte
// load per lane per 64 chunks into the wave's own LDS region, from where each
// lane reads its row's 8 bytes.  (8-byte loads by every lane, four lanes to
// an address, cost several times the code loads' issue time.)  The loads are
// unconditional (lanes past the last chunk repeat it).
template <int P>
struct PieceGather {
    static constexpr int N = (8 * P + 63) / 64;
    u32x4 v[N];
    // piece_addr(p): the global address of piece p, as an integer (a select
    // among pointers can become a lookup table in scratch memory)
    template <typename F>
    __device__ __forceinline__ void issue(F piece_addr) {
        typedef __attribute__((address_space(1))) const u32x4 global_u32x4;
        const int lane = __lane_id();
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int c = i * 64 + lane < 8 * P ? i * 64 + lane : 8 * P - 1;
            const uint64_t a = piece_addr(c >> 3) + (uint64_t)(c & 7) * 16;
            v[i] = __builtin_nontemporal_load(reinterpret_cast<global_u32x4 *>(a));
        }
    }
    // into a region of N x 64 chunks (lanes past the last chunk store their
    // repeat into the spare slots: no branch, so the compiler's waits stay
    // exact)
    __device__ __forceinline__ void store(u32x4 *lds) const {
        const int lane = __lane_id();
#pragma unroll
        for (int i = 0; i < N; ++i) lds[i * 64 + lane] = v[i];
    }
};
// row rr of piece p in a gathered region
__device__ __forceinline__ u32x2 piece_row(const u32x4 *lds, int p, int rr) {
    return reinterpret_cast<const u32x2 *>(lds)[p * 16 + rr];
}

template <int FMT, int MT>
__device__ __forceinline__ void gateup_load_x(GateUpUnit<FMT, MT> &U, int u, int gq,
                                              const uint16_t *const *xrow) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            U.A[mt][j] = *reinterpret_cast<const u32x4 *>(xrow[mt] + u * 128 + j * 32 + gq * 8);
}

// The weight operand of block J: Q2 exact codes q, Q3 q - 4 (both exact)
template <int J, bool F16, int FMT>
__device__ __forceinline__ u32x4 block_operand(uint32_t lo_dw, uint32_t hi_w) {
    if constexpr (FMT == MOE_FMT_Q3_B32)
        return q3_operand<J, F16>(lo_dw, hi_w);
    else
        return lo_operand<J & 1, F16>(lo_dw);
}

__device__ __forceinline__ float half_of(const u32x2 &v, int j) {
    return half_bits_to_float((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
}

// IMAX = number of valid D rows per lane group i (compile time): 1 for a
// single-token batch, 2 for two tokens, 4 otherwise.  The epilogue touches
// only those rows, so small batches pay no selects.
// RS: result registers between successive rows used (token rows spread
// over the matrix rows: accumulator i takes result register i RS)
template <int FMT, int MT, int IMAX, int J, int RS = 1>
__device__ __forceinline__ void gateup_block(const GateUpUnit<FMT, MT> &U, f32x4 *ag, f32x4 *au) {
    const u32x4 ones = {kOneBf16x2, kOneBf16x2, kOneBf16x2, kOneBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const u32x4 Bg = block_operand<J, false, FMT>(U.lg[J >> 1], U.hg);
    const u32x4 Bu = block_operand<J, false, FMT>(U.lu[J >> 1], U.hu);
    const float dg = half_of(U.sg, J), du = half_of(U.su, J);
    float mgv = 0.f, muv = 0.f;
    if constexpr (FMT == MOE_FMT_Q2_B32) {
        mgv = half_of(U.mg, J);
        muv = half_of(U.mu, J);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 pg = mfma_bf16(U.A[mt][J], Bg, zero);
        f32x4 pu = mfma_bf16(U.A[mt][J], Bu, zero);
        if constexpr (FMT == MOE_FMT_Q3_B32) {
            // x . (q - 4) in one matrix op (the operand holds q - 4)
#pragma unroll
            for (int i = 0; i < IMAX; ++i) {
                ag[mt][i] = fmaf(dg, pg[i * RS], ag[mt][i]);
                au[mt][i] = fmaf(du, pu[i * RS], au[mt][i]);
            }
        } else {
            const f32x4 xs = mfma_bf16(U.A[mt][J], ones, zero);
#pragma unroll
            for (int i = 0; i < IMAX; ++i) {
                ag[mt][i] = fmaf(dg, pg[i * RS], fmaf(mgv, xs[i * RS], ag[mt][i]));
                au[mt][i] = fmaf(du, pu[i * RS], fmaf(muv, xs[i * RS], au[mt][i]));
            }
        }
    }
}

#ifndef MOE_DECODE_BATCH
#define MOE_DECODE_BATCH 4
#endif
constexpr int kBatch = MOE_DECODE_BATCH;   // units prefetched per wave per batch
// gate/up: units per wave per batch, NB = 16 / NW (K = d_model = 2048 is 16
// units: one batch per wave)
// down: K = d_ff = 768 is 6 units, 3 per wave of two; a batch of 4 held a
// fourth, unused unit's registers (166 -> 128 VGPRs at 16 tokens)
constexpr int kDownBatch = 3;

constexpr size_t kXsMaxBytes = 32768;   // x staged in LDS by the gate/up kernel (up to 8 tokens)
// One gate/up task: 16 h columns (row tile nt) of one expert group, for all
// of the group's rows.  The NW waves of the workgroup split K and meet in LDS
// (red); wave 0 applies SwiGLU and writes h as fp16 hi + lo.
//
// The 16 matrix rows are the batch's tokens themselves (T <= 16), not the
// group's rows, so the activation loads depend on nothing and go out with
// the weights; a group row's token (its pair's entry in sorted_pair) is
// needed only when wave 0 picks its row out of the sums.  Each output row is
// the same dot product either way.  XL: x is first copied into LDS once per
// workgroup (global-to-LDS, no registers held) and the activation operands
// are read from there; TPW > 1: one workgroup of TPW x NW waves serves TPW
// column tiles with that one copy.
// The exponent a of the largest magnitude of x_t (0 for a zero row), from the
// largest bf16 magnitude bits (sign cleared): 2^a <= max|x_t| < 2^(a+1).
__device__ __forceinline__ int exp_of_max_bits(uint32_t mx) {
    const int ef = (int)(mx >> 7);
    return mx == 0u ? 0 : (ef == 0 ? -126 : ef - 127);
}
__device__ __forceinline__ uint32_t max_mag_bf16x8(const u32x4 &v, uint32_t mx) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = v[q] & 0x7fffu, hi = (v[q] >> 16) & 0x7fffu;
        mx = lo > mx ? lo : mx;
        mx = hi > mx ? hi : mx;
    }
    return mx;
}

// SP: matrix rows per token (x staged for SP > 1).  Token t fills rows
// SP t .. SP t + SP - 1, so with SP = 4 (up to 4 tokens) lane group t holds
// token t's sums in its first result register and the per-block epilogue
// runs one FMA per matrix (RI = 1), and with SP = 2 (up to 8 tokens) lane
// group g holds tokens 2g and 2g + 1 in registers 0 and 2 (RI = 2); with the
// tokens in rows 0 .. T-1 (SP = 1) only the first lane groups held useful
// rows, while all four ran T FMAs.
__host__ __device__ constexpr int spread_ri(int sp, int imax) { return sp == 1 ? imax : (4 / sp < imax ? 4 / sp : imax); }
template <int FMT, int IMAX, int NW, bool XL, int TPW, int NB = 16 / NW, int SP = 1, int RI = spread_ri(SP, IMAX)>
__device__ __forceinline__ void gateup_task(const QMatDev &gate, const QMatDev &up, const QMatDev &sgate,
                                            const QMatDev &sup, const uint16_t *__restrict__ x, int T, int k, int d,
                                            int f, const int32_t *__restrict__ sorted_pair, const Group &grp,
                                            int nt, float (*red)[2][RI][64], uint32_t (*redx)[16],
                                            uint16_t *__restrict__ h_hi, uint16_t *__restrict__ h_lo,
                                            int32_t *__restrict__ hx, uint16_t *xs, u32x4 *pieces) {
    static_assert(NW > 1, "token rows: K split over waves");
    static_assert(TPW == 1 || XL, "several tiles per workgroup share the staged x");
    static_assert(SP == 1 || (XL && (SP == 2 || SP == 4)), "spread token rows: x staged, 2 or 4 rows per token");
    const int lane = __lane_id();
    // TPW tiles per workgroup: waves [NW g, NW g + NW) take tile nt + g
    const int wall = wave_uniform(threadIdx.x >> 6);
    const int wv = wall % NW, tg = wall / NW;
    nt += tg;
    red += tg * NW;
    redx += tg * NW;
    const int gq = lane >> 4, rr = lane & 15;
    const bool shared = grp.expert < 0;
    const QMatDev Wg = shared ? sgate : gate;
    const QMatDev Wu = shared ? sup : up;
    const int e = shared ? 0 : grp.expert;
    const int KC = d / 128;
    const size_t ubase = ((size_t)e * (f / 16) + nt) * KC;
    const int nrows = grp.nrows;

    // the pair of output row r = lane % 16 (rows past the group's last row
    // use its last row, never stored): one register, loaded unconditionally
    // before the weights, read by wave 0 at the end through a lane shuffle
    int rtok;
    {
        const int r = rr < nrows ? rr : nrows - 1;
        rtok = shared ? r : sorted_pair[grp.row0 + r];
    }
    f32x4 ag[1], au[1];
    ag[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    au[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the token row of this lane's matrix row
    const int xr = rr / SP < T ? rr / SP : T - 1;
    const uint16_t *xrow[1] = {x + (size_t)xr * d};
    const int cpr = d / 8;                // 16-byte chunks per x row
    uint32_t xmax = 0u;                   // largest |x| bits of this lane's row over its K slices
    GateUpUnit<FMT, 1> U[NB];
    // scale pieces of a batch: unit b, matrix m (gate, up), plane (scale, Q2 min)
    constexpr int NPL = FMT == MOE_FMT_Q2_B32 ? 2 : 1;
    constexpr int NP = NB * 2 * NPL;
    u32x4 *const pw = pieces + (size_t)wall * 64 * PieceGather<NP>::N;   // this wave's region
    // plane base addresses as integers, chosen by selects
    const uint64_t gs = (uint64_t)Wg.scale, gm = (uint64_t)Wg.min, us = (uint64_t)Wu.scale, um = (uint64_t)Wu.min;
    auto gather = [=](int u0) {
        PieceGather<NP> g;
        g.issue([=](int p) {
            const int b = p / (2 * NPL), m = (p / NPL) & 1, pl = p % NPL;
            const int u = u0 + NW * b < KC ? u0 + NW * b : KC - 1;
            // three selects; the empty asm keeps them selects (folded, they
            // become a table in scratch memory)
            uint64_t base = m == 0 && pl == 1 ? gm : gs;
            __asm__ volatile("" : "+v"(base));
            base = m == 1 && pl == 0 ? us : base;
            __asm__ volatile("" : "+v"(base));
            base = m == 1 && pl == 1 ? um : base;
            return base + (ubase + u) * 128;
        });
        return g;
    };
    PieceGather<NP> pg = gather(wv);
    // unconditional (clamped past KC; those units are not used): a load in a
    // branch makes the compiler's waits conservative
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int u = wv + NW * b;
        gateup_load_codes(U[b], Wg, Wu, ubase + (u < KC ? u : KC - 1), lane);
    }
    // XL: x was staged and waited for by every wave before the barrier that
    // published the group.  The largest |x| of each token row (for h's
    // scaling) comes from the staged rows once, wave wv taking rows wv,
    // wv + NW, ..., while this wave's first weights are in flight: tracked
    // per unit instead, it cost as many VALU instructions as the
    // dequantisation.
    if constexpr (XL) {
        for (int t = wv; t < T; t += NW) {
            uint32_t m = 0u;
            for (int c = lane; c < cpr; c += 64)
                m = max_mag_bf16x8(*reinterpret_cast<const u32x4 *>(xs + ((size_t)t * cpr + (c ^ (t & 7))) * 8), m);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const uint32_t v = (uint32_t)__shfl_xor((int)m, o, 64);
                m = v > m ? v : m;
            }
            if (lane == 0) redx[wv][t] = m;
        }
    }
    for (int u0 = wv; u0 < KC; u0 += NW * NB) {
        if (u0 != wv) {
            pg = gather(u0);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int u = u0 + NW * b;
                gateup_load_codes(U[b], Wg, Wu, ubase + (u < KC ? u : KC - 1), lane);
            }
        }
        __asm__ volatile("" ::: "memory");
        // the scales landed before the codes (issued first): stage and read them
        pg.store(pw);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            U[b].sg = piece_row(pw, (b * 2 + 0) * NPL, rr);
            U[b].su = piece_row(pw, (b * 2 + 1) * NPL, rr);
            if constexpr (FMT == MOE_FMT_Q2_B32) {
                U[b].mg = piece_row(pw, (b * 2 + 0) * NPL + 1, rr);
                U[b].mu = piece_row(pw, (b * 2 + 1) * NPL + 1, rr);
            }
        }
        if constexpr (!XL) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int u = u0 + NW * b;
                if (u < KC) gateup_load_x(U[b], u, gq, xrow);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (u0 + NW * b < KC) {
                if constexpr (XL) {
                    const int u = u0 + NW * b;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = u * 16 + j * 4 + gq;
                        U[b].A[0][j] = *reinterpret_cast<const u32x4 *>(
                            xs + ((size_t)xr * cpr + (c ^ (xr & 7))) * 8);
                    }
                }
                if constexpr (!XL) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) xmax = max_mag_bf16x8(U[b].A[0][j], xmax);
                }
                gateup_block<FMT, 1, RI, 0, SP>(U[b], ag, au);
                gateup_block<FMT, 1, RI, 1, SP>(U[b], ag, au);
                gateup_block<FMT, 1, RI, 2, SP>(U[b], ag, au);
                gateup_block<FMT, 1, RI, 3, SP>(U[b], ag, au);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < RI; ++i) {
        red[wv][0][i][lane] = ag[0][i];
        red[wv][1][i][lane] = au[0][i];
    }
    // !XL: the row's (lane rr's token) largest |x| over the four lane groups
    if constexpr (!XL) {
        uint32_t o = (uint32_t)__shfl_xor((int)xmax, 16, 64);
        xmax = o > xmax ? o : xmax;
        o = (uint32_t)__shfl_xor((int)xmax, 32, 64);
        xmax = o > xmax ? o : xmax;
        if (lane < 16) redx[wv][lane] = xmax;
    }
    __syncthreads();
    if (wv != 0) return;
    // output row r = 4 gq + i (SP = 4: r = gq) takes the sums of its token's
    // matrix rows: token t's are in lane group SP t / 4, accumulator
    // t % (4 / SP)
    const int n = nt * 16 + rr;
#pragma unroll
    for (int i = 0; i < (SP == 4 ? 1 : IMAX); ++i) {
        const int r = SP == 4 ? gq : 4 * gq + i;
        const int tk = __shfl(rtok, r, 64);
        if (r >= nrows) continue;
        const int t = shared ? tk : tk / k;
        const int sl = ((SP * t) >> 2) * 16 + rr, si = t % (4 / SP);
        float gs = red[0][0][si][sl], us = red[0][1][si][sl];
        uint32_t mx = XL ? redx[t % NW][t] : redx[0][t];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) {
            gs += red[w2][0][si][sl];
            us += red[w2][1][si][sl];
            if constexpr (!XL) mx = redx[w2][t] > mx ? redx[w2][t] : mx;
        }
        // h * 2^-2a = (g 2^-a) sigmoid(g) (u 2^-a): exact scalings
        const int a = exp_of_max_bits(mx);
        const float h = swiglu(gs, us, a);
        const _Float16 hh = static_cast<_Float16>(h);
        const float rem = h - static_cast<float>(hh);
        const size_t off = (size_t)(grp.hrow0 + r) * f + n;
        h_hi[off] = __builtin_bit_cast(uint16_t, hh);
        h_lo[off] = f32_to_f16_bits(rem);
        if (nt == 0) hx[grp.hrow0 + r] = a;
    }
}

template <int FMT, int MT>
struct DownUnit {
    u32x2 lw, sw, mw;
    uint32_t hw;
    u32x4 A[MT][4];
};

template <int FMT, int MT, int IMAX, int J>
__device__ __forceinline__ void down_block(const DownUnit<FMT, MT> &U, f32x4 *acc) {
    const u32x4 ones = {kOneF16x2, kOneF16x2, kOneF16x2, kOneF16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const u32x4 B = block_operand<J, true, FMT>(U.lw[J >> 1], U.hw);
    const float dv = half_of(U.sw, J);
    float mv = 0.f;
    if constexpr (FMT == MOE_FMT_Q2_B32) mv = half_of(U.mw, J);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const f32x4 p = mfma_f16(U.A[mt][J], B, zero);
        if constexpr (FMT == MOE_FMT_Q3_B32) {
            // h . (q - 4) in one matrix op
#pragma unroll
            for (int i = 0; i < IMAX; ++i) acc[mt][i] = fmaf(dv, p[i], acc[mt][i]);
        } else {
            const f32x4 hs = mfma_f16(U.A[mt][J], ones, zero);
#pragma unroll
            for (int i = 0; i < IMAX; ++i) acc[mt][i] = fmaf(dv, p[i], fmaf(mv, hs[i], acc[mt][i]));
        }
    }
}

// SPREAD form (at most 4 group rows): group row r's h_hi fills matrix rows
// 4r, 4r + 1 and its h_lo rows 4r + 2, 4r + 3, so lane group r holds both in
// result registers 0 and 2: two epilogue FMAs per block (Q2: four) where the
// stacked form (hi rows 0-7 over lo rows 8-15) ran one per row on every lane.
// The same products and sums per row: y is bit-identical to the stacked
// form's.
template <int FMT, int J>
__device__ __forceinline__ void down_block_spread(const DownUnit<FMT, 1> &U, float (&acc)[2]) {
    const u32x4 ones = {kOneF16x2, kOneF16x2, kOneF16x2, kOneF16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const u32x4 B = block_operand<J, true, FMT>(U.lw[J >> 1], U.hw);
    const float dv = half_of(U.sw, J);
    const f32x4 p = mfma_f16(U.A[0][J], B, zero);
    if constexpr (FMT == MOE_FMT_Q3_B32) {
        acc[0] = fmaf(dv, p[0], acc[0]);
        acc[1] = fmaf(dv, p[2], acc[1]);
    } else {
        const float mv = half_of(U.mw, J);
        const f32x4 hs = mfma_f16(U.A[0][J], ones, zero);
        acc[0] = fmaf(dv, p[0], fmaf(mv, hs[0], acc[0]));
        acc[1] = fmaf(dv, p[2], fmaf(mv, hs[2], acc[1]));
    }
}

// Down-projection weights of one batch of a wave's units (units u0 + NW b),
// loadable before h is needed: the weights do not depend on it.
template <int FMT, int MT, int NW>
struct DownW {
    static constexpr int NB = kDownBatch;
    static constexpr int NPL = FMT == MOE_FMT_Q2_B32 ? 2 : 1;   // scale (and Q2 min) pieces per unit
    u32x2 lw[NB];
    uint32_t hw[NB];
    PieceGather<NB * NPL> pg;
};

template <int FMT, int MT, int NW>
__device__ __forceinline__ void down_load_w(DownW<FMT, MT, NW> &Wt, const QMatDev &down, const QMatDev &sdown,
                                            int d, int f, const Group &grp, int ot, int u0) {
    const int lane = __lane_id(), rr = lane & 15;
    const bool shared = grp.expert < 0;
    const QMatDev W = shared ? sdown : down;
    const int e = shared ? 0 : grp.expert;
    const int KC = f / 128;
    const size_t ubase = ((size_t)e * (d / 16) + ot) * KC;
    constexpr int NB = DownW<FMT, MT, NW>::NB, NPL = DownW<FMT, MT, NW>::NPL;
    (void)rr;
    // the batch's scale pieces first (piece p: unit p / NPL, plane p % NPL)
    {
        const uint64_t sc = (uint64_t)W.scale, mn = (uint64_t)W.min;
        Wt.pg.issue([=](int p) {
            int u = u0 + NW * (p / NPL);
            u = u < KC ? u : KC - 1;
            uint64_t base = p % NPL ? mn : sc;
            __asm__ volatile("" : "+v"(base));
            return base + (ubase + u) * 128;
        });
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        int u = u0 + NW * b;
        u = u < KC ? u : KC - 1;   // clamped: unconditional loads, unused past KC
        const size_t unit = ubase + u;
        auto ld = [](const auto *p) { return __builtin_nontemporal_load(p); };   // read once
        Wt.lw[b] = ld(reinterpret_cast<const u32x2 *>(W.lo + unit * 512 + lane * 8));
        if constexpr (FMT == MOE_FMT_Q3_B32) Wt.hw[b] = ld(reinterpret_cast<const uint32_t *>(W.hi + unit * 256 + lane * 4));
    }
}

// One down task: 16 outputs (row tile ot) of one expert group, all rows; the
// NW waves of the task (index wq) split K = d_ff.  Wt holds the first batch
// of weights (units wq + NW b), loaded by the caller.  A tile row rr < 8
// holds h_hi of group row 8 mt + rr, row 8 + rr its h_lo; D rows 4 gq + i:
// hi rows in lanes gq = 0, 1 and lo rows in gq = 2, 3.
// HL: the group's h rows (hi and lo, at most 8 each) are staged in LDS by
// global-to-LDS copies: stored row S = (lo ? nrows : 0) + r, chunk c of it at
// S * (f / 8) + (c ^ (S & 7)); the A operands are read from there.
template <int FMT, int MT, int IMAX, int NW, bool DEV, bool HL, bool SPREAD = false, int RI = SPREAD ? 2 : IMAX>
__device__ __forceinline__ void down_task(DownW<FMT, MT, NW> &Wt, const QMatDev &down, const QMatDev &sdown,
                                          const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
                                          const int32_t *__restrict__ hx, int d, int f, const Group &grp, int ot,
                                          int wq, float (*red)[MT][RI][64], float *__restrict__ y_pairs,
                                          float *__restrict__ y_shared, uint16_t *hs, u32x4 *pieces) {
    static_assert(!HL || MT == 1, "staged h: groups of at most 8 rows");
    static_assert(!SPREAD || MT == 1, "spread rows: groups of at most 4 rows");
    const int lane = __lane_id();
    const int gq = lane >> 4, rr = lane & 15;
    const int KC = f / 128;
    const int nrows = grp.nrows;
    // the exponents of this lane's output rows (y = acc * 2^2a), loaded
    // early: their latency runs under the weights'
    int ya[MT][IMAX];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < IMAX; ++i) {
            int r = SPREAD ? gq : mt * 8 + gq * 4 + i;
            r = r < nrows ? r : nrows - 1;
            ya[mt][i] = wq == 0 ? 2 * hx[grp.hrow0 + r] : 0;
        }
    const int cpr = f / 8;
    const uint16_t *hrow[MT];
    // this lane's A row: group row ar, its h_lo half if alo
    const int ar = SPREAD ? rr >> 2 : rr & 7;
    const bool alo = SPREAD ? (rr & 3) >= 2 : rr >= 8;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int r = mt * 8 + ar;
        r = r < nrows ? r : nrows - 1;
        hrow[mt] = (alo ? h_lo : h_hi) + (size_t)(grp.hrow0 + r) * f;
    }
    int srow = 0;   // HL: this lane's stored row
    if constexpr (HL) {
        const int r = ar < nrows ? ar : nrows - 1;
        srow = (alo ? nrows : 0) + r;
        const int nch = 2 * nrows * cpr;
        for (int q = wq; q * 64 < nch; q += NW) {
            const int L = q * 64 + lane;
            if (L < nch) {
                const int S = L / cpr, cs = L - S * cpr;
                const int hr = S < nrows ? S : S - nrows;
                const uint16_t *src = (S < nrows ? h_hi : h_lo) + (size_t)(grp.hrow0 + hr) * f;
                copy_to_lds16(src + (size_t)(cs ^ (S & 7)) * 8, hs + (size_t)q * 512);
            }
        }
        wait_vm<0>();   // the copies and the first weights
        __syncthreads();
    }
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float acs[2] = {0.f, 0.f};   // SPREAD: this lane's row, h_hi and h_lo halves
    constexpr int NB = DownW<FMT, MT, NW>::NB;
    for (int u0 = wq; u0 < KC; u0 += NW * NB) {
        if (u0 != wq) down_load_w<FMT, MT, NW>(Wt, down, sdown, d, f, grp, ot, u0);
        constexpr int NPL = DownW<FMT, MT, NW>::NPL;
        Wt.pg.store(pieces);
        DownUnit<FMT, MT> U[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int u = u0 + NW * b;
            u = u < KC ? u : KC - 1;
            U[b].lw = Wt.lw[b];
            U[b].sw = piece_row(pieces, b * NPL, rr);
            if constexpr (FMT == MOE_FMT_Q2_B32) U[b].mw = piece_row(pieces, b * NPL + 1, rr);
            if constexpr (FMT == MOE_FMT_Q3_B32) U[b].hw = Wt.hw[b];
            if constexpr (!HL) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) U[b].A[mt][j] =
                            *reinterpret_cast<const u32x4 *>(hrow[mt] + u * 128 + j * 32 + gq * 8);
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (u0 + NW * b < KC) {
                if constexpr (HL) {
                    const int u = u0 + NW * b;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int c = u * 16 + j * 4 + gq;
                        U[b].A[0][j] = *reinterpret_cast<const u32x4 *>(hs + ((size_t)srow * cpr + (c ^ (srow & 7))) * 8);
                    }
                }
                if constexpr (SPREAD) {
                    down_block_spread<FMT, 0>(U[b], acs);
                    down_block_spread<FMT, 1>(U[b], acs);
                    down_block_spread<FMT, 2>(U[b], acs);
                    down_block_spread<FMT, 3>(U[b], acs);
                } else {
                    down_block<FMT, MT, IMAX, 0>(U[b], acc);
                    down_block<FMT, MT, IMAX, 1>(U[b], acc);
                    down_block<FMT, MT, IMAX, 2>(U[b], acc);
                    down_block<FMT, MT, IMAX, 3>(U[b], acc);
                }
            }
        }
    }
    if constexpr (NW > 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < RI; ++i) red[wq][mt][i][lane] = SPREAD ? acs[i] : acc[mt][i];
        __syncthreads();
        if (wq == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < RI; ++i) {
                    float v = red[0][mt][i][lane];
#pragma unroll
                    for (int w2 = 1; w2 < NW; ++w2) v += red[w2][mt][i][lane];
                    if constexpr (SPREAD)
                        acs[i] = v;
                    else
                        acc[mt][i] = v;
                }
        }
    }
    if (wq != 0) return;
    if constexpr (SPREAD) {
        // lane group gq: group row gq, h_hi + h_lo in one lane
        const int r = gq;
        if (r < nrows) {
            const float y = ldexpf(acs[0] + acs[1], ya[0][0]);
            const int o = ot * 16 + rr;
            float *dst = grp.expert < 0 ? y_shared + (size_t)r * d + o : y_pairs + (size_t)(grp.row0 + r) * d + o;
            if constexpr (DEV)
                store_dev(dst, y);   // read by another workgroup of this launch
            else
                *dst = y;
        }
        return;
    }
    // hi (rows 0..7, lanes 0..31) + lo (rows 8..15, lanes 32..63)
    const int o = ot * 16 + rr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < IMAX; ++i) {
            const float y = ldexpf(acc[mt][i] + __shfl_xor(acc[mt][i], 32, 64), ya[mt][i]);
            const int r = mt * 8 + gq * 4 + i;
            if (gq >= 2 || r >= nrows) continue;
            float *dst = grp.expert < 0 ? y_shared + (size_t)r * d + o
                                        : y_pairs + (size_t)(grp.row0 + r) * d + o;
            if constexpr (DEV)
                store_dev(dst, y);   // read by another workgroup of this launch
            else
                *dst = y;
        }
}

constexpr int kTileMaxT = 4;    // down_tile_kernel: T <= 4, k <= 16 (pairs and merge in LDS)
constexpr int kTileMaxK = 16;

// The fused combine (moe_combine's sum for one 16-column output tile).  Every
// workgroup of the tile (one per group slot, empty slots included) arrives
// after its y stores have completed at device scope; the last to arrive
// computes out[t][16 ot .. 16 ot + 16) for every token exactly as the
// combine kernel does (shared term first, then j order, one fma per pair)
// and restores the tile's counter to zero.
struct CombineArgs {
    const int32_t *pair_pos;
    const float *w;
    float *out;
    int32_t *counters;   // one per tile, kCntLine apart
    int T, k;
};

__device__ __forceinline__ void combine_tile(const CombineArgs &cb, const float *y_pairs, const float *y_shared,
                                             int d, int ot, int n_arrivals) {
    __shared__ int last;
    int32_t *counter = cb.counters + (size_t)kCntLine * ot;
    publish_then_count(counter, n_arrivals, last);
    if (!last) return;
    constexpr int B = 8;   // pairs whose rows are loaded together
    const int k = cb.k;
    for (int i = threadIdx.x; i < cb.T * 16; i += blockDim.x) {
        const int t = i >> 4, c = ot * 16 + (i & 15);
        const int32_t *pp = cb.pair_pos + (size_t)t * k;
        const float *ww = cb.w + (size_t)t * k;
        float acc = load_dev(y_shared + (size_t)t * d + c);
        for (int j0 = 0; j0 < k; j0 += B) {
            int p[B];
            float wj[B], v[B];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const int j = j0 + b < k ? j0 + b : k - 1;
                p[b] = pp[j];
                wj[b] = ww[j];
            }
#pragma unroll
            for (int b = 0; b < B; ++b) v[b] = load_dev(y_pairs + (size_t)(p[b] >= 0 ? p[b] : 0) * d + c);
#pragma unroll
            for (int b = 0; b < B; ++b)
                if (j0 + b < k && p[b] >= 0) acc = fmaf(wj[b], v[b], acc);
        }
        cb.out[(size_t)t * d + c] = acc;
    }
    if (threadIdx.x == 0) store_dev_int(counter, 0);
}

// ---------------------------------------------------------------- kernels
// grid: (d_ff/16 row tiles, group slots slot0 + blockIdx.y: slot 0 the shared
// expert, slots 1 .. min(E, P) the routed groups); NW waves split K.  The
// first tile of each slot also records the slot's group (nrows 0: none) in
// `table`, so the down kernel reads it with one load.  NB: units each wave
// has in flight per batch (fewer hold fewer registers).
template <int FMT, int IMAX, int NW, bool XL, int TPW, int NB = 16 / NW, int SP = 1>
__global__ __launch_bounds__(64 * NW * TPW) __attribute__((amdgpu_waves_per_eu(IMAX > 2 && NB == 2 ? 5 : 1)))
void gateup_small_kernel(
    QMatDev gate, QMatDev up, QMatDev sgate, QMatDev sup, const uint16_t *__restrict__ x, int T,
    int k, int d, int f, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_pair, uint16_t *__restrict__ h_hi,
    uint16_t *__restrict__ h_lo, int32_t *__restrict__ hx, Group *__restrict__ table, int slot0) {
    __shared__ float red[NW * TPW][2][spread_ri(SP, IMAX)][64];
    __shared__ uint32_t redx[NW * TPW][16];
    // per wave: a batch's scale pieces (16 units' worth: 2 matrices x 2 planes)
    __shared__ u32x4 pieces[NW * TPW][8 * NB * 2 * 2];
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];   // XL: x, T * d halves
    if constexpr (XL) {
        // x [T][d] into LDS once per workgroup by global-to-LDS copies (no
        // registers held), issued first: x does not depend on the group.
        // Chunk c of row r goes to r * cpr + (c ^ (r & 7)), so the T rows
        // read at one column fall in different banks.
        const int cpr = d / 8, nch = T * cpr, lane = __lane_id();
        const int wall = wave_uniform(threadIdx.x >> 6);
        for (int q = wall; q * 64 < nch; q += NW * TPW) {
            const int L = q * 64 + lane;
            if (L < nch) {
                const int r = L / cpr, cs = L - r * cpr;
                copy_to_lds16(x + (size_t)r * d + (size_t)(cs ^ (r & 7)) * 8, xs_dyn + (size_t)q * 512);
            }
        }
    }
    // one wave looks the group up; the others take it from LDS
    __shared__ Group grp_s;
    __shared__ int found_s;
    if (threadIdx.x < 64) {
        Group g;
        const bool f0 = find_group(offsets, E, T, T * k, slot0 + (int)blockIdx.y, g);
        if (threadIdx.x == 0) {
            grp_s = g;
            found_s = f0;
        }
    }
    // meet: every wave's x copies are in LDS and the group is known to all
    // (nothing else is in flight yet, so the full drain costs nothing)
    __syncthreads();
    const Group grp = grp_s;
    const bool found = found_s != 0;
    // the first tile of each slot records the slot's group for the down
    // kernel, after its own loads (a store issued before them would delay
    // them: the memory counter retires in order)
    const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
    if (!found) {
        if (rec) *reinterpret_cast<u32x4 *>(&table[blockIdx.y]) = u32x4{0u, 0u, 0u, 0u};
        return;
    }
    gateup_task<FMT, IMAX, NW, XL, TPW, NB, SP>(gate, up, sgate, sup, x, T, k, d, f, sorted_pair, grp,
                                        (int)blockIdx.x * TPW, red, redx, h_hi, h_lo, hx, xs_dyn, &pieces[0][0]);
    if (rec) *reinterpret_cast<u32x4 *>(&table[blockIdx.y]) = __builtin_bit_cast(u32x4, grp);
}

// grid: (d_model/16 row tiles, group slots); NW waves split K = d_ff.  FUSE:
// the last workgroup of each row tile also computes the tile of out.
template <int FMT, int MT, int IMAX, int NW, bool FUSE, bool HL, bool SPREAD = false>
__global__ __launch_bounds__(64 * NW) void down_small_kernel(
    QMatDev down, QMatDev sdown, const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
    const int32_t *__restrict__ hx, int d, int f, const Group *__restrict__ table, float *__restrict__ y_pairs,
    float *__restrict__ y_shared, CombineArgs cb) {
    __shared__ float red[NW][MT][SPREAD ? 2 : IMAX][64];
    __shared__ u32x4 pieces[NW][64 * PieceGather<kDownBatch * 2>::N];   // per wave: a batch's scale pieces
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];   // HL: the group's h rows
    const Group grp = table[blockIdx.y];   // written by the gate/up kernel
    if (grp.nrows != 0) {
        const int wq = wave_uniform(threadIdx.x >> 6);
        DownW<FMT, MT, NW> Wt;
        down_load_w<FMT, MT, NW>(Wt, down, sdown, d, f, grp, blockIdx.x, wq);
        down_task<FMT, MT, IMAX, NW, FUSE, HL, SPREAD>(Wt, down, sdown, h_hi, h_lo, hx, d, f, grp, blockIdx.x, wq, red,
                                               y_pairs, y_shared, xs_dyn, pieces[wq]);
    }
    if constexpr (FUSE) combine_tile(cb, y_pairs, y_shared, d, blockIdx.x, gridDim.y);
}


// Down projection for batches of at most 4 tokens and d_ff <= 768: one
// workgroup per 16-row output tile and chunk of up to 16 group slots, one
// wave per slot over all of K = d_ff, so no partial sums cross waves.  Each
// wave copies its group's h rows (hi, then lo) into an LDS region of its own
// and waits for nothing but its own copies.  FUSE with a single chunk (T = 1
// at top-10: 11 slots) also merges each token's outputs for the tile in the
// workgroup -- shared term first, then the pairs in j order, one fma each,
// moe_combine's order -- with no counter and no re-read; with several
// chunks each arrives on the tile's counter after its y stores and the last
// one merges from memory (combine_tile).
constexpr int kTileUnits = 6;   // d_ff / 128 <= 6
// LDS halves per wave of down_tile_kernel: the group's h rows (hi and lo, RMAX
// each), and first the scale pieces of its units (a region of whole 64-chunk
// blocks)
template <int FMT, int RMAX>
__host__ __device__ constexpr int tile_region_halves(int f) {
    const int np = kTileUnits * (FMT == MOE_FMT_Q2_B32 ? 2 : 1);
    const int pieces = ((8 * np + 63) / 64) * 64 * 8;
    return 2 * RMAX * f > pieces ? 2 * RMAX * f : pieces;
}
template <int FMT, int RMAX, bool FUSE>
__global__ __launch_bounds__(64 * 16) void down_tile_kernel(
    QMatDev down, QMatDev sdown, const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
    const int32_t *__restrict__ hx, int d, int f, const Group *__restrict__ table, int slots, int nchunks,
    float *__restrict__ y_pairs, float *__restrict__ y_shared, CombineArgs cb) {
    extern __shared__ __attribute__((aligned(16))) uint16_t hs_dyn[];   // per wave: 2 RMAX rows of f halves
    __shared__ float ylds[(kTileMaxT * kTileMaxK + kTileMaxT) * 16];   // y by row (pairs, then shared)
    __shared__ int32_t pp_s[kTileMaxT * kTileMaxK];
    __shared__ float w_s[kTileMaxT * kTileMaxK];
    const int lane = __lane_id(), gq = lane >> 4, rr = lane & 15;
    const int wv = wave_uniform(threadIdx.x >> 6), CH = blockDim.x >> 6;
    const int ot = blockIdx.x, slot = blockIdx.y * CH + wv;
    const int T = cb.T, k = cb.k, P = T * k;
    const bool merge_here = FUSE && nchunks == 1;
    if (merge_here) {
        // the routing of the batch, for the merge (written by earlier kernels)
        for (int i = threadIdx.x; i < P; i += blockDim.x) {
            pp_s[i] = cb.pair_pos[i];
            w_s[i] = cb.w[i];
        }
    }
    Group grp{0, 0, 0, 0};
    if (slot < slots) grp = table[slot];
    const int n = grp.nrows;
    float yv[RMAX];
    if (n > 0) {
        const int KC = f / 128, cpr = f / 8;
        uint16_t *hs = hs_dyn + (size_t)wv * tile_region_halves<FMT, RMAX>(f);
        const bool shared = grp.expert < 0;
        const QMatDev W = shared ? sdown : down;
        const size_t ubase = ((size_t)(shared ? 0 : grp.expert) * (d / 16) + ot) * KC;
        // 0. the block scales (and Q2 minimums) of the wave's units, first:
        //    piece p = unit p / NPL, plane p % NPL (staged through the wave's
        //    h region before h lands there)
        constexpr int NPL = FMT == MOE_FMT_Q2_B32 ? 2 : 1;
        constexpr int NP = kTileUnits * NPL;
        PieceGather<NP> pg;
        {
            const uint64_t sc = (uint64_t)W.scale, mn = (uint64_t)W.min;
            pg.issue([=](int p) {
                const int b = p / NPL;
                uint64_t base = p % NPL ? mn : sc;
                __asm__ volatile("" : "+v"(base));
                return base + (ubase + (b < KC ? b : KC - 1)) * 128;
            });
        }
        // 1. the group's h rows, loaded into registers first and written to
        //    this wave's LDS once they land (register loads, not global-to-LDS
        //    copies: the compiler then waits for exactly these and leaves the
        //    weights in flight; every tile's workgroup reads the same rows, so
        //    they are plain loads that stay in L2).  Stored row S < n is h_hi row S, S >= n h_lo
        //    row S - n; chunk c of row S at S * cpr + (c ^ (S & 7)) (the rows
        //    read at one column fall in different banks).
        constexpr int QMAX = 3 * RMAX;   // 16-byte chunks per lane: 2 RMAX rows of <= 96
        const int nch = 2 * n * cpr;
        u32x4 hv[QMAX];
#pragma unroll
        for (int q = 0; q < QMAX; ++q) {
            const int L = q * 64 + lane < nch ? q * 64 + lane : 0;   // unconditional, clamped
            const int S = L / cpr, cs = L - S * cpr;
            const int hr = S < n ? S : S - n;
            const uint16_t *src = (S < n ? h_hi : h_lo) + (size_t)(grp.hrow0 + hr) * f;
            hv[q] = *reinterpret_cast<const u32x4 *>(src + (size_t)(cs ^ (S & 7)) * 8);
        }
        // 2. the rows' exponents (y = acc 2^2a)
        int ya[RMAX];
#pragma unroll
        for (int i = 0; i < RMAX; ++i) {
            const int r = 4 * gq + i < n ? 4 * gq + i : n - 1;
            ya[i] = 2 * hx[grp.hrow0 + r];
        }
        // 3. all of the wave's codes (unconditional, clamped past KC)
        DownUnit<FMT, 1> U[kTileUnits];
#pragma unroll
        for (int b = 0; b < kTileUnits; ++b) {
            const size_t unit = ubase + (b < KC ? b : KC - 1);
            auto ld = [](const auto *p) { return __builtin_nontemporal_load(p); };
            U[b].lw = ld(reinterpret_cast<const u32x2 *>(W.lo + unit * 512 + lane * 8));
            if constexpr (FMT == MOE_FMT_Q3_B32) U[b].hw = ld(reinterpret_cast<const uint32_t *>(W.hi + unit * 256 + lane * 4));
            __asm__ volatile("" ::: "memory");   // issue in unit order: unit 0 lands first
        }
        // the scales through the h region, then h itself (LDS accesses of one
        // wave complete in order)
        pg.store(reinterpret_cast<u32x4 *>(hs));
#pragma unroll
        for (int b = 0; b < kTileUnits; ++b) {
            U[b].sw = piece_row(reinterpret_cast<const u32x4 *>(hs), b * NPL, rr);
            if constexpr (FMT == MOE_FMT_Q2_B32) U[b].mw = piece_row(reinterpret_cast<const u32x4 *>(hs), b * NPL + 1, rr);
        }
#pragma unroll
        for (int q = 0; q < QMAX; ++q)
            if (q * 64 + lane < nch) *reinterpret_cast<u32x4 *>(hs + (size_t)(q * 64 + lane) * 8) = hv[q];
        const int srow = (rr < 8 ? 0 : n) + ((rr & 7) < n ? (rr & 7) : n - 1);
        f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int b = 0; b < kTileUnits; ++b) {
            if (b < KC) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = b * 16 + j * 4 + gq;
                    U[b].A[0][j] = *reinterpret_cast<const u32x4 *>(hs + ((size_t)srow * cpr + (c ^ (srow & 7))) * 8);
                }
                down_block<FMT, 1, RMAX, 0>(U[b], acc);
                down_block<FMT, 1, RMAX, 1>(U[b], acc);
                down_block<FMT, 1, RMAX, 2>(U[b], acc);
                down_block<FMT, 1, RMAX, 3>(U[b], acc);
            }
        }
        // hi rows (lanes gq 0, 1) + lo rows (gq 2, 3)
#pragma unroll
        for (int i = 0; i < RMAX; ++i) {
            yv[i] = ldexpf(acc[0][i] + __shfl_xor(acc[0][i], 32, 64), ya[i]);
            const int r = 4 * gq + i;
            if (merge_here && gq < 2 && r < n) ylds[(shared ? P + r : grp.row0 + r) * 16 + rr] = yv[i];
        }
    }
    // y to memory: after the merge's barrier when merging here (a barrier
    // waits for this workgroup's outstanding stores to complete)
    auto store_y = [&](bool dev) {
        if (n == 0) return;
        const int o = ot * 16 + rr;
#pragma unroll
        for (int i = 0; i < RMAX; ++i) {
            const int r = 4 * gq + i;
            if (gq >= 2 || r >= n) continue;
            float *dst = grp.expert < 0 ? y_shared + (size_t)r * d + o : y_pairs + (size_t)(grp.row0 + r) * d + o;
            if (dev)
                store_dev(dst, yv[i]);   // read by another workgroup of this launch
            else
                *dst = yv[i];
        }
    };
    if constexpr (!FUSE) {
        store_y(false);
    } else {
        if (!merge_here) {
            store_y(true);
            combine_tile(cb, y_pairs, y_shared, d, ot, nchunks);
            return;
        }
        // only LDS traffic to wait for: no global store is outstanding
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        wg_barrier();
        // shared term first, then j order, one fma per pair (moe_combine's
        // order); the pair positions and weights of a batch of 8 picks, then
        // their y values, are read before the first fma (a read, then a
        // dependent read, per pick cost two LDS round trips each)
        constexpr int B = 8;
        for (int i = threadIdx.x; i < T * 16; i += blockDim.x) {
            const int t = i >> 4, c = i & 15;
            float acc = ylds[(P + t) * 16 + c];
            for (int j0 = 0; j0 < k; j0 += B) {
                int p[B];
                float wj[B], v[B];
#pragma unroll
                for (int b = 0; b < B; ++b) {
                    const int j = j0 + b < k ? j0 + b : k - 1;   // clamped: read, not used
                    p[b] = pp_s[t * k + j];
                    wj[b] = w_s[t * k + j];
                }
#pragma unroll
                for (int b = 0; b < B; ++b) v[b] = ylds[(p[b] >= 0 ? p[b] : 0) * 16 + c];
#pragma unroll
                for (int b = 0; b < B; ++b)
                    if (j0 + b < k && p[b] >= 0) acc = fmaf(wj[b], v[b], acc);
            }
            cb.out[(size_t)t * d + ot * 16 + c] = acc;
        }
        store_y(false);
    }
}

static QMatDev qm(const moe_qmat &m) { return QMatDev{m.lo, m.hi, m.scale, m.min}; }

// h_hi, h_lo [rows][f] (each padded to 128 elements), the group table, then
// the rows' exponents hx [rows]
size_t ffn_small_ws_bytes(int d, int f, int E, int T, int k) {
    (void)d;
    const size_t rows = (size_t)T * k + T;
    const size_t P = (size_t)T * k;
    const size_t slots = 1 + ((size_t)E < P ? (size_t)E : P);
    return 2 * (((rows * f + 127) / 128) * 128) * sizeof(uint16_t) + ((slots * sizeof(Group) + 255) / 256) * 256 +
           rows * sizeof(int32_t) + 256;
}

template <int FMT, int MTD, int IMAX>
static void launch_small_fmt(const moe_layer &L, const uint16_t *x, int T, int k,
                             const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                             float *y_shared, uint16_t *h_hi, uint16_t *h_lo, int32_t *hx, Group *table,
                             int parts, const CombineArgs &cb, hipStream_t s) {
    const int d = L.d_model, f = L.d_ff, E = L.n_experts;
    const int P = T * k;
    const int slot0 = (parts & kFfnShared) ? 0 : 1;
    const int slots = ((parts & kFfnShared) ? 1 : 0) + ((parts & kFfnRouted) ? (E < P ? E : P) : 0);
    if (slots == 0) return;
#ifndef MOE_GU_WAVES
#define MOE_GU_WAVES 8
#endif
#ifndef MOE_DN_WAVES
#define MOE_DN_WAVES 2
#endif
    // waves per workgroup (split K): eight for one or two tokens; from three
    // tokens on there are enough groups that four keep more workgroups resident
    constexpr int NWG = IMAX <= 2 ? MOE_GU_WAVES : 4, NWD = MOE_DN_WAVES;
    // up to eight tokens: x staged in LDS (32 KiB at most), which frees the
    // registers that held it, so more waves keep weight loads in flight, and
    // reads each x byte from L2 once per workgroup instead of once per wave
    // and lane group
    const size_t xbytes = (size_t)T * d * 2;
    // one token (and k <= 16, d_ff <= 768): the down projection runs per
    // 16-column output tile (down_tile_kernel), one wave per group.  Without
    // the merge, eight or more group slots are split over two workgroups per
    // tile, so all CUs take part (FFN 13.7 -> 13.0 us at T = 1, top-10);
    // with it, one workgroup holds every group of its tile and merges in LDS
    // (a merge across two workgroups, through device-scope float adds into
    // a cleared out, took the fused call from 14.7 to 21 us)
    const bool tile_path = MTD == 1 && T == 1 && k <= kTileMaxK && f <= 128 * kTileUnits && f % 128 == 0;
    int CH = 0, nchunks = 0;
    unsigned tile_lds = 0;
    if (tile_path) {
        CH = !cb.out && slots >= 8 ? (slots + 1) / 2 : slots;
        CH = CH < 16 ? CH : 16;
        const int region = tile_region_halves<FMT, IMAX>(f) * 2;   // bytes per wave
        const int lds_ch = 49152 / region;                          // waves whose regions fit 48 KiB
        CH = CH < lds_ch ? CH : lds_ch;
        nchunks = (slots + CH - 1) / CH;
        tile_lds = (unsigned)(CH * region);
    }
    if (IMAX > 2 && T <= 4 && xbytes <= kXsMaxBytes)
        // three or four tokens: batches of two units per wave, so that five
        // workgroups fit a CU (96 VGPRs, 28 KiB of LDS) and every real
        // group's workgroups are resident at once (with four-unit batches,
        // 124 VGPRs, only four fit and the last groups ran as a second
        // round: workload 2 +3.5%, T = 4 Q2 +3%; at T = 8 it lost 0.5%)
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, true, 1, 2, 4>), dim3(f / 16, slots),
                           dim3(64 * NWG), (unsigned)xbytes, s, qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up),
                           x, T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, hx, table, slot0);
    else if (IMAX == 2 && xbytes <= kXsMaxBytes)
        // two tokens: rows 0-3 and 4-7, one epilogue FMA per matrix
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, true, 1, 16 / NWG, 4>), dim3(f / 16, slots),
                           dim3(64 * NWG), (unsigned)xbytes, s, qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up),
                           x, T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, hx, table, slot0);
    else if (T <= 8 && xbytes <= kXsMaxBytes)
        // five to eight tokens: two rows per token
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, true, 1, 16 / NWG, IMAX == 4 ? 2 : 1>), dim3(f / 16, slots),
                           dim3(64 * NWG), (unsigned)xbytes, s, qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up),
                           x, T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, hx, table, slot0);
    else if (IMAX >= 2 && T <= 16 && xbytes <= 2 * kXsMaxBytes && (f / 16) % 2 == 0)
        // 9 to 16 tokens: x takes up to 64 KiB, so one workgroup of eight
        // waves serves two column tiles with one copy
        // (four waves per tile: the LDS of x and of eight waves' sums would
        // pass 64 KiB)
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, 4, IMAX >= 2, IMAX >= 2 ? 2 : 1>), dim3(f / 32, slots),
                           dim3(2 * 64 * 4), (unsigned)xbytes, s, qm(L.gate), qm(L.up), qm(L.sh_gate),
                           qm(L.sh_up), x, T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, hx, table, slot0);
    else
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, false, 1>), dim3(f / 16, slots),
                           dim3(64 * NWG), 0, s, qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up), x,
                           T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, hx, table, slot0);
    // one token: the tile kernel (measured at T = 4 with 41 groups in chunks
    // of 4 it lost to one workgroup per group and tile)
    if (tile_path) {
        constexpr int RMAX = IMAX;
        const unsigned lds = tile_lds;
        if (cb.out)
            hipLaunchKernelGGL((down_tile_kernel<FMT, RMAX, true>), dim3(d / 16, nchunks), dim3(64 * CH), lds, s,
                               qm(L.down), qm(L.sh_down), h_hi, h_lo, hx, d, f, table, slots, nchunks, y_pairs,
                               y_shared, cb);
        else
            hipLaunchKernelGGL((down_tile_kernel<FMT, RMAX, false>), dim3(d / 16, nchunks), dim3(64 * CH), lds, s,
                               qm(L.down), qm(L.sh_down), h_hi, h_lo, hx, d, f, table, slots, nchunks, y_pairs,
                               y_shared, cb);
        return;
    }
    // up to four tokens: the group's h rows (at most T of hi and of lo)
    // staged in LDS (measured: T = 1 +0.7%, T = 2 +9%, T = 4 +3% on Q2,
    // neutral on Q3; at T = 8 it lost 1.5%)
    const size_t hbytes = (size_t)2 * T * f * 2;
    constexpr bool HLOK = MTD == 1;
    const bool hl = HLOK && T <= 4 && hbytes <= kXsMaxBytes;
    // up to 4 tokens (groups of at most 4 rows): the spread row form
    auto launch_down = [&](auto spread_c) {
        constexpr bool SP = decltype(spread_c)::value;
        if (cb.out && hl)
            hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, true, HLOK, SP>), dim3(d / 16, slots),
                               dim3(64 * NWD), (unsigned)hbytes, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, hx, d, f,
                               table, y_pairs, y_shared, cb);
        else if (cb.out)
            hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, true, false, SP>), dim3(d / 16, slots),
                               dim3(64 * NWD), 0, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, hx, d, f, table,
                               y_pairs, y_shared, cb);
        else if (hl)
            hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, false, HLOK, SP>), dim3(d / 16, slots),
                               dim3(64 * NWD), (unsigned)hbytes, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, hx, d, f,
                               table, y_pairs, y_shared, cb);
        else
            hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, false, false, SP>), dim3(d / 16, slots),
                               dim3(64 * NWD), 0, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, hx, d, f, table,
                               y_pairs, y_shared, cb);
    };
    if constexpr (MTD == 1) {
        if (T <= 4) {
            launch_down(std::true_type{});
            return;
        }
    }
    launch_down(std::false_type{});
}

template <int FMT>
static void launch_small_t(const moe_layer &L, const uint16_t *x, int T, int k,
                           const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                           float *y_shared, uint16_t *h_hi, uint16_t *h_lo, int32_t *hx, Group *table,
                           int parts, const CombineArgs &cb, hipStream_t s) {
    // down M tiles: 8 rows (hi over lo) per tile; gate/up: one 16-token tile
    if (T == 1)
        launch_small_fmt<FMT, 1, 1>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, hx, table,
                                    parts, cb, s);
    else if (T == 2)
        launch_small_fmt<FMT, 1, 2>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, hx, table,
                                    parts, cb, s);
    else if (T <= 8)
        launch_small_fmt<FMT, 1, 4>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, hx, table,
                                    parts, cb, s);
    else   // T <= 16
        launch_small_fmt<FMT, 2, 4>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, hx, table,
                                    parts, cb, s);
}

hipError_t launch_ffn_small(const moe_layer &L, const uint16_t *x, int T, int k,
                            const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                            float *y_shared, void *ws, int parts, hipStream_t s,
                            const int32_t *pair_pos, const float *topk_w, float *out) {
    const size_t rows = (size_t)T * k + T;
    uint16_t *h_hi = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + kWsHeader);
    uint16_t *h_lo = h_hi + ((rows * L.d_ff + 127) / 128) * 128;
    Group *table = reinterpret_cast<Group *>(h_lo + ((rows * L.d_ff + 127) / 128) * 128);
    const size_t slots = 1 + ((size_t)L.n_experts < (size_t)T * k ? (size_t)L.n_experts : (size_t)T * k);
    int32_t *hx = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(table) +
                                              ((slots * sizeof(Group) + 255) / 256) * 256);
    const CombineArgs cb{pair_pos, topk_w, out,
                         reinterpret_cast<int32_t *>(static_cast<char *>(ws) + kCombineCnt), T, k};
    if (L.format == MOE_FMT_Q2_B32)
        launch_small_t<MOE_FMT_Q2_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, hx, table,
                                        parts, cb, s);
    else
        launch_small_t<MOE_FMT_Q3_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, hx, table,
                                        parts, cb, s);
    return hipGetLastError();
}

}  // namespace moe
