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
//     (two masks + four converts per 16 codes); Q3's third bit is a second
//     operand holding 4*bit;
//   - the 32-wide K block is exactly one 16x16x32 matrix-core step, so the
//     product codes x activations comes out per block, and the block scale and
//     minimum are applied in fp32: acc += d*P + m*X (Q2) or d*(P - 4X) (Q3),
//     X = sum of the block's activations (a matrix-core step against ones).
//   Weights are therefore used exactly (no rounding of d*q + m), and all sums
//   are fp32.
//   - gate/up: A = the batch's x rows (bf16, exact; each group row then takes
//     its token's sums); h = silu(g)*u in fp32 is written as fp16 hi + fp16
//     lo (22 significant bits).
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

template <int FMT, int MT>
__device__ __forceinline__ void gateup_load_w(GateUpUnit<FMT, MT> &U, const QMatDev &Wg,
                                              const QMatDev &Wu, size_t unit, int lane, int rr) {
    // each weight is read once per call: nontemporal
    auto ld = [](const auto *p) { return __builtin_nontemporal_load(p); };
    U.lg = ld(reinterpret_cast<const u32x2 *>(Wg.lo + unit * 512 + lane * 8));
    U.lu = ld(reinterpret_cast<const u32x2 *>(Wu.lo + unit * 512 + lane * 8));
    if constexpr (FMT == MOE_FMT_Q3_B32) {
        U.hg = ld(reinterpret_cast<const uint32_t *>(Wg.hi + unit * 256 + lane * 4));
        U.hu = ld(reinterpret_cast<const uint32_t *>(Wu.hi + unit * 256 + lane * 4));
    }
    U.sg = ld(reinterpret_cast<const u32x2 *>(Wg.scale + unit * 64 + rr * 4));
    U.su = ld(reinterpret_cast<const u32x2 *>(Wu.scale + unit * 64 + rr * 4));
    if constexpr (FMT == MOE_FMT_Q2_B32) {
        U.mg = ld(reinterpret_cast<const u32x2 *>(Wg.min + unit * 64 + rr * 4));
        U.mu = ld(reinterpret_cast<const u32x2 *>(Wu.min + unit * 64 + rr * 4));
    }
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

template <int J, bool F16, int FMT>
__device__ __forceinline__ void block_operands(uint32_t lo_dw, uint32_t hi_w, u32x4 &B, u32x4 &H) {
    B = lo_operand<J & 1, F16>(lo_dw);
    if constexpr (FMT == MOE_FMT_Q3_B32) H = hi_operand<J, F16>(hi_w);
}

__device__ __forceinline__ float half_of(const u32x2 &v, int j) {
    return half_bits_to_float((uint16_t)(v[j >> 1] >> (16 * (j & 1))));
}

// IMAX = number of valid D rows per lane group i (compile time): 1 for a
// single-token batch, 2 for two tokens, 4 otherwise.  The epilogue touches
// only those rows, so small batches pay no selects.
template <int FMT, int MT, int IMAX, int J>
__device__ __forceinline__ void gateup_block(const GateUpUnit<FMT, MT> &U, f32x4 *ag, f32x4 *au) {
    const u32x4 ones = {kOneBf16x2, kOneBf16x2, kOneBf16x2, kOneBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    u32x4 Bg, Bu, Hg, Hu;
    block_operands<J, false, FMT>(U.lg[J >> 1], U.hg, Bg, Hg);
    block_operands<J, false, FMT>(U.lu[J >> 1], U.hu, Bu, Hu);
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
            pg = mfma_bf16(U.A[mt][J], Hg, pg);
            pu = mfma_bf16(U.A[mt][J], Hu, pu);
        }
        const f32x4 xs = mfma_bf16(U.A[mt][J], ones, zero);
#pragma unroll
        for (int i = 0; i < IMAX; ++i) {
            if constexpr (FMT == MOE_FMT_Q2_B32) {
                ag[mt][i] = fmaf(dg, pg[i], fmaf(mgv, xs[i], ag[mt][i]));
                au[mt][i] = fmaf(du, pu[i], fmaf(muv, xs[i], au[mt][i]));
            } else {
                ag[mt][i] = fmaf(dg, fmaf(-4.0f, xs[i], pg[i]), ag[mt][i]);
                au[mt][i] = fmaf(du, fmaf(-4.0f, xs[i], pu[i]), au[mt][i]);
            }
        }
    }
}

#ifndef MOE_DECODE_BATCH
#define MOE_DECODE_BATCH 4
#endif
constexpr int kBatch = MOE_DECODE_BATCH;   // units prefetched per wave per batch
// down: K = d_ff = 768 is 6 units, 3 per wave of two; a batch of 4 held a
// fourth, unused unit's registers (166 -> 128 VGPRs at 16 tokens)
constexpr int kDownBatch = 3;

constexpr size_t kXsMaxBytes = 32768;   // x staged in LDS by the gate/up kernel (up to 8 tokens)
constexpr int kPfPieces = 4;   // 16-byte pieces per thread (covers 3 down tiles)

// The down-projection weights of output tiles ot = nt, nt + G, nt + 2G, ...
// (G gate/up tiles per group: with G and the down grid's width multiples of
// 8, each such tile's down workgroup runs on the XCD of this one), read while
// the gate/up work runs so that the down kernel finds them in the caches
// instead of paying a full memory latency after its group lookup.  The
// values are only held until the caller consumes them.  Used for single-token
// batches (11 groups): there the FFN gains ~0.6 us; with 4 or 16 tokens (22
// to 140 groups) the extra loads slowed gate/up by more than down gained.
template <int FMT>
__device__ __forceinline__ void down_prefetch(u32x4 (&pf)[kPfPieces], const QMatDev &down,
                                              const QMatDev &sdown, int d, int f, const Group &grp,
                                              int nt, int G) {
    const QMatDev W = grp.expert < 0 ? sdown : down;
    const int e = grp.expert < 0 ? 0 : grp.expert;
    const int KC = f / 128, OT = d / 16;
    // pieces of one tile: codes (32 per unit), Q3 third bits (16), scales (8), Q2 minimums (8)
    const int n_lo = KC * 32, n_hi = FMT == MOE_FMT_Q3_B32 ? KC * 16 : 0, n_sc = KC * 8;
    const int P = n_lo + n_hi + 2 * n_sc - (FMT == MOE_FMT_Q3_B32 ? n_sc : 0);
    const int ntile = (OT - nt + G - 1) / G;   // tiles nt + G m < OT
#pragma unroll
    for (int i = 0; i < kPfPieces; ++i) {
        int q = (int)threadIdx.x + (int)blockDim.x * i;
        q = q < ntile * P ? q : 0;   // unconditional loads: spare threads re-read piece 0
        const int tq = q / P, pp = q - tq * P;
        int ot = nt + G * tq;
        ot = ot < OT ? ot : OT - 1;   // (only when no tile is left: f > d)
        const size_t ub = ((size_t)e * OT + ot) * KC;
        const uint8_t *src;
        if (pp < n_lo)
            src = W.lo + ub * 512 + (size_t)pp * 16;
        else if (pp < n_lo + n_hi)
            src = W.hi + ub * 256 + (size_t)(pp - n_lo) * 16;
        else if (pp < n_lo + n_hi + n_sc)
            src = reinterpret_cast<const uint8_t *>(W.scale) + ub * 128 + (size_t)(pp - n_lo - n_hi) * 16;
        else
            src = reinterpret_cast<const uint8_t *>(W.min) + ub * 128 + (size_t)(pp - n_lo - n_hi - n_sc) * 16;
        pf[i] = *reinterpret_cast<const u32x4 *>(src);
    }
}

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
template <int FMT, int IMAX, int NW, bool XL, int TPW>
__device__ __forceinline__ void gateup_task(const QMatDev &gate, const QMatDev &up, const QMatDev &sgate,
                                            const QMatDev &sup, const uint16_t *__restrict__ x, int T, int k, int d,
                                            int f, const int32_t *__restrict__ sorted_pair, const Group &grp,
                                            int nt, float (*red)[2][IMAX][64], uint16_t *__restrict__ h_hi,
                                            uint16_t *__restrict__ h_lo, const QMatDev &down,
                                            const QMatDev &sdown, uint16_t *xs) {
    static_assert(NW > 1, "token rows: K split over waves");
    static_assert(TPW == 1 || XL, "several tiles per workgroup share the staged x");
    constexpr bool kPrefetch = IMAX == 1 && TPW == 1;   // single-token batch
    const int lane = __lane_id();
    // TPW tiles per workgroup: waves [NW g, NW g + NW) take tile nt + g
    const int wall = wave_uniform(threadIdx.x >> 6);
    const int wv = wall % NW, tg = wall / NW;
    nt += tg;
    red += tg * NW;
    const int gq = lane >> 4, rr = lane & 15;
    const bool shared = grp.expert < 0;
    const QMatDev Wg = shared ? sgate : gate;
    const QMatDev Wu = shared ? sup : up;
    const int e = shared ? 0 : grp.expert;
    const int KC = d / 128;
    const size_t ubase = ((size_t)e * (f / 16) + nt) * KC;
    const int nrows = grp.nrows;

    // token of output row 4 gq + i; lanes past the group's last row use its
    // last row (never stored), so the loads are unconditional and go out
    // together, before the weights
    int otok[IMAX];
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
        int r = 4 * gq + i;
        r = r < nrows ? r : nrows - 1;
        otok[i] = shared ? r : sorted_pair[grp.row0 + r];
    }
    f32x4 ag[1], au[1];
    ag[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    au[0] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int xr = rr < T ? rr : T - 1;   // the token row of this lane's matrix row
    const uint16_t *xrow[1] = {x + (size_t)xr * d};
    const int cpr = d / 8;                // 16-byte chunks per x row
    u32x4 pf[kPfPieces];
    GateUpUnit<FMT, 1> U[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        const int u = wv + NW * b;
        if (u < KC) gateup_load_w(U[b], Wg, Wu, ubase + u, lane, rr);
    }
    if constexpr (XL) {
        // x [T][d] into LDS once per workgroup by global-to-LDS copies (no
        // registers held): chunk c of row r goes to r * cpr + (c ^ (r & 7)),
        // so the T rows read at one column fall in different banks
        const int nch = T * cpr;
        for (int q = wall; q * 64 < nch; q += NW * TPW) {
            const int L = q * 64 + lane;
            if (L < nch) {
                const int r = L / cpr, cs = L - r * cpr;
                copy_to_lds16(x + (size_t)r * d + (size_t)(cs ^ (r & 7)) * 8, xs + (size_t)q * 512);
            }
        }
        wait_vm<0>();   // the copies and the first weights
        __syncthreads();
    }
    for (int u0 = wv; u0 < KC; u0 += NW * kBatch) {
        if (u0 != wv) {
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int u = u0 + NW * b;
                if (u < KC) gateup_load_w(U[b], Wg, Wu, ubase + u, lane, rr);
            }
        }
        __asm__ volatile("" ::: "memory");
        if constexpr (!XL) {
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int u = u0 + NW * b;
                if (u < KC) gateup_load_x(U[b], u, gq, xrow);
            }
        }
        if (kPrefetch && u0 == wv) {
            __asm__ volatile("" ::: "memory");
            down_prefetch<FMT>(pf, down, sdown, d, f, grp, nt, f / 16);
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
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
                gateup_block<FMT, 1, IMAX, 0>(U[b], ag, au);
                gateup_block<FMT, 1, IMAX, 1>(U[b], ag, au);
                gateup_block<FMT, 1, IMAX, 2>(U[b], ag, au);
                gateup_block<FMT, 1, IMAX, 3>(U[b], ag, au);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
        red[wv][0][i][lane] = ag[0][i];
        red[wv][1][i][lane] = au[0][i];
    }
    __syncthreads();
    if (wv != 0) {
        if constexpr (kPrefetch)
#pragma unroll
            for (int i = 0; i < kPfPieces; ++i) __asm__ volatile("" ::"v"(pf[i]));
        return;
    }
    // output row r = 4 gq + i takes the sums of its token's matrix row
    const int n = nt * 16 + rr;
#pragma unroll
    for (int i = 0; i < IMAX; ++i) {
        const int r = 4 * gq + i;
        if (r >= nrows) continue;
        const int t = shared ? otok[i] : otok[i] / k;
        const int sl = (t >> 2) * 16 + rr, si = t & 3;
        float gs = red[0][0][si][sl], us = red[0][1][si][sl];
#pragma unroll
        for (int w2 = 1; w2 < NW; ++w2) {
            gs += red[w2][0][si][sl];
            us += red[w2][1][si][sl];
        }
        const float h = swiglu(gs, us);
        const _Float16 hh = static_cast<_Float16>(h);
        const float rem = h - static_cast<float>(hh);
        const size_t off = (size_t)(grp.hrow0 + r) * f + n;
        h_hi[off] = __builtin_bit_cast(uint16_t, hh);
        h_lo[off] = f32_to_f16_bits(rem);
    }
    if constexpr (kPrefetch)
#pragma unroll
        for (int i = 0; i < kPfPieces; ++i) __asm__ volatile("" ::"v"(pf[i]));
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
    u32x4 B, H;
    block_operands<J, true, FMT>(U.lw[J >> 1], U.hw, B, H);
    const float dv = half_of(U.sw, J);
    float mv = 0.f;
    if constexpr (FMT == MOE_FMT_Q2_B32) mv = half_of(U.mw, J);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        f32x4 p = mfma_f16(U.A[mt][J], B, zero);
        if constexpr (FMT == MOE_FMT_Q3_B32) p = mfma_f16(U.A[mt][J], H, p);
        const f32x4 hs = mfma_f16(U.A[mt][J], ones, zero);
#pragma unroll
        for (int i = 0; i < IMAX; ++i) {
            if constexpr (FMT == MOE_FMT_Q2_B32)
                acc[mt][i] = fmaf(dv, p[i], fmaf(mv, hs[i], acc[mt][i]));
            else
                acc[mt][i] = fmaf(dv, fmaf(-4.0f, hs[i], p[i]), acc[mt][i]);
        }
    }
}

// Down-projection weights of one batch of a wave's units (units u0 + NW b),
// loadable before h is needed: the weights do not depend on it.
template <int FMT, int MT, int NW>
struct DownW {
    static constexpr int NB = kDownBatch;
    u32x2 lw[NB], sw[NB], mw[NB];
    uint32_t hw[NB];
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
#pragma unroll
    for (int b = 0; b < DownW<FMT, MT, NW>::NB; ++b) {
        int u = u0 + NW * b;
        u = u < KC ? u : KC - 1;   // clamped: unconditional loads, unused past KC
        const size_t unit = ubase + u;
        auto ld = [](const auto *p) { return __builtin_nontemporal_load(p); };   // read once
        Wt.lw[b] = ld(reinterpret_cast<const u32x2 *>(W.lo + unit * 512 + lane * 8));
        if constexpr (FMT == MOE_FMT_Q3_B32) Wt.hw[b] = ld(reinterpret_cast<const uint32_t *>(W.hi + unit * 256 + lane * 4));
        Wt.sw[b] = ld(reinterpret_cast<const u32x2 *>(W.scale + unit * 64 + rr * 4));
        if constexpr (FMT == MOE_FMT_Q2_B32) Wt.mw[b] = ld(reinterpret_cast<const u32x2 *>(W.min + unit * 64 + rr * 4));
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
template <int FMT, int MT, int IMAX, int NW, bool DEV, bool HL>
__device__ __forceinline__ void down_task(DownW<FMT, MT, NW> &Wt, const QMatDev &down, const QMatDev &sdown,
                                          const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
                                          int d, int f, const Group &grp, int ot, int wq,
                                          float (*red)[MT][IMAX][64], float *__restrict__ y_pairs,
                                          float *__restrict__ y_shared, uint16_t *hs) {
    static_assert(!HL || MT == 1, "staged h: groups of at most 8 rows");
    const int lane = __lane_id();
    const int gq = lane >> 4, rr = lane & 15;
    const int KC = f / 128;
    const int nrows = grp.nrows;
    const int cpr = f / 8;
    const uint16_t *hrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        int r = mt * 8 + (rr & 7);
        r = r < nrows ? r : nrows - 1;
        hrow[mt] = (rr < 8 ? h_hi : h_lo) + (size_t)(grp.hrow0 + r) * f;
    }
    int srow = 0;   // HL: this lane's stored row
    if constexpr (HL) {
        const int r = (rr & 7) < nrows ? (rr & 7) : nrows - 1;
        srow = (rr < 8 ? 0 : nrows) + r;
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
    constexpr int NB = DownW<FMT, MT, NW>::NB;
    for (int u0 = wq; u0 < KC; u0 += NW * NB) {
        if (u0 != wq) down_load_w<FMT, MT, NW>(Wt, down, sdown, d, f, grp, ot, u0);
        DownUnit<FMT, MT> U[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int u = u0 + NW * b;
            u = u < KC ? u : KC - 1;
            U[b].lw = Wt.lw[b];
            U[b].sw = Wt.sw[b];
            if constexpr (FMT == MOE_FMT_Q2_B32) U[b].mw = Wt.mw[b];
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
                down_block<FMT, MT, IMAX, 0>(U[b], acc);
                down_block<FMT, MT, IMAX, 1>(U[b], acc);
                down_block<FMT, MT, IMAX, 2>(U[b], acc);
                down_block<FMT, MT, IMAX, 3>(U[b], acc);
            }
        }
    }
    if constexpr (NW > 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < IMAX; ++i) red[wq][mt][i][lane] = acc[mt][i];
        __syncthreads();
        if (wq == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < IMAX; ++i) {
                    float v = red[0][mt][i][lane];
#pragma unroll
                    for (int w2 = 1; w2 < NW; ++w2) v += red[w2][mt][i][lane];
                    acc[mt][i] = v;
                }
        }
    }
    if (wq != 0) return;
    // hi (rows 0..7, lanes 0..31) + lo (rows 8..15, lanes 32..63)
    const int o = ot * 16 + rr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < IMAX; ++i) {
            const float y = acc[mt][i] + __shfl_xor(acc[mt][i], 32, 64);
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
// `table`, so the down kernel reads it with one load.
template <int FMT, int IMAX, int NW, bool XL, int TPW>
__global__ __launch_bounds__(64 * NW * TPW) void gateup_small_kernel(
    QMatDev gate, QMatDev up, QMatDev sgate, QMatDev sup, const uint16_t *__restrict__ x, int T,
    int k, int d, int f, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_pair, uint16_t *__restrict__ h_hi,
    uint16_t *__restrict__ h_lo, Group *__restrict__ table, QMatDev down, QMatDev sdown, int slot0) {
    __shared__ float red[NW * TPW][2][IMAX][64];
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];   // XL: x, T * d halves
    Group grp;
    const bool found = find_group(offsets, E, T, T * k, slot0 + (int)blockIdx.y, grp);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const Group none{0, 0, 0, 0};
        *reinterpret_cast<u32x4 *>(&table[blockIdx.y]) = __builtin_bit_cast(u32x4, found ? grp : none);
    }
    if (!found) return;
    gateup_task<FMT, IMAX, NW, XL, TPW>(gate, up, sgate, sup, x, T, k, d, f, sorted_pair, grp,
                                        (int)blockIdx.x * TPW, red, h_hi, h_lo, down, sdown, xs_dyn);
}

// grid: (d_model/16 row tiles, group slots); NW waves split K = d_ff.  FUSE:
// the last workgroup of each row tile also computes the tile of out.
template <int FMT, int MT, int IMAX, int NW, bool FUSE, bool HL>
__global__ __launch_bounds__(64 * NW) void down_small_kernel(
    QMatDev down, QMatDev sdown, const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
    int d, int f, const Group *__restrict__ table, float *__restrict__ y_pairs,
    float *__restrict__ y_shared, CombineArgs cb) {
    __shared__ float red[NW][MT][IMAX][64];
    extern __shared__ __attribute__((aligned(16))) uint16_t xs_dyn[];   // HL: the group's h rows
    const Group grp = table[blockIdx.y];   // written by the gate/up kernel
    if (grp.nrows != 0) {
        const int wq = wave_uniform(threadIdx.x >> 6);
        DownW<FMT, MT, NW> Wt;
        down_load_w<FMT, MT, NW>(Wt, down, sdown, d, f, grp, blockIdx.x, wq);
        down_task<FMT, MT, IMAX, NW, FUSE, HL>(Wt, down, sdown, h_hi, h_lo, d, f, grp, blockIdx.x, wq, red,
                                               y_pairs, y_shared, xs_dyn);
    }
    if constexpr (FUSE) combine_tile(cb, y_pairs, y_shared, d, blockIdx.x, gridDim.y);
}

static QMatDev qm(const moe_qmat &m) { return QMatDev{m.lo, m.hi, m.scale, m.min}; }

// h_hi, h_lo [rows][f] (each padded to 128 elements), then the group table
size_t ffn_small_ws_bytes(int d, int f, int E, int T, int k) {
    (void)d;
    const size_t rows = (size_t)T * k + T;
    const size_t P = (size_t)T * k;
    const size_t slots = 1 + ((size_t)E < P ? (size_t)E : P);
    return 2 * (((rows * f + 127) / 128) * 128) * sizeof(uint16_t) + slots * sizeof(Group) + 256;
}

template <int FMT, int MTD, int IMAX>
static void launch_small_fmt(const moe_layer &L, const uint16_t *x, int T, int k,
                             const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                             float *y_shared, uint16_t *h_hi, uint16_t *h_lo, Group *table, int parts,
                             const CombineArgs &cb, hipStream_t s) {
    const int d = L.d_model, f = L.d_ff, E = L.n_experts;
    const int P = T * k;
    const int slot0 = (parts & kFfnShared) ? 0 : 1;
    const int slots = ((parts & kFfnShared) ? 1 : 0) + ((parts & kFfnRouted) ? (E < P ? E : P) : 0);
    if (slots == 0) return;
#ifndef MOE_GU_WAVES
#define MOE_GU_WAVES 4
#endif
#ifndef MOE_DN_WAVES
#define MOE_DN_WAVES 2
#endif
    constexpr int NWG = MOE_GU_WAVES, NWD = MOE_DN_WAVES;   // waves per workgroup (split K)
    // up to eight tokens: x staged in LDS (32 KiB at most), which frees the
    // registers that held it, so more waves keep weight loads in flight, and
    // reads each x byte from L2 once per workgroup instead of once per wave
    // and lane group
    const size_t xbytes = (size_t)T * d * 2;
    if (T <= 8 && xbytes <= kXsMaxBytes)
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, true, 1>), dim3(f / 16, slots),
                           dim3(64 * NWG), (unsigned)xbytes, s, qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up),
                           x, T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, table, qm(L.down), qm(L.sh_down),
                           slot0);
    else if (IMAX >= 2 && T <= 16 && xbytes <= 2 * kXsMaxBytes && (f / 16) % 2 == 0)
        // 9 to 16 tokens: x takes up to 64 KiB, so one workgroup of eight
        // waves serves two column tiles with one copy
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, IMAX >= 2, IMAX >= 2 ? 2 : 1>), dim3(f / 32, slots),
                           dim3(2 * 64 * NWG), (unsigned)xbytes, s, qm(L.gate), qm(L.up), qm(L.sh_gate),
                           qm(L.sh_up), x, T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, table, qm(L.down),
                           qm(L.sh_down), slot0);
    else
        hipLaunchKernelGGL((gateup_small_kernel<FMT, IMAX, NWG, false, 1>), dim3(f / 16, slots),
                           dim3(64 * NWG), 0, s, qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up), x,
                           T, k, d, f, E, offsets, sorted_pair, h_hi, h_lo, table, qm(L.down), qm(L.sh_down),
                           slot0);
    // up to four tokens: the group's h rows (at most T of hi and of lo)
    // staged in LDS (measured: T = 1 +0.7%, T = 2 +9%, T = 4 +3% on Q2,
    // neutral on Q3; at T = 8 it lost 1.5%)
    const size_t hbytes = (size_t)2 * T * f * 2;
    constexpr bool HLOK = MTD == 1;
    const bool hl = HLOK && T <= 4 && hbytes <= kXsMaxBytes;
    if (cb.out && hl)
        hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, true, HLOK>), dim3(d / 16, slots),
                           dim3(64 * NWD), (unsigned)hbytes, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, d, f,
                           table, y_pairs, y_shared, cb);
    else if (cb.out)
        hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, true, false>), dim3(d / 16, slots),
                           dim3(64 * NWD), 0, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, d, f, table,
                           y_pairs, y_shared, cb);
    else if (hl)
        hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, false, HLOK>), dim3(d / 16, slots),
                           dim3(64 * NWD), (unsigned)hbytes, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, d, f,
                           table, y_pairs, y_shared, cb);
    else
        hipLaunchKernelGGL((down_small_kernel<FMT, MTD, IMAX, NWD, false, false>), dim3(d / 16, slots),
                           dim3(64 * NWD), 0, s, qm(L.down), qm(L.sh_down), h_hi, h_lo, d, f, table,
                           y_pairs, y_shared, cb);
}

template <int FMT>
static void launch_small_t(const moe_layer &L, const uint16_t *x, int T, int k,
                           const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                           float *y_shared, uint16_t *h_hi, uint16_t *h_lo, Group *table, int parts,
                           const CombineArgs &cb, hipStream_t s) {
    // down M tiles: 8 rows (hi over lo) per tile; gate/up: one 16-token tile
    if (T == 1)
        launch_small_fmt<FMT, 1, 1>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, table,
                                    parts, cb, s);
    else if (T == 2)
        launch_small_fmt<FMT, 1, 2>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, table,
                                    parts, cb, s);
    else if (T <= 8)
        launch_small_fmt<FMT, 1, 4>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, table,
                                    parts, cb, s);
    else   // T <= 16
        launch_small_fmt<FMT, 2, 4>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, table,
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
    const CombineArgs cb{pair_pos, topk_w, out,
                         reinterpret_cast<int32_t *>(static_cast<char *>(ws) + kCombineCnt), T, k};
    if (L.format == MOE_FMT_Q2_B32)
        launch_small_t<MOE_FMT_Q2_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, table,
                                        parts, cb, s);
    else
        launch_small_t<MOE_FMT_Q3_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, table,
                                        parts, cb, s);
    return hipGetLastError();
}

}  // namespace moe
