// ffn_small.hip -- expert FFN when every expert group has few rows (decode,
// MTP verify: T <= 32 tokens).
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
//   - gate/up: A = x rows of the group (bf16, exact); h = silu(g)*u in fp32 is
//     written as fp16 hi + fp16 lo (22 significant bits).
//   - down: A stacks the group's h_hi rows over its h_lo rows in one 16-row
//     tile, so one fp16 matrix-core step covers both halves.
//   - four waves of a workgroup split K; partial sums meet in LDS in a fixed
//     order.
#include "common.h"

namespace moe {

constexpr uint32_t kOneBf16x2 = 0x3F803F80u;
constexpr uint32_t kOneF16x2 = 0x3C003C00u;

__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

template <int FMT, int MT>
__global__ __launch_bounds__(256) void gateup_small_kernel(
    QMatDev gate, QMatDev up, QMatDev sgate, QMatDev sup, const uint16_t *__restrict__ x, int T,
    int k, int d, int f, int E, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ sorted_pair, uint16_t *__restrict__ h_hi,
    uint16_t *__restrict__ h_lo) {
    __shared__ float red[4][MT][2][4][64];
    const int nt = blockIdx.x;
    const int slot = blockIdx.y;
    const int P = T * k;
    Group grp;
    if (!find_group(offsets, E, T, P, slot, grp)) return;
    const int lane = __lane_id();
    const int wv = wave_uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, rr = lane & 15;
    const bool shared = grp.expert < 0;
    const QMatDev Wg = shared ? sgate : gate;
    const QMatDev Wu = shared ? sup : up;
    const int e = shared ? 0 : grp.expert;
    const int KC = d / 128;
    const size_t ubase = ((size_t)e * (f / 16) + nt) * KC;
    const int nrows = grp.nrows;
    const int imax = nrows >= 4 ? 4 : nrows;

    // activation rows owned by this lane as A-operand row rr of each M tile
    const uint16_t *xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + rr;
        xrow[mt] = nullptr;
        if (r < nrows) {
            const int t = shared ? r : sorted_pair[grp.row0 + r] / k;
            xrow[mt] = x + (size_t)t * d;
        }
    }
    f32x4 ag[MT], au[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        ag[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        au[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones = {kOneBf16x2, kOneBf16x2, kOneBf16x2, kOneBf16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    for (int u = wv; u < KC; u += 4) {
        const size_t U = ubase + u;
        const u32x2 lg = *reinterpret_cast<const u32x2 *>(Wg.lo + U * 512 + lane * 8);
        const u32x2 lu = *reinterpret_cast<const u32x2 *>(Wu.lo + U * 512 + lane * 8);
        uint32_t hg = 0, hu = 0;
        if constexpr (FMT == MOE_FMT_Q3_B32) {
            hg = *reinterpret_cast<const uint32_t *>(Wg.hi + U * 256 + lane * 4);
            hu = *reinterpret_cast<const uint32_t *>(Wu.hi + U * 256 + lane * 4);
        }
        const u32x2 sg = *reinterpret_cast<const u32x2 *>(Wg.scale + U * 64 + rr * 4);
        const u32x2 su = *reinterpret_cast<const u32x2 *>(Wu.scale + U * 64 + rr * 4);
        u32x2 mg = {0u, 0u}, mu = {0u, 0u};
        if constexpr (FMT == MOE_FMT_Q2_B32) {
            mg = *reinterpret_cast<const u32x2 *>(Wg.min + U * 64 + rr * 4);
            mu = *reinterpret_cast<const u32x2 *>(Wu.min + U * 64 + rr * 4);
        }
        u32x4 A[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                A[mt][j] = u32x4{0u, 0u, 0u, 0u};
                if (xrow[mt])
                    A[mt][j] = *reinterpret_cast<const u32x4 *>(xrow[mt] + u * 128 + j * 32 + gq * 8);
            }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t dwg = lg[j >> 1], dwu = lu[j >> 1];
            u32x4 Bg, Bu, Hg, Hu;
            if (j & 1) {
                Bg = lo_operand<1, false>(dwg);
                Bu = lo_operand<1, false>(dwu);
            } else {
                Bg = lo_operand<0, false>(dwg);
                Bu = lo_operand<0, false>(dwu);
            }
            if constexpr (FMT == MOE_FMT_Q3_B32) {
                switch (j) {
                    case 0: Hg = hi_operand<0, false>(hg); Hu = hi_operand<0, false>(hu); break;
                    case 1: Hg = hi_operand<1, false>(hg); Hu = hi_operand<1, false>(hu); break;
                    case 2: Hg = hi_operand<2, false>(hg); Hu = hi_operand<2, false>(hu); break;
                    default: Hg = hi_operand<3, false>(hg); Hu = hi_operand<3, false>(hu); break;
                }
            }
            const uint32_t sgw = sg[j >> 1] >> (16 * (j & 1));
            const uint32_t suw = su[j >> 1] >> (16 * (j & 1));
            const float dg = half_bits_to_float((uint16_t)sgw), du = half_bits_to_float((uint16_t)suw);
            float mgv = 0.f, muv = 0.f;
            if constexpr (FMT == MOE_FMT_Q2_B32) {
                mgv = half_bits_to_float((uint16_t)(mg[j >> 1] >> (16 * (j & 1))));
                muv = half_bits_to_float((uint16_t)(mu[j >> 1] >> (16 * (j & 1))));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 pg = mfma_bf16(A[mt][j], Bg, zero);
                f32x4 pu = mfma_bf16(A[mt][j], Bu, zero);
                if constexpr (FMT == MOE_FMT_Q3_B32) {
                    pg = mfma_bf16(A[mt][j], Hg, pg);
                    pu = mfma_bf16(A[mt][j], Hu, pu);
                }
                const f32x4 xs = mfma_bf16(A[mt][j], ones, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < imax || mt > 0) {
                        if constexpr (FMT == MOE_FMT_Q2_B32) {
                            ag[mt][i] += dg * pg[i] + mgv * xs[i];
                            au[mt][i] += du * pu[i] + muv * xs[i];
                        } else {
                            ag[mt][i] += dg * (pg[i] - 4.0f * xs[i]);
                            au[mt][i] += du * (pu[i] - 4.0f * xs[i]);
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            red[wv][mt][0][i][lane] = ag[mt][i];
            red[wv][mt][1][i][lane] = au[mt][i];
        }
    __syncthreads();
    if (wv != 0) return;
    const int n = nt * 16 + rr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + gq * 4 + i;
            if (r >= nrows) continue;
            const float gs = (red[0][mt][0][i][lane] + red[1][mt][0][i][lane]) +
                             (red[2][mt][0][i][lane] + red[3][mt][0][i][lane]);
            const float us = (red[0][mt][1][i][lane] + red[1][mt][1][i][lane]) +
                             (red[2][mt][1][i][lane] + red[3][mt][1][i][lane]);
            const float h = swiglu(gs, us);
            const _Float16 hh = static_cast<_Float16>(h);
            const float rem = h - static_cast<float>(hh);
            const size_t off = (size_t)(grp.hrow0 + r) * f + n;
            h_hi[off] = __builtin_bit_cast(uint16_t, hh);
            h_lo[off] = f32_to_f16_bits(rem);
        }
}

template <int FMT, int MT>
__global__ __launch_bounds__(256) void down_small_kernel(
    QMatDev down, QMatDev sdown, const uint16_t *__restrict__ h_hi, const uint16_t *__restrict__ h_lo,
    int T, int k, int d, int f, int E, const int32_t *__restrict__ offsets,
    float *__restrict__ y_pairs, float *__restrict__ y_shared) {
    __shared__ float red[4][MT][4][64];
    const int ot = blockIdx.x;
    const int slot = blockIdx.y;
    const int P = T * k;
    Group grp;
    if (!find_group(offsets, E, T, P, slot, grp)) return;
    const int lane = __lane_id();
    const int wv = wave_uniform(threadIdx.x >> 6);
    const int gq = lane >> 4, rr = lane & 15;
    const bool shared = grp.expert < 0;
    const QMatDev W = shared ? sdown : down;
    const int e = shared ? 0 : grp.expert;
    const int KC = f / 128;
    const size_t ubase = ((size_t)e * (d / 16) + ot) * KC;
    const int nrows = grp.nrows;
    const int imax = nrows >= 4 ? 4 : nrows;

    // A-operand row rr: rows 0..7 = h_hi of group rows 8mt.., rows 8..15 = h_lo
    const uint16_t *hrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 8 + (rr & 7);
        hrow[mt] = nullptr;
        if (r < nrows) hrow[mt] = (rr < 8 ? h_hi : h_lo) + (size_t)(grp.hrow0 + r) * f;
    }
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = {kOneF16x2, kOneF16x2, kOneF16x2, kOneF16x2};
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    for (int u = wv; u < KC; u += 4) {
        const size_t U = ubase + u;
        const u32x2 lw = *reinterpret_cast<const u32x2 *>(W.lo + U * 512 + lane * 8);
        uint32_t hw = 0;
        if constexpr (FMT == MOE_FMT_Q3_B32)
            hw = *reinterpret_cast<const uint32_t *>(W.hi + U * 256 + lane * 4);
        const u32x2 sw = *reinterpret_cast<const u32x2 *>(W.scale + U * 64 + rr * 4);
        u32x2 mw = {0u, 0u};
        if constexpr (FMT == MOE_FMT_Q2_B32)
            mw = *reinterpret_cast<const u32x2 *>(W.min + U * 64 + rr * 4);
        u32x4 A[MT][4];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                A[mt][j] = u32x4{0u, 0u, 0u, 0u};
                if (hrow[mt])
                    A[mt][j] = *reinterpret_cast<const u32x4 *>(hrow[mt] + u * 128 + j * 32 + gq * 8);
            }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 B = (j & 1) ? lo_operand<1, true>(lw[j >> 1]) : lo_operand<0, true>(lw[j >> 1]);
            u32x4 H;
            if constexpr (FMT == MOE_FMT_Q3_B32) {
                switch (j) {
                    case 0: H = hi_operand<0, true>(hw); break;
                    case 1: H = hi_operand<1, true>(hw); break;
                    case 2: H = hi_operand<2, true>(hw); break;
                    default: H = hi_operand<3, true>(hw); break;
                }
            }
            const float dv = half_bits_to_float((uint16_t)(sw[j >> 1] >> (16 * (j & 1))));
            float mv = 0.f;
            if constexpr (FMT == MOE_FMT_Q2_B32)
                mv = half_bits_to_float((uint16_t)(mw[j >> 1] >> (16 * (j & 1))));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 p = mfma_f16(A[mt][j], B, zero);
                if constexpr (FMT == MOE_FMT_Q3_B32) p = mfma_f16(A[mt][j], H, p);
                const f32x4 hs = mfma_f16(A[mt][j], ones, zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < imax || mt > 0) {
                        if constexpr (FMT == MOE_FMT_Q2_B32)
                            acc[mt][i] += dv * p[i] + mv * hs[i];
                        else
                            acc[mt][i] += dv * (p[i] - 4.0f * hs[i]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wv][mt][i][lane] = acc[mt][i];
    __syncthreads();
    if (wv != 0) return;
    // sum the four K slices, then hi (rows 0..7, lanes 0..31) + lo (rows 8..15, lanes 32..63)
    const int o = ot * 16 + rr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float part = (red[0][mt][i][lane] + red[1][mt][i][lane]) +
                               (red[2][mt][i][lane] + red[3][mt][i][lane]);
            const float y = part + __shfl_xor(part, 32, 64);
            const int r = mt * 8 + gq * 4 + i;
            if (gq >= 2 || r >= nrows) continue;
            if (shared)
                y_shared[(size_t)r * d + o] = y;
            else
                y_pairs[(size_t)(grp.row0 + r) * d + o] = y;
        }
}

static QMatDev qm(const moe_qmat &m) { return QMatDev{m.lo, m.hi, m.scale, m.min}; }

size_t ffn_small_ws_bytes(int d, int f, int E, int T, int k) {
    (void)d;
    (void)E;
    const size_t rows = (size_t)T * k + T;
    return 2 * rows * f * sizeof(uint16_t) + 256;
}

template <int FMT, int MTG, int MTD>
static void launch_small_fmt(const moe_layer &L, const uint16_t *x, int T, int k,
                             const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                             float *y_shared, uint16_t *h_hi, uint16_t *h_lo, hipStream_t s) {
    const int d = L.d_model, f = L.d_ff, E = L.n_experts;
    const int P = T * k;
    const int slots = 1 + (E < P ? E : P);
    hipLaunchKernelGGL((gateup_small_kernel<FMT, MTG>), dim3(f / 16, slots), dim3(256), 0, s,
                       qm(L.gate), qm(L.up), qm(L.sh_gate), qm(L.sh_up), x, T, k, d, f, E, offsets,
                       sorted_pair, h_hi, h_lo);
    hipLaunchKernelGGL((down_small_kernel<FMT, MTD>), dim3(d / 16, slots), dim3(256), 0, s,
                       qm(L.down), qm(L.sh_down), h_hi, h_lo, T, k, d, f, E, offsets, y_pairs,
                       y_shared);
}

hipError_t launch_ffn_small(const moe_layer &L, const uint16_t *x, int T, int k,
                            const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                            float *y_shared, void *ws, hipStream_t s) {
    const size_t rows = (size_t)T * k + T;
    uint16_t *h_hi = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + kWsHeader);
    uint16_t *h_lo = h_hi + ((rows * L.d_ff + 127) / 128) * 128;
    // M tiles: gate/up 16 rows per tile, down 8 rows (hi over lo) per tile
    if (L.format == MOE_FMT_Q2_B32) {
        if (T <= 8)
            launch_small_fmt<MOE_FMT_Q2_B32, 1, 1>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, s);
        else if (T <= 16)
            launch_small_fmt<MOE_FMT_Q2_B32, 1, 2>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, s);
        else
            launch_small_fmt<MOE_FMT_Q2_B32, 2, 4>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, s);
    } else {
        if (T <= 8)
            launch_small_fmt<MOE_FMT_Q3_B32, 1, 1>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, s);
        else if (T <= 16)
            launch_small_fmt<MOE_FMT_Q3_B32, 1, 2>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, s);
        else
            launch_small_fmt<MOE_FMT_Q3_B32, 2, 4>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, h_hi, h_lo, s);
    }
    return hipGetLastError();
}

}  // namespace moe
