// ffn_prefill.hip -- expert FFN for large token batches (prompt chunks).
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 …", section
// "긴 프롬프트와 긴 컨텍스트 처리": prompts are read in chunks of up to 8,192
// tokens; section "Strata의 동작 원리": each token uses 10 of 512 routed experts
// plus the shared expert; [guide] tech.okbari.net "Strata와 Qwen3.8-Flash-Next…",
// section "24GB에 들어가는 원리": a wide batch touches many experts at once.
//
// Grouped GEMM on the matrix cores (v_mfma_f32_16x16x32_f16, fp32 accumulate):
//   gate/up:  [rows of group g] x d  .  (W_gate_g | W_up_g)^T   -> h = silu(g)*u
//   down:     [rows of group g] x f  .  W_down_g^T              -> y (fp32)
// Work items are (group, 128-row chunk, column tile).  A prepass builds the
// item table on the device from the dispatch offsets (the shared expert's
// chunks first, then every non-empty routed expert), so no host readback is
// needed and heavily loaded experts simply contribute more items.
//
// Operands:
//   A (activations): x converted once to fp16 (exact for bf16 values in fp16
//     range), or h; a 128-row tile per K step goes global -> registers -> LDS.
//   B (weights): never touches LDS.  The storage unit (16 rows x 128 columns,
//     lane-major) gives each lane exactly its 16x16x32 B-fragment bytes; the
//     lane turns codes into fp16 with the fp4 convert and applies the block
//     scale with one packed fp16 FMA per two weights: fp16(d*q + m) rounded
//     once (Q3: fp16(d*(q-4))).
// Precision: routed experts use the fp16-rounded weights and fp16 h; the
// shared expert (weight 1 in every token's output) uses exact weights as fp16
// hi + lo and h as fp16 hi + lo (the product lo*lo, below 2^-22 relative, is
// dropped).  Max |err| / rms(out) stays near 1.1e-3 on these workloads.
#include "common.h"

namespace moe {

constexpr int PF_MT = 128;           // rows per work item
constexpr int PF_KS = 128;           // K per step (one storage unit per row tile)
constexpr int PF_APITCH = PF_KS + 8; // fp16 elements per LDS row (16 B pad)

struct PfItem {
    int32_t expert;  // -1 = shared
    int32_t row0;    // first row (sorted position, or token for the shared expert)
    int32_t nrows;
    int32_t hrow0;   // first row in the h buffer
};


// ---------------------------------------------------------------- prepass
// One block of 1024 threads.  Shared-expert chunks first, then routed experts
// in index order.
__global__ __launch_bounds__(1024) void pf_build_items_kernel(const int32_t *__restrict__ offsets,
                                                              int E, int T, int P,
                                                              PfItem *__restrict__ items,
                                                              int32_t *__restrict__ n_items) {
    __shared__ int cnt[1024];
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    const int lane = __lane_id(), wv = tid >> 6;
    const int shared_ch = (T + PF_MT - 1) / PF_MT;
    int rows = 0, nch = 0;
    if (tid < E) {
        rows = offsets[tid + 1] - offsets[tid];
        nch = (rows + PF_MT - 1) / PF_MT;
    }
    // exclusive scan of nch over experts
    const int incl = wave_incl_scan(nch);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    if (wv == 0) {
        const int s = lane < 16 ? wsum[lane] : 0;
        const int si = wave_incl_scan(s);
        if (lane < 16) wsum[lane] = si - s;
    }
    __syncthreads();
    const int base = shared_ch + incl - nch + wsum[wv];
    if (tid < E) {
        const int r0 = offsets[tid];
        for (int c = 0; c < nch; ++c) {
            const int n = rows - c * PF_MT < PF_MT ? rows - c * PF_MT : PF_MT;
            items[base + c] = PfItem{tid, r0 + c * PF_MT, n, r0 + c * PF_MT};
        }
    }
    for (int c = tid; c < shared_ch; c += 1024) {
        const int n = T - c * PF_MT < PF_MT ? T - c * PF_MT : PF_MT;
        items[c] = PfItem{-1, c * PF_MT, n, P + c * PF_MT};
    }
    cnt[tid] = tid < E ? nch : 0;
    __syncthreads();
    if (tid == 0) {
        int tot = shared_ch;
        for (int e = 0; e < E; ++e) tot += cnt[e];
        n_items[0] = tot;
    }
}

__global__ __launch_bounds__(256) void pf_x_to_f16_kernel(const uint16_t *__restrict__ x,
                                                          uint16_t *__restrict__ x16, size_t n8) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
        const u32x4 v = reinterpret_cast<const u32x4 *>(x)[i];
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = __uint_as_float(v[q] << 16), b = __uint_as_float(v[q] & 0xffff0000u);
            const _Float16 ha = static_cast<_Float16>(a), hb = static_cast<_Float16>(b);
            o[q] = (uint32_t)__builtin_bit_cast(uint16_t, ha) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
        }
        reinterpret_cast<u32x4 *>(x16)[i] = o;
    }
}

// ------------------------------------------------------------ B fragments
// Lane (g = lane/16, rr = lane%16) holds, per storage unit, 8 bytes of codes
// (blocks j = 0..3, 8 codes each), a Q3 hi word, and its row's 4 scales/mins.
template <int FMT>
struct BRaw {
    u32x2 lo;
    uint32_t hi;
    u32x2 sc, mn;
};

template <int FMT>
__device__ __forceinline__ void load_braw(BRaw<FMT> &b, const QMatDev &W, size_t unit, int lane, int rr) {
    b.lo = *reinterpret_cast<const u32x2 *>(W.lo + unit * 512 + lane * 8);
    if constexpr (FMT == MOE_FMT_Q3_B32) b.hi = *reinterpret_cast<const uint32_t *>(W.hi + unit * 256 + lane * 4);
    b.sc = *reinterpret_cast<const u32x2 *>(W.scale + unit * 64 + rr * 4);
    if constexpr (FMT == MOE_FMT_Q2_B32) b.mn = *reinterpret_cast<const u32x2 *>(W.min + unit * 64 + rr * 4);
}

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
__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, uint32_t b) {
    uint32_t r;
    __asm__("v_pk_add_f16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// fp16(w) for the 8 weights of block J (rounded once).
template <int FMT, int J>
__device__ __forceinline__ u32x4 bfrag_f16(const BRaw<FMT> &b) {
    const u32x4 q = lo_operand<J & 1, true>(b.lo[J >> 1]);      // exact codes 0..3 as fp16
    const uint32_t d = half_pair(b.sc, J);
    u32x4 r;
    if constexpr (FMT == MOE_FMT_Q2_B32) {
        const uint32_t m = half_pair(b.mn, J);
        r.x = pk_fma_f16(q.x, d, m);
        r.y = pk_fma_f16(q.y, d, m);
        r.z = pk_fma_f16(q.z, d, m);
        r.w = pk_fma_f16(q.w, d, m);
    } else {
        const u32x4 h4 = hi_operand<J, true>(b.hi);               // 4*bit2 as fp16
        // -4d, exact: fp16 bits of d with the exponent raised by 2 and the sign set
        const uint32_t m4 = pk_fma_f16(d, 0xC400C400u /* -4.0, -4.0 */, 0u);
        r.x = pk_fma_f16(pk_add_f16(q.x, h4.x), d, m4);
        r.y = pk_fma_f16(pk_add_f16(q.y, h4.y), d, m4);
        r.z = pk_fma_f16(pk_add_f16(q.z, h4.z), d, m4);
        r.w = pk_fma_f16(pk_add_f16(q.w, h4.w), d, m4);
    }
    return r;
}

// exact weights split as fp16 hi + lo: w = fp32(d*q + m) (exact), hi = fp16(w),
// lo = fp16(w - hi).  qword holds two fp16 codes (Q3: lo + 4*bit2).
template <int FMT>
__device__ __forceinline__ void split_pair(uint32_t qword, float d, float m, uint32_t &hi, uint32_t &lo) {
    const float q0 = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(qword & 0xffffu)));
    const float q1 = static_cast<float>(__builtin_bit_cast(_Float16, (uint16_t)(qword >> 16)));
    float w0, w1;
    if constexpr (FMT == MOE_FMT_Q2_B32) {
        w0 = fmaf(q0, d, m);
        w1 = fmaf(q1, d, m);
    } else {
        w0 = d * (q0 - 4.0f);
        w1 = d * (q1 - 4.0f);
    }
    const _Float16 h0 = (_Float16)w0, h1 = (_Float16)w1;
    const _Float16 l0 = (_Float16)(w0 - (float)h0), l1 = (_Float16)(w1 - (float)h1);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
}

template <int FMT, int J>
__device__ __forceinline__ void bfrag_split(const BRaw<FMT> &b, u32x4 &hi, u32x4 &lo) {
    u32x4 q = lo_operand<J & 1, true>(b.lo[J >> 1]);
    if constexpr (FMT == MOE_FMT_Q3_B32) {
        const u32x4 h4 = hi_operand<J, true>(b.hi);
        q.x = pk_add_f16(q.x, h4.x);
        q.y = pk_add_f16(q.y, h4.y);
        q.z = pk_add_f16(q.z, h4.z);
        q.w = pk_add_f16(q.w, h4.w);
    }
    const float d = half_bits_to_float((uint16_t)(b.sc[J >> 1] >> (16 * (J & 1))));
    float m = 0.f;
    if constexpr (FMT == MOE_FMT_Q2_B32) m = half_bits_to_float((uint16_t)(b.mn[J >> 1] >> (16 * (J & 1))));
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_pair<FMT>(q.x, d, m, h0, l0);
    split_pair<FMT>(q.y, d, m, h1, l1);
    split_pair<FMT>(q.z, d, m, h2, l2);
    split_pair<FMT>(q.w, d, m, h3, l3);
    hi = u32x4{h0, h1, h2, h3};
    lo = u32x4{l0, l1, l2, l3};
}

// ------------------------------------------------------------- the GEMMs
// MODE 0: gate/up (K = d).  Wave w of the workgroup owns h columns
//   [n0 + 32w, n0 + 32w + 32): B subtiles 0,1 = gate rows, 2,3 = up rows.
// MODE 1: down (K = f).  Wave w owns output columns [n0 + 64w, +64).
// SPLIT: exact hi+lo weights (and for MODE 1, h hi+lo as A) -- shared expert.
template <int FMT, int MODE, bool SPLIT>
__global__ __launch_bounds__(256, 1) void pf_gemm_kernel(
    QMatDev W0, QMatDev W1, const PfItem *__restrict__ items, const int32_t *__restrict__ n_items,
    int item_base, int n_tiles, const uint16_t *__restrict__ a_src, const uint16_t *__restrict__ a_lo,
    const int32_t *__restrict__ sorted_pair, int k, int d, int f, uint16_t *__restrict__ h_out,
    uint16_t *__restrict__ h_lo_out, float *__restrict__ y_pairs, float *__restrict__ y_shared,
    int T) {
    constexpr int NA = (MODE == 1 && SPLIT) ? 2 : 1;   // A tiles (h hi, h lo)
    __shared__ __attribute__((aligned(16))) _Float16 As[NA][PF_MT * PF_APITCH];
    __shared__ int arow[PF_MT];
    const int bid = blockIdx.x;
    const int it = item_base + bid / n_tiles;
    const int nt = bid % n_tiles;
    PfItem item;
    if (SPLIT) {
        // shared expert: items are the first ceil(T/128) entries
        if (it >= (T + PF_MT - 1) / PF_MT) return;
    } else {
        if (it >= n_items[0]) return;
    }
    item = items[it];
    if (!SPLIT && item.expert < 0) return;
    const int tid = threadIdx.x, lane = __lane_id();
    const int wv = wave_uniform(tid >> 6);
    const int gq = lane >> 4, rr = lane & 15;
    const int K = MODE == 0 ? d : f;
    const int KC = K / 128;
    const int nrows = item.nrows;
    const int e = item.expert < 0 ? 0 : item.expert;
    // h_lo holds the shared rows only, indexed by token: row = h row - hrow0 + row0
    const long lo_delta = (long)item.row0 - item.hrow0;

    // A row sources (rows past the item's end reuse its last row; never stored)
    if (tid < PF_MT) {
        const int r = tid < nrows ? tid : nrows - 1;
        int src;
        if (MODE == 0)
            src = item.expert < 0 ? item.row0 + r : sorted_pair[item.row0 + r] / k;
        else
            src = item.hrow0 + r;
        arow[tid] = src;
    }
    // B row tiles of this wave: unit index base for each of the 4 subtiles
    size_t ubase[4];
    QMatDev Wsub[4];
    if (MODE == 0) {
        const int rows_per_exp = f / 16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int tile = (nt * 128 + wv * 32) / 16 + (s & 1);
            ubase[s] = ((size_t)e * rows_per_exp + tile) * KC;
            Wsub[s] = s < 2 ? W0 : W1;
        }
    } else {
        // d is a multiple of 128, so a wave's 64 columns are all in range or
        // all past d; past d the wave reads the last tile and stores nothing
        const int rows_per_exp = d / 16;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            int tile = (nt * 256 + wv * 64) / 16 + s;
            tile = tile < rows_per_exp ? tile : rows_per_exp - 1;
            ubase[s] = ((size_t)e * rows_per_exp + tile) * KC;
            Wsub[s] = W0;
        }
    }
    __syncthreads();

    // accumulators: 8 m-subtiles x 4 n-subtiles
    f32x4 acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nsub = (nrows + 15) / 16;

    // A staging: 128 rows x 128 fp16 = 2048 x 16 B; thread loads 8 chunks
    u32x4 areg[NA][8];
    auto load_a = [&](int kc) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 4, col = (c & 15) * 8;
            const size_t off = (size_t)arow[row] * K + kc * 128 + col;
            areg[0][i] = *reinterpret_cast<const u32x4 *>(a_src + off);
            if constexpr (NA == 2)
                areg[1][i] = *reinterpret_cast<const u32x4 *>(a_lo + off + lo_delta * K);
        }
    };
    auto store_a = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 4, col = (c & 15) * 8;
#pragma unroll
            for (int t = 0; t < NA; ++t)
                *reinterpret_cast<u32x4 *>(&As[t][row * PF_APITCH + col]) = areg[t][i];
        }
    };
    BRaw<FMT> braw[4];
    auto load_b = [&](int kc) {
#pragma unroll
        for (int s = 0; s < 4; ++s) load_braw(braw[s], Wsub[s], ubase[s] + kc, lane, rr);
    };

    load_a(0);
    load_b(0);
    for (int kc = 0; kc < KC; ++kc) {
        store_a();
        BRaw<FMT> bcur[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) bcur[s] = braw[s];
        __syncthreads();
        if (kc + 1 < KC) {
            load_a(kc + 1);
            load_b(kc + 1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 bf[4], bl[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if constexpr (SPLIT) {
                    switch (j) {
                        case 0: bfrag_split<FMT, 0>(bcur[s], bf[s], bl[s]); break;
                        case 1: bfrag_split<FMT, 1>(bcur[s], bf[s], bl[s]); break;
                        case 2: bfrag_split<FMT, 2>(bcur[s], bf[s], bl[s]); break;
                        default: bfrag_split<FMT, 3>(bcur[s], bf[s], bl[s]); break;
                    }
                } else {
                    switch (j) {
                        case 0: bf[s] = bfrag_f16<FMT, 0>(bcur[s]); break;
                        case 1: bf[s] = bfrag_f16<FMT, 1>(bcur[s]); break;
                        case 2: bf[s] = bfrag_f16<FMT, 2>(bcur[s]); break;
                        default: bf[s] = bfrag_f16<FMT, 3>(bcur[s]); break;
                    }
                }
            }
#pragma unroll
            for (int ms = 0; ms < 8; ++ms) {
                if (ms < nsub) {
                    const int arow_l = ms * 16 + rr;
                    const u32x4 af = *reinterpret_cast<const u32x4 *>(&As[0][arow_l * PF_APITCH + j * 32 + gq * 8]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        acc[ms][s] = mfma_f16(af, bf[s], acc[ms][s]);
                        if constexpr (SPLIT) acc[ms][s] = mfma_f16(af, bl[s], acc[ms][s]);
                    }
                    if constexpr (NA == 2) {
                        const u32x4 al = *reinterpret_cast<const u32x4 *>(&As[1][arow_l * PF_APITCH + j * 32 + gq * 8]);
#pragma unroll
                        for (int s = 0; s < 4; ++s) acc[ms][s] = mfma_f16(al, bf[s], acc[ms][s]);
                    }
                }
            }
        }
        __syncthreads();
    }

    // epilogue
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
        if (ms >= nsub) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = ms * 16 + gq * 4 + i;
            if (r >= nrows) continue;
            if constexpr (MODE == 0) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const float hv = swiglu(acc[ms][s][i], acc[ms][s + 2][i]);
                    const int col = nt * 128 + wv * 32 + s * 16 + rr;
                    const size_t off = (size_t)(item.hrow0 + r) * f + col;
                    const _Float16 hh = static_cast<_Float16>(hv);
                    h_out[off] = __builtin_bit_cast(uint16_t, hh);
                    if constexpr (SPLIT) {
                        const _Float16 hl = static_cast<_Float16>(hv - static_cast<float>(hh));
                        h_lo_out[(size_t)(item.row0 + r) * f + col] = __builtin_bit_cast(uint16_t, hl);
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int col = nt * 256 + wv * 64 + s * 16 + rr;
                    if (col >= d) continue;
                    if (item.expert < 0)
                        y_shared[(size_t)(item.row0 + r) * d + col] = acc[ms][s][i];
                    else
                        y_pairs[(size_t)(item.row0 + r) * d + col] = acc[ms][s][i];
                }
            }
        }
    }
}

// ------------------------------------------------------------------ host
struct PfWs {
    PfItem *items;
    int32_t *n_items;
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
    w.n_items = reinterpret_cast<int32_t *>(p);
    p += 256;
    w.items = reinterpret_cast<PfItem *>(p);
    p += align256(pf_max_items(E, T, k) * sizeof(PfItem));
    w.x16 = reinterpret_cast<uint16_t *>(p);
    p += align256((size_t)T * d * 2);
    w.h = reinterpret_cast<uint16_t *>(p);
    p += align256(((size_t)T * k + T) * f * 2);
    w.h_lo = reinterpret_cast<uint16_t *>(p);
    return w;
}

size_t ffn_prefill_ws_bytes(int d, int f, int E, int T, int k) {
    return 256 + align256(pf_max_items(E, T, k) * sizeof(PfItem)) + align256((size_t)T * d * 2) +
           align256(((size_t)T * k + T) * f * 2) + align256((size_t)T * f * 2);
}

template <int FMT>
static void pf_launch_fmt(const moe_layer &L, const uint16_t *x, int T, int k, const int32_t *offsets,
                          const int32_t *sorted_pair, float *y_pairs, float *y_shared, const PfWs &w,
                          hipStream_t s) {
    const int d = L.d_model, f = L.d_ff, E = L.n_experts;
    const int P = T * k;
    const QMatDev g{L.gate.lo, L.gate.hi, L.gate.scale, L.gate.min};
    const QMatDev u{L.up.lo, L.up.hi, L.up.scale, L.up.min};
    const QMatDev dn{L.down.lo, L.down.hi, L.down.scale, L.down.min};
    const QMatDev sg{L.sh_gate.lo, L.sh_gate.hi, L.sh_gate.scale, L.sh_gate.min};
    const QMatDev su{L.sh_up.lo, L.sh_up.hi, L.sh_up.scale, L.sh_up.min};
    const QMatDev sd{L.sh_down.lo, L.sh_down.hi, L.sh_down.scale, L.sh_down.min};
    const int sh_items = (T + PF_MT - 1) / PF_MT;
    const int max_items = (int)pf_max_items(E, T, k);
    const int nt_gu = f / 128, nt_dn = (d + 255) / 256;
    hipLaunchKernelGGL(pf_build_items_kernel, dim3(1), dim3(1024), 0, s, offsets, E, T, P, w.items,
                       w.n_items);
    const size_t n8 = (size_t)T * d / 8;
    size_t blocks = (n8 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(pf_x_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, w.x16, n8);
    // gate/up: shared (exact), routed
    hipLaunchKernelGGL((pf_gemm_kernel<FMT, 0, true>), dim3(sh_items * nt_gu), dim3(256), 0, s, sg, su,
                       w.items, w.n_items, 0, nt_gu, w.x16, nullptr, sorted_pair, k, d, f, w.h, w.h_lo,
                       y_pairs, y_shared, T);
    hipLaunchKernelGGL((pf_gemm_kernel<FMT, 0, false>), dim3((max_items - sh_items) * nt_gu), dim3(256), 0,
                       s, g, u, w.items, w.n_items, sh_items, nt_gu, w.x16, nullptr, sorted_pair, k, d, f,
                       w.h, w.h_lo, y_pairs, y_shared, T);
    // down: shared (exact weights, h hi + lo), routed
    hipLaunchKernelGGL((pf_gemm_kernel<FMT, 1, true>), dim3(sh_items * nt_dn), dim3(256), 0, s, sd, sd,
                       w.items, w.n_items, 0, nt_dn, w.h, w.h_lo, sorted_pair, k, d, f, w.h, w.h_lo,
                       y_pairs, y_shared, T);
    hipLaunchKernelGGL((pf_gemm_kernel<FMT, 1, false>), dim3((max_items - sh_items) * nt_dn), dim3(256), 0,
                       s, dn, dn, w.items, w.n_items, sh_items, nt_dn, w.h, nullptr, sorted_pair, k, d, f,
                       w.h, w.h_lo, y_pairs, y_shared, T);
}

hipError_t launch_ffn_prefill(const moe_layer &L, const uint16_t *x, int T, int k,
                              const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                              float *y_shared, void *ws, hipStream_t s) {
    const PfWs w = pf_carve(ws, L.d_model, L.d_ff, L.n_experts, T, k);
    if (L.format == MOE_FMT_Q2_B32)
        pf_launch_fmt<MOE_FMT_Q2_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, w, s);
    else
        pf_launch_fmt<MOE_FMT_Q3_B32>(L, x, T, k, offsets, sorted_pair, y_pairs, y_shared, w, s);
    return hipGetLastError();
}

}  // namespace moe
