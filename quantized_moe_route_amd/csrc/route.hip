// route.hip -- router logits, top-k selection and routing weights.
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 Qwen3.8-Flash-
// Next만을 위해 만든 추론 엔진", section "Strata의 동작 원리 / 그래픽카드, RAM, SSD에
// 나눠 담은 전문가": the router runs on the GPU for every token and layer and
// names the experts the token uses; section "Strata 소개": 10 of 512 per layer.
//
// Small T (decode, MTP verify): one launch.  The d x E router matrix (4 MiB
// fp32 at d=2048, E=512) is the only large read, so it is split over
// (E/64 column slices) x (d/128 row chunks) workgroups -- 128 of them at the
// full shape -- each reading 128 rows x 64 columns once.  Partial sums are
// reduced in a fixed order by the last workgroup to arrive, which also runs
// the top-k, so the result is deterministic and needs no second launch.
//
// Large T (prefill): a matrix-core GEMM.  fp32 router weights are split
// exactly into three bf16 terms (truncation: hi + mid + lo == w), x is already
// bf16, so every product is exact and only the fp32 accumulation order
// differs from a plain fp32 dot product.  A second kernel does the top-k, one
// wave per token.
#include "common.h"

namespace moe {

// --------------------------------------------------------------- top-k (wave)
// Cross-lane steps use DPP (register-file lane permutes) inside each row of
// 16 lanes and v_readlane across the four rows; no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// (v, i) beats (w, j): larger value, then lower index; i == INT_MAX is empty.
__device__ __forceinline__ bool beats(float v, int i, float w, int j) {
    return i != 0x7fffffff && (j == 0x7fffffff || v > w || (v == w && i < j));
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float &v, int &i) {
    const float ov = dpp_f<CTRL>(v);
    const int oi = dpp_i<CTRL>(i);
    if (beats(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void argmax_bcast_step(float &v, int &i) {
    // rows outside ROW_MASK keep their own value (old operand)
    const float ov = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
    const int oi = __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xF, false);
    if (beats(ov, oi, v, i)) {
        v = ov;
        i = oi;
    }
}
// Wave-wide arg-max, all in VALU: four DPP steps give every lane its row's
// best, row_bcast15/row_bcast31 carry rows 0..2 into row 3, and one readlane
// of lane 63 makes the result uniform.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
    argmax_step<0xB1>(v, i);   // quad_perm [1,0,3,2]
    argmax_step<0x4E>(v, i);   // quad_perm [2,3,0,1]
    argmax_step<0x141>(v, i);  // row_half_mirror
    argmax_step<0x140>(v, i);  // row_mirror
    argmax_bcast_step<0x142, 0xA>(v, i);  // row_bcast:15 -> rows 1, 3
    argmax_bcast_step<0x143, 0xC>(v, i);  // row_bcast:31 -> rows 2, 3
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    i = __builtin_amdgcn_readlane(i, 63);
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    v += dpp_f<0x140>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
           __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}

// One wave selects the k largest of E (<= 64*PER) logits: larger value first,
// equal values (including -0.0 vs +0.0) by lower index.  Lane l owns experts
// l, l+64, ... and keeps the best of its remaining ones; each round takes the
// wave-wide best and only the lane that owned it rescans.  Weights: softmax
// over the k selected logits.  `sel`/`seli` are LDS scratch of >= k entries.
template <int PER, bool DEV_LOADS>
__device__ void wave_topk(const float *lg, int E, int k, int32_t *__restrict__ ids,
                          float *__restrict__ w, float *sel, int *seli) {
    const int l = __lane_id();
    float v[PER];
    uint32_t alive = 0;
    // unconditional loads at clamped indices, so they are all in flight at once
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = l + 64 * i;
        const bool ok = e < E;
        const int ec = ok ? e : 0;
        v[i] = DEV_LOADS ? load_dev(&lg[ec]) : lg[ec];
        alive |= ok ? 1u << i : 0u;
    }
    auto local_best = [&](float &bv, int &bi) {
        bv = 0.0f;
        bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            // ascending index: strict > keeps the lowest index among equals
            const bool take = ((alive >> i) & 1u) && (bi == 0x7fffffff || v[i] > bv);
            bv = take ? v[i] : bv;
            bi = take ? l + 64 * i : bi;
        }
    };
    float lv;
    int li;
    local_best(lv, li);
    for (int j = 0; j < k; ++j) {
        float bv = lv;
        int bi = li;
        wave_argmax(bv, bi);
        if (l == 0) {
            sel[j] = bv;
            seli[j] = bi;
        }
        if ((bi & 63) == l) {
            alive &= ~(1u << (bi >> 6));
            local_best(lv, li);
        }
    }
    // lane 0 wrote sel[]/seli[]; make the LDS writes complete before other lanes read
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const float l0 = sel[0];
    float part = 0.0f;
    for (int j = l; j < k; j += 64) part += expf(sel[j] - l0);
    const float inv = 1.0f / wave_sum(part);
    for (int j = l; j < k; j += 64) {
        w[j] = expf(sel[j] - l0) * inv;
        ids[j] = seli[j];
    }
}

template <bool DEV_LOADS>
__device__ __forceinline__ void wave_topk_any(const float *lg, int E, int k, int32_t *ids, float *w,
                                              float *sel, int *seli) {
    if (E <= 64)
        wave_topk<1, DEV_LOADS>(lg, E, k, ids, w, sel, seli);
    else if (E <= 128)
        wave_topk<2, DEV_LOADS>(lg, E, k, ids, w, sel, seli);
    else if (E <= 256)
        wave_topk<4, DEV_LOADS>(lg, E, k, ids, w, sel, seli);
    else if (E <= 512)
        wave_topk<8, DEV_LOADS>(lg, E, k, ids, w, sel, seli);
    else
        wave_topk<16, DEV_LOADS>(lg, E, k, ids, w, sel, seli);
}

// ------------------------------------------- top-k on ordered keys (wave)
// For k <= 64, one wave per token.  Each logit becomes an unsigned key that
// orders like the float (sign-magnitude mapped to offset binary; -0.0 read as
// +0.0); 0 marks an empty or already taken entry, which no finite logit maps
// to.  Lane l owns experts l, l + 64, ...; each round takes the wave maximum
// key with six DPP max steps, finds the lanes holding it by ballot and, only
// on a tie, the lowest expert among them by a second reduction.  The owner
// clears the entry; lane j keeps the j-th selection in registers.
__device__ __forceinline__ uint32_t ord_key(float v) {
    uint32_t f = __float_as_uint(v);
    if (f == 0x80000000u) f = 0u;
    return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}
__device__ __forceinline__ float ord_value(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
// The lanes a row mask leaves out read the operation's identity (0 for max,
// all ones for min), so the move folds into one max/min with a DPP operand.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
    return o > v ? o : v;
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_min_u32(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, CTRL, ROW_MASK, 0xF, false);
    return o < v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = dpp_max_u32<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
    v = dpp_max_u32<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
    v = dpp_max_u32<0x141, 0xF>(v);   // row_half_mirror
    v = dpp_max_u32<0x140, 0xF>(v);   // row_mirror
    v = dpp_max_u32<0x142, 0xA>(v);   // row_bcast:15 -> rows 1, 3
    v = dpp_max_u32<0x143, 0xC>(v);   // row_bcast:31 -> rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = dpp_min_u32<0xB1, 0xF>(v);
    v = dpp_min_u32<0x4E, 0xF>(v);
    v = dpp_min_u32<0x141, 0xF>(v);
    v = dpp_min_u32<0x140, 0xF>(v);
    v = dpp_min_u32<0x142, 0xA>(v);
    v = dpp_min_u32<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

template <int PER>
__device__ void wave_topk_ord(const float *__restrict__ lg, int E, int k, int32_t *__restrict__ ids,
                              float *__restrict__ w, int32_t *ids_lds = nullptr) {
    const int l = __lane_id();
    uint32_t key[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = l + 64 * i;
        const float v = lg[e < E ? e : 0];
        key[i] = e < E ? ord_key(v) : 0u;
    }
    // lane's best: largest key, lowest slot among equals (a pairwise tree,
    // the right half taken only when strictly larger)
    auto local_best = [&](uint32_t &bk, int &bs) {
        uint32_t kk[PER];
        int ss[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            kk[i] = key[i];
            ss[i] = i;
        }
#pragma unroll
        for (int h = 1; h < PER; h *= 2)
#pragma unroll
            for (int i = 0; i + h < PER; i += 2 * h) {
                const bool take = kk[i + h] > kk[i];
                kk[i] = take ? kk[i + h] : kk[i];
                ss[i] = take ? ss[i + h] : ss[i];
            }
        bk = kk[0];
        bs = ss[0];
    };
    uint32_t bk;
    int bs;
    local_best(bk, bs);
    uint32_t my_key = 0u;   // lane j: the j-th pick
    int my_id = 0;
    for (int j = 0; j < k; ++j) {
        const uint32_t m = wave_max_u32(bk);
        const unsigned long long hold = __ballot(bk == m);
        int e;
        if (__builtin_expect(__popcll(hold) != 1, 0))
            e = (int)wave_min_u32(bk == m ? (uint32_t)(l + 64 * bs) : 0xffffffffu);
        else {
            const int owner = __builtin_ctzll(hold);
            e = owner + 64 * __builtin_amdgcn_readlane(bs, owner);
        }
        my_key = l == j ? m : my_key;
        my_id = l == j ? e : my_id;
        // the owner clears its pick; every lane rescans (same issue cost as
        // the owner alone, and no branch)
        const int slot = wave_uniform(e >> 6);
        key[slot] = l == (e & 63) ? 0u : key[slot];
        local_best(bk, bs);
    }
    const float l0 = ord_value((uint32_t)__builtin_amdgcn_readlane((int)my_key, 0));
    const float ev = l < k ? expf(ord_value(my_key) - l0) : 0.0f;
    const float inv = 1.0f / wave_sum(ev);
    if (l < k) {
        w[l] = ev * inv;
        ids[l] = my_id;
        if (ids_lds) ids_lds[l] = my_id;
    }
}


__device__ __forceinline__ void wave_topk_ord_any(const float *lg, int E, int k, int32_t *ids, float *w,
                                                  int32_t *ids_lds = nullptr) {
    if (E <= 64)
        wave_topk_ord<1>(lg, E, k, ids, w, ids_lds);
    else if (E <= 128)
        wave_topk_ord<2>(lg, E, k, ids, w, ids_lds);
    else if (E <= 256)
        wave_topk_ord<4>(lg, E, k, ids, w, ids_lds);
    else if (E <= 512)
        wave_topk_ord<8>(lg, E, k, ids, w, ids_lds);
    else
        wave_topk_ord<16>(lg, E, k, ids, w, ids_lds);
}

// ------------------------------------------------------- small T: one launch
// grid: (ceil(E/64) column slices, d/128 row chunks, ceil(T/8) token tiles),
// 512 threads: wave w of a workgroup owns 16 router rows, lane = one expert
// column, for the tile's (up to) 8 tokens.  Partial sums go out at device
// scope; the last workgroup of a tile to arrive adds the d/128 partials of
// every (token, expert) of the tile in chunk order, writes the logits and
// runs the top-k from LDS.  Tiles are independent (a counter line each).
constexpr int kMaxSmallT = kRouteTile;

// With offsets given (a batch of one tile, k <= 64), the last workgroup also
// lists the pairs by expert, as moe_dispatch does, from the ids it has just
// picked: one launch instead of two.
__global__ __launch_bounds__(512) void route_small_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ w, int32_t *__restrict__ counters, float *__restrict__ partial,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pair_pos,
    int tail_from) {
    __shared__ float red[8][kMaxSmallT][64];
    __shared__ int32_t sel_ids[kMaxSmallT * kWaveTopkMaxK];   // the batch's picks, for the listing
    __shared__ uint32_t emask[1024];                          // listing: tokens (bits) per expert
    __shared__ int32_t eoff[1024];                            // listing: first position per expert
    __shared__ int32_t wtot[8];
    // one LDS pool: the logits [T][E] for the register top-k (k <= 64), or
    // the serial top-k's per-wave scratch (k > 64)
    constexpr int kPoolBytes = 2 * 8 * 1024 * 4;
    static_assert(kMaxSmallT * 1024 * 4 <= kPoolBytes, "pool too small for the logits");
    __shared__ __attribute__((aligned(16))) unsigned char pool[kPoolBytes];
    __shared__ int last_flag;
    float *lgs = reinterpret_cast<float *>(pool);                       // [T][E], k <= 64
    float *sel = reinterpret_cast<float *>(pool);                       // [8][1024], k > 64
    int *seli = reinterpret_cast<int *>(pool + 8 * 1024 * 4);           // [8][1024], k > 64
    const int cs = blockIdx.x;
    const int kc = blockIdx.y;
    const int n_kc = gridDim.y;
    // this workgroup's token tile: tokens [t0, t0 + T)
    const int t0 = blockIdx.z * kRouteTile;
    T = T - t0 < kRouteTile ? T - t0 : kRouteTile;
    x += (size_t)t0 * d;
    logits += (size_t)t0 * E;
    ids += (size_t)t0 * k;
    w += (size_t)t0 * k;
    partial += (size_t)blockIdx.z * n_kc * kRouteTile * E;
    int32_t *const counter = counters + kCntLine * blockIdx.z;
    const int tid = threadIdx.x;
    const int col = tid & 63;
    const int wv = wave_uniform(tid >> 6);
    const int e = cs * 64 + col;

    // 16 router rows per thread, all loads in flight together
    const int c0 = kc * 128 + wv * 16;
    // unconditional loads at clamped indices (columns past E and tokens past T
    // are computed and discarded), so they are all in flight at once
    const int ec = e < E ? e : E - 1;
    float wrv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) wrv[r] = wr[(size_t)(c0 + r) * E + ec];
    u32x4 xv[kMaxSmallT][2];
#pragma unroll
    for (int t = 0; t < kMaxSmallT; ++t) {
        const int tc = t < T ? t : 0;
        xv[t][0] = *reinterpret_cast<const u32x4 *>(x + (size_t)tc * d + c0);
        xv[t][1] = *reinterpret_cast<const u32x4 *>(x + (size_t)tc * d + c0 + 8);
    }
#pragma unroll
    for (int t = 0; t < kMaxSmallT; ++t) {
        float a_ = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t word = xv[t][r >> 3][(r >> 1) & 3];
            const float xf = __uint_as_float((r & 1) ? (word & 0xffff0000u) : (word << 16));
            a_ += xf * wrv[r];
        }
        red[wv][t][col] = a_;
    }
    __syncthreads();
    if (wv == 0 && e < E) {
        for (int t = 0; t < T; ++t) {
            float s_ = red[0][t][col];
#pragma unroll
            for (int w2 = 1; w2 < 8; ++w2) s_ += red[w2][t][col];
            store_dev(&partial[((size_t)kc * T + t) * E + e], s_);
        }
    }
    publish_then_count(counter, gridDim.x * gridDim.y, last_flag);
    if (!last_flag) return;
    if (tid == 0) store_dev_int(counter, 0);
    // last workgroup: sum the partials of every (token, expert) in chunk
    // order.  A thread takes up to four (token, expert) entries per pass, with
    // all their partial loads in flight together.
    for (int idx0 = tid; idx0 < T * E; idx0 += 4 * 512) {
        const int left = (T * E - (idx0 - tid) + 511) / 512;   // uniform over the block
        const int nu = left < 4 ? left : 4;
        float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int q0 = 0; q0 < n_kc; q0 += 16) {
            float v[4][16];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (u >= nu) break;
                const int idx = idx0 + u * 512 < T * E ? idx0 + u * 512 : idx0;
                const int t = idx / E, ee = idx - t * E;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int qc = q0 + i < n_kc ? q0 + i : n_kc - 1;
                    v[u][i] = load_dev(&partial[((size_t)qc * T + t) * E + ee]);
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (u >= nu) break;
#pragma unroll
                for (int i = 0; i < 16; ++i) sum[u] += q0 + i < n_kc ? v[u][i] : 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = idx0 + u * 512;
            if (u >= nu || idx >= T * E) continue;
            const int ee = idx % E;
            const float s_ = bias ? sum[u] + bias[ee] : sum[u];
            logits[idx] = s_;
            if (k <= kWaveTopkMaxK) lgs[idx] = s_;
        }
    }
    __syncthreads();
    // one wave per token
    if (k <= kWaveTopkMaxK) {
        for (int t = wv; t < T; t += 8)
            wave_topk_ord_any(lgs + t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                              offsets ? sel_ids + t * k : nullptr);
        if (!offsets) return;
        // The listing: a token picks an expert at most once, so the pairs of
        // expert e are the tokens in emask[e]; pair p = t k + j goes to
        // (pairs of lower experts) + (tokens before t in emask[e]), the
        // position a stable sort by expert gives.  Bit 31 marks an expert
        // some token picked at a rank below tail_from (route tail-skip; with
        // tail_from = k every picked expert): the others list no pairs.
        constexpr uint32_t KEEP = 1u << 31;
        for (int e = tid; e < 1024; e += 512) emask[e] = 0u;
        __syncthreads();
        const int P = T * k;
        if (tid < P) atomicOr(&emask[sel_ids[tid]], (1u << (tid / k)) | (tid % k < tail_from ? KEEP : 0u));
        __syncthreads();
        // exclusive scan of the per-expert counts, two experts per thread
        const int e0 = 2 * tid;
        auto kept_count = [](uint32_t m) { return (m & KEEP) ? __popc(m & ~KEEP) : 0; };
        const int c0 = kept_count(emask[e0]), c1 = kept_count(emask[e0 + 1]);
        const int incl = wave_incl_scan(c0 + c1);
        if (__lane_id() == 63) wtot[wv] = incl;
        __syncthreads();
        int base = 0;
        for (int w2 = 0; w2 < wv; ++w2) base += wtot[w2];
        const int ex = base + incl - (c0 + c1);
        eoff[e0] = ex;
        eoff[e0 + 1] = ex + c0;
        if (e0 < E) offsets[e0] = ex;
        if (e0 + 1 < E) offsets[e0 + 1] = ex + c0;
        if (tid == 511) offsets[E] = base + incl;   // all pairs (slots past E count none)
        __syncthreads();
        if (tid < P) {
            const int e = sel_ids[tid], t = tid / k;
            const uint32_t m = emask[e];
            if (m & KEEP) {
                const int pos = eoff[e] + __popc(m & ((1u << t) - 1u));
                sorted_pair[pos] = tid;
                pair_pos[tid] = pos;
            } else {
                pair_pos[tid] = -1;
            }
        }
        return;
    }
    // large k: serial selection per token from the logits just written
    for (int t = wv; t < T; t += 8)
        wave_topk_any<false>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                             sel + wv * 1024, seli + wv * 1024);
}

size_t route_ws_bytes(int d, int E, int T) {
    if (T > kRouteSmallTMax) return router_gemm_ws_bytes(d, E);
    const size_t tiles = (size_t)(T + kRouteTile - 1) / kRouteTile;
    return (size_t)(d / 128) * tiles * kRouteTile * E * sizeof(float);
}

hipError_t launch_route_small(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, int k, int32_t *ids, float *w, void *ws,
                              hipStream_t s, int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos,
                              int tail_from) {
    int32_t *counters = reinterpret_cast<int32_t *>(ws);
    float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kWsHeader);
    dim3 grid((E + 63) / 64, d / 128, (T + kRouteTile - 1) / kRouteTile);
    hipLaunchKernelGGL(route_small_kernel, grid, dim3(512), 0, s, x, wr, bias, logits, T, d, E, k,
                       ids, w, counters, partial, offsets, sorted_pair, pair_pos, tail_from < 0 ? k : tail_from);
    return hipGetLastError();
}

// ------------------------------------------------------------ top-k kernel
// Logits given: one wave per token, four tokens per workgroup.  k <= 64 keeps
// every selection in registers; larger k selects serially through LDS.
__global__ __launch_bounds__(256) void topk_wave_kernel(const float *__restrict__ logits, int T,
                                                        int E, int k, int32_t *__restrict__ ids,
                                                        float *__restrict__ w) {
    const int wv = wave_uniform(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    wave_topk_ord_any(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
    __shared__ float sel[4][1024];
    __shared__ int seli[4][1024];
    const int wv = wave_uniform(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    wave_topk_any<false>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                         sel[wv], seli[wv]);
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w,
                       hipStream_t s) {
    if (k <= kWaveTopkMaxK)
        hipLaunchKernelGGL(topk_wave_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k,
                           ids, w);
    else
        hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
    return hipGetLastError();
}

// ------------------------------------------------------- large T: MFMA GEMM
// The fp32 router matrix is split exactly into three bf16 terms by truncation
// (hi + mid + lo == w; the last remainder has at most 8 significant bits) and
// stored transposed, [3][E][d], in the workspace.  x is bf16 already, so every
// product is exact and only the fp32 accumulation order differs from a plain
// fp32 dot product.
//
// GEMM: one workgroup of four waves (2 x 2) per 256 tokens x 64 experts; a
// wave owns 128 tokens x 32 experts, four 32x32x16 MFMA tiles, each fed the
// three weight terms.  K advances 32 at a time through a ring of five LDS
// stages (140 KiB) filled by global->LDS DMA (28 KiB a stage: 256 rows of x and 3 x 64
// rows of weight terms, 64 bytes each).  16-byte chunk c of row r is stored
// at chunk c ^ ((r >> 1) & 3) of its row, so the 32 rows an operand read
// touches fall on distinct banks.  Workgroups are dealt to the eight XCDs so
// that the expert tiles of one token tile share an XCD, and its L2 serves x.
constexpr int RG_TM = 256, RG_TN = 64, RG_KS = 32, RG_NS = 5;
constexpr int RG_ABYTES = RG_TM * RG_KS * 2;        // 16 KiB of x
constexpr int RG_BBYTES = 3 * RG_TN * RG_KS * 2;    // 12 KiB of weight terms
constexpr int RG_STAGE = RG_ABYTES + RG_BBYTES;
constexpr int RG_AI = RG_ABYTES / 1024 / 4;         // 1 KiB DMA copies per wave and stage: 4
constexpr int RG_BI = RG_BBYTES / 1024 / 4;         // 3
constexpr int RG_VM = RG_AI + RG_BI;                // vector-memory ops per stage and wave

__device__ __forceinline__ void split3(float v, uint16_t &h, uint16_t &m, uint16_t &lo) {
    const uint32_t u = __float_as_uint(v);
    h = (uint16_t)(u >> 16);
    const float r1 = v - __uint_as_float(u & 0xffff0000u);
    const uint32_t u1 = __float_as_uint(r1);
    m = (uint16_t)(u1 >> 16);
    const float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
    lo = (uint16_t)(__float_as_uint(r2) >> 16);
}

// wr [d][E] fp32 -> wt [3][E][d] bf16 terms.  Block = 64 k x 64 experts.
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ wr, int d,
                                                           int E, uint16_t *__restrict__ wt) {
    __shared__ float tile[64][65];
    const int k0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    for (int i = tid; i < 64 * 64; i += 256) {
        const int r = i >> 6, c = i & 63;
        tile[r][c] = e0 + c < E ? wr[(size_t)(k0 + r) * E + e0 + c] : 0.0f;
    }
    __syncthreads();
    const int el = tid >> 2, kq = (tid & 3) * 16;   // expert row, 16 consecutive k
    if (e0 + el >= E) return;
    uint32_t h[8], m[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint16_t h0, m0, l0, h1, m1, l1;
        split3(tile[kq + 2 * i][el], h0, m0, l0);
        split3(tile[kq + 2 * i + 1][el], h1, m1, l1);
        h[i] = h0 | ((uint32_t)h1 << 16);
        m[i] = m0 | ((uint32_t)m1 << 16);
        lo[i] = l0 | ((uint32_t)l1 << 16);
    }
    const size_t o = (size_t)(e0 + el) * d + k0 + kq;
    const size_t term = (size_t)E * d;
    u32x4 *p0 = reinterpret_cast<u32x4 *>(wt + o);
    u32x4 *p1 = reinterpret_cast<u32x4 *>(wt + term + o);
    u32x4 *p2 = reinterpret_cast<u32x4 *>(wt + 2 * term + o);
    p0[0] = u32x4{h[0], h[1], h[2], h[3]};
    p0[1] = u32x4{h[4], h[5], h[6], h[7]};
    p1[0] = u32x4{m[0], m[1], m[2], m[3]};
    p1[1] = u32x4{m[4], m[5], m[6], m[7]};
    p2[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    p2[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
}

__device__ __forceinline__ f32x16 mfma32_bf16(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 1) void router_mfma_kernel(const uint16_t *__restrict__ x,
                                                             const uint16_t *__restrict__ wt,
                                                             const float *__restrict__ bias,
                                                             float *__restrict__ logits, int T,
                                                             int d, int E, int n_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[RG_NS * RG_STAGE];
    const int l = __lane_id();
    const int wv = wave_uniform(threadIdx.x >> 6);
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int t = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
    const int m0 = (t / n_n) * RG_TM, n0 = (t % n_n) * RG_TN;

    // DMA sources of this lane: copy q covers 16 rows of 64 bytes; lane l
    // fills physical chunk l % 4 of row 16 (q % 4) + l / 4 of its region
    const char *asrc[RG_AI];
    const char *bsrc[RG_BI];
#pragma unroll
    for (int i = 0; i < RG_AI; ++i) {
        const int q = wv * RG_AI + i;
        const int r = 16 * q + (l >> 2);
        const int c = (l & 3) ^ ((r >> 1) & 3);
        const int row = m0 + r < T ? m0 + r : T - 1;
        asrc[i] = reinterpret_cast<const char *>(x + (size_t)row * d + c * 8);
    }
#pragma unroll
    for (int j = 0; j < RG_BI; ++j) {
        const int q = wv * RG_BI + j;
        const int term = q >> 2, n = 16 * (q & 3) + (l >> 2);
        const int c = (l & 3) ^ ((n >> 1) & 3);
        const int e = n0 + n < E ? n0 + n : E - 1;
        bsrc[j] = reinterpret_cast<const char *>(wt + ((size_t)term * E + e) * d + c * 8);
    }
    auto issue = [&](int kc) {
        uint8_t *sb = lds + (kc % RG_NS) * RG_STAGE;
        const size_t ko = (size_t)kc * (RG_KS * 2);
#pragma unroll
        for (int i = 0; i < RG_AI; ++i) copy_to_lds16(asrc[i] + ko, sb + (wv * RG_AI + i) * 1024);
#pragma unroll
        for (int j = 0; j < RG_BI; ++j)
            copy_to_lds16(bsrc[j] + ko, sb + RG_ABYTES + (wv * RG_BI + j) * 1024);
    };

    // operand reads: lane l reads row (l % 32) of a 32-row block, logical
    // chunk 2 s + l / 32 for k sub-step s
    const int wm = (wv >> 1) * 128, wn = (wv & 1) * 32;
    int lane_off[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
        lane_off[s] = (l & 31) * 64 + (((2 * s + (l >> 5)) ^ (((l & 31) >> 1) & 3)) * 16);

    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    struct Frags {
        u32x4 a[4], b[3];
    };
    // Each read first waits for every LDS read in flight: those were issued a
    // sub-step earlier, before the matrix ops just done, so the wait is short,
    // and the compiler, which places one full wait before the first use of
    // loop-carried LDS data, then has nothing left to wait for.  The
    // scheduling fence keeps the reads ahead of the matrix ops that follow.
    auto read = [&](Frags &f, int kc, int s) {
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
        const uint8_t *sb = lds + (kc % RG_NS) * RG_STAGE;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f.a[i] = *reinterpret_cast<const u32x4 *>(sb + (wm + 32 * i) * 64 + lane_off[s]);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            f.b[j] = *reinterpret_cast<const u32x4 *>(sb + RG_ABYTES + j * (RG_TN * 64) + wn * 64 +
                                                      lane_off[s]);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto mma = [&](const Frags &f) {
#pragma unroll
        for (int j = 2; j >= 0; --j)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = mfma32_bf16(f.a[i], f.b[j], acc[i]);
    };
    const int nk = d / RG_KS;
    static_assert(RG_NS - 2 <= 3, "arrive() waits for at most three later stages");
    // wait until stage kc has landed, when at most `ahead` later stages have
    // been issued, then meet the other waves
    auto arrive = [&](int kc, int ahead) {
        const int after = (nk - 1 - kc) < ahead ? (nk - 1 - kc) : ahead;
        if (after >= 3)
            wait_vm<3 * RG_VM>();
        else if (after == 2)
            wait_vm<2 * RG_VM>();
        else if (after == 1)
            wait_vm<RG_VM>();
        else
            wait_vm<0>();
        wg_barrier();
    };

    // Operand reads run one k sub-step ahead of the matrix ops.  The barrier
    // for stage kc + 1 sits between the two sub-steps of stage kc; the stage
    // refilled after it (kc + RG_NS - 1, in the ring slot of kc - 1) was last
    // read in the previous iteration.
    // the epilogue's kernel arguments are loaded here: a scalar load still in
    // flight inside the loop would turn each LDS wait there into a full one
    __asm__ volatile("" ::"s"(bias), "s"(logits));
    for (int kc = 0; kc < RG_NS - 1 && kc < nk; ++kc) issue(kc);
    arrive(0, RG_NS - 2);
    Frags f0, f1;
    read(f0, 0, 0);
    for (int kc = 0; kc < nk - 1; ++kc) {
        read(f1, kc, 1);
        mma(f0);
        arrive(kc + 1, RG_NS - 3);
        if (kc + RG_NS - 1 < nk) issue(kc + RG_NS - 1);
        read(f0, kc + 1, 0);
        mma(f1);
    }
    read(f1, nk - 1, 1);
    mma(f0);
    mma(f1);
    // D: lane l holds expert column l % 32, tokens 8 (r / 4) + 4 (l / 32) + r % 4
    const int n = n0 + wn + (l & 31);
    if (n >= E) return;
    const float bb = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
            if (m < T) logits[(size_t)m * E + n] = bias ? acc[i][r] + bb : acc[i][r];
        }
}

size_t router_gemm_ws_bytes(int d, int E) { return (size_t)3 * E * d * sizeof(uint16_t); }

hipError_t launch_router_gemm(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, void *ws, hipStream_t s) {
    uint16_t *wt = reinterpret_cast<uint16_t *>(static_cast<char *>(ws) + kWsHeader);
    hipLaunchKernelGGL(router_split_kernel, dim3(d / 64, (E + 63) / 64), dim3(256), 0, s, wr, d, E,
                       wt);
    const int n_m = (T + RG_TM - 1) / RG_TM, n_n = (E + RG_TN - 1) / RG_TN;
    hipLaunchKernelGGL(router_mfma_kernel, dim3(n_m * n_n), dim3(256), 0, s, x, wt, bias, logits, T,
                       d, E, n_n);
    return hipGetLastError();
}

}  // namespace moe
