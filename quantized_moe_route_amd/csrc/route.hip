// route.hip -- router logits, top-k selection and routing weights.
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 Qwen3.8-Flash-
// Next만을 위해 만든 추론 엔진", section "Strata의 동작 원리 / 그래픽카드, RAM, SSD에
// 나눠 담은 전문가": the router runs on the GPU for every token and layer and
// names the experts the token uses; section "Strata 소개": 10 of 512 per layer.
//
// Small T (decode, MTP verify): one launch.  The d x E router matrix (4 MiB
// fp32 at d=2048, E=512) is the only large read, so it is split over
// (E/32 column slices) x (d/128 row chunks) workgroups -- 256 of them at the
// full shape, one per compute unit -- each reading 128 rows x 32 columns
// (whole 128-byte lines) once.  The tile's last workgroup to finish adds
// the partial sums in a fixed order and selects the top k, one wave per
// token.  The result is deterministic and needs no second launch.
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

// ------------------------------------------- order-preserving keys
// Each logit becomes an unsigned key that orders like the float
// (sign-magnitude mapped to offset binary; -0.0 read as +0.0); 0 marks an
// empty entry, which no finite logit maps to.
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
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = dpp_min_u32<0xB1, 0xF>(v);
    v = dpp_min_u32<0x4E, 0xF>(v);
    v = dpp_min_u32<0x141, 0xF>(v);
    v = dpp_min_u32<0x140, 0xF>(v);
    v = dpp_min_u32<0x142, 0xA>(v);
    v = dpp_min_u32<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// ------------------------------------------------------- small T: one launch
// Two phases in one launch, for tiles of up to 8 tokens:
//   A. grid (ceil(E/32) column slices x d/128 row chunks, token tiles), 256
//      threads.  A workgroup reads its 128 rows x 32 columns of the router
//      matrix -- whole 128-byte lines, 16 bytes per lane, all loads in
//      flight at once -- multiplies them with the tile's x rows, sums its 32
//      row groups in a fixed order and publishes the 32 x Tt partial sums at
//      device scope.  It arrives on its column slice's counter; the slice's
//      last workgroup arrives on the tile's counter (two levels of 16
//      arrivals instead of one of 256: arrivals on one line are served one
//      after another).
//   B. The tile's last workgroup adds each logit's d/128 partial sums in
//      row-chunk order (fixed), adds the bias and writes the logits; then,
//      one wave per token, selects the top k (wave_select) and writes ids and
//      weights.  With offsets given (one tile, k <= 64) it also lists the
//      pairs by expert, as moe_dispatch does.
// Every sum runs in a fixed order and the selection is exact, so the result
// does not depend on arrival order.
constexpr int kRS = 32;                  // router columns per workgroup (one 128-byte line)
constexpr int kRK = 128;                 // router rows per workgroup
constexpr int kRT = kRouteTile;          // tokens per tile
constexpr int kRSMax = 1024 / kRS;       // column slices at E = 1024
constexpr int kRGroup = 4;               // tokens per selection round (one wave each)
constexpr int kRRow = 1024 + 64;         // LDS key row per token: 64 P keys, then the survivors' zero pad
static_assert(kRouteSliceCntLines == kRouteSmallTMax / kRouteTile * kRSMax, "one counter line per tile and slice");

__device__ __forceinline__ unsigned long long route_key(float v, int e) {
    return ((unsigned long long)ord_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(unsigned long long key) { return ord_value((uint32_t)(key >> 32)); }
__device__ __forceinline__ int key_expert(unsigned long long key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }
__device__ __forceinline__ unsigned long long max_u64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Inclusive prefix sum over the wave in registers: four row shifts, then the
// row broadcasts carry each row's total into the rows above.
__device__ __forceinline__ int wave_scan_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
    return v;
}

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_u64(unsigned long long v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return max_u64(v, ((unsigned long long)hi << 32) | lo);
}
// The maximum over each aligned group of L lanes (L a power of two <= 64).
__device__ __forceinline__ unsigned long long group_max_u64(unsigned long long v, int L) {
    if (L > 1) v = dpp_max_u64<0xB1>(v);    // quad_perm [1,0,3,2]
    if (L > 2) v = dpp_max_u64<0x4E>(v);    // quad_perm [2,3,0,1]
    if (L > 4) v = dpp_max_u64<0x141>(v);   // row_half_mirror: the two quads of each 8
    if (L > 8) v = dpp_max_u64<0x140>(v);   // row_mirror: the two halves of each 16
    if (L > 16) v = max_u64(v, __shfl_xor(v, 16, 64));
    if (L > 32) v = max_u64(v, __shfl_xor(v, 32, 64));
    return v;
}
// The same on 32-bit words.
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v, int L) {
    if (L > 1) v = dpp_max_u32<0xB1, 0xF>(v);
    if (L > 2) v = dpp_max_u32<0x4E, 0xF>(v);
    if (L > 4) v = dpp_max_u32<0x141, 0xF>(v);
    if (L > 8) v = dpp_max_u32<0x140, 0xF>(v);
    if (L > 16) v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
    if (L > 32) v = max(v, (uint32_t)__shfl_xor((int)v, 32, 64));
    return v;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((unsigned long long)hi << 32) | lo;
}

// The k (<= 64) largest keys of a wave; lane j returns the j-th (0 in lanes
// >= k).  Lane l holds v[i], the key of item l + 64 i (0 = no item; keys are
// unique, and a present key's low word, the inverted expert, is nonzero) and
// the wave holds at least k items.  A lower bound prunes first, on the value
// words alone: the lanes form G >= k groups of L = 64 / G; the k-th largest
// of the G group maxima (of value words), x, is reached by at least k keys,
// so every key of the top k has a value word >= x.  The keys whose value word
// reaches x -- a few more than k for typical logits -- are compacted into LDS
// and ranked exactly (full keys) against each other.  Per-wave LDS scratch:
// M of 64 words, sel of 64 keys, S of 64 P + 16 keys.
template <int P>
__device__ unsigned long long wave_select(const unsigned long long (&v)[P], int k, uint32_t *M,
                                          unsigned long long *sel, unsigned long long *S) {
    const int l = __lane_id();
    int G = 1;
    while (G < k) G <<= 1;
    const int lg = 6 - __builtin_ctz(G);    // log2 of L = 64 / G
    uint32_t hv[P];
#pragma unroll
    for (int i = 0; i < P; ++i) hv[i] = (uint32_t)(v[i] >> 32);
    uint32_t gm = hv[0];
#pragma unroll
    for (int i = 1; i < P; ++i) gm = max(gm, hv[i]);
    gm = group_max_u32(gm, 1 << lg);
    // the group maxima, padded with zeros to whole reads of 16
    const int Gp = (G + 15) & ~15;
    if (l < Gp) M[l] = 0u;
    if ((l & ((1 << lg) - 1)) == 0) M[l >> lg] = gm;
    int rk = 0;   // group maxima above this lane's
    for (int j0 = 0; j0 < Gp; j0 += 16) {
        u32x4 o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = *reinterpret_cast<const u32x4 *>(M + j0 + 4 * q);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) rk += o[q][c] > gm ? 1 : 0;
    }
    // x: the least group maximum with fewer than k maxima above it (0 when
    // fewer than k groups hold a key: then every key stays)
    const uint32_t x = wave_min_u32(rk < k ? gm : 0xFFFFFFFFu);
    bool kp[P];
    if (x != 0u) {
#pragma unroll
        for (int i = 0; i < P; ++i) kp[i] = hv[i] >= x;
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i) kp[i] = v[i] != 0ull;
    }
    // survivors, compacted in lane order
    int c = 0;
#pragma unroll
    for (int i = 0; i < P; ++i) c += kp[i] ? 1 : 0;
    const int incl = wave_scan_dpp(c);
    const int n = __builtin_amdgcn_readlane(incl, 63);
    int pos = incl - c;
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (kp[i]) S[pos++] = v[i];
    if (l < 16) S[n + l] = 0ull;   // zero keys rank below every key
    // exact ranks: 16 LDS reads in flight per step
    for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + l;
        const unsigned long long key = S[i < n ? i : n];
        int rank = 0;
        for (int j0 = 0; j0 < n; j0 += 16) {
            unsigned long long o[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) o[j] = S[j0 + j];
#pragma unroll
            for (int j = 0; j < 16; ++j) rank += o[j] > key ? 1 : 0;
        }
        if (i < n && rank < k) sel[rank] = key;
    }
    return l < k ? sel[l] : 0ull;
}

// One token's selection from its LDS key row (row[e] for e < 64 P, zero past
// E): ids, weights (softmax over the k picks) and, if asked, the picks in
// ids_lds for the listing.  The row is reused as the survivors' scratch.
// Lane j < k returns pick j's expert, the other lanes -1.
template <int P>
__device__ int select_token(unsigned long long *row, int k, uint32_t *M, unsigned long long *sel,
                            int32_t *__restrict__ ids, float *__restrict__ w, int32_t *ids_lds) {
    const int l = __lane_id();
    unsigned long long v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = row[l + 64 * i];
    const unsigned long long my = wave_select<P>(v, k, M, sel, row);
    const float lv = key_value(my);
    const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), 0));
    const float ev = l < k ? expf(lv - l0) : 0.0f;
    const float inv = 1.0f / wave_sum(ev);
    int e = -1;
    if (l < k) {
        e = key_expert(my);
        ids[l] = e;
        w[l] = ev * inv;
        if (ids_lds) ids_lds[l] = e;
    }
    return e;
}

// The listing of moe_dispatch from the batch's picks (ids_s [T][k] in LDS):
// a token picks an expert at most once, so the pairs of expert e are the
// tokens in emask[e]; pair p = t k + j goes to (pairs of lower experts) +
// (tokens before t in emask[e]), the position a stable sort by expert gives.
// Bit 31 marks an expert some token picked at a rank below tail_from (route
// tail-skip; with tail_from = k every picked expert): the others list no
// pairs.  Called by all 256 threads; T <= 8, k <= 64.
__device__ void list_pairs(const int32_t *ids_s, int T, int E, int k, int tail_from, uint32_t *emask,
                           int32_t *eoff, int32_t *wtot, int32_t *__restrict__ offsets,
                           int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pair_pos) {
    constexpr uint32_t KEEP = 1u << 31;
    const int tid = threadIdx.x, wv = tid >> 6;
    for (int e = tid; e < 1024; e += 256) emask[e] = 0u;
    lds_barrier();
    const int P = T * k;
    for (int p = tid; p < P; p += 256)
        atomicOr(&emask[ids_s[p]], (1u << (p / k)) | (p % k < tail_from ? KEEP : 0u));
    lds_barrier();
    // exclusive scan of the per-expert counts, four experts per thread
    auto kept_count = [](uint32_t m) { return (m & KEEP) ? __popc(m & ~KEEP) : 0; };
    const int e0 = 4 * tid;
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        c[i] = kept_count(emask[e0 + i]);
        sum += c[i];
    }
    const int incl = wave_scan_dpp(sum);
    if (__lane_id() == 63) wtot[wv] = incl;
    lds_barrier();
    int run = incl - sum;
    for (int w2 = 0; w2 < wv; ++w2) run += wtot[w2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        eoff[e0 + i] = run;
        if (e0 + i < E) offsets[e0 + i] = run;
        run += c[i];
    }
    if (tid == 255) offsets[E] = run;   // all (kept) pairs; slots past E count none
    lds_barrier();
    for (int p = tid; p < P; p += 256) {
        const int e = ids_s[p], t = p / k;
        const uint32_t m = emask[e];
        if (m & KEEP) {
            const int pos = eoff[e] + __popc(m & ((1u << t) - 1u));
            sorted_pair[pos] = p;
            pair_pos[p] = pos;
        } else {
            pair_pos[p] = -1;
        }
    }
}

// The listing for a single token (pairs p = j) from its kept picks (ranks j
// < tail_from) as bits of an expert mask, bit e & 31 of word e >> 5 (E <=
// 1024): pair j's position and offsets[e] both count the kept picks with a
// lower expert (a token picks an expert once).  mark_one, by the selecting
// wave (lane j < k holds pick j's expert): sets the bits in words bits[0 ..
// 31] (cleared beforehand; bits[32] stays zero), stores each word's exclusive
// prefix count in cnt[0 .. 32] and lists the pairs.  After a barrier,
// offsets_one fills offsets[0 .. E] from the words (all threads).
__device__ void mark_one(int e_pick, int k, int tail_from, uint32_t *bits, int32_t *cnt,
                         int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pair_pos) {
    const int l = __lane_id();
    const int kk = tail_from < k ? tail_from : k;   // picks 0 .. kk-1 are kept
    if (l < kk) atomicOr(&bits[e_pick >> 5], 1u << (e_pick & 31));
    // the same wave reads the words back: its LDS operations run in order
    const uint32_t m = l < 32 ? bits[l] : 0u;
    const int c = __popc(m);
    const int below = wave_scan_dpp(c) - c;
    if (l <= 32) cnt[l] = below;
    const int wd = l < kk ? e_pick >> 5 : 0;
    const uint32_t mw = (uint32_t)__shfl((int)m, wd, 64);
    const int bw = __shfl(below, wd, 64);
    if (l < kk) {
        const int pos = bw + __popc(mw & ((1u << (e_pick & 31)) - 1u));
        pair_pos[l] = pos;
        sorted_pair[pos] = l;
    } else if (l < k) {
        pair_pos[l] = -1;
    }
}
__device__ void offsets_one(const uint32_t *bits, const int32_t *cnt, int E, int32_t *__restrict__ offsets) {
    for (int e = threadIdx.x; e <= E; e += 256) {
        const int wd = e >> 5;
        offsets[e] = cnt[wd] + __popc(bits[wd] & ((1u << (e & 31)) - 1u));
    }
}

// Device-coherent 16-byte load (sc1: served by the level all XCDs share)
// through a buffer resource; byte offsets past `bytes` read zero.
__device__ __forceinline__ f32x4 load_dev_f4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 16));
}

// TT: token slots (1, 2, 4 or 8; >= the tile's token count)
template <bool VEC, int TT>
__global__ __launch_bounds__(256) void route_small_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int k, int32_t *__restrict__ ids, float *__restrict__ w,
    int32_t *__restrict__ tile_cnt, int32_t *__restrict__ slice_cnt, float *__restrict__ partial,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_pair, int32_t *__restrict__ pair_pos,
    int tail_from) {
    // key rows of kRGroup tokens (B); phase A's cross-wave sums and the
    // serial selection's scratch (k > 64) live in the same memory
    __shared__ __attribute__((aligned(16))) unsigned long long keys[kRGroup][kRRow];
    __shared__ __attribute__((aligned(16))) unsigned long long wscr[4][128];   // per wave: M, sel
    __shared__ __attribute__((aligned(16))) uint16_t xT[kRK][TT];             // A: x, rows x tokens
    __shared__ int32_t sel_ids[kRT * kWaveTopkMaxK];                          // B: the picks, for the listing
    __shared__ uint32_t emask[1024];
    __shared__ int32_t eoff[1024];
    __shared__ int32_t wtot[4];
    __shared__ int last_flag, tile_flag;
    static_assert(4 * TT * 4 * kRS * 4 <= sizeof(keys), "phase A's pair sums fit the key rows");

    const int ES = (E + kRS - 1) / kRS, KC = d / kRK;
    const int slice = blockIdx.x % ES, kc = blockIdx.x / ES, tt = blockIdx.y;
    const int t0 = tt * kRT;
    const int Tt = T - t0 < kRT ? T - t0 : kRT;
    const int tid = threadIdx.x, l = __lane_id();
    const int wv = wave_uniform(tid >> 6);
    // partial sums of the tile: [ES][KC][kRT][kRS]
    float *const ptile = partial + (size_t)tt * ES * KC * (kRT * kRS);

    // ------------------------------------------------------------- phase A
    {
        const int eq = l & 7, rs = l >> 3;
        const int e0 = slice * kRS + eq * 4;
        // row chunk 0 adds the bias to its partial sums (a 0-byte resource
        // elsewhere reads zeros); loaded with the router rows
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float *>(bias), 0, (bias && kc == 0) ? E * (int)sizeof(float) : 0, 0x00020000);
        const float bias_e = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(brs, 4 * (slice * kRS + (tid & (kRS - 1))), 0, 0));
        float wv4[4][4];
        // unconditional loads at clamped addresses (columns past E are
        // computed and dropped), all in flight together
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = kc * kRK + wv * 32 + i * 8 + rs;
            const float *src = wr + (size_t)row * E;
            if constexpr (VEC) {
                const int ec = e0 < E ? e0 : E - 4;
                const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(src + ec));
#pragma unroll
                for (int c = 0; c < 4; ++c) wv4[i][c] = v[c];
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) wv4[i][c] = src[e0 + c < E ? e0 + c : E - 1];
            }
        }
        // x: 16 chunks of 8 rows per token, transposed into xT (token slots
        // past the tile's end are zero)
        if (tid < 16 * TT) {
            const int t = tid >> 4, ch = tid & 15;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (t < Tt) v = *reinterpret_cast<const u32x4 *>(x + (size_t)(t0 + t) * d + kc * kRK + ch * 8);
#pragma unroll
            for (int j = 0; j < 8; ++j) xT[ch * 8 + j][t] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
        }
        lds_barrier();
        float acc[TT][4];
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[t][c] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wv * 32 + i * 8 + rs;
            uint32_t xw[(TT + 1) / 2];
#pragma unroll
            for (int q = 0; q < (TT + 1) / 2; ++q)
                xw[q] = TT == 1 ? (uint32_t)xT[row][0] : reinterpret_cast<const uint32_t *>(&xT[row][0])[q];
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const uint32_t word = xw[t >> 1];
                const float xf = __uint_as_float((t & 1) ? (word & 0xffff0000u) : (word << 16));
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[t][c] = fmaf(xf, wv4[i][c], acc[t][c]);
            }
        }
        // the 8 row lanes of a wave (same eq): row pairs (rs, rs ^ 1) in the
        // lane (rotation by 8 within each 16-lane row, no LDS), the four
        // pair sums through LDS; the sum over rows is then
        // ((p01 + p23) + (p45 + p67)) per wave and the waves add in order
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[t][c] += __int_as_float(
                    __builtin_amdgcn_update_dpp(0, __float_as_int(acc[t][c]), 0x128, 0xF, 0xF, false));
        float *red = reinterpret_cast<float *>(&keys[0][0]);   // [4 waves][TT][4 pairs][32]
        if ((rs & 1) == 0) {
#pragma unroll
            for (int t = 0; t < TT; ++t)
                *reinterpret_cast<f32x4 *>(&red[((wv * TT + t) * 4 + (rs >> 1)) * kRS + eq * 4]) =
                    f32x4{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
        }
        __syncthreads();
        if (tid < TT * kRS) {
            const int t = tid / kRS, e = tid % kRS;
            if (t < Tt) {
                float sw[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float *q = &red[((w * TT + t) * 4) * kRS + e];
                    sw[w] = (q[0] + q[kRS]) + (q[2 * kRS] + q[3 * kRS]);
                }
                const float s = (((sw[0] + sw[1]) + sw[2]) + sw[3]) + bias_e;
                store_dev(&ptile[(((size_t)slice * KC + kc) * kRT + t) * kRS + e], s);
            }
        }
    }
    // two-level arrival: the slice's counter, then (its last chunk) the tile's
    int32_t *const scnt = slice_cnt + (size_t)(tt * kRSMax + slice) * kCntLine;
    publish_then_count(scnt, KC, last_flag);
    if (!last_flag) return;
    int32_t *const tcnt = tile_cnt + (size_t)tt * kCntLine;
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(tcnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        tile_flag = old == ES - 1;
    }
    __syncthreads();
    if (!tile_flag) return;
    const bool listing = offsets != nullptr;
    // one token: the listing's expert mask, cleared before the first barrier
    // below (the selecting wave sets it)
    if (listing && Tt == 1 && tid <= 32) emask[tid] = 0u;
    // The tile's last workgroup resets the tile's counters at its very end: a
    // store issued before its loads would delay them (the memory counter
    // retires in order).

    // ------------------------------------------------------------- phase B
    const int E4 = (E + 3) >> 2;
    const int Pk = E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;   // keys per lane
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(ptile, 0, ES * KC * (kRT * kRS) * (int)sizeof(float), 0x00020000);
    const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(logits, 0, T * E * (int)sizeof(float), 0x00020000);
    for (int g0 = 0; g0 < Tt; g0 += kRGroup) {
        const int nt = Tt - g0 < kRGroup ? Tt - g0 : kRGroup;
        const int items = nt * E4;   // (token, 4 experts)
        // logits and keys, two items per thread per round; each item's d/128
        // partial sums are added in row-chunk order, all loads in flight
        for (int it0 = 0; it0 < items; it0 += 512) {
            const int nh = it0 + 256 < items ? 2 : 1;   // items per thread this round
            int itm[2];
            f32x4 s[2];
            uint32_t off0[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int it = it0 + h * 256 + tid;
                itm[h] = it;
                const int itc = it < items ? it : 0;
                const int t = itc / E4, e4 = itc - t * E4;
                const int sl = e4 >> 3, q = e4 & 7;
                // byte offset of (slice, chunk 0, token, quad); chunks 1 KiB apart
                off0[h] = (uint32_t)((((sl * KC) * kRT + g0 + t) * kRS + q * 4) * 4);
                s[h] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            int q0 = 0;
            constexpr uint32_t kChunkBytes = kRT * kRS * 4;
            if (nh == 2) {
                // both items' loads in flight before the first add
                for (; q0 + 16 <= KC; q0 += 16) {
                    f32x4 pa[16], pb[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) pa[j] = load_dev_f4(prs, off0[0] + (uint32_t)(q0 + j) * kChunkBytes);
#pragma unroll
                    for (int j = 0; j < 16; ++j) pb[j] = load_dev_f4(prs, off0[1] + (uint32_t)(q0 + j) * kChunkBytes);
#pragma unroll
                    for (int j = 0; j < 16; ++j) s[0] += pa[j];
#pragma unroll
                    for (int j = 0; j < 16; ++j) s[1] += pb[j];
                }
                for (; q0 < KC; ++q0) {
                    s[0] += load_dev_f4(prs, off0[0] + (uint32_t)q0 * kChunkBytes);
                    s[1] += load_dev_f4(prs, off0[1] + (uint32_t)q0 * kChunkBytes);
                }
            } else {
                for (; q0 + 16 <= KC; q0 += 16) {
                    f32x4 pa[16];
#pragma unroll
                    for (int j = 0; j < 16; ++j) pa[j] = load_dev_f4(prs, off0[0] + (uint32_t)(q0 + j) * kChunkBytes);
#pragma unroll
                    for (int j = 0; j < 16; ++j) s[0] += pa[j];
                }
                for (; q0 < KC; ++q0) s[0] += load_dev_f4(prs, off0[0] + (uint32_t)q0 * kChunkBytes);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (itm[h] < items) {
                    const int t = itm[h] / E4, e4 = itm[h] - t * E4;
                    unsigned long long kq[4];
                    float *const lrow = logits + (size_t)(t0 + g0 + t) * E;
                    if constexpr (VEC) {
                        // one 16-byte device-coherent store (the large-k
                        // selection below re-reads the logits)
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s[h]), lrs,
                                                               (int)(((size_t)(lrow - logits) + 4 * e4) * 4), 0, 16);
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int e = 4 * e4 + c;
                        kq[c] = 0ull;
                        if (e < E) {
                            if constexpr (!VEC) store_dev(&lrow[e], s[h][c]);
                            kq[c] = route_key(s[h][c], e);
                        }
                    }
                    u32x4 lo, hi;
                    lo = u32x4{(uint32_t)kq[0], (uint32_t)(kq[0] >> 32), (uint32_t)kq[1], (uint32_t)(kq[1] >> 32)};
                    hi = u32x4{(uint32_t)kq[2], (uint32_t)(kq[2] >> 32), (uint32_t)kq[3], (uint32_t)(kq[3] >> 32)};
                    *reinterpret_cast<u32x4 *>(&keys[t][4 * e4]) = lo;
                    *reinterpret_cast<u32x4 *>(&keys[t][4 * e4 + 2]) = hi;
                }
            }
        }
        // zero keys from 4 ceil(E/4) to the row's 64 Pk
        const int pad0 = 4 * E4, padn = 64 * Pk - pad0;
        for (int i = tid; i < nt * padn; i += 256) keys[i / padn][pad0 + i % padn] = 0ull;
        // LDS only: the logits stores may land later (for large k, re-read
        // below from memory, wait for them first)
        if (k > kWaveTopkMaxK) __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (wv < nt) {
            const int t = g0 + wv;
            int32_t *const id_t = ids + (size_t)(t0 + t) * k;
            float *const w_t = w + (size_t)(t0 + t) * k;
            if (k <= kWaveTopkMaxK) {
                uint32_t *M = reinterpret_cast<uint32_t *>(wscr[wv]);
                unsigned long long *sel = wscr[wv] + 64;
                int32_t *il = listing && Tt > 1 ? sel_ids + t * k : nullptr;
                int e_pick;
                switch (Pk) {
                case 1: e_pick = select_token<1>(keys[wv], k, M, sel, id_t, w_t, il); break;
                case 2: e_pick = select_token<2>(keys[wv], k, M, sel, id_t, w_t, il); break;
                case 4: e_pick = select_token<4>(keys[wv], k, M, sel, id_t, w_t, il); break;
                case 8: e_pick = select_token<8>(keys[wv], k, M, sel, id_t, w_t, il); break;
                default: e_pick = select_token<16>(keys[wv], k, M, sel, id_t, w_t, il); break;
                }
                if (listing && Tt == 1) mark_one(e_pick, k, tail_from, emask, eoff, sorted_pair, pair_pos);
            } else {
                // large k: the serial wave top-k on the logits just written
                // (device-scope loads), scratch in this wave's key row
                float *selv = reinterpret_cast<float *>(keys[wv]);
                int *seli = reinterpret_cast<int *>(selv + 1024);
                wave_topk_any<true>(logits + (size_t)(t0 + t) * E, E, k, id_t, w_t, selv, seli);
            }
        }
        lds_barrier();   // the key rows serve the next group
    }
    if (listing) {
        if (Tt == 1)
            offsets_one(emask, eoff, E, offsets);
        else
            list_pairs(sel_ids, Tt, E, k, tail_from, emask, eoff, wtot, offsets, sorted_pair, pair_pos);
    }
    // zero the tile's counters for the next call (every arrival is in)
    if (tid < ES) store_dev_int(slice_cnt + (size_t)(tt * kRSMax + tid) * kCntLine, 0);
    if (tid == 0) store_dev_int(tcnt, 0);
}

// workspace after the header: the partial sums [tiles][ES][d/128][kRT][kRS]
size_t route_ws_bytes(int d, int E, int T) {
    if (T > kRouteSmallTMax) return router_gemm_ws_bytes(d, E);
    const size_t tiles = (size_t)(T + kRT - 1) / kRT, ES = (size_t)(E + kRS - 1) / kRS;
    return tiles * ES * (size_t)(d / kRK) * kRT * kRS * sizeof(float);
}

template <bool VEC>
static void launch_route_small_v(dim3 grid, int TT, hipStream_t s, const uint16_t *x, const float *wr,
                                 const float *bias, float *logits, int T, int d, int E, int k, int32_t *ids, float *w,
                                 int32_t *tile_cnt, int32_t *slice_cnt, float *partial, int32_t *offsets,
                                 int32_t *sorted_pair, int32_t *pair_pos, int tail_from) {
#define MOE_ROUTE_LAUNCH(TTV)                                                                                        \
    hipLaunchKernelGGL((route_small_kernel<VEC, TTV>), grid, dim3(256), 0, s, x, wr, bias, logits, T, d, E, k, ids, \
                       w, tile_cnt, slice_cnt, partial, offsets, sorted_pair, pair_pos, tail_from)
    if (TT == 1)
        MOE_ROUTE_LAUNCH(1);
    else if (TT == 2)
        MOE_ROUTE_LAUNCH(2);
    else if (TT == 4)
        MOE_ROUTE_LAUNCH(4);
    else
        MOE_ROUTE_LAUNCH(8);
#undef MOE_ROUTE_LAUNCH
}

hipError_t launch_route_small(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, int k, int32_t *ids, float *w, void *ws,
                              hipStream_t s, int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos,
                              int tail_from) {
    char *base = static_cast<char *>(ws);
    int32_t *tile_cnt = reinterpret_cast<int32_t *>(base);
    int32_t *slice_cnt = reinterpret_cast<int32_t *>(base + kRouteSliceCnt);
    float *partial = reinterpret_cast<float *>(base + kWsHeader);
    const int ES = (E + kRS - 1) / kRS, KC = d / kRK;
    const dim3 grid(ES * KC, (T + kRT - 1) / kRT);
    // token slots: the batch itself up to one tile, else full tiles
    const int TT = T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8;
    const int tf = tail_from < 0 ? k : tail_from;
    if (E % 4 == 0)
        launch_route_small_v<true>(grid, TT, s, x, wr, bias, logits, T, d, E, k, ids, w, tile_cnt, slice_cnt, partial,
                                   offsets, sorted_pair, pair_pos, tf);
    else
        launch_route_small_v<false>(grid, TT, s, x, wr, bias, logits, T, d, E, k, ids, w, tile_cnt, slice_cnt,
                                    partial, offsets, sorted_pair, pair_pos, tf);
    return hipGetLastError();
}

// ------------------------------------------------------------ top-k kernel
// Logits given, k > 64: one wave per token, four tokens per workgroup, the
// selection serial through LDS.
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

// Logits given, k <= 64: one wave per token, four tokens per workgroup, the
// pruned selection of the one-launch router (wave_select: a lower bound from
// group maxima of the value words, then exact ranks of the keys above it)
// on the token's keys staged in LDS: a few LDS round trips per token instead
// of k serial max-and-clear rounds over the wave.
template <int P>
__global__ __launch_bounds__(256) void topk_sel_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                       int32_t *__restrict__ ids, float *__restrict__ w) {
    __shared__ __attribute__((aligned(16))) unsigned long long rows[4][64 * P + 16];
    __shared__ __attribute__((aligned(16))) unsigned long long scr[4][128];   // per wave: M, sel
    const int wv = wave_uniform(threadIdx.x >> 6), l = __lane_id();
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    const float *lg = logits + (size_t)t * E;
    float v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int e = l + 64 * i;
        v[i] = lg[e < E ? e : 0];
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int e = l + 64 * i;
        rows[wv][e] = e < E ? route_key(v[i], e) : 0ull;
    }
    // each lane reads back only what it wrote; the selection's exchanges are
    // within the wave, whose LDS operations complete in order
    select_token<P>(rows[wv], k, reinterpret_cast<uint32_t *>(scr[wv]), scr[wv] + 64, ids + (size_t)t * k,
                    w + (size_t)t * k, nullptr);
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w,
                       hipStream_t s) {
    const dim3 grid((T + 3) / 4), blk(256);
    if (k <= kWaveTopkMaxK) {
        if (E <= 64)
            hipLaunchKernelGGL(topk_sel_kernel<1>, grid, blk, 0, s, logits, T, E, k, ids, w);
        else if (E <= 128)
            hipLaunchKernelGGL(topk_sel_kernel<2>, grid, blk, 0, s, logits, T, E, k, ids, w);
        else if (E <= 256)
            hipLaunchKernelGGL(topk_sel_kernel<4>, grid, blk, 0, s, logits, T, E, k, ids, w);
        else if (E <= 512)
            hipLaunchKernelGGL(topk_sel_kernel<8>, grid, blk, 0, s, logits, T, E, k, ids, w);
        else
            hipLaunchKernelGGL(topk_sel_kernel<16>, grid, blk, 0, s, logits, T, E, k, ids, w);
    } else
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
