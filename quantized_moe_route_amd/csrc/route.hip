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

// -------------------------------------------------- top-k by ranking (block)
// For k <= 32: every logit becomes a 64-bit key that orders exactly like
// (larger value, then lower index): the float bits mapped to an unsigned
// order (with -0.0 read as +0.0) in the high word, the complemented index in
// the low word.  Keys are distinct, so ranks are a permutation.
//   phase 1: each 64-expert chunk ranks its members against the chunk; the
//            ones ranked < k are the chunk's candidates (slot chunk*k + rank);
//   phase 2: each candidate's rank among its token's candidates is its
//            position in the output.
// No serial rounds: both phases are independent compares read from LDS.
constexpr int kRankMaxK = 32;

__device__ __forceinline__ unsigned long long topk_key(float v, int e) {
    uint32_t f = __float_as_uint(v);
    if (f == 0x80000000u) f = 0u;                        // -0.0 ties with +0.0
    const uint32_t ord = (f & 0x80000000u) ? ~f : (f | 0x80000000u);
    return ((unsigned long long)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ float key_value(unsigned long long key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

// keys [T][E] and cand [T][nch*k] in LDS; all threads of the block call this.
template <int NT>
__device__ void block_topk_rank(const unsigned long long *keys, unsigned long long *cand, int T, int E,
                                int k, int32_t *__restrict__ ids, float *__restrict__ w,
                                unsigned long long *sel /* LDS [T][k] */) {
    const int tid = threadIdx.x;
    const int nch = (E + 63) / 64;
    const int nslot = nch * k;
    // phase 1: task = (token, chunk, member)
    for (int task = tid; task < T * nch * 64; task += NT) {
        const int t = task / (nch * 64);
        const int rem = task - t * nch * 64;
        const int c = rem >> 6, m = rem & 63;
        const int e = c * 64 + m;
        const int clen = (E - c * 64) < 64 ? (E - c * 64) : 64;
        if (m < clen) {
            const unsigned long long my = keys[t * E + e];
            const unsigned long long *ck = keys + t * E + c * 64;
            int rank = 0;
            for (int j = 0; j < clen; ++j) rank += ck[j] > my ? 1 : 0;
            if (rank < k) cand[t * nslot + c * k + rank] = my;
        }
        if (m < k && m >= clen) cand[t * nslot + c * k + m] = 0ull;   // short last chunk
    }
    __syncthreads();
    // phase 2: task = (token, slot)
    for (int task = tid; task < T * nslot; task += NT) {
        const int t = task / nslot;
        const unsigned long long my = cand[task];
        if (my == 0ull) continue;
        const unsigned long long *tc = cand + t * nslot;
        int rank = 0;
        for (int j = 0; j < nslot; ++j) rank += tc[j] > my ? 1 : 0;
        if (rank < k) sel[t * k + rank] = my;
    }
    __syncthreads();
    // weights: softmax over the selected logits, one wave per token
    const int wv = tid >> 6, l = __lane_id();
    for (int t = wv; t < T; t += NT / 64) {
        const float l0 = key_value(sel[t * k]);
        float ev = 0.0f;
        if (l < k) ev = expf(key_value(sel[t * k + l]) - l0);
        const float inv = 1.0f / wave_sum(ev);
        if (l < k) {
            w[(size_t)t * k + l] = ev * inv;
            ids[(size_t)t * k + l] = (int)~(uint32_t)sel[t * k + l];
        }
    }
}

// ------------------------------------------------------- small T: one launch
// grid: (ceil(E/64) column slices, d/128 row chunks), 512 threads: wave w of
// a workgroup owns 16 router rows, lane = one expert column.  Partial sums go
// out at device scope; the last of all workgroups to arrive adds the d/128
// partials of every (token, expert) in chunk order, writes the logits and
// runs the top-k from LDS.
constexpr int kMaxSmallT = 8;

__global__ __launch_bounds__(512) void route_small_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ w, int32_t *__restrict__ counters, float *__restrict__ partial) {
    __shared__ float red[8][kMaxSmallT][64];
    // one LDS pool: ranking top-k (keys, candidates, selection) or, for k > 32,
    // the serial top-k's per-wave scratch
    constexpr int kKeyBytes = kMaxSmallT * 1024 * 8, kCandBytes = kMaxSmallT * 16 * kRankMaxK * 8;
    constexpr int kSelBytes = kMaxSmallT * kRankMaxK * 8;
    constexpr int kPoolBytes = kKeyBytes + kCandBytes + kSelBytes;
    static_assert(kPoolBytes >= 2 * 8 * 1024 * 4, "pool too small for the serial top-k");
    __shared__ __attribute__((aligned(16))) unsigned char pool[kPoolBytes];
    __shared__ int last_flag;
    unsigned long long *keys = reinterpret_cast<unsigned long long *>(pool);
    unsigned long long *cand = reinterpret_cast<unsigned long long *>(pool + kKeyBytes);
    unsigned long long *selk = reinterpret_cast<unsigned long long *>(pool + kKeyBytes + kCandBytes);
    float *sel = reinterpret_cast<float *>(pool);                      // [8][1024], k > 32 only
    int *seli = reinterpret_cast<int *>(pool + 8 * 1024 * 4);           // [8][1024], k > 32 only
    const int cs = blockIdx.x;
    const int kc = blockIdx.y;
    const int n_kc = gridDim.y;
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
    publish_then_count(&counters[kCntRouteAll], gridDim.x * gridDim.y, last_flag);
    if (!last_flag) return;
    if (tid == 0) store_dev_int(&counters[kCntRouteAll], 0);
    // last workgroup: sum the partials of every (token, expert) in chunk order
    for (int idx = tid; idx < T * E; idx += 512) {
        const int t = idx / E, ee = idx - t * E;
        float s_ = 0.0f;
        for (int q0 = 0; q0 < n_kc; q0 += 16) {
            float v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qc = q0 + i < n_kc ? q0 + i : n_kc - 1;
                v[i] = load_dev(&partial[((size_t)qc * T + t) * E + ee]);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) s_ += q0 + i < n_kc ? v[i] : 0.0f;
        }
        if (bias) s_ = s_ + bias[ee];
        logits[(size_t)t * E + ee] = s_;
        keys[t * E + ee] = topk_key(s_, ee);
    }
    __syncthreads();
    if (k <= kRankMaxK) {
        block_topk_rank<512>(keys, cand, T, E, k, ids, w, selk);
        return;
    }
    // large k: serial selection per token from the logits just written
    for (int t = wv; t < T; t += 8)
        wave_topk_any<false>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k,
                             sel + wv * 1024, seli + wv * 1024);
}

size_t route_ws_bytes(int d, int E, int T) {
    if (T > kMaxSmallT) return 0;
    return (size_t)(d / 128) * T * E * sizeof(float);
}

hipError_t launch_route_small(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, int k, int32_t *ids, float *w, void *ws,
                              hipStream_t s) {
    int32_t *counters = reinterpret_cast<int32_t *>(ws);
    float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kWsHeader);
    dim3 grid((E + 63) / 64, d / 128);
    hipLaunchKernelGGL(route_small_kernel, grid, dim3(512), 0, s, x, wr, bias, logits, T, d, E, k,
                       ids, w, counters, partial);
    return hipGetLastError();
}

// ------------------------------------------------------------ top-k kernel
// Logits given: two tokens per 256-thread workgroup ranked as above; for
// k > 32 one wave per token selects serially.
__global__ __launch_bounds__(256) void topk_rank_kernel(const float *__restrict__ logits, int T,
                                                        int E, int k, int32_t *__restrict__ ids,
                                                        float *__restrict__ w) {
    __shared__ unsigned long long keys[2 * 1024];
    __shared__ unsigned long long cand[2 * 16 * kRankMaxK];
    __shared__ unsigned long long selk[2 * kRankMaxK];
    const int t0 = blockIdx.x * 2;
    const int nt = (T - t0) < 2 ? (T - t0) : 2;
    for (int i = threadIdx.x; i < nt * E; i += 256) {
        const int t = i / E, e = i - t * E;
        keys[i] = topk_key(logits[(size_t)(t0 + t) * E + e], e);
    }
    __syncthreads();
    block_topk_rank<256>(keys, cand, nt, E, k, ids + (size_t)t0 * k, w + (size_t)t0 * k, selk);
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
    if (k <= kRankMaxK)
        hipLaunchKernelGGL(topk_rank_kernel, dim3((T + 1) / 2), dim3(256), 0, s, logits, T, E, k,
                           ids, w);
    else
        hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, T, E, k, ids, w);
    return hipGetLastError();
}

// ------------------------------------------------------- large T: MFMA GEMM
// Tile: 64 tokens x 64 experts per workgroup, K step 32.  Four waves in a 2x2
// grid, each owning 32x32 = 2x2 MFMA 16x16 tiles.  LDS holds the x tile
// (bf16, [64][32]) and the three bf16 terms of the router tile, transposed to
// [n][k] so each lane reads 8 consecutive k with one 16-byte load.
constexpr int RG_M = 64, RG_N = 64, RG_K = 32, RG_PAD = 8;

__device__ __forceinline__ void split3(float v, uint16_t &h, uint16_t &m, uint16_t &lo) {
    uint32_t u = __float_as_uint(v);
    h = (uint16_t)(u >> 16);
    float r1 = v - __uint_as_float(u & 0xffff0000u);
    uint32_t u1 = __float_as_uint(r1);
    m = (uint16_t)(u1 >> 16);
    float r2 = r1 - __uint_as_float(u1 & 0xffff0000u);
    lo = (uint16_t)(__float_as_uint(r2) >> 16);   // r2 has <= 8 significant bits: exact
}

__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits, int T, int d,
                                                          int E) {
    __shared__ __attribute__((aligned(16))) uint16_t As[RG_M][RG_K + RG_PAD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[3][RG_N][RG_K + RG_PAD];
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wv = wave_uniform(tid >> 6);
    const int m0 = blockIdx.x * RG_M, n0 = blockIdx.y * RG_N;
    const int wm = (wv >> 1) * 32, wn = (wv & 1) * 32;
    f32x4 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < d; k0 += RG_K) {
        // A: 64 rows x 32 bf16 = 256 x 16 B
        {
            const int r = tid >> 2, c = (tid & 3) * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (m0 + r < T) v = *reinterpret_cast<const u32x4 *>(x + (size_t)(m0 + r) * d + k0 + c);
            *reinterpret_cast<u32x4 *>(&As[r][c]) = v;
        }
        // B: 32 k-rows x 64 experts fp32 = 512 float4: two per thread
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + q * 256;
            const int kr = idx >> 4, nc = (idx & 15) * 4;
            float4 v = {0.f, 0.f, 0.f, 0.f};
            const float *p = wr + (size_t)(k0 + kr) * E + n0 + nc;
            if (n0 + nc + 3 < E) {
                v = *reinterpret_cast<const float4 *>(p);
            } else {
                if (n0 + nc + 0 < E) v.x = p[0];
                if (n0 + nc + 1 < E) v.y = p[1];
                if (n0 + nc + 2 < E) v.z = p[2];
            }
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint16_t h, m, lo;
                split3(vv[i], h, m, lo);
                Bs[0][nc + i][kr] = h;
                Bs[1][nc + i][kr] = m;
                Bs[2][nc + i][kr] = lo;
            }
        }
        __syncthreads();
        const int g = lane >> 4, rr = lane & 15;
        u32x4 af[2], bfr[3][2];
#pragma unroll
        for (int a = 0; a < 2; ++a) af[a] = *reinterpret_cast<const u32x4 *>(&As[wm + a * 16 + rr][g * 8]);
#pragma unroll
        for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                bfr[t3][b] = *reinterpret_cast<const u32x4 *>(&Bs[t3][wn + b * 16 + rr][g * 8]);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                acc[a][b] = mfma_bf16(af[a], bfr[2][b], acc[a][b]);
                acc[a][b] = mfma_bf16(af[a], bfr[1][b], acc[a][b]);
                acc[a][b] = mfma_bf16(af[a], bfr[0][b], acc[a][b]);
            }
        __syncthreads();
    }
    // D: lane holds rows 4*(lane/16)+i, column lane%16
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int n = n0 + wn + b * 16 + (lane & 15);
            if (n >= E) continue;
            const float bb = bias ? bias[n] : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = m0 + wm + a * 16 + 4 * (lane >> 4) + i;
                if (m < T) logits[(size_t)m * E + n] = bias ? acc[a][b][i] + bb : acc[a][b][i];
            }
        }
}

hipError_t launch_router_gemm(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, hipStream_t s) {
    dim3 grid((T + RG_M - 1) / RG_M, (E + RG_N - 1) / RG_N);
    hipLaunchKernelGGL(router_gemm_kernel, grid, dim3(256), 0, s, x, wr, bias, logits, T, d, E);
    return hipGetLastError();
}

}  // namespace moe
