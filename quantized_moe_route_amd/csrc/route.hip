// route.hip -- router logits, top-k selection and routing weights.
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 Qwen3.8-Flash-
// Next만을 위해 만든 추론 엔진", section "Strata의 동작 원리 / 그래픽카드, RAM, SSD에
// 나눠 담은 전문가": the router runs on the GPU for every token and layer and
// names the experts the token uses; section "Strata 소개": 10 of 512 per layer.
//
// Small T (decode, MTP verify): one launch.  The d x E router matrix (4 MiB
// fp32 at d=2048, E=512) is the only large read, so it is split over
// (E/64 column slices) x (d/64 row chunks) workgroups -- 256 of them at the
// full shape -- each reading 64 rows x 64 columns once.  Partial sums are
// reduced in a fixed order by the last workgroup to arrive per column slice,
// and the last slice to finish runs the top-k, so the result is deterministic
// and needs no second launch.
//
// Large T (prefill): a matrix-core GEMM.  fp32 router weights are split
// exactly into three bf16 terms (truncation: hi + mid + lo == w), x is already
// bf16, so every product is exact and only the fp32 accumulation order
// differs from a plain fp32 dot product.  A second kernel does the top-k, one
// wave per token.
#include "common.h"

namespace moe {

// --------------------------------------------------------------- top-k (wave)
// One wave selects the k largest of E (<= 1024) logits: larger value first,
// equal values (including -0.0 vs +0.0) by lower index.  Lane l owns experts
// l, l+64, ... .  Weights: softmax over the k selected logits.
__device__ void wave_topk(const float *__restrict__ lg, int E, int k, int32_t *__restrict__ ids,
                          float *__restrict__ w, float *sel /* LDS, >= k floats */) {
    const int l = __lane_id();
    const int per = (E + 63) / 64;
    float v[16];
    uint32_t alive = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = l + 64 * i;
        v[i] = 0.0f;
        if (i < per && e < E) {
            v[i] = lg[e];
            alive |= 1u << i;
        }
    }
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((alive >> i) & 1u) {
                // entries are visited in ascending index, so strict > keeps the lowest index
                if (bi == 0x7fffffff || v[i] > bv) {
                    bv = v[i];
                    bi = l + 64 * i;
                }
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float ov = __shfl_xor(bv, o, 64);
            const int oi = __shfl_xor(bi, o, 64);
            const bool take = (oi != 0x7fffffff) &&
                              (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
            if (take) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == l) alive &= ~(1u << (bi >> 6));
        if (l == 0) {
            ids[j] = bi;
            sel[j] = bv;
        }
    }
    // lane 0 wrote sel[]; make the LDS writes complete before other lanes read
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const float l0 = sel[0];
    float part = 0.0f;
    for (int j = l; j < k; j += 64) part += expf(sel[j] - l0);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    const float inv = 1.0f / part;
    for (int j = l; j < k; j += 64) w[j] = expf(sel[j] - l0) * inv;
}

// ------------------------------------------------------- small T: one launch
constexpr int kMaxSmallT = 8;

__global__ __launch_bounds__(256) void route_small_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    float *__restrict__ logits, int T, int d, int E, int k, int32_t *__restrict__ ids,
    float *__restrict__ w, int32_t *__restrict__ counters, float *__restrict__ partial) {
    __shared__ float red[4][kMaxSmallT][64];
    __shared__ float sel[4][1024];
    __shared__ int last_flag;
    const int cs = blockIdx.x;        // 64-column slice
    const int kc = blockIdx.y;        // 64-row chunk
    const int n_kc = gridDim.y;
    const int n_cs = gridDim.x;
    const int tid = threadIdx.x;
    const int col = tid & 63;
    const int wv = wave_uniform(tid >> 6);
    const int e = cs * 64 + col;

    float acc[kMaxSmallT];
#pragma unroll
    for (int t = 0; t < kMaxSmallT; ++t) acc[t] = 0.0f;
    const int c0 = kc * 64 + wv * 16;
    if (e < E) {
#pragma unroll 4
        for (int r = 0; r < 16; ++r) {
            const int c = c0 + r;
            const float wv_ = wr[(size_t)c * E + e];
#pragma unroll
            for (int t = 0; t < kMaxSmallT; ++t)
                if (t < T) acc[t] += bf16_bits_to_float(x[(size_t)t * d + c]) * wv_;
        }
    }
#pragma unroll
    for (int t = 0; t < kMaxSmallT; ++t) red[wv][t][col] = acc[t];
    __syncthreads();
    if (wv == 0 && e < E) {
        for (int t = 0; t < T; ++t) {
            const float s = (red[0][t][col] + red[1][t][col]) + (red[2][t][col] + red[3][t][col]);
            partial[((size_t)kc * T + t) * E + e] = s;
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const int old = atomicAdd(&counters[kCntRouteSlice + cs], 1);
        last_flag = (old == n_kc - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    // last arrival for this slice: reduce the n_kc partials in chunk order
    if (wv == 0 && e < E) {
        for (int t = 0; t < T; ++t) {
            float s = 0.0f;
            for (int q = 0; q < n_kc; ++q) s += partial[((size_t)q * T + t) * E + e];
            if (bias) s = s + bias[e];
            logits[(size_t)t * E + e] = s;
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        counters[kCntRouteSlice + cs] = 0;
        const int old = atomicAdd(&counters[kCntRouteAll], 1);
        last_flag = (old == n_cs - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    if (tid == 0) counters[kCntRouteAll] = 0;
    for (int t = wv; t < T; t += 4)
        wave_topk(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, sel[wv]);
}

size_t route_ws_bytes(int d, int E, int T) {
    if (T > kMaxSmallT) return 0;
    return (size_t)(d / 64) * T * E * sizeof(float);
}

hipError_t launch_route_small(const uint16_t *x, const float *wr, const float *bias, float *logits,
                              int T, int d, int E, int k, int32_t *ids, float *w, void *ws,
                              hipStream_t s) {
    int32_t *counters = reinterpret_cast<int32_t *>(ws);
    float *partial = reinterpret_cast<float *>(static_cast<char *>(ws) + kWsHeader);
    dim3 grid((E + 63) / 64, d / 64);
    hipLaunchKernelGGL(route_small_kernel, grid, dim3(256), 0, s, x, wr, bias, logits, T, d, E, k,
                       ids, w, counters, partial);
    return hipGetLastError();
}

// ------------------------------------------------------------ top-k kernel
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k, int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
    __shared__ float sel[4][1024];
    const int wv = wave_uniform(threadIdx.x >> 6);
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;
    wave_topk(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, sel[wv]);
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int32_t *ids, float *w,
                       hipStream_t s) {
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
