// combine.hip -- weighted merge of each token's expert outputs.
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 …", section
// "Strata의 동작 원리 / 그래픽카드, RAM, SSD에 나눠 담은 전문가": the GPU merges the
// results of all experts, then the next layer starts.
//   out[t] = y_shared[t] + sum_j w[t][j] * y_pairs[pair_pos[t*k+j]]
// A pure streaming gather: one thread per 4 output columns, fp32, shared term
// first then j = 0..k-1 (fixed order, deterministic).  The pair positions and
// weights of a batch of 10 j are loaded first, then the batch's 10 rows all
// at once (nontemporal: each row is read once), so each thread keeps 10 row
// loads in flight instead of one.  A pair
// that route tail-skip dropped (pair_pos -1) adds nothing (its load reads
// row 0, unused).
#include "common.h"

namespace moe {

// pairs whose rows are loaded together: a top-10 token's rows all at once
constexpr int kCombineBatch = 10;

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y_pairs,
                                                      const float *__restrict__ y_shared,
                                                      const int32_t *__restrict__ pair_pos,
                                                      const float *__restrict__ w, int T, int k,
                                                      int d, float *__restrict__ out) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    const int32_t *pp = pair_pos + (size_t)t * k;
    const float *ww = w + (size_t)t * k;
    float4 acc = *reinterpret_cast<const float4 *>(y_shared + (size_t)t * d + c);
    for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
        int p[kCombineBatch];
        float wj[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            const int j = j0 + i < k ? j0 + i : k - 1;   // clamped: loaded, not used
            p[i] = pp[j];
            wj[i] = ww[j];
        }
        float4 v[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            // each y row is read once: nontemporal loads keep it out of the caches
            const f32x4 t = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4 *>(y_pairs + (size_t)(p[i] >= 0 ? p[i] : 0) * d + c));
            v[i] = make_float4(t[0], t[1], t[2], t[3]);
        }
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
            if (j0 + i < k && p[i] >= 0) {
                acc.x += wj[i] * v[i].x;
                acc.y += wj[i] * v[i].y;
                acc.z += wj[i] * v[i].z;
                acc.w += wj[i] * v[i].w;
            }
        }
    }
    *reinterpret_cast<float4 *>(out + (size_t)t * d + c) = acc;
}

hipError_t launch_combine(const float *y_pairs, const float *y_shared, const int32_t *pair_pos,
                          const float *w, int T, int k, int d, float *out, hipStream_t s) {
    dim3 grid((d / 4 + 255) / 256, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, y_pairs, y_shared, pair_pos, w, T, k,
                       d, out);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4 *__restrict__ p, size_t n16,
                                                        uint8_t *__restrict__ tail, size_t ntail) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        p[i] = uint4{0u, 0u, 0u, 0u};
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<uint4 *>(p), n16, static_cast<uint8_t *>(p) + n16 * 16,
                       bytes - n16 * 16);
    return hipGetLastError();
}

}  // namespace moe
