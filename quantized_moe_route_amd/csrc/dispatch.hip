// dispatch.hip -- expert-sorted permutation of the token-expert pairs.
//
// [forum] discuss.pytorch.kr "Strata: 12GB 그래픽카드 PC에서 125B 모델 …", section
// "Strata의 동작 원리 / 그래픽카드, RAM, SSD에 나눠 담은 전문가": once the router has
// named the experts, the work is split among the places that compute them.
// With every expert resident in HBM the split is a stable counting sort of
// the pairs by expert, done on the device (no host round trip).
//
// Stability without atomics on positions: tokens are taken in chunks of 64
// (one wave, lane = token).  A token selects an expert at most once, so within
// a chunk the pairs of expert e form a 64-bit token mask, built with LDS
// atomic OR.  The rank of a pair inside its expert segment is then
//   (pairs of e in earlier chunks) + popcount(mask & lanes below this one),
// which is exactly the position a stable sort by (expert, pair index) gives.
#include "common.h"

namespace moe {

__device__ __forceinline__ unsigned long long below_mask(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// one wave: OR each token's bit into masks[e] for its k experts
__device__ __forceinline__ void build_chunk_masks(const int32_t *__restrict__ ids, int T, int k,
                                                  int chunk, unsigned long long *masks) {
    const int lane = __lane_id();
    const int t = chunk * 64 + lane;
    if (t < T) {
        const unsigned long long bit = 1ull << lane;
        for (int j = 0; j < k; ++j) atomicOr(&masks[ids[(size_t)t * k + j]], bit);
    }
}

__device__ __forceinline__ void write_chunk_positions(const int32_t *__restrict__ ids, int T, int k,
                                                      int chunk, const unsigned long long *masks,
                                                      const int32_t *base /* [E] for chunk */,
                                                      int32_t *__restrict__ sorted_pair,
                                                      int32_t *__restrict__ pair_pos) {
    const int lane = __lane_id();
    const int t = chunk * 64 + lane;
    if (t >= T) return;
    const unsigned long long lt = below_mask(lane);
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int pos = base[e] + __popcll(masks[e] & lt);
        const int p = t * k + j;
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
    }
}

// In-place exclusive scan of v[0..n) (n <= 1024) by a block of exactly 1024
// threads (16 waves).
__device__ void block_excl_scan_1024(int *v, int n, int *wsum /* LDS [16] */) {
    const int tid = threadIdx.x;
    const int lane = __lane_id(), wv = tid >> 6;
    const int x = tid < n ? v[tid] : 0;
    const int incl = wave_incl_scan(x);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    if (wv == 0) {
        const int s = lane < 16 ? wsum[lane] : 0;
        const int si = wave_incl_scan(s);
        if (lane < 16) wsum[lane] = si - s;
    }
    __syncthreads();
    if (tid < n) v[tid] = incl - x + wsum[wv];
}

// ------------------------------------------------------------ fused, small P
constexpr int kSmallMaskEntries = 4096;   // n_chunks * E

__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t *__restrict__ ids, int T,
                                                              int E, int k,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ sorted_pair,
                                                              int32_t *__restrict__ pair_pos) {
    __shared__ unsigned long long masks[kSmallMaskEntries];
    __shared__ int32_t cbase[kSmallMaskEntries];
    __shared__ int32_t tot[1024];
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int n_chunks = (T + 63) / 64;
    for (int i = tid; i < n_chunks * E; i += 1024) masks[i] = 0ull;
    __syncthreads();
    for (int c = wv; c < n_chunks; c += 16) build_chunk_masks(ids, T, k, c, masks + (size_t)c * E);
    __syncthreads();
    // per expert: prefix over chunks
    if (tid < E) {
        int run = 0;
        for (int c = 0; c < n_chunks; ++c) {
            cbase[c * E + tid] = run;
            run += __popcll(masks[c * E + tid]);
        }
        tot[tid] = run;
    }
    __syncthreads();
    block_excl_scan_1024(tot, E, wsum);
    __syncthreads();
    if (tid < E) {
        offsets[tid] = tot[tid];
        for (int c = 0; c < n_chunks; ++c) cbase[c * E + tid] += tot[tid];
    }
    if (tid == 0) offsets[E] = T * k;
    __syncthreads();
    for (int c = wv; c < n_chunks; c += 16)
        write_chunk_positions(ids, T, k, c, masks + (size_t)c * E, cbase + (size_t)c * E,
                              sorted_pair, pair_pos);
}

// ----------------------------------------------------------- three passes
__global__ __launch_bounds__(64) void dispatch_count_kernel(const int32_t *__restrict__ ids, int T,
                                                            int E, int k,
                                                            int32_t *__restrict__ cnt) {
    __shared__ unsigned long long masks[1024];
    const int c = blockIdx.x;
    for (int i = threadIdx.x; i < E; i += 64) masks[i] = 0ull;
    __syncthreads();
    build_chunk_masks(ids, T, k, c, masks);
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += 64) cnt[(size_t)c * E + i] = __popcll(masks[i]);
}

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t *__restrict__ cnt, int n_chunks,
                                                             int E, int P,
                                                             int32_t *__restrict__ offsets) {
    __shared__ int32_t tot[1024];
    __shared__ int wsum[16];
    const int tid = threadIdx.x;
    if (tid < E) {
        int run = 0;
        for (int c = 0; c < n_chunks; ++c) {
            const int v = cnt[(size_t)c * E + tid];
            cnt[(size_t)c * E + tid] = run;
            run += v;
        }
        tot[tid] = run;
    }
    __syncthreads();
    block_excl_scan_1024(tot, E, wsum);
    __syncthreads();
    if (tid < E) {
        const int o = tot[tid];
        offsets[tid] = o;
        for (int c = 0; c < n_chunks; ++c) cnt[(size_t)c * E + tid] += o;
    }
    if (tid == 0) offsets[E] = P;
}

__global__ __launch_bounds__(64) void dispatch_place_kernel(const int32_t *__restrict__ ids, int T,
                                                            int E, int k,
                                                            const int32_t *__restrict__ cbase,
                                                            int32_t *__restrict__ sorted_pair,
                                                            int32_t *__restrict__ pair_pos) {
    __shared__ unsigned long long masks[1024];
    const int c = blockIdx.x;
    for (int i = threadIdx.x; i < E; i += 64) masks[i] = 0ull;
    __syncthreads();
    build_chunk_masks(ids, T, k, c, masks);
    __syncthreads();
    write_chunk_positions(ids, T, k, c, masks, cbase + (size_t)c * E, sorted_pair, pair_pos);
}

static bool dispatch_fits_small(int E, int T) {
    return (size_t)((T + 63) / 64) * E <= (size_t)kSmallMaskEntries;
}

size_t dispatch_ws_bytes(int E, int T, int k) {
    (void)k;
    if (dispatch_fits_small(E, T)) return 0;
    return (size_t)((T + 63) / 64) * E * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t *ids, int T, int E, int k, int32_t *offsets,
                           int32_t *sorted_pair, int32_t *pair_pos, void *ws, hipStream_t s) {
    if (dispatch_fits_small(E, T)) {
        hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, s, ids, T, E, k, offsets,
                           sorted_pair, pair_pos);
        return hipGetLastError();
    }
    const int n_chunks = (T + 63) / 64;
    int32_t *cnt = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + kWsHeader);
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(n_chunks), dim3(64), 0, s, ids, T, E, k, cnt);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, n_chunks, E, T * k,
                       offsets);
    hipLaunchKernelGGL(dispatch_place_kernel, dim3(n_chunks), dim3(64), 0, s, ids, T, E, k, cnt,
                       sorted_pair, pair_pos);
    return hipGetLastError();
}

}  // namespace moe
