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
//
// Route tail-skip (opt-in; same page, same section: an expert that every token
// of the batch picked only at 7th place or lower of its top 10 is not
// computed).  With a rank threshold tail_from, expert e is kept iff some token
// picks it at a rank j < tail_from; the pairs of the other experts are left
// out of the listing (pair_pos = -1) and offsets count kept pairs only.  The
// kernels take a keep flag per expert (nullptr: every pair is kept).
//
// Ids are caller input here, so every id is range-checked before it indexes
// anything: a pair whose id lies outside [0, E) is left out of the listing
// (pair_pos = -1) and sets bit kErrIdRange of the workspace's error word; a
// token that names one expert twice sets bit kErrIdRepeat (its two pairs then
// share one position, so every listed entry is still a valid pair).
#include "common.h"

namespace moe {

__device__ __forceinline__ unsigned long long below_mask(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ bool id_ok(int e, int E) { return (unsigned)e < (unsigned)E; }

// one wave: OR each token's bit into masks[e] for its k experts (kept ones,
// if keep is given); with mark given, also flag mark[e] for the experts
// picked at a rank below tail_from.  Ids outside [0, E) and repeated ids are
// reported in *err (the workspace's error word).
__device__ __forceinline__ void build_chunk_masks(const int32_t *__restrict__ ids, int T, int E, int k,
                                                  int chunk, unsigned long long *masks,
                                                  const int32_t *keep, int32_t *err,
                                                  int32_t *mark = nullptr, int tail_from = 0) {
    const int lane = __lane_id();
    const int t = chunk * 64 + lane;
    if (t < T) {
        const unsigned long long bit = 1ull << lane;
        int bad = 0;
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            if (!id_ok(e, E)) {
                bad |= kErrIdRange;
                continue;
            }
            if (!keep || keep[e]) {
                const unsigned long long old = atomicOr(&masks[e], bit);
                if (old & bit) bad |= kErrIdRepeat;
            }
            if (mark && j < tail_from) mark[e] = 1;
        }
        if (bad && err) atomicOr(err, bad);
    }
}

__device__ __forceinline__ void write_chunk_positions(const int32_t *__restrict__ ids, int T, int E, int k,
                                                      int chunk, const unsigned long long *masks,
                                                      const int32_t *base /* [E] for chunk */,
                                                      int32_t *__restrict__ sorted_pair,
                                                      int32_t *__restrict__ pair_pos,
                                                      const int32_t *keep) {
    const int lane = __lane_id();
    const int t = chunk * 64 + lane;
    if (t >= T) return;
    const unsigned long long lt = below_mask(lane);
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int p = t * k + j;
        if (!id_ok(e, E) || (keep && !keep[e])) {
            pair_pos[p] = -1;
            continue;
        }
        const int pos = base[e] + __popcll(masks[e] & lt);
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
    }
}

// keep[e] = 1 iff some token picks e at a rank below tail_from (keep zeroed
// before); every writer stores the same value
__device__ __forceinline__ void mark_kept(const int32_t *__restrict__ ids, int T, int E, int k, int tail_from,
                                          int32_t *keep, int i0, int stride) {
    const int n = T * (tail_from < k ? tail_from : k);
    const int kh = tail_from < k ? tail_from : k;
    for (int i = i0; i < n; i += stride) {
        const int t = i / kh, j = i - t * kh;
        const int e = ids[(size_t)t * k + j];
        if (id_ok(e, E)) keep[e] = 1;   // a bad id is reported by the count pass
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

template <bool TAIL>
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t *__restrict__ ids, int T,
                                                              int E, int k, int tail_from,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ sorted_pair,
                                                              int32_t *__restrict__ pair_pos,
                                                              int32_t *__restrict__ err) {
    __shared__ unsigned long long masks[kSmallMaskEntries];
    __shared__ int32_t cbase[kSmallMaskEntries];
    __shared__ int32_t tot[1024];
    __shared__ int wsum[16];
    __shared__ int32_t keep_s[TAIL ? 1024 : 1];
    const int32_t *keep = TAIL ? keep_s : nullptr;
    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int n_chunks = (T + 63) / 64;
    for (int i = tid; i < n_chunks * E; i += 1024) masks[i] = 0ull;
    if constexpr (TAIL)
        for (int e = tid; e < E; e += 1024) keep_s[e] = 0;
    __syncthreads();
    // masks of every pair; with tail-skip the same pass flags the kept experts
    for (int c = wv; c < n_chunks; c += 16)
        build_chunk_masks(ids, T, E, k, c, masks + (size_t)c * E, nullptr, err, TAIL ? keep_s : nullptr,
                          tail_from);
    __syncthreads();
    // per expert: prefix over chunks (a dropped expert counts no pairs)
    int run = 0;
    if (tid < E) {
        const bool kept = !TAIL || keep_s[tid];
        for (int c = 0; c < n_chunks; ++c) {
            cbase[c * E + tid] = run;
            run += kept ? __popcll(masks[c * E + tid]) : 0;
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
    if (tid == E - 1) offsets[E] = tot[tid] + run;   // all (kept) pairs
    __syncthreads();
    for (int c = wv; c < n_chunks; c += 16)
        write_chunk_positions(ids, T, E, k, c, masks + (size_t)c * E, cbase + (size_t)c * E,
                              sorted_pair, pair_pos, keep);
}

// large batches, tail-skip: keep flags in the workspace (zeroed just before)
__global__ __launch_bounds__(256) void dispatch_keep_kernel(const int32_t *__restrict__ ids, int T, int E,
                                                            int k, int tail_from, int32_t *__restrict__ keep) {
    mark_kept(ids, T, E, k, tail_from, keep, blockIdx.x * 256 + threadIdx.x, gridDim.x * 256);
}

// ----------------------------------------------------------- three passes
// 1. count: cnt[c][e] = pairs of expert e in chunk c (chunk-major, so a wave's
//    64 lanes touch 64 consecutive experts).
__global__ __launch_bounds__(64) void dispatch_count_kernel(const int32_t *__restrict__ ids, int T,
                                                            int E, int k, const int32_t *keep,
                                                            int32_t *__restrict__ cnt, int32_t *__restrict__ err) {
    __shared__ unsigned long long masks[1024];
    const int c = blockIdx.x;
    for (int i = threadIdx.x; i < E; i += 64) masks[i] = 0ull;
    __syncthreads();
    build_chunk_masks(ids, T, E, k, c, masks, keep, err);
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += 64) cnt[(size_t)c * E + i] = __popcll(masks[i]);
}

// 2. scan, one workgroup per 64 experts (lane = expert), 16 waves splitting
//    the chunks: cnt[c][e] := pairs of e in chunks before c, tot[e] := all
//    pairs of e.  Loads go out 16 at a time.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int32_t *__restrict__ cnt, int n_chunks,
                                                             int E, int32_t *__restrict__ tot) {
    __shared__ int32_t seg[16][64];
    const int l = __lane_id(), wv = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + l;
    const int per = (n_chunks + 15) / 16;
    const int c0 = wv * per;
    const int c1 = c0 + per < n_chunks ? c0 + per : n_chunks;
    const bool ok = e < E;
    int sum = 0;
    if (ok) {
        for (int cb = c0; cb < c1; cb += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) {
                const int c = cb + i < c1 ? cb + i : c1 - 1;
                v[i] = cnt[(size_t)c * E + e];
            }
#pragma unroll
            for (int i = 0; i < kScanBatch; ++i) sum += cb + i < c1 ? v[i] : 0;
        }
    }
    seg[wv][l] = sum;
    __syncthreads();
    int run = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int v = seg[q][l];
        run += q < wv ? v : 0;
        total += v;
    }
    if (!ok) return;
    if (wv == 0) tot[e] = total;
    for (int cb = c0; cb < c1; cb += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            const int c = cb + i < c1 ? cb + i : c1 - 1;
            v[i] = cnt[(size_t)c * E + e];
        }
#pragma unroll
        for (int i = 0; i < kScanBatch; ++i) {
            if (cb + i < c1) {
                cnt[(size_t)(cb + i) * E + e] = run;
                run += v[i];
            }
        }
    }
}

// 3. place, one wave per chunk: expert offsets = exclusive scan of tot (each
//    lane sums a run of up to 16 experts, then a wave scan), written out by
//    chunk 0; position = offsets[e] + cnt[c][e] + earlier lanes of the chunk.
__global__ __launch_bounds__(64) void dispatch_place_kernel(const int32_t *__restrict__ ids, int T,
                                                            int E, int k, const int32_t *keep,
                                                            const int32_t *__restrict__ cnt,
                                                            const int32_t *__restrict__ tot,
                                                            int32_t *__restrict__ offsets,
                                                            int32_t *__restrict__ sorted_pair,
                                                            int32_t *__restrict__ pair_pos) {
    __shared__ unsigned long long masks[1024];
    __shared__ int32_t off[1024];
    const int c = blockIdx.x;
    const int lane = __lane_id();
    for (int i = lane; i < E; i += 64) masks[i] = 0ull;
    const int per = (E + 63) / 64;   // <= 16
    const int e0 = lane * per;
    int v[16];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = e0 + i;
        v[i] = (i < per && e < E) ? tot[e] : 0;
        sum += v[i];
    }
    int run = wave_incl_scan(sum) - sum;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = e0 + i;
        if (i < per && e < E) {
            off[e] = run;
            if (c == 0) offsets[e] = run;
        }
        run += v[i];
    }
    if (c == 0 && lane == 63) offsets[E] = run;
    __syncthreads();
    // errors were reported by the count pass over the same ids
    build_chunk_masks(ids, T, E, k, c, masks, keep, nullptr);
    __syncthreads();
    const int t = c * 64 + lane;
    if (t >= T) return;
    const unsigned long long lt = below_mask(lane);
    for (int j = 0; j < k; ++j) {
        const int e = ids[(size_t)t * k + j];
        const int p = t * k + j;
        if (!id_ok(e, E) || (keep && !keep[e])) {
            pair_pos[p] = -1;
            continue;
        }
        const int pos = off[e] + cnt[(size_t)c * E + e] + __popcll(masks[e] & lt);
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
    }
}

static bool dispatch_fits_small(int E, int T) {
    return (size_t)((T + 63) / 64) * E <= (size_t)kSmallMaskEntries;
}

// cnt [n_chunks][E], then tot [E], then the tail-skip keep flags [E]
size_t dispatch_ws_bytes(int E, int T, int k) {
    (void)k;
    if (dispatch_fits_small(E, T)) return 0;
    return ((size_t)((T + 63) / 64) * E + 2 * (size_t)E) * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t *ids, int T, int E, int k, int tail_from, int32_t *offsets,
                           int32_t *sorted_pair, int32_t *pair_pos, void *ws, hipStream_t s) {
    const bool tail = tail_from < k;
    int32_t *err = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + kWsErrorWord);
    if (dispatch_fits_small(E, T)) {
        if (tail)
            hipLaunchKernelGGL(dispatch_small_kernel<true>, dim3(1), dim3(1024), 0, s, ids, T, E, k,
                               tail_from, offsets, sorted_pair, pair_pos, err);
        else
            hipLaunchKernelGGL(dispatch_small_kernel<false>, dim3(1), dim3(1024), 0, s, ids, T, E, k,
                               tail_from, offsets, sorted_pair, pair_pos, err);
        return hipGetLastError();
    }
    const int n_chunks = (T + 63) / 64;
    int32_t *cnt = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + kWsHeader);
    int32_t *tot = cnt + (size_t)n_chunks * E;
    int32_t *keep = nullptr;
    if (tail) {
        keep = tot + E;
        hipError_t e = launch_fill_zero(keep, (size_t)E * sizeof(int32_t), s);
        if (e != hipSuccess) return e;
        const int n = T * (tail_from > 0 ? tail_from : 1);
        int blocks = (n + 255) / 256;
        blocks = blocks < 1024 ? blocks : 1024;
        hipLaunchKernelGGL(dispatch_keep_kernel, dim3(blocks), dim3(256), 0, s, ids, T, E, k, tail_from, keep);
    }
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(n_chunks), dim3(64), 0, s, ids, T, E, k, keep, cnt, err);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3((E + 63) / 64), dim3(1024), 0, s, cnt, n_chunks, E,
                       tot);
    hipLaunchKernelGGL(dispatch_place_kernel, dim3(n_chunks), dim3(64), 0, s, ids, T, E, k, keep, cnt, tot,
                       offsets, sorted_pair, pair_pos);
    return hipGetLastError();
}

}  // namespace moe
