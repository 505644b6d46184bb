// abi.hip -- the extern "C" entry points of libmoe: host-side validation, then
// the kernel launches.  Declarations and contracts: include/moe.h.
#include <stdint.h>

#include <mutex>

#include "common.h"

using namespace moe;

namespace {

// Scratch of moe_expert_ffn_noalloc: a fixed device array instead of a
// caller workspace.  Each GPU the library runs on holds its own copy for the
// life of the process.  Host code never uses the array's name as an address
// (on the host it is only a stand-in symbol): the device address is looked up
// once per device with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on first use).
moe_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return MOE_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

constexpr int kMaxE = 1024;
constexpr int kMaxDim = 16384;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
inline bool ok_dim(int v) { return v > 0 && v <= kMaxDim && v % 128 == 0; }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline moe_status launched(hipError_t e) {
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_HIP;
    }
    return MOE_OK;
}

bool check_qmat(const moe_qmat &m, int fmt) {
    if (!m.lo || !m.scale) return false;
    if (!aligned16(m.lo) || !aligned16(m.scale)) return false;
    if (fmt == MOE_FMT_Q2_B32) {
        if (m.hi || !m.min || !aligned16(m.min)) return false;
    } else {
        if (m.min || !m.hi || !aligned16(m.hi)) return false;
    }
    return true;
}

// route needs the header always (counters) plus its partial sums
size_t route_need(int d, int E, int T) { return kWsHeader + route_ws_bytes(d, E, T); }
size_t dispatch_need(int E, int T, int k) { return kWsHeader + dispatch_ws_bytes(E, T, k); }
size_t ffn_need(int d, int f, int E, int T, int k) {
    if (T <= kSmallTMax) return kWsHeader + ffn_small_ws_bytes(d, f, E, T, k);
    if (T <= kPfMidTMax) return kWsHeader + ffn_prefill_mid_ws_bytes(d, f, E, T, k);
    return kWsHeader + ffn_prefill_ws_bytes(d, f, E, T, k);
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported format or shape";
        case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
        case MOE_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

moe_status moe_validate_ids(const int32_t *topk_ids_host, int32_t T, int32_t E, int32_t k) {
    if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k >= INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!topk_ids_host) return MOE_ERR_INVALID_ARGUMENT;
    // seen[e] holds the last token (+1) that named expert e
    int32_t seen[kMaxE] = {0};
    for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
            const int32_t e = topk_ids_host[(int64_t)t * k + j];
            if (e < 0 || e >= E || seen[e] == t + 1) return MOE_ERR_INVALID_ARGUMENT;
            seen[e] = t + 1;
        }
    return MOE_OK;
}

size_t moe_workspace_size(int32_t d_model, int32_t d_ff, int32_t E, int32_t T, int32_t k) {
    if (d_model <= 0 || d_ff <= 0 || E <= 0 || T < 0 || k <= 0) return 0;
    size_t need = route_need(d_model, E, T);
    const size_t b = dispatch_need(E, T, k);
    const size_t c = ffn_need(d_model, d_ff, E, T, k);
    if (b > need) need = b;
    if (c > need) need = c;
    return (need + 255) & ~(size_t)255;
}

moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream) {
    if (!ws || !aligned256(ws) || ws_bytes < kWsHeader) return MOE_ERR_WORKSPACE;
    return launched(launch_fill_zero(ws, ws_bytes, as_stream(stream)));
}

moe_status moe_route(const uint16_t *x_bf16, const float *w_router, const float *bias,
                     float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                     int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k >= INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (!logits || !topk_ids || !topk_w) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w))
        return MOE_ERR_INVALID_ARGUMENT;
    if (w_router) {
        if (!x_bf16 || !aligned16(x_bf16) || !aligned16(w_router)) return MOE_ERR_INVALID_ARGUMENT;
        if (bias && !aligned16(bias)) return MOE_ERR_INVALID_ARGUMENT;
        if (!ok_dim(d_model)) return MOE_ERR_UNSUPPORTED;
    } else {
        if (x_bf16 || bias) return MOE_ERR_INVALID_ARGUMENT;
    }
    if (!ws || !aligned256(ws)) return MOE_ERR_WORKSPACE;
    if (w_router && ws_bytes < route_need(d_model, E, T)) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    hipStream_t s = as_stream(stream);
    if (!w_router) return launched(launch_topk(logits, T, E, k, topk_ids, topk_w, s));
    if (T <= kRouteSmallTMax)
        return launched(launch_route_small(x_bf16, w_router, bias, logits, T, d_model, E, k,
                                           topk_ids, topk_w, ws, s));
    hipError_t e = launch_router_gemm(x_bf16, w_router, bias, logits, T, d_model, E, ws, s);
    if (e != hipSuccess) return launched(e);
    return launched(launch_topk(logits, T, E, k, topk_ids, topk_w, s));
}

static moe_status dispatch_checked(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k,
                                   int32_t tail_from, int32_t *offsets, int32_t *sorted_pair,
                                   int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream) {
    if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (tail_from < 0 || tail_from > k) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k >= INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (!topk_ids || !offsets || !sorted_pair || !pair_pos) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(topk_ids) || !aligned16(offsets) || !aligned16(sorted_pair) ||
        !aligned16(pair_pos))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!ws || !aligned256(ws) || ws_bytes < dispatch_need(E, T, k)) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    return launched(launch_dispatch(topk_ids, T, E, k, tail_from, offsets, sorted_pair, pair_pos, ws,
                                    as_stream(stream)));
}

moe_status moe_dispatch(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k,
                        int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos, void *ws,
                        size_t ws_bytes, void *stream) {
    return dispatch_checked(topk_ids, T, E, k, k, offsets, sorted_pair, pair_pos, ws, ws_bytes, stream);
}

moe_status moe_dispatch_tail_skip(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k,
                                  int32_t tail_from, int32_t *offsets, int32_t *sorted_pair,
                                  int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream) {
    return dispatch_checked(topk_ids, T, E, k, tail_from, offsets, sorted_pair, pair_pos, ws, ws_bytes,
                            stream);
}

static moe_status route_dispatch_checked(const uint16_t *x_bf16, const float *w_router, const float *bias,
                                         float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                                         int32_t tail_from, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                                         int32_t *sorted_pair, int32_t *pair_pos, void *ws, size_t ws_bytes,
                                         void *stream) {
    // the checks of both calls, before anything is enqueued
    if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (tail_from < 0 || tail_from > k) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k >= INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (!w_router || !x_bf16 || !logits || !topk_ids || !topk_w || !offsets || !sorted_pair || !pair_pos)
        return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x_bf16) || !aligned16(w_router) || (bias && !aligned16(bias)) || !aligned16(logits) ||
        !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(offsets) || !aligned16(sorted_pair) ||
        !aligned16(pair_pos))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!ok_dim(d_model)) return MOE_ERR_UNSUPPORTED;
    if (!ws || !aligned256(ws) || ws_bytes < route_need(d_model, E, T) || ws_bytes < dispatch_need(E, T, k))
        return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    if (T <= kRouteTile && k <= kWaveTopkMaxK)
        return launched(launch_route_small(x_bf16, w_router, bias, logits, T, d_model, E, k, topk_ids,
                                           topk_w, ws, as_stream(stream), offsets, sorted_pair, pair_pos,
                                           tail_from));
    const moe_status st = moe_route(x_bf16, w_router, bias, logits, T, d_model, E, k, topk_ids, topk_w, ws,
                                    ws_bytes, stream);
    if (st != MOE_OK) return st;
    return dispatch_checked(topk_ids, T, E, k, tail_from, offsets, sorted_pair, pair_pos, ws, ws_bytes, stream);
}

moe_status moe_route_dispatch(const uint16_t *x_bf16, const float *w_router, const float *bias,
                              float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                              int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *sorted_pair,
                              int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream) {
    return route_dispatch_checked(x_bf16, w_router, bias, logits, T, d_model, E, k, k, topk_ids, topk_w, offsets,
                                  sorted_pair, pair_pos, ws, ws_bytes, stream);
}

moe_status moe_route_dispatch_tail_skip(const uint16_t *x_bf16, const float *w_router, const float *bias,
                                        float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                                        int32_t tail_from, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                                        int32_t *sorted_pair, int32_t *pair_pos, void *ws, size_t ws_bytes,
                                        void *stream) {
    return route_dispatch_checked(x_bf16, w_router, bias, logits, T, d_model, E, k, tail_from, topk_ids, topk_w,
                                  offsets, sorted_pair, pair_pos, ws, ws_bytes, stream);
}

static moe_status ffn_checked(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                              const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                              float *y_shared, int parts, void *ws, size_t ws_bytes, void *stream,
                              bool validate_only = false) {
    if (!layer) return MOE_ERR_INVALID_ARGUMENT;
    const moe_layer &L = *layer;
    if (L.format != MOE_FMT_Q2_B32 && L.format != MOE_FMT_Q3_B32) return MOE_ERR_UNSUPPORTED;
    if (!ok_dim(L.d_model) || !ok_dim(L.d_ff)) return MOE_ERR_UNSUPPORTED;
    if (L.n_experts < 1 || L.n_experts > kMaxE) return MOE_ERR_INVALID_ARGUMENT;
    if (T < 0) return MOE_ERR_INVALID_ARGUMENT;
    if ((parts & kFfnRouted) && (k < 1 || k > L.n_experts)) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k >= INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (!x_bf16 || !aligned16(x_bf16)) return MOE_ERR_INVALID_ARGUMENT;
    if (parts & kFfnRouted) {
        if (!check_qmat(L.gate, L.format) || !check_qmat(L.up, L.format) || !check_qmat(L.down, L.format))
            return MOE_ERR_INVALID_ARGUMENT;
        if (!offsets || !sorted_pair || !y_pairs) return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned16(offsets) || !aligned16(sorted_pair) || !aligned16(y_pairs))
            return MOE_ERR_INVALID_ARGUMENT;
    }
    if (parts & kFfnShared) {
        if (!check_qmat(L.sh_gate, L.format) || !check_qmat(L.sh_up, L.format) ||
            !check_qmat(L.sh_down, L.format))
            return MOE_ERR_INVALID_ARGUMENT;
        if (!y_shared || !aligned16(y_shared)) return MOE_ERR_INVALID_ARGUMENT;
    }
    if (!ws || !aligned256(ws) || ws_bytes < ffn_need(L.d_model, L.d_ff, L.n_experts, T, k))
        return MOE_ERR_WORKSPACE;
    if (T == 0 || validate_only) return MOE_OK;
    hipStream_t s = as_stream(stream);
    if (T <= kSmallTMax)
        return launched(launch_ffn_small(L, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, ws,
                                         parts, s));
    hipError_t e = T <= kPfMidTMax ? launch_ffn_prefill_mid(L, x_bf16, T, k, offsets, sorted_pair, y_pairs,
                                                            y_shared, ws, parts, s)
                                   : launch_ffn_prefill(L, x_bf16, T, k, offsets, sorted_pair, y_pairs,
                                                        y_shared, ws, parts, s);
    if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
    return launched(e);
}

moe_status moe_expert_ffn(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                          const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                          float *y_shared, void *ws, size_t ws_bytes, void *stream) {
    return ffn_checked(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, kFfnBoth, ws, ws_bytes,
                       stream);
}

moe_status moe_routed_ffn(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                          const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs, void *ws,
                          size_t ws_bytes, void *stream) {
    return ffn_checked(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, nullptr, kFfnRouted, ws, ws_bytes,
                       stream);
}

moe_status moe_shared_ffn(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, float *y_shared,
                          void *ws, size_t ws_bytes, void *stream) {
    // k = 0: the workspace holds the shared expert's rows only
    return ffn_checked(layer, x_bf16, T, 0, nullptr, nullptr, nullptr, y_shared, kFfnShared, ws, ws_bytes,
                       stream);
}

moe_status moe_expert_ffn_noalloc(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                                  const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                                  float *y_shared, void *stream) {
    // every check of moe_expert_ffn except the workspace's (a stand-in
    // address that passes the alignment test and an unbounded size)
    const moe_status st = ffn_checked(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, kFfnBoth,
                                      reinterpret_cast<void *>((uintptr_t)256), SIZE_MAX, stream,
                                      /*validate_only=*/true);
    if (st != MOE_OK) return st;
    if (T > kSmallTMax) return MOE_ERR_UNSUPPORTED;
    if (ffn_need(layer->d_model, layer->d_ff, layer->n_experts, T, k) > kStaticScratchBytes)
        return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    void *ws = nullptr;
    const moe_status sst = scratch_of_current_device(&ws);
    if (sst != MOE_OK) return sst;
    // the small-batch kernels write every scratch byte they read (h rows,
    // group table) earlier in the same call: nothing must start at zero
    return launched(launch_ffn_small(*layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, ws, kFfnBoth,
                                     as_stream(stream)));
}

moe_status moe_expert_ffn_combine(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                                  const int32_t *offsets, const int32_t *sorted_pair, const int32_t *pair_pos,
                                  const float *topk_w, float *y_pairs, float *y_shared, float *out, void *ws,
                                  size_t ws_bytes, void *stream) {
    if (!pair_pos || !topk_w || !out || !aligned16(pair_pos) || !aligned16(topk_w) || !aligned16(out))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!layer) return MOE_ERR_INVALID_ARGUMENT;
    if (T > kFuseCombineTMax || T == 0) {
        // one call after the other
        const moe_status st = moe_expert_ffn(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, ws,
                                             ws_bytes, stream);
        if (st != MOE_OK) return st;
        return moe_combine(y_pairs, y_shared, pair_pos, topk_w, T, k, layer->d_model, out, stream);
    }
    // validation of both calls, then the fused launch
    const moe_status st = ffn_checked(layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, kFfnBoth,
                                      ws, ws_bytes, stream, /*validate_only=*/true);
    if (st != MOE_OK) return st;
    return launched(launch_ffn_small(*layer, x_bf16, T, k, offsets, sorted_pair, y_pairs, y_shared, ws, kFfnBoth,
                                     as_stream(stream), pair_pos, topk_w, out));
}

moe_status moe_combine(const float *y_pairs, const float *y_shared, const int32_t *pair_pos,
                       const float *topk_w, int32_t T, int32_t k, int32_t d_model, float *out,
                       void *stream) {
    if (T < 0 || k < 1 || k > kMaxE) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k >= INT32_MAX) return MOE_ERR_INVALID_ARGUMENT;
    if (!ok_dim(d_model)) return MOE_ERR_UNSUPPORTED;
    if (!y_pairs || !y_shared || !pair_pos || !topk_w || !out) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(y_pairs) || !aligned16(y_shared) || !aligned16(pair_pos) ||
        !aligned16(topk_w) || !aligned16(out))
        return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    return launched(launch_combine(y_pairs, y_shared, pair_pos, topk_w, T, k, d_model, out,
                                   as_stream(stream)));
}

}  // extern "C"
