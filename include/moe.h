/*
 * moe.h -- C ABI of libmoe: the routed, block-quantized Mixture-of-Experts
 * layer (top-k routed experts plus one shared expert, 2-3-bit weights), on one
 * AMD Instinct MI355X (gfx950).
 *
 * Where the operations come from (the pages this library follows):
 *   [forum] discuss.pytorch.kr, "Strata: 12GB 그래픽카드 PC에서 125B 모델
 *           Qwen3.8-Flash-Next만을 위해 만든 추론 엔진":
 *           section "Strata 소개" -- each layer selects 10 of 512 experts;
 *           section "Strata의 동작 원리 / 그래픽카드, RAM, SSD에 나눠 담은 전문가"
 *           -- per layer the router picks the expert ids, the ids are split
 *           among the places that compute them, and the GPU merges the results
 *           before the next layer; the router and the shared expert always sit
 *           on the GPU;
 *           section "추측 후 검증: MTP 층을 이용한 투기적 디코딩" -- the verify pass
 *           runs 1 + 3 tokens through the layers at once;
 *           section "긴 프롬프트와 긴 컨텍스트 처리" -- prompts are read in chunks
 *           of up to 8,192 tokens.
 *   [guide] tech.okbari.net, "Strata와 Qwen3.8-Flash-Next: RTX 4090 Windows 실행
 *           가이드", section "Strata, Qwen, GSQ-RCO는 서로 다른 구성 요소다" --
 *           48 layers; per MoE layer 10 of 512 routed experts plus 1 shared
 *           expert are active.
 *   [video] kangdaejong.com, "2026-10-09 strata-qwen-flash-next-soulseeker"
 *           summary, section "픽업" -- the selected experts' compressed weights
 *           are decompressed and computed on the GPU.
 * The pages give no formulas, tensor shapes or bit layouts.  The readings this
 * library takes: softmax over the E logits, top-k, renormalised over the k;
 * SwiGLU experts h = silu(x Wg^T) * (x Wu^T), y = h Wd^T; the shared expert is
 * added with weight 1; weights are stored in the block-32 formats below.
 *
 * Conventions for every call
 *   - Array pointers are DEVICE pointers owned by the caller (e.g. allocated
 *     through PyTorch).  `moe_layer` is a host struct holding device pointers;
 *     it is read during the call and not kept.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on `stream` and returns; the library never allocates,
 *     frees or synchronises.  Results are ready when the stream reaches them.
 *   - Arguments are validated on the host before anything is enqueued.  On any
 *     error nothing is enqueued and no output is written.
 *   - T == 0 is valid: MOE_OK, nothing enqueued.
 *   - Errors: MOE_ERR_INVALID_ARGUMENT (null pointer where one is required,
 *     bad size, misaligned pointer), MOE_ERR_UNSUPPORTED (unknown format or a
 *     shape outside the supported set), MOE_ERR_WORKSPACE (workspace too small
 *     or misaligned), MOE_ERR_HIP (a kernel launch failed; the HIP error is
 *     cleared).  Faults inside kernels surface at the caller's next
 *     synchronisation, as HIP reports them.
 *   - Supported shapes: 1 <= k <= E <= 1024; d_model and d_ff multiples of 128
 *     and at most 16384; T * k < 2^31.  Every pointer is 16-byte aligned.
 *   - Integer results (ids, offsets, permutation) are bit-exact and identical
 *     run to run; float results are deterministic on a given device.
 *   - Calls on different streams are independent only if they use different
 *     workspaces.
 *
 * Block-32 weight formats (rows x K matrix, K the reduction axis, blocks of 32
 * consecutive K elements share one scale):
 *   MOE_FMT_Q2_B32  2-bit codes q in 0..3, fp16 scale d, fp16 min m:
 *                   w = d*q + m                     (0.375 bytes per weight)
 *   MOE_FMT_Q3_B32  3-bit codes q in 0..7, fp16 scale d:
 *                   w = d*(q - 4)                   (0.4375 bytes per weight)
 * Storage order (rows % 16 == 0, K % 128 == 0).  The matrix is cut into units
 * of 16 rows x 128 columns, unit u = (r/16)*(K/128) + k/128.  Inside a unit:
 * rr = r%16, block j = (k%128)/32, eighth g = (k%32)/8, s = k%8, c = s%4.
 *   lo    512 bytes per unit.  Byte ((g*16 + rr)*4 + j)*2 + s/4 holds the low
 *         two code bits of four columns; column c of the four is at bit
 *         4*(c&1) + 2*(c>>1) (so bits 1:0 = c0, 3:2 = c2, 5:4 = c1, 7:6 = c3).
 *   hi    (Q3 only) 256 bytes per unit: little-endian 32-bit word g*16 + rr,
 *         bit 4*n + t holds code bit 2, with n = 4*(j%2) + 2*(s/4) + s%2 and
 *         t = 2*(j/2) + (s/2)%2 (the bit of the code whose low bits are in
 *         nibble n of the word's 32-bit lo dword j/2 at bits 1:0 of the
 *         nibble when t is even, at bits 3:2 when t is odd).
 *   scale 64 fp16 per unit, element rr*4 + j.
 *   min   (Q2 only) 64 fp16 per unit, element rr*4 + j.
 * n matrices of one kind are stacked expert-major (expert e starts at unit
 * e*(rows/16)*(K/128)).  Each plane is a separate array.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

/* The workspace's error word: an int32 at this byte offset of every
 * workspace.  Kernels that find their device-side input breaking a stated
 * precondition set bits here instead of touching memory out of bounds; the
 * bits stay set until moe_workspace_init clears the workspace.  A caller that
 * wants to know reads the 4 bytes back (e.g. after a synchronisation). */
#define MOE_WS_ERROR_OFFSET 3968
#define MOE_WS_ERR_ID_RANGE 1  /* moe_dispatch*: an id outside [0, E)   */
#define MOE_WS_ERR_ID_REPEAT 2 /* moe_dispatch*: a token names an expert twice */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status;

typedef enum { MOE_FMT_Q2_B32 = 1, MOE_FMT_Q3_B32 = 2 } moe_format;

/* n stacked rows x K matrices in the storage order above. */
typedef struct {
    const uint8_t *lo;     /* required                                  */
    const uint8_t *hi;     /* Q3: required; Q2: must be NULL            */
    const uint16_t *scale; /* fp16 bits, required                       */
    const uint16_t *min;   /* Q2: required (fp16 bits); Q3: must be NULL */
} moe_qmat;

/* One MoE layer.  Routed: n = n_experts matrices each; shared: n = 1.
 * gate, up: rows = d_ff, K = d_model.   down: rows = d_model, K = d_ff. */
typedef struct {
    int32_t format; /* moe_format */
    int32_t d_model;
    int32_t d_ff;
    int32_t n_experts;
    moe_qmat gate, up, down;
    moe_qmat sh_gate, sh_up, sh_down;
} moe_layer;

/*
 * moe_route -- router scores, top-k selection and routing weights.
 * [forum] "Strata의 동작 원리": the router runs on the GPU for every token of
 * every layer and names the k experts the token uses ("Strata 소개": 10 of 512).
 *
 *   logits[t][e] = sum_c x[t][c] * Wr[c][e]  (+ bias[e])      fp32
 *   ids[t][0..k) = the k largest logits[t][.], in descending order; equal
 *                  values (also -0.0 vs +0.0) rank the lower expert first
 *   w[t][j]      = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0), l_j = logit of ids[t][j]
 *                  (= softmax over all E, restricted to the top k, renormalised)
 *
 * x_bf16   [T][d_model] bfloat16 bits, row-major.
 * w_router [d_model][E] fp32, E contiguous.  If NULL, `logits` is an INPUT
 *          [T][E] (x_bf16 and bias must then be NULL): only selection and
 *          weights are computed.
 * bias     [E] fp32 or NULL.
 * logits   [T][E] fp32, written (or read, see above).  Must be finite.
 * topk_ids [T][k] int32, topk_w [T][k] fp32: written.
 * ws       workspace of at least moe_workspace_size(d_model, *, E, T, k) bytes,
 *          256-byte aligned, zero-filled once by moe_workspace_init.
 */
moe_status moe_route(const uint16_t *x_bf16, const float *w_router, const float *bias,
                     float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                     int32_t *topk_ids, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_dispatch -- group the P = T*k token-expert pairs by expert.
 * [forum] "Strata의 동작 원리": once the ids are known the experts are split
 * among their executors; here every expert is resident, so the split becomes
 * an expert-sorted permutation consumed by moe_expert_ffn.
 *
 * Pair p = t*k + j names token t and its j-th expert topk_ids[t][j].
 *   offsets     [E+1] int32: offsets[e] = number of pairs with expert < e;
 *               offsets[E] = P.
 *   sorted_pair [P] int32: pairs ordered by expert, ascending p within an
 *               expert (stable).   pair_pos [P] int32: inverse permutation,
 *               sorted_pair[pair_pos[p]] == p.
 * Every id must lie in [0, E) and a token's k ids must be distinct (as
 * moe_route produces them); other input is a precondition violation.  It is
 * detected on the device: a pair whose id lies outside [0, E) is left out of
 * the listing (pair_pos = -1, offsets[E] counts the listed pairs) and sets
 * MOE_WS_ERR_ID_RANGE in the workspace's error word; a repeated id sets
 * MOE_WS_ERR_ID_REPEAT (both pairs then share one position).  Either way every
 * listed entry is a valid pair, so the later calls stay in bounds.
 * moe_validate_ids checks the same conditions on a host copy.
 */
moe_status moe_dispatch(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k,
                        int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * moe_dispatch_tail_skip -- moe_dispatch with route tail-skip (opt-in, lossy).
 * [forum] "Strata의 동작 원리 / 그래픽카드, RAM, SSD에 나눠 담은 전문가": an expert
 * that every token of the batch picked only at 7th place or lower of its
 * top 10 is not computed, and the other routing weights are left as they are
 * (there the rule covers only experts outside VRAM; every expert is resident
 * here, so it applies to all of them).
 *
 * tail_from in [0, k]: expert e is kept iff some token picks it at a rank
 * j < tail_from (0-based; the page's rule is tail_from = 6 for k = 10).  The
 * pairs of the other experts are dropped: pair_pos[p] = -1, and they appear in
 * neither sorted_pair nor offsets (offsets[E] = number of kept pairs <= P).
 * Kept pairs are listed exactly as moe_dispatch lists them.  tail_from = k
 * gives moe_dispatch's result.  moe_expert_ffn computes only the listed rows;
 * moe_combine leaves dropped pairs out.  Same preconditions, workspace and
 * errors as moe_dispatch; tail_from outside [0, k] is MOE_ERR_INVALID_ARGUMENT.
 */
moe_status moe_dispatch_tail_skip(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k,
                                  int32_t tail_from, int32_t *offsets, int32_t *sorted_pair,
                                  int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_route_dispatch -- moe_route followed by moe_dispatch, in one launch
 * where the batch allows it.  [forum] "Strata의 동작 원리": per layer the
 * router's picks go straight on to the split among executors; a decode layer
 * is a chain of small steps, so each launch saved is time saved per layer.
 *
 * Writes exactly what moe_route then moe_dispatch (same arguments) write:
 * logits, topk_ids, topk_w, offsets, sorted_pair, pair_pos.  w_router and
 * x_bf16 must be given (no logits input).  With T <= 8 and k <= 64 one kernel
 * does both; otherwise the two calls are enqueued in turn.  ws must suffice
 * for both (moe_workspace_size does).  Errors: those of the two calls,
 * checked before anything is enqueued.
 */
moe_status moe_route_dispatch(const uint16_t *x_bf16, const float *w_router, const float *bias,
                              float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                              int32_t *topk_ids, float *topk_w, int32_t *offsets, int32_t *sorted_pair,
                              int32_t *pair_pos, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_route_dispatch_tail_skip -- moe_route followed by moe_dispatch_tail_skip
 * (same tail_from), in one launch where the batch allows it (T <= 8 and
 * k <= 64), as moe_route_dispatch does for moe_dispatch.  Writes exactly what
 * the two calls write; tail_from outside [0, k] is MOE_ERR_INVALID_ARGUMENT.
 */
moe_status moe_route_dispatch_tail_skip(const uint16_t *x_bf16, const float *w_router, const float *bias,
                                        float *logits, int32_t T, int32_t d_model, int32_t E, int32_t k,
                                        int32_t tail_from, int32_t *topk_ids, float *topk_w, int32_t *offsets,
                                        int32_t *sorted_pair, int32_t *pair_pos, void *ws, size_t ws_bytes,
                                        void *stream);

/*
 * moe_expert_ffn -- the selected experts and the shared expert.
 * [forum] "Strata의 동작 원리" and [guide] "Strata, Qwen, GSQ-RCO…": 10 routed
 * experts plus one shared expert per token per layer; [video] "픽업": the
 * 2-3-bit expert weights are decompressed and computed on the GPU.
 *
 * For sorted position i (expert e with offsets[e] <= i < offsets[e+1], token
 * t = sorted_pair[i] / k), and for the shared expert on every token t:
 *   h = silu(x_t . Wg_e^T) * (x_t . Wu_e^T),  silu(z) = z / (1 + exp(-z))
 *   y = h . Wd_e^T
 * y_pairs  [T*k][d_model] fp32: row i = position i (expert-sorted order).
 * y_shared [T][d_model] fp32: the shared expert on each token.
 * offsets and sorted_pair as written by moe_dispatch (or
 * moe_dispatch_tail_skip) for the same T, k, E; rows past offsets[E] of
 * y_pairs are not written.
 * Weights are dequantised exactly in fp32 when few rows share an expert
 * (decode); larger groups use fp16 matrix-core tiles with fp32 accumulation.
 */
moe_status moe_expert_ffn(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                          const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                          float *y_shared, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_routed_ffn, moe_shared_ffn -- the two halves of moe_expert_ffn.
 * [forum] "Strata의 동작 원리": the shared expert is always resident and
 * needs no routing decision; [local] localai.co.kr guide, section "0.1.43의
 * GPU별 측정 결과를 살펴봐요": copies are overlapped with the decode work they
 * do not depend on.  moe_shared_ffn needs only x, so a caller can run it on a
 * second stream while moe_route / moe_dispatch run, then moe_routed_ffn, and
 * join the streams before moe_combine.
 *
 * moe_routed_ffn writes exactly the y_pairs of moe_expert_ffn (same
 * arguments); moe_shared_ffn exactly its y_shared [T][d_model].  Each reads
 * only its own expert matrices (the shared ones may be null for
 * moe_routed_ffn and the routed ones for moe_shared_ffn).  Workspace: as
 * moe_expert_ffn; moe_workspace_size(d_model, d_ff, E, T, k) with any k >= 1
 * suffices for moe_shared_ffn.  Two calls that run at the same time need
 * separate workspaces.  Errors as moe_expert_ffn.
 */
moe_status moe_routed_ffn(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                          const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs, void *ws,
                          size_t ws_bytes, void *stream);
moe_status moe_shared_ffn(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, float *y_shared,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_combine -- moe_expert_ffn followed by moe_combine.
 * [forum] "Strata의 동작 원리": the GPU merges every expert's result, then the
 * next layer starts; a decode layer is a chain of small steps, so each launch
 * saved is time saved per layer.
 *
 * Writes exactly what moe_expert_ffn then moe_combine (same arguments) write:
 * y_pairs, y_shared and out, bit for bit.  With T <= 4 the expert kernels do
 * the merge themselves (the last workgroup of each 16-column output tile to
 * finish sums that tile), one launch less than the two calls; otherwise the
 * two calls are enqueued in turn.  Workspace as moe_expert_ffn; its counters
 * are zero again when the call ends.  Errors: those of the two calls.
 */
moe_status moe_expert_ffn_combine(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                                  const int32_t *offsets, const int32_t *sorted_pair, const int32_t *pair_pos,
                                  const float *topk_w, float *y_pairs, float *y_shared, float *out, void *ws,
                                  size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_noalloc -- moe_expert_ffn without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call allocates
 * nothing; its scratch is a fixed 8 MiB device array inside the library
 * (each GPU the library runs on holds one copy until the process ends),
 * located on the current device, which must be the device of `stream`.
 *
 * Same arguments (minus ws, ws_bytes), results and validation as
 * moe_expert_ffn, bit-identical to it, for decode-sized batches only: T <= 16
 * and moe_workspace_size(d_model, d_ff, E, T, k) <= 8 MiB (e.g. d_model=2048,
 * d_ff=768, E=512, k=10 at every T <= 16).  Larger sizes return
 * MOE_ERR_UNSUPPORTED and enqueue nothing.  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (different streams, or
 * concurrent host threads whose work runs at once) race and must not be
 * issued; calls ordered on one stream are fine.  Nothing in the array has to
 * start at zero (each call writes what it reads).  MOE_ERR_HIP if the array's
 * device address cannot be found.
 */
moe_status moe_expert_ffn_noalloc(const moe_layer *layer, const uint16_t *x_bf16, int32_t T, int32_t k,
                                  const int32_t *offsets, const int32_t *sorted_pair, float *y_pairs,
                                  float *y_shared, void *stream);

/*
 * moe_combine -- merge the expert outputs of each token.
 * [forum] "Strata의 동작 원리": the GPU merges every expert's result, then the
 * next layer starts.
 *   out[t][:] = y_shared[t][:] + sum_{j<k} topk_w[t][j] * y_pairs[pair_pos[t*k+j]][:]
 * where a pair with pair_pos -1 (dropped by moe_dispatch_tail_skip) adds
 * nothing.  out [T][d_model] fp32, overwritten.  Needs no workspace.
 */
moe_status moe_combine(const float *y_pairs, const float *y_shared, const int32_t *pair_pos,
                       const float *topk_w, int32_t T, int32_t k, int32_t d_model, float *out,
                       void *stream);

/*
 * moe_validate_ids -- host-side check of the routing ids that moe_dispatch
 * expects: topk_ids_host is a HOST array [T][k]; every id must lie in [0, E)
 * and a token's k ids must be distinct.  Returns MOE_OK, or
 * MOE_ERR_INVALID_ARGUMENT (bad sizes, a null pointer, or an id that breaks
 * the conditions).  Touches no device and enqueues nothing.
 */
moe_status moe_validate_ids(const int32_t *topk_ids_host, int32_t T, int32_t E, int32_t k);

/* Workspace bytes that suffice for every call above with these sizes. */
size_t moe_workspace_size(int32_t d_model, int32_t d_ff, int32_t E, int32_t T, int32_t k);

/* Zero-fill a workspace (enqueued on `stream`).  Needed once after
 * allocation; every call leaves the workspace's counters zero again. */
moe_status moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

const char *moe_status_string(moe_status s);
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
