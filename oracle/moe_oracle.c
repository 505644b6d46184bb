/*
 * moe_oracle.c -- plain CPU reference of the routed, block-quantized MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  The GPU library shares no
 * code, header, table or helper with it.
 *
 * Sources (the pages this follows):
 *   [forum]  discuss.pytorch.kr, "Strata: 12GB 그래픽카드 PC에서 125B 모델
 *            Qwen3.8-Flash-Next만을 위해 만든 추론 엔진"; section "Strata의 동작
 *            원리 / 그래픽카드, RAM, SSD에 나눠 담은 전문가" (per-layer flow: the
 *            router picks 10 expert ids, the experts are computed, the GPU merges
 *            the results) and section "Strata 소개" (10 of 512 experts per layer).
 *   [guide]  tech.okbari.net, "Strata와 Qwen3.8-Flash-Next: RTX 4090 Windows 실행
 *            가이드"; section "Strata, Qwen, GSQ-RCO는 서로 다른 구성 요소다"
 *            (48 layers, 10 of 512 routed experts plus 1 shared expert per MoE
 *            layer).
 * The pages give no formulas.  Where they are silent this file takes the plain
 * textbook reading of a top-k softmax-routed SwiGLU MoE layer:
 *   - softmax over all E logits, keep the k largest, renormalise over those k;
 *   - ties between equal logits go to the lower expert index (-0.0 == +0.0);
 *   - the shared expert is added with weight 1 (the pages name no gate for it);
 *   - SwiGLU: h = silu(x.Wg) * (x.Wu), y = h.Wd;
 *   - block-32 weights along K: Q2 w = d*q + m, Q3 w = d*(q - 4), with the
 *     library's tiled storage order (restated below, independently of the GPU
 *     sources).
 * Everything is evaluated in double from the packed bytes; results are stored
 * as fp32.  Functions here are written for clarity, not speed.
 *
 * Storage order of one rows x K matrix (rows % 16 == 0, K % 128 == 0):
 *   unit u = (r/16) * (K/128) + k/128 ; rr = r%16 ; j = (k%128)/32 ;
 *   g = (k%32)/8 ; s = k%8.
 *   lo   : 512 B per unit, byte (((g*16+rr)*4+j)*2 + s/4); within that byte
 *          the 2-bit code of s%4 = c sits at bit 4*(c&1) + 2*(c>>1).
 *   hi   : (Q3) 256 B per unit, 32-bit word (g*16+rr), bit 4*n + t with
 *          n = 4*(j%2) + 2*(s/4) + s%2 and t = 2*(j/2) + (s/2)%2 (the third
 *          bit of the code whose low bits sit in nibble n of the lane's lo
 *          dword j/2, or of that dword shifted right by 2 when t is odd).
 *   scale: 64 fp16 per unit, element rr*4 + j.      min: same as scale (Q2).
 *   n matrices are stacked expert-major.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_Q2 1
#define ORACLE_Q3 2

typedef struct {
    const uint8_t *lo;
    const uint8_t *hi;
    const uint16_t *scale;
    const uint16_t *min;
} oracle_qmat;

/* ------------------------------------------------------------------ numbers */

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 / 1024 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp(1.0 + f / 1024.0, e - 15);
    return sign ? -v : v;
}

/* --------------------------------------------------------------- dequantise */

/* Integer code (0..3 for Q2, 0..7 for Q3) of element (r, k) of matrix `e`. */
int oracle_code(const oracle_qmat *m, int fmt, int rows, int K, int e, int r, int k)
{
    long units_per_mat = (long)(rows / 16) * (K / 128);
    long u = (long)e * units_per_mat + (long)(r / 16) * (K / 128) + k / 128;
    int rr = r % 16, j = (k % 128) / 32, g = (k % 32) / 8, s = k % 8;
    int c = s % 4;
    uint8_t byte = m->lo[u * 512 + ((g * 16 + rr) * 4 + j) * 2 + s / 4];
    int q = (byte >> (4 * (c & 1) + 2 * (c >> 1))) & 3;
    if (fmt == ORACLE_Q3) {
        const uint8_t *wp = m->hi + u * 256 + (g * 16 + rr) * 4;
        uint32_t word = (uint32_t)wp[0] | ((uint32_t)wp[1] << 8) | ((uint32_t)wp[2] << 16) |
                        ((uint32_t)wp[3] << 24);
        int n = 4 * (j % 2) + 2 * (s / 4) + s % 2, t = 2 * (j / 2) + (s / 2) % 2;
        q |= (int)((word >> (4 * n + t)) & 1) << 2;
    }
    return q;
}

/* Exact real value of element (r, k) of matrix `e`. */
double oracle_weight(const oracle_qmat *m, int fmt, int rows, int K, int e, int r, int k)
{
    long units_per_mat = (long)(rows / 16) * (K / 128);
    long u = (long)e * units_per_mat + (long)(r / 16) * (K / 128) + k / 128;
    long si = u * 64 + (r % 16) * 4 + (k % 128) / 32;
    double d = oracle_fp16_to_double(m->scale[si]);
    int q = oracle_code(m, fmt, rows, K, e, r, k);
    if (fmt == ORACLE_Q2)
        return d * q + oracle_fp16_to_double(m->min[si]);
    return d * (q - 4);
}

/* Dense double copy of matrix `e`: out[r*K + k]. */
void oracle_dequant_matrix(const oracle_qmat *m, int fmt, int rows, int K, int e, double *out)
{
    for (int r = 0; r < rows; ++r)
        for (int k = 0; k < K; ++k)
            out[(long)r * K + k] = oracle_weight(m, fmt, rows, K, e, r, k);
}

/* ------------------------------------------------------------------ routing */

/* logits[t][e] = fp32( sum_c x[t][c] * Wr[c][e] ) (+ bias[e], added in fp32). */
void oracle_router_logits(const uint16_t *x, const float *wr, const float *bias,
                          int T, int d, int E, float *logits)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int c = 0; c < d; ++c)
                s += oracle_bf16_to_double(x[(long)t * d + c]) * (double)wr[(long)c * E + e];
            float l = (float)s;
            if (bias)
                l = l + bias[e];
            logits[(long)t * E + e] = l;
        }
}

/* Per token: p = softmax over all E logits; ids = the k experts with the
 * largest logits in descending order (equal logits: lower index first);
 * w_j = p_ids[j] / sum_j' p_ids[j'].  Selection compares the fp32 logits. */
void oracle_topk_softmax(const float *logits, int T, int E, int k, int32_t *ids, float *w)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (long)t * E;
        char *taken = calloc((size_t)E, 1);
        double *p = malloc(sizeof(double) * (size_t)E);
        /* softmax over all experts */
        double mx = -INFINITY;
        for (int e = 0; e < E; ++e)
            if (l[e] > mx)
                mx = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp((double)l[e] - mx);
            z += p[e];
        }
        for (int e = 0; e < E; ++e)
            p[e] /= z;
        /* k rounds of "largest remaining, lowest index on ties" */
        double psum = 0.0;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            ids[(long)t * k + j] = best;
            psum += p[best];
        }
        for (int j = 0; j < k; ++j)
            w[(long)t * k + j] = (float)(p[ids[(long)t * k + j]] / psum);
        free(p);
        free(taken);
    }
}

/* ----------------------------------------------------------------- dispatch */

/* Expert-major listing of the P = T*k token-expert pairs p = t*k + j.
 * Within one expert, pairs keep ascending p.  offsets has E+1 entries.
 * sorted_pair[i] = pair at sorted position i; pair_pos[p] = its position. */
void oracle_dispatch(const int32_t *ids, int T, int k, int E,
                     int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos)
{
    long P = (long)T * k;
    long n = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)n;
        for (long p = 0; p < P; ++p)
            if (ids[p] == e) {
                sorted_pair[n] = (int32_t)p;
                pair_pos[p] = (int32_t)n;
                ++n;
            }
    }
    offsets[E] = (int32_t)n;
}

/* Route tail-skip.  [forum] section "Strata의 동작 원리 / 그래픽카드, RAM, SSD에
 * 나눠 담은 전문가": an expert that every token of the batch picked only at
 * 7th place or lower of its top 10 is not computed (there, only for experts
 * outside VRAM; the other routing weights are left as they are).  Here:
 * expert e is kept iff some pair (t, j) with rank j < tail_from (0-based)
 * selects it.  The pairs of the other experts are dropped: pair_pos = -1, and
 * they appear in neither sorted_pair nor offsets.  Kept pairs are listed as
 * oracle_dispatch lists them.  tail_from = k keeps every pair. */
void oracle_tail_keep(const int32_t *ids, int T, int k, int E, int tail_from, char *keep)
{
    memset(keep, 0, (size_t)E);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k && j < tail_from; ++j) keep[ids[(long)t * k + j]] = 1;
}

void oracle_dispatch_tail_skip(const int32_t *ids, int T, int k, int E, int tail_from,
                               int32_t *offsets, int32_t *sorted_pair, int32_t *pair_pos)
{
    long P = (long)T * k;
    char *keep = malloc((size_t)E);
    oracle_tail_keep(ids, T, k, E, tail_from, keep);
    long n = 0;
    for (int e = 0; e < E; ++e) {
        offsets[e] = (int32_t)n;
        for (long p = 0; p < P; ++p)
            if (ids[p] == e) {
                if (keep[e]) {
                    sorted_pair[n] = (int32_t)p;
                    pair_pos[p] = (int32_t)n;
                    ++n;
                } else {
                    pair_pos[p] = -1;
                }
            }
    }
    offsets[E] = (int32_t)n;
    free(keep);
}

/* ------------------------------------------------------------------- expert */

/* One expert applied to one token row, with the expert's matrices given dense:
 *   gt_n = sum_c x_c Wg[n][c], u_n = sum_c x_c Wu[n][c],
 *   h_n  = gt_n / (1 + exp(-gt_n)) * u_n,
 *   y_o  = sum_n h_n Wd[o][n].
 * Wg, Wu: [f][d]; Wd: [d][f].  h (length f, may be NULL) and y (length d). */
void oracle_swiglu_row(const double *Wg, const double *Wu, const double *Wd, int d, int f,
                       const uint16_t *x_row, double *h_out, double *y_out)
{
    double *xv = malloc(sizeof(double) * (size_t)d);
    double *h = malloc(sizeof(double) * (size_t)f);
    for (int c = 0; c < d; ++c)
        xv[c] = oracle_bf16_to_double(x_row[c]);
    for (int n = 0; n < f; ++n) {
        double gt = 0.0, u = 0.0;
        for (int c = 0; c < d; ++c) {
            gt += xv[c] * Wg[(long)n * d + c];
            u += xv[c] * Wu[(long)n * d + c];
        }
        h[n] = gt / (1.0 + exp(-gt)) * u;
        if (h_out)
            h_out[n] = h[n];
    }
    for (int o = 0; o < d; ++o) {
        double y = 0.0;
        for (int n = 0; n < f; ++n)
            y += h[n] * Wd[(long)o * f + n];
        y_out[o] = y;
    }
    free(h);
    free(xv);
}

/* Rows of the expert FFN for explicit (expert, token) pairs.  Row r uses
 * expert row_expert[r] (-1 = the shared expert) on token row_token[r].
 * The rows are grouped by expert and cut into chunks of at most
 * ORACLE_ROW_CHUNK rows; each chunk dequantises its expert to dense doubles
 * and evaluates its rows with oracle_swiglu_row.  Chunks run in parallel (an
 * expert used by thousands of rows, such as the shared one, is split over
 * threads); every row is computed the same way whichever thread takes it.
 * Results (double) go to y[r][0..d) and, if h != NULL, h[r][0..f). */
#define ORACLE_ROW_CHUNK 128

void oracle_expert_rows_f64(const oracle_qmat *gate, const oracle_qmat *up,
                            const oracle_qmat *down, const oracle_qmat *sh_gate,
                            const oracle_qmat *sh_up, const oracle_qmat *sh_down, int fmt,
                            int d, int f, int E, const uint16_t *x, int n_rows,
                            const int32_t *row_expert, const int32_t *row_token, double *y,
                            double *h)
{
    /* rows listed expert by expert (index E stands for the shared expert) */
    long *count = calloc((size_t)E + 2, sizeof(long));
    for (int r = 0; r < n_rows; ++r)
        count[(row_expert[r] < 0 ? E : row_expert[r]) + 1] += 1;
    for (int e = 0; e <= E; ++e)
        count[e + 1] += count[e];
    int *by_expert = malloc(sizeof(int) * ((size_t)n_rows + 1));
    long *fill = malloc(sizeof(long) * ((size_t)E + 1));
    memcpy(fill, count, sizeof(long) * ((size_t)E + 1));
    for (int r = 0; r < n_rows; ++r)
        by_expert[fill[row_expert[r] < 0 ? E : row_expert[r]]++] = r;
    /* chunks: (expert, first listed row, number of rows) */
    long n_chunks = 0;
    for (int e = 0; e <= E; ++e)
        n_chunks += (count[e + 1] - count[e] + ORACLE_ROW_CHUNK - 1) / ORACLE_ROW_CHUNK;
    long *chunk = malloc(sizeof(long) * 3 * ((size_t)n_chunks + 1));
    long c = 0;
    for (int e = 0; e <= E; ++e)
        for (long i = count[e]; i < count[e + 1]; i += ORACLE_ROW_CHUNK) {
            chunk[3 * c] = e;
            chunk[3 * c + 1] = i;
            chunk[3 * c + 2] = count[e + 1] - i < ORACLE_ROW_CHUNK ? count[e + 1] - i : ORACLE_ROW_CHUNK;
            ++c;
        }
#pragma omp parallel
    {
        double *Wg = malloc(sizeof(double) * (size_t)f * d);
        double *Wu = malloc(sizeof(double) * (size_t)f * d);
        double *Wd = malloc(sizeof(double) * (size_t)d * f);
        long have = -1; /* expert held in Wg, Wu, Wd by this thread */
#pragma omp for schedule(dynamic, 1)
        for (long i = 0; i < n_chunks; ++i) {
            const long e = chunk[3 * i];
            if (e != have) {
                if (e == E) {
                    oracle_dequant_matrix(sh_gate, fmt, f, d, 0, Wg);
                    oracle_dequant_matrix(sh_up, fmt, f, d, 0, Wu);
                    oracle_dequant_matrix(sh_down, fmt, d, f, 0, Wd);
                } else {
                    oracle_dequant_matrix(gate, fmt, f, d, (int)e, Wg);
                    oracle_dequant_matrix(up, fmt, f, d, (int)e, Wu);
                    oracle_dequant_matrix(down, fmt, d, f, (int)e, Wd);
                }
                have = e;
            }
            for (long q = chunk[3 * i + 1]; q < chunk[3 * i + 1] + chunk[3 * i + 2]; ++q) {
                const int r = by_expert[q];
                oracle_swiglu_row(Wg, Wu, Wd, d, f, x + (long)row_token[r] * d,
                                  h ? h + (long)r * f : NULL, y + (long)r * d);
            }
        }
        free(Wd);
        free(Wu);
        free(Wg);
    }
    free(chunk);
    free(fill);
    free(by_expert);
    free(count);
}

/* fp32-stored variant of oracle_expert_rows_f64 (y and h rounded once). */
void oracle_expert_rows(const oracle_qmat *gate, const oracle_qmat *up, const oracle_qmat *down,
                        const oracle_qmat *sh_gate, const oracle_qmat *sh_up,
                        const oracle_qmat *sh_down, int fmt, int d, int f, int E,
                        const uint16_t *x, int n_rows, const int32_t *row_expert,
                        const int32_t *row_token, float *y, float *h)
{
    double *yd = malloc(sizeof(double) * (size_t)n_rows * d);
    double *hd = h ? malloc(sizeof(double) * (size_t)n_rows * f) : NULL;
    oracle_expert_rows_f64(gate, up, down, sh_gate, sh_up, sh_down, fmt, d, f, E, x, n_rows,
                           row_expert, row_token, yd, hd);
    for (long i = 0; i < (long)n_rows * d; ++i)
        y[i] = (float)yd[i];
    if (h)
        for (long i = 0; i < (long)n_rows * f; ++i)
            h[i] = (float)hd[i];
    free(hd);
    free(yd);
}

/* ------------------------------------------------------------------ combine */

/* out[t] = y_shared[t] + sum_{j<k} w[t][j] * y_pairs[pair_pos[t*k+j]], in double;
 * a dropped pair (pair_pos < 0, route tail-skip) adds nothing. */
void oracle_combine(const float *y_pairs, const float *y_shared, const int32_t *pair_pos,
                    const float *w, int T, int k, int d, float *out)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < d; ++o) {
            double acc = y_shared[(long)t * d + o];
            for (int j = 0; j < k; ++j) {
                const int32_t pos = pair_pos[(long)t * k + j];
                if (pos < 0) continue;
                acc += (double)w[(long)t * k + j] * (double)y_pairs[(long)pos * d + o];
            }
            out[(long)t * d + o] = (float)acc;
        }
}

/* ---------------------------------------------------------------- the layer */

/* The whole layer for T tokens:
 *   route (logits given, or computed from x, Wr, bias) -> top-k softmax
 *   weights -> k routed experts + the shared expert per token -> weighted sum.
 * With tail_from < k the routed experts of the batch that only appear at
 * ranks >= tail_from are skipped (route tail-skip, oracle_tail_keep); their
 * terms are left out and the other weights are not changed.
 * The expert outputs stay in double up to the final sum, so this is the
 * closed-form value of the layer (the routing weights are the fp32 values
 * stored in w).  If logits_in is NULL the logits are computed with
 * oracle_router_logits.  ids and w (T*k) are outputs. */
void oracle_layer(const oracle_qmat *gate, const oracle_qmat *up, const oracle_qmat *down,
                  const oracle_qmat *sh_gate, const oracle_qmat *sh_up, const oracle_qmat *sh_down,
                  int fmt, int d, int f, int E, int k, int T, const uint16_t *x,
                  const float *wr, const float *bias, const float *logits_in, int tail_from,
                  int32_t *ids, float *w, float *out)
{
    float *logits = NULL;
    const float *lg = logits_in;
    if (!lg) {
        logits = malloc(sizeof(float) * (size_t)T * E);
        oracle_router_logits(x, wr, bias, T, d, E, logits);
        lg = logits;
    }
    oracle_topk_softmax(lg, T, E, k, ids, w);
    char *keep = malloc((size_t)E);
    oracle_tail_keep(ids, T, k, E, tail_from, keep);
    /* row t*(k+1)+j: token t with its j-th expert; j == k is the shared expert */
    int n_rows = T * (k + 1);
    int32_t *re = malloc(sizeof(int32_t) * (size_t)n_rows);
    int32_t *rt = malloc(sizeof(int32_t) * (size_t)n_rows);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j <= k; ++j) {
            re[t * (k + 1) + j] = (j == k) ? -1 : ids[(long)t * k + j];
            rt[t * (k + 1) + j] = t;
        }
    double *yall = malloc(sizeof(double) * (size_t)n_rows * d);
    oracle_expert_rows_f64(gate, up, down, sh_gate, sh_up, sh_down, fmt, d, f, E, x, n_rows, re,
                           rt, yall, NULL);
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < d; ++o) {
            double acc = yall[((long)t * (k + 1) + k) * d + o];
            for (int j = 0; j < k; ++j)
                if (keep[ids[(long)t * k + j]])
                    acc += (double)w[(long)t * k + j] * yall[((long)t * (k + 1) + j) * d + o];
            out[(long)t * d + o] = (float)acc;
        }
    free(keep);
    free(yall);
    free(rt);
    free(re);
    free(logits);
}

int oracle_num_threads(void) { return omp_get_max_threads(); }
