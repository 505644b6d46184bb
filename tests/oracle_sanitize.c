/*
 * oracle_sanitize.c -- drives every entry point of oracle/moe_oracle.c on
 * small seeded inputs, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles and runs
 * it on the CPU).  Any out-of-bounds access, leak, use after free, signed
 * overflow or misaligned access in the oracle aborts the run with a report.
 *
 * Shapes cover the tiny workload (d=256, f=128, E=16, top-2 + shared, T=4),
 * the degenerate cases (E = k = 1, k = E, T = 0, a single token) and both
 * formats.  A few invariants are checked too (dispatch is a permutation, the
 * routing weights sum to 1), so a run that computes nonsense also fails.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const uint8_t *lo;
    const uint8_t *hi;
    const uint16_t *scale;
    const uint16_t *min;
} oracle_qmat;

double oracle_bf16_to_double(uint16_t b);
double oracle_fp16_to_double(uint16_t h);
int oracle_code(const oracle_qmat *m, int fmt, int rows, int K, int e, int r, int k);
double oracle_weight(const oracle_qmat *m, int fmt, int rows, int K, int e, int r, int k);
void oracle_dequant_matrix(const oracle_qmat *m, int fmt, int rows, int K, int e, double *out);
void oracle_router_logits(const uint16_t *x, const float *wr, const float *bias, int T, int d, int E,
                          float *logits);
void oracle_topk_softmax(const float *logits, int T, int E, int k, int32_t *ids, float *w);
void oracle_dispatch(const int32_t *ids, int T, int k, int E, int32_t *offsets, int32_t *sorted_pair,
                     int32_t *pair_pos);
void oracle_tail_keep(const int32_t *ids, int T, int k, int E, int tail_from, char *keep);
void oracle_dispatch_tail_skip(const int32_t *ids, int T, int k, int E, int tail_from, int32_t *offsets,
                               int32_t *sorted_pair, int32_t *pair_pos);
void oracle_expert_rows(const oracle_qmat *gate, const oracle_qmat *up, const oracle_qmat *down,
                        const oracle_qmat *sh_gate, const oracle_qmat *sh_up, const oracle_qmat *sh_down,
                        int fmt, int d, int f, int E, const uint16_t *x, int n_rows,
                        const int32_t *row_expert, const int32_t *row_token, float *y, float *h);
void oracle_combine(const float *y_pairs, const float *y_shared, const int32_t *pair_pos, const float *w,
                    int T, int k, int d, float *out);
void oracle_layer(const oracle_qmat *gate, const oracle_qmat *up, const oracle_qmat *down,
                  const oracle_qmat *sh_gate, const oracle_qmat *sh_up, const oracle_qmat *sh_down, int fmt,
                  int d, int f, int E, int k, int T, const uint16_t *x, const float *wr, const float *bias,
                  const float *logits_in, int tail_from, int32_t *ids, float *w, float *out);
int oracle_num_threads(void);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* splitmix64 */
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static double uniform(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

/* fp16 bits of a value in [0.005, 0.015] (normal range: exponent 2^-8 .. 2^-7) */
static uint16_t fp16_bits_of(double v)
{
    int e;
    double m = frexp(v, &e); /* v = m * 2^e, m in [0.5, 1) */
    int frac = (int)((m * 2.0 - 1.0) * 1024.0 + 0.5);
    int ex = e - 1 + 15;
    if (frac == 1024) {
        frac = 0;
        ++ex;
    }
    return (uint16_t)((ex << 10) | frac);
}

typedef struct {
    uint8_t *lo, *hi;
    uint16_t *scale, *min;
    oracle_qmat q;
} owned_qmat;

static void make_qmat(owned_qmat *m, int fmt, int n, int rows, int K)
{
    const size_t w = (size_t)n * rows * K;
    m->lo = malloc(w / 4);
    m->hi = fmt == 2 ? malloc(w / 8) : NULL;
    m->scale = malloc(sizeof(uint16_t) * (w / 32));
    m->min = fmt == 1 ? malloc(sizeof(uint16_t) * (w / 32)) : NULL;
    for (size_t i = 0; i < w / 4; ++i) m->lo[i] = (uint8_t)next_u64();
    if (m->hi)
        for (size_t i = 0; i < w / 8; ++i) m->hi[i] = (uint8_t)next_u64();
    for (size_t i = 0; i < w / 32; ++i) {
        const double dsc = 0.005 + 0.01 * uniform();
        m->scale[i] = fp16_bits_of(dsc);
        if (m->min) m->min[i] = (uint16_t)(fp16_bits_of(1.5 * dsc) | 0x8000u); /* about -1.5 d */
    }
    m->q.lo = m->lo;
    m->q.hi = m->hi;
    m->q.scale = m->scale;
    m->q.min = m->min;
}

static void free_qmat(owned_qmat *m)
{
    free(m->lo);
    free(m->hi);
    free(m->scale);
    free(m->min);
}

static int failures = 0;
#define CHECK(cond, ...)                       \
    do {                                       \
        if (!(cond)) {                         \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");             \
            ++failures;                        \
        }                                      \
    } while (0)

static void run_case(int fmt, int d, int f, int E, int k, int T, int with_bias, int tail_from)
{
    owned_qmat g, u, dn, sg, su, sd;
    make_qmat(&g, fmt, E, f, d);
    make_qmat(&u, fmt, E, f, d);
    make_qmat(&dn, fmt, E, d, f);
    make_qmat(&sg, fmt, 1, f, d);
    make_qmat(&su, fmt, 1, f, d);
    make_qmat(&sd, fmt, 1, d, f);
    const int P = T * k;
    uint16_t *x = malloc(sizeof(uint16_t) * ((size_t)T * d + 1));
    for (long i = 0; i < (long)T * d; ++i) {
        /* bf16 of a value in (-3, 3): keep the top 16 bits of a float */
        float v = (float)(6.0 * uniform() - 3.0);
        uint32_t b;
        memcpy(&b, &v, 4);
        x[i] = (uint16_t)(b >> 16);
    }
    float *wr = malloc(sizeof(float) * (size_t)d * E);
    for (long i = 0; i < (long)d * E; ++i) wr[i] = (float)((uniform() - 0.5) / sqrt((double)d));
    float *bias = NULL;
    if (with_bias) {
        bias = malloc(sizeof(float) * (size_t)E);
        for (int e = 0; e < E; ++e) bias[e] = (float)(-1.1 * log(1.0 + e));
    }
    float *logits = malloc(sizeof(float) * ((size_t)T * E + 1));
    int32_t *ids = malloc(sizeof(int32_t) * ((size_t)P + 1));
    float *w = malloc(sizeof(float) * ((size_t)P + 1));
    int32_t *offsets = malloc(sizeof(int32_t) * ((size_t)E + 1));
    int32_t *sp = malloc(sizeof(int32_t) * ((size_t)P + 1));
    int32_t *pp = malloc(sizeof(int32_t) * ((size_t)P + 1));
    float *out = malloc(sizeof(float) * ((size_t)T * d + 1));

    oracle_router_logits(x, wr, bias, T, d, E, logits);
    /* force ties on the first token: integer-valued logits */
    if (T > 0)
        for (int e = 0; e < E; ++e) logits[e] = (float)(e % 3);
    oracle_topk_softmax(logits, T, E, k, ids, w);
    for (int t = 0; t < T; ++t) {
        double s = 0.0;
        for (int j = 0; j < k; ++j) {
            CHECK(ids[t * k + j] >= 0 && ids[t * k + j] < E, "id out of range");
            s += w[t * k + j];
        }
        CHECK(fabs(s - 1.0) < 1e-5, "weights of token %d sum to %g", t, s);
    }
    oracle_dispatch(ids, T, k, E, offsets, sp, pp);
    CHECK(offsets[0] == 0 && offsets[E] == P, "offsets ends");
    for (int p = 0; p < P; ++p) CHECK(sp[pp[p]] == p, "pair_pos is not the inverse of sorted_pair");
    char *keep = malloc((size_t)E);
    oracle_tail_keep(ids, T, k, E, tail_from, keep);
    oracle_dispatch_tail_skip(ids, T, k, E, tail_from, offsets, sp, pp);
    for (int p = 0; p < P; ++p)
        if (pp[p] >= 0) CHECK(sp[pp[p]] == p, "tail-skip listing");
    free(keep);

    /* expert rows: every pair plus the shared rows, then the combine */
    int32_t *re = malloc(sizeof(int32_t) * ((size_t)P + T + 1));
    int32_t *rt = malloc(sizeof(int32_t) * ((size_t)P + T + 1));
    oracle_dispatch(ids, T, k, E, offsets, sp, pp);
    for (int i = 0; i < P; ++i) {
        re[i] = ids[sp[i]];
        rt[i] = sp[i] / k;
    }
    for (int t = 0; t < T; ++t) {
        re[P + t] = -1;
        rt[P + t] = t;
    }
    float *y = malloc(sizeof(float) * ((size_t)(P + T) * d + 1));
    float *h = malloc(sizeof(float) * ((size_t)(P + T) * f + 1));
    oracle_expert_rows(&g.q, &u.q, &dn.q, &sg.q, &su.q, &sd.q, fmt, d, f, E, x, P + T, re, rt, y, h);
    oracle_combine(y, y + (size_t)P * d, pp, w, T, k, d, out);
    float *out2 = malloc(sizeof(float) * ((size_t)T * d + 1));
    int32_t *ids2 = malloc(sizeof(int32_t) * ((size_t)P + 1));
    float *w2 = malloc(sizeof(float) * ((size_t)P + 1));
    oracle_layer(&g.q, &u.q, &dn.q, &sg.q, &su.q, &sd.q, fmt, d, f, E, k, T, x, NULL, NULL, logits, k, ids2, w2,
                 out2);
    for (long i = 0; i < (long)T * d; ++i) {
        const double ref = out2[i];
        CHECK(fabs(out[i] - ref) <= 1e-4 * (fabs(ref) + 1e-3), "layer != combine of rows at %ld", i);
        if (failures > 20) break;
    }
    /* the layer again from x (router inside) and with route tail-skip */
    oracle_layer(&g.q, &u.q, &dn.q, &sg.q, &su.q, &sd.q, fmt, d, f, E, k, T, x, wr, bias, NULL, tail_from, ids2,
                 w2, out2);
    /* element accessors on a few positions */
    if (E > 0) {
        double dense_first = 0.0;
        double *dense = malloc(sizeof(double) * (size_t)f * d);
        oracle_dequant_matrix(&g.q, fmt, f, d, E - 1, dense);
        dense_first = dense[0];
        CHECK(dense_first == oracle_weight(&g.q, fmt, f, d, E - 1, 0, 0), "dequant vs weight");
        CHECK(oracle_code(&g.q, fmt, f, d, E - 1, f - 1, d - 1) < (fmt == 1 ? 4 : 8), "code range");
        free(dense);
    }

    free(w2);
    free(ids2);
    free(out2);
    free(h);
    free(y);
    free(rt);
    free(re);
    free(out);
    free(pp);
    free(sp);
    free(offsets);
    free(w);
    free(ids);
    free(logits);
    free(bias);
    free(wr);
    free(x);
    free_qmat(&g);
    free_qmat(&u);
    free_qmat(&dn);
    free_qmat(&sg);
    free_qmat(&su);
    free_qmat(&sd);
}

int main(void)
{
    CHECK(oracle_bf16_to_double(0x3F80) == 1.0, "bf16 one");
    CHECK(oracle_fp16_to_double(0x3C00) == 1.0, "fp16 one");
    CHECK(oracle_fp16_to_double(0x0001) == ldexp(1.0, -24), "fp16 smallest subnormal");
    CHECK(isinf(oracle_fp16_to_double(0x7C00)), "fp16 inf");
    CHECK(oracle_num_threads() >= 1, "threads");
    /* fmt, d, f, E, k, T, bias, tail_from */
    run_case(1, 256, 128, 16, 2, 4, 0, 1);  /* the tiny workload */
    run_case(2, 256, 128, 16, 2, 4, 1, 2);
    run_case(1, 128, 128, 1, 1, 3, 0, 0);   /* one expert */
    run_case(2, 128, 256, 8, 8, 5, 1, 4);   /* k = E */
    run_case(1, 128, 128, 4, 2, 0, 0, 1);   /* no tokens */
    run_case(2, 384, 128, 64, 10, 1, 1, 6); /* one token, top-10 */
    run_case(1, 128, 128, 32, 4, 70, 0, 2); /* more than 64 tokens */
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle sanitizer run ok\n");
    return 0;
}
