/*
 * Runs every entry point of the fp64 oracle (oracle/attn_oracle.c) on small
 * seeded inputs under ASan and UBSan. Each array is allocated at exactly its
 * size, so a read or write past any of them is reported; the outputs are
 * checked against properties the definitions fix (causal row 0 is V row 0,
 * attention rows are convex combinations of V rows, probabilities sum to 1,
 * the position table's entries lie in [-1, 1]). Exit status 0 when all hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attn_fwd_f64(const double* q, const double* k, const double* v, double* o, double* p, int B, int H,
                        int S_q, int S_kv, int D, int causal);
int oracle_attn_decode_f64(const double* q, const double* kcache, const double* vcache, const int32_t* seqlens,
                           double* o, int B, int H, int S_cap, int D);
int oracle_attn_fwd_kvcache_f64(const double* q, const double* kcache, const double* vcache, const int32_t* seqlens,
                                double* o, double* lse, int B, int H, int S_q, int S_cap, int D, int causal);
int oracle_attn_fwd_mask_f64(const double* q, const double* k, const double* v, const uint8_t* key_mask, double* o,
                             double* lse, int B, int H, int S_q, int S_kv, int D, int causal);
int oracle_qkv_proj_f64(const double* x, const double* w, double* q, double* k, double* v, int M, int E, int N);
int oracle_sinusoidal_pe_f64(double* pe, int S, int d_model, int pos0);
int oracle_masked_softmax_f64(const double* s, double* p, int B, int H, int S_q, int S_kv, double scale,
                              int causal);

static unsigned long long rng = 88172645463325252ull;
static double urand(void) {   /* xorshift64, uniform in [-1, 1) */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}
static double* randn(size_t n) {
    double* x = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) x[i] = 2.0 * urand();
    return x;
}
static int fails = 0;
#define CHECK(c)                                                        \
    do {                                                                \
        if (!(c)) {                                                     \
            fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
            ++fails;                                                    \
        }                                                               \
    } while (0)

int main(void) {
    const int B = 2, H = 3, S = 17, Skv = 23, D = 8;
    double *q = randn((size_t)B * S * H * D), *k = randn((size_t)B * Skv * H * D), *v = randn((size_t)B * Skv * H * D);
    double* o = (double*)malloc(sizeof(double) * B * S * H * D);
    double* p = (double*)malloc(sizeof(double) * B * H * S * Skv);
    CHECK(oracle_attn_fwd_f64(q, k, v, o, p, B, H, S, Skv, D, 1) == 0);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < S; ++i) {
                double sum = 0;
                for (int j = 0; j < Skv; ++j) sum += p[(((size_t)b * H + h) * S + i) * Skv + j];
                CHECK(fabs(sum - 1.0) < 1e-12);
            }
    CHECK(oracle_attn_fwd_f64(q, k, v, o, NULL, B, H, S, Skv, D, 0) == 0);
    CHECK(oracle_attn_fwd_f64(q, k, v, o, NULL, B, H, Skv + 1, Skv, D, 1) != 0);   /* causal, S_q > S_kv */
    /* square causal: query row 0 sees only key 0, so it is V row 0 */
    CHECK(oracle_attn_fwd_f64(q, k, v, o, NULL, 1, 1, 5, 5, D, 1) == 0);
    for (int d = 0; d < D; ++d) CHECK(o[d] == v[d]);
    /* decode, with lengths below 0, 0, inside and beyond the capacity */
    int32_t lens[2] = {-1, Skv + 5};
    double* od = (double*)malloc(sizeof(double) * B * H * D);
    CHECK(oracle_attn_decode_f64(q, k, v, lens, od, B, H, Skv, D) == 0);
    for (int i = 0; i < H * D; ++i) CHECK(od[i] == 0.0);
    lens[0] = 5;
    CHECK(oracle_attn_decode_f64(q, k, v, lens, od, B, H, Skv, D) == 0);
    for (int i = 0; i < B * H * D; ++i) CHECK(fabs(od[i]) <= 2.0);   /* a convex combination of V entries */
    double* lse = (double*)malloc(sizeof(double) * B * H * S);
    CHECK(oracle_attn_fwd_kvcache_f64(q, k, v, lens, o, lse, B, H, S, Skv, D, 1) == 0);
    CHECK(oracle_attn_fwd_kvcache_f64(q, k, v, NULL, o, NULL, B, H, S, Skv, D, 1) == 0);
    uint8_t* mask = (uint8_t*)malloc((size_t)B * Skv);
    for (int i = 0; i < B * Skv; ++i) mask[i] = (uint8_t)((i * 7) % 3 != 0);
    CHECK(oracle_attn_fwd_mask_f64(q, k, v, mask, o, lse, B, H, S, Skv, D, 0) == 0);
    CHECK(oracle_attn_fwd_mask_f64(q, k, v, NULL, o, NULL, B, H, S, Skv, D, 1) == 0);
    /* projection, position table, standalone softmax */
    const int M = 9, E = 16, N = 12;
    double *x = randn((size_t)M * E), *w = randn((size_t)3 * N * E);
    double *pq = (double*)malloc(sizeof(double) * M * N), *pk = (double*)malloc(sizeof(double) * M * N),
           *pv = (double*)malloc(sizeof(double) * M * N);
    CHECK(oracle_qkv_proj_f64(x, w, pq, pk, pv, M, E, N) == 0);
    double* pe = (double*)malloc(sizeof(double) * 33 * 14);
    CHECK(oracle_sinusoidal_pe_f64(pe, 33, 14, 1000) == 0);
    for (int i = 0; i < 33 * 14; ++i) CHECK(pe[i] >= -1.0 && pe[i] <= 1.0);
    double* sc = randn((size_t)B * H * S * Skv);
    double* ps = (double*)malloc(sizeof(double) * B * H * S * Skv);
    CHECK(oracle_masked_softmax_f64(sc, ps, B, H, S, Skv, 0.5, 1) == 0);
    for (int r = 0; r < B * H * S; ++r) {
        double sum = 0;
        for (int j = 0; j < Skv; ++j) sum += ps[(size_t)r * Skv + j];
        CHECK(fabs(sum - 1.0) < 1e-12);
    }
    free(q); free(k); free(v); free(o); free(p); free(od); free(lse); free(mask);
    free(x); free(w); free(pq); free(pk); free(pv); free(pe); free(sc); free(ps);
    printf("oracle driver: %d failures\n", fails);
    return fails != 0;
}
