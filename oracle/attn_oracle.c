/*
 * attn_oracle.c -- fp64 CPU oracle for masked (causal) multi-head attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes is the plain definition, written out step by step:
 *
 *   S = Q K^T / sqrt(D)                       (all S_q x S_kv entries, fp64)
 *   S[i][j] = -inf  where the causal mask hides key j from query i
 *   P = softmax(S) row by row (subtract the row max, exp, divide by the sum)
 *   O = P V
 *
 *   - definition and causal mask M (0 where visible, -inf elsewhere):
 *     "Hand-written Masked Multi-Head Attention CUDA kernel" page, section 2
 *     (its "O = AV^T" is read as O = A.V, the product the other pages use);
 *   - key j visible to query i iff j <= i: same page, section 2.2;
 *   - the unfused form softmax(QK^T/sqrt(d))V, masked positions set to -inf
 *     so that exp gives exactly 0, and the subtraction of the row max:
 *     "Week-4 CUDA notes" page, section 2.2;
 *   - tensors are [B, S, H, D] row-major: MMHA page, section 2.1.
 *
 * Readings where the pages are silent (listed again in the design notes):
 *   - the diagonal is visible (j <= i);
 *   - when S_q != S_kv the queries are the LAST S_q positions of the key
 *     sequence: query i sits at absolute position i + (S_kv - S_q), so key j
 *     is visible iff j <= i + S_kv - S_q.  Causal with S_q > S_kv is rejected;
 *   - no clamp of the running max (the MMHA page's section 2.3 clamp is not
 *     part of the definition);
 *   - decode: query b attends keys 0 .. len_b-1 of its cache; len_b <= 0 gives
 *     an all-zero output row and len_b > S_cap is clamped to S_cap;
 *   - KV-cache prefill: entry b of a cache holds len_b valid rows and its S_q
 *     queries are the last S_q positions (query i at len_b - S_q + i); a
 *     query that sees no key at all gets a zero output row;
 *   - the log-sum-exp of a row is ln(sum_j exp(S[i][j])) over its visible
 *     keys (the log of the softmax denominator), -inf for a row with none;
 *   - key-padding mask: a byte per (b, key), 0 hides the key from every
 *     query of entry b (its score is -inf, so exp gives exactly 0: "Week-4
 *     CUDA notes" page, section 2.2); it combines with the causal rule, and
 *     a row left with no visible key is a zero row. Hidden keys still enter
 *     O = P V with weight 0, so their values must be finite.
 *
 * The score matrix of one (b, h) is materialised in full (S_q*S_kv doubles),
 * the three stages run as three separate passes over it, and OpenMP only
 * splits the rows of a pass between threads; every value is computed by the
 * same plain loop whatever the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* Element (b, s, h, d) of a [B, S, H, D] row-major tensor. */
static size_t at(long b, long s, long h, long d, long S, long H, long D) {
    return (size_t)(((b * S + s) * H + h) * D + d);
}

/*
 * One (b, h) head: q rows i < S_q of a [*, S_qdim, H, D] tensor, keys/values
 * j < S_kv of [*, S_kdim, H, D] tensors (S_kdim >= S_kv lets a KV cache of
 * capacity S_kdim be used with S_kv valid tokens). p_out, when not NULL,
 * receives the S_q x S_kv probability matrix of this head.
 */
static int oracle_head(const double* q, const double* k, const double* v, double* o,
                       double* p_out, double* lse_out, long b, long h, long H, long D,
                       long S_q, long S_qdim, long S_kv, long S_kdim, int causal,
                       const uint8_t* kmask /* this entry's S_kv key bytes, or NULL */,
                       double* S /* scratch, S_q*S_kv */) {
    const double scale = 1.0 / sqrt((double)D);
    const long off = S_kv - S_q; /* absolute position of query i is i + off */
    long i;

    /* Pass 1: scores S = Q K^T * scale, masked entries (causal rule or key
     * mask) set to -inf. */
#pragma omp parallel for schedule(static)
    for (i = 0; i < S_q; ++i) {
        double* row = S + (size_t)i * (size_t)S_kv;
        for (long j = 0; j < S_kv; ++j) {
            if ((causal && j > i + off) || (kmask && kmask[j] == 0)) {
                row[j] = -INFINITY;
                continue;
            }
            double dot = 0.0;
            for (long d = 0; d < D; ++d)
                dot += q[at(b, i, h, d, S_qdim, H, D)] * k[at(b, j, h, d, S_kdim, H, D)];
            row[j] = dot * scale;
        }
    }

    /* Pass 2: softmax of each row: subtract the row max, exponentiate
     * (exp(-inf) is exactly 0), divide by the row sum. The log-sum-exp of
     * the row is m + ln(l). A row with no visible key is all zeros. */
#pragma omp parallel for schedule(static)
    for (i = 0; i < S_q; ++i) {
        double* row = S + (size_t)i * (size_t)S_kv;
        double m = -INFINITY;
        for (long j = 0; j < S_kv; ++j)
            if (row[j] > m) m = row[j];
        if (m == -INFINITY) {
            for (long j = 0; j < S_kv; ++j) row[j] = 0.0;
            if (lse_out) lse_out[(size_t)(b * H + h) * (size_t)S_q + (size_t)i] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (long j = 0; j < S_kv; ++j) {
            row[j] = exp(row[j] - m);
            l += row[j];
        }
        for (long j = 0; j < S_kv; ++j) row[j] = row[j] / l;
        if (lse_out) lse_out[(size_t)(b * H + h) * (size_t)S_q + (size_t)i] = m + log(l);
    }

    /* Pass 3: O = P V. Each output element is the sum over j = 0, 1, ...
     * S_kv-1 in that order; the j loop is outside the d loop only so that
     * value rows are read contiguously. */
#pragma omp parallel for schedule(static)
    for (i = 0; i < S_q; ++i) {
        const double* row = S + (size_t)i * (size_t)S_kv;
        double* out = o + at(b, i, h, 0, S_qdim, H, D);
        for (long d = 0; d < D; ++d) out[d] = 0.0;
        for (long j = 0; j < S_kv; ++j) {
            const double pj = row[j];
            const double* vrow = v + at(b, j, h, 0, S_kdim, H, D);
            for (long d = 0; d < D; ++d) out[d] += pj * vrow[d];
        }
    }

    if (p_out) {
        double* dst = p_out + (size_t)(b * H + h) * (size_t)S_q * (size_t)S_kv;
        memcpy(dst, S, sizeof(double) * (size_t)S_q * (size_t)S_kv);
    }
    return ORACLE_OK;
}

/*
 * Prefill / general forward.
 *   q, o : [B, S_q, H, D];  k, v : [B, S_kv, H, D];  fp64, row-major.
 *   p    : optional [B, H, S_q, S_kv] probabilities (NULL to skip).
 * Returns ORACLE_EINVAL for a non-positive size, causal with S_q > S_kv, or a
 * causal flag other than 0/1; ORACLE_ENOMEM if the score matrix cannot be
 * allocated.
 */
int oracle_attn_fwd_f64(const double* q, const double* k, const double* v, double* o,
                        double* p, int B, int H, int S_q, int S_kv, int D, int causal) {
    if (B <= 0 || H <= 0 || S_q <= 0 || S_kv <= 0 || D <= 0) return ORACLE_EINVAL;
    if (causal != 0 && causal != 1) return ORACLE_EINVAL;
    if (causal && S_q > S_kv) return ORACLE_EINVAL;
    double* S = (double*)malloc(sizeof(double) * (size_t)S_q * (size_t)S_kv);
    if (!S) return ORACLE_ENOMEM;
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < H; ++h)
            oracle_head(q, k, v, o, p, NULL, b, h, H, D, S_q, S_q, S_kv, S_kv, causal, NULL, S);
    free(S);
    return ORACLE_OK;
}

/*
 * Single-query decode against a KV cache.
 *   q, o            : [B, 1, H, D]
 *   kcache, vcache  : [B, S_cap, H, D]
 *   seqlens         : int32[B]; query b sees cache slots 0 .. len_b-1.
 * len_b <= 0 writes a zero row; len_b > S_cap is treated as S_cap. Slots at
 * or beyond len_b are never read. This is the forward above with S_q = 1 and
 * S_kv = len_b (causal or not makes no difference for one query that is the
 * last position).
 */
int oracle_attn_decode_f64(const double* q, const double* kcache, const double* vcache,
                           const int32_t* seqlens, double* o, int B, int H, int S_cap, int D) {
    if (B <= 0 || H <= 0 || S_cap <= 0 || D <= 0) return ORACLE_EINVAL;
    double* S = (double*)malloc(sizeof(double) * (size_t)S_cap);
    if (!S) return ORACLE_ENOMEM;
    for (long b = 0; b < B; ++b) {
        long n = seqlens[b];
        if (n > S_cap) n = S_cap;
        for (long h = 0; h < H; ++h) {
            if (n <= 0) {
                for (long d = 0; d < D; ++d) o[at(b, 0, h, d, 1, H, D)] = 0.0;
                continue;
            }
            oracle_head(q, kcache, vcache, o, NULL, NULL, b, h, H, D, 1, 1, n, S_cap, 1, NULL, S);
        }
    }
    free(S);
    return ORACLE_OK;
}

/*
 * Chunk of queries against a KV cache (chunked prefill), with the
 * log-sum-exp of every query row.
 *   q, o            : [B, S_q, H, D]
 *   kcache, vcache  : [B, S_cap, H, D]
 *   seqlens         : int32[B] or NULL; entry b holds len_b valid rows,
 *                     len_b clamped to [0, S_cap] (NULL: S_cap). Query i of
 *                     entry b sits at position len_b - S_q + i.
 *   lse             : optional [B, H, S_q] (NULL to skip)
 * Each (b, h) is the forward above over the len_b valid rows (S_kv = len_b);
 * the query positions may be negative, and such rows see no key: zero output,
 * log-sum-exp -inf. len_b == 0 makes every row of the entry such a row.
 */
int oracle_attn_fwd_kvcache_f64(const double* q, const double* kcache, const double* vcache,
                                const int32_t* seqlens, double* o, double* lse, int B, int H, int S_q,
                                int S_cap, int D, int causal) {
    if (B <= 0 || H <= 0 || S_q <= 0 || S_cap <= 0 || D <= 0) return ORACLE_EINVAL;
    if (causal != 0 && causal != 1) return ORACLE_EINVAL;
    double* S = (double*)malloc(sizeof(double) * (size_t)S_q * (size_t)S_cap);
    if (!S) return ORACLE_ENOMEM;
    for (long b = 0; b < B; ++b) {
        long n = seqlens ? seqlens[b] : S_cap;
        if (n > S_cap) n = S_cap;
        if (n < 0) n = 0;
        for (long h = 0; h < H; ++h) {
            if (n == 0) {
                for (long i = 0; i < S_q; ++i) {
                    for (long d = 0; d < D; ++d) o[at(b, i, h, d, S_q, H, D)] = 0.0;
                    if (lse) lse[(size_t)(b * H + h) * (size_t)S_q + (size_t)i] = -INFINITY;
                }
                continue;
            }
            oracle_head(q, kcache, vcache, o, NULL, lse, b, h, H, D, S_q, S_q, n, S_cap, causal, NULL, S);
        }
    }
    free(S);
    return ORACLE_OK;
}

/*
 * Forward with a key-padding mask, plus the log-sum-exp of every row.
 *   q, o     : [B, S_q, H, D];  k, v : [B, S_kv, H, D]
 *   key_mask : uint8 [B, S_kv]; 0 hides key j of entry b from all its
 *              queries (NULL: every key visible, the forward above)
 *   lse      : optional [B, H, S_q] (NULL to skip)
 * The causal rule (bottom-right aligned) applies as well when causal is 1.
 * A row with no visible key gets a zero output row and log-sum-exp -inf.
 */
int oracle_attn_fwd_mask_f64(const double* q, const double* k, const double* v, const uint8_t* key_mask,
                             double* o, double* lse, int B, int H, int S_q, int S_kv, int D, int causal) {
    if (B <= 0 || H <= 0 || S_q <= 0 || S_kv <= 0 || D <= 0) return ORACLE_EINVAL;
    if (causal != 0 && causal != 1) return ORACLE_EINVAL;
    if (causal && S_q > S_kv) return ORACLE_EINVAL;
    double* S = (double*)malloc(sizeof(double) * (size_t)S_q * (size_t)S_kv);
    if (!S) return ORACLE_ENOMEM;
    for (long b = 0; b < B; ++b)
        for (long h = 0; h < H; ++h)
            oracle_head(q, k, v, o, NULL, lse, b, h, H, D, S_q, S_q, S_kv, S_kv, causal,
                        key_mask ? key_mask + (size_t)b * (size_t)S_kv : NULL, S);
    free(S);
    return ORACLE_OK;
}

/*
 * Q, K and V projections of the input rows, as one GEMM with the three
 * weight matrices stacked ("Hand-written Masked Multi-Head Attention CUDA
 * kernel" page, section 2: Q = X W_Q, K = X W_K, V = X W_V; "Week-4 CUDA
 * notes" page, section 2.1: the three projections are one concatenated
 * GEMM in practice).
 *   x        : [M, E]      input rows (M = B*S tokens, E = model width)
 *   w        : [3*N, E]    stacked weights, output-major: row n of block
 *                          0 / 1 / 2 holds the E weights of output column n
 *                          of Q / K / V (N = H*D)
 *   q, k, v  : [M, N]      = [B, S, H, D] row-major
 * Each output is the plain dot product sum_e x[m][e] * w[c*N + n][e] in
 * fp64, e ascending.
 */
int oracle_qkv_proj_f64(const double* x, const double* w, double* q, double* k, double* v, int M, int E, int N) {
    if (M <= 0 || E <= 0 || N <= 0) return ORACLE_EINVAL;
    double* out[3] = {q, k, v};
    long m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        const double* xrow = x + (size_t)m * (size_t)E;
        for (int c = 0; c < 3; ++c)
            for (long n = 0; n < N; ++n) {
                const double* wrow = w + ((size_t)c * (size_t)N + (size_t)n) * (size_t)E;
                double acc = 0.0;
                for (long e = 0; e < E; ++e) acc += xrow[e] * wrow[e];
                out[c][(size_t)m * (size_t)N + (size_t)n] = acc;
            }
    }
    return ORACLE_OK;
}

/*
 * Sinusoidal position encoding ("Week-4 CUDA notes" page, section 2.3):
 *   pe[s][2i]   = sin(pos / 10000^(2i/d_model))
 *   pe[s][2i+1] = cos(pos / 10000^(2i/d_model)),   pos = pos0 + s
 * for s < S and i < d_model/2, fp64, the formula as written (the power taken
 * directly). d_model must be even.
 */
int oracle_sinusoidal_pe_f64(double* pe, int S, int d_model, int pos0) {
    if (S <= 0 || d_model <= 0 || (d_model & 1) || pos0 < 0) return ORACLE_EINVAL;
    long s;
#pragma omp parallel for schedule(static)
    for (s = 0; s < S; ++s) {
        const double pos = (double)pos0 + (double)s;
        for (long i = 0; i < d_model / 2; ++i) {
            const double angle = pos / pow(10000.0, (double)(2 * i) / (double)d_model);
            pe[(size_t)s * (size_t)d_model + (size_t)(2 * i)] = sin(angle);
            pe[(size_t)s * (size_t)d_model + (size_t)(2 * i + 1)] = cos(angle);
        }
    }
    return ORACLE_OK;
}

/*
 * Row softmax of a score matrix under the causal rule, the stage the MMHA
 * page's section 1 describes on its own (a generic softmax would process
 * the masked upper triangle too), with the masked positions set to -inf
 * before it ("Week-4 CUDA notes" page, section 2.2):
 *   s, p : [B, H, S_q, S_kv] row-major; row i of a (b, h) sees keys
 *          j <= i + S_kv - S_q when causal, all keys otherwise
 *   p[i][j] = exp(scale*s[i][j] - m_i) / sum_j' exp(scale*s[i][j'] - m_i)
 *   over the visible j (m_i their maximum), 0 where masked; a row with no
 *   visible key is all zeros. Masked scores are never read.
 */
int oracle_masked_softmax_f64(const double* s, double* p, int B, int H, int S_q, int S_kv, double scale, int causal) {
    if (B <= 0 || H <= 0 || S_q <= 0 || S_kv <= 0) return ORACLE_EINVAL;
    if (causal != 0 && causal != 1) return ORACLE_EINVAL;
    const long rows = (long)B * H * S_q;
    const long off = (long)S_kv - S_q;
    long r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        const long i = r % S_q;
        const double* srow = s + (size_t)r * (size_t)S_kv;
        double* prow = p + (size_t)r * (size_t)S_kv;
        long n = causal ? i + off + 1 : S_kv;   /* visible keys 0 .. n-1 */
        if (n > S_kv) n = S_kv;
        if (n < 0) n = 0;
        for (long j = 0; j < S_kv; ++j) prow[j] = 0.0;
        if (n == 0) continue;
        double m = -INFINITY;
        for (long j = 0; j < n; ++j)
            if (scale * srow[j] > m) m = scale * srow[j];
        double l = 0.0;
        for (long j = 0; j < n; ++j) {
            prow[j] = exp(scale * srow[j] - m);
            l += prow[j];
        }
        for (long j = 0; j < n; ++j) prow[j] = prow[j] / l;
    }
    return ORACLE_OK;
}

/* Threads the OpenMP runtime will use for the passes above (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
