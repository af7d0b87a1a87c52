/*
 * hca_oracle.c - plain fp64 CPU oracle for Heavily Compressed Attention (HCA).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU path is
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no source with the HIP library and
 * includes none of its headers; the only thing both sides share is the seeded
 * input generator, which holds none of the method's arithmetic.
 *
 * What HCA computes, from the pages:
 *   - aitest123.com, "ERNIE-5.5-Flash-Base开源：280B总参数，激活仅14B",
 *     section 模型结构: 37 of 43 layers use HCA, which keeps one cache entry
 *     for every 128 tokens.
 *   - yilup.net, section 架構設計：稀疏 MoE 與混合注意力機制, and
 *     blog.derekhsu.net (ERNIE-5.5-Flash-Base translation), section
 *     潛在閘控稀疏注意力: each query attends to those entries plus a short
 *     window of recent uncompressed tokens; HCA heads are 512 wide.
 *   - lininn.cn, "2800 亿参数的模型，每次只叫醒 140 亿", section
 *     43 层里，37 层只读摘要: the uncompressed window is the latest 128 tokens.
 *   - blog.derekhsu.net, section 低秩閘控注意力: the attention output is
 *     multiplied elementwise by a learned gate.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - an entry is the arithmetic mean of its block's rows (K and V
 *     separately), stored as bfloat16 (round to nearest, ties to even);
 *   - one shared K/V head for all query heads;
 *   - entry b is visible to the query at position t iff b*block+block-1 <= t;
 *   - the window is raw positions max(0, t-window+1) .. t;
 *   - one softmax over the union of visible entries and window rows;
 *   - scores are scale * <q, k> (scale = 1/sqrt(512) for the real layer);
 *   - the gate is sigmoid(G) with the pre-sigmoid logits G given per
 *     (token, head, channel).
 *
 * Everything is IEEE double.  bfloat16 inputs are widened exactly; nothing
 * is rounded except a compressed entry, which the pages' own design stores
 * in the cache (so it is rounded to bfloat16 here as well).
 *
 * Return codes: 0 on success, a negative number on an argument that does
 * not describe a valid problem.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_EBADARG (-1)
#define ORACLE_ERANGE  (-2)
#define ORACLE_ENOMEM  (-3)

/* bfloat16 bits -> double.  A bfloat16 is the upper half of a binary32. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* double -> bfloat16 bits, round to nearest, ties to even.
 * bfloat16 keeps 8 significant bits and the binary32 exponent range, so the
 * quantum of a normal value with 2^(e-1) <= |x| < 2^e is 2^(e-8); subnormal
 * quantum is 2^-133.  Scaling by powers of two is exact, and nearbyint rounds
 * ties to even in the default rounding mode. */
static uint16_t round_bf16(double x)
{
    if (isnan(x)) return 0x7FC0;
    if (x == 0.0 || isinf(x)) {
        float f = (float)x;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        return (uint16_t)(u >> 16);
    }
    int e;
    frexp(x, &e);
    int q = e - 8;
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(x, -q)), q);
    float f = (float)r; /* exact, or +-inf past the largest finite value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

uint16_t hca_oracle_round_bf16(double x) { return round_bf16(x); }
double hca_oracle_widen_bf16(uint16_t b) { return widen_bf16(b); }

int hca_oracle_threads(void) { return omp_get_max_threads(); }

/*
 * Block compression: entry[b][d] = bf16( (1/block) * sum_{i<block} x[b*block+i][d] ).
 * The sum runs in index order in double; every one of the floor(T/block)
 * complete blocks gets an entry; a trailing partial block gets none.
 * x is [T, ld] (ld >= D), out is [floor(T/block), D].
 */
int hca_oracle_compress(const uint16_t *x, int64_t T, int64_t ld, int D, int block,
                        uint16_t *out)
{
    if (!x || !out || T < 0 || D <= 0 || block <= 0 || ld < D) return ORACLE_EBADARG;
    int64_t nb = T / block;
    for (int64_t b = 0; b < nb; ++b) {
        for (int d = 0; d < D; ++d) {
            double s = 0.0;
            for (int i = 0; i < block; ++i)
                s += widen_bf16(x[(b * block + i) * ld + d]);
            out[b * D + d] = round_bf16(s / (double)block);
        }
    }
    return 0;
}

/* One (query, head) row: softmax over the listed keys, weighted sum of the
 * listed values, times the sigmoid gate.  keys/vals are n pointers to
 * D-element bfloat16 rows.  s is scratch of n doubles. */
static void attend_row(const uint16_t *q, const uint16_t *g, const uint16_t *const *keys,
                       const uint16_t *const *vals, int64_t n, int D, double scale,
                       double *s, double *out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += widen_bf16(q[d]) * widen_bf16(keys[j][d]);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) acc += s[j] * widen_bf16(vals[j][d]);
        double gate = 1.0 / (1.0 + exp(-widen_bf16(g[d])));
        out[d] = (acc / z) * gate;
    }
}

/*
 * Attention for an arbitrary list of query positions (prefill rows).
 *   q, g    [n, H, D]     query rows and gate logits; row i is at position tpos[i]
 *   k, v    [Tkv, D]      raw rows for positions kv_start .. kv_start+Tkv-1
 *   ck, cv  [Nc, D]       compressed entries for blocks 0 .. Nc-1
 *   out     [n, H, D]     double
 * For a query at position t the keys are the entries b < Nc with
 * b*block+block-1 <= t, then the raw positions max(0, t-window+1) .. t.
 * Returns ORACLE_ERANGE if a needed raw row lies outside [kv_start, kv_start+Tkv).
 */
int hca_oracle_attn(const uint16_t *q, const uint16_t *g, const int64_t *tpos, int64_t n,
                    const uint16_t *k, const uint16_t *v, int64_t Tkv, int64_t kv_start,
                    const uint16_t *ck, const uint16_t *cv, int64_t Nc, int H, int D,
                    int block, int window, double scale, double *out, int nthreads)
{
    if (!q || !g || !tpos || !out || n < 0 || H <= 0 || D <= 0 || block <= 0 || window <= 0 ||
        Nc < 0 || Tkv < 0)
        return ORACLE_EBADARG;
    if ((Nc > 0 && (!ck || !cv)) || (Tkv > 0 && (!k || !v))) return ORACLE_EBADARG;
    for (int64_t i = 0; i < n; ++i) {
        int64_t t = tpos[i];
        int64_t lo = t - window + 1 < 0 ? 0 : t - window + 1;
        if (t < 0 || lo < kv_start || t >= kv_start + Tkv) return ORACLE_ERANGE;
    }
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    int64_t maxkeys = Nc + window;
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        const uint16_t **keys = malloc(sizeof(*keys) * (size_t)maxkeys);
        const uint16_t **vals = malloc(sizeof(*vals) * (size_t)maxkeys);
        double *s = malloc(sizeof(*s) * (size_t)maxkeys);
        if (!keys || !vals || !s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp barrier
        if (!failed) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n * H; ++r) {
                int64_t i = r / H;
                int h = (int)(r % H);
                int64_t t = tpos[i];
                int64_t nk = 0;
                for (int64_t b = 0; b < Nc; ++b) {
                    if (b * block + block - 1 <= t) {
                        keys[nk] = ck + b * D;
                        vals[nk] = cv + b * D;
                        ++nk;
                    }
                }
                int64_t lo = t - window + 1 < 0 ? 0 : t - window + 1;
                for (int64_t p = lo; p <= t; ++p) {
                    keys[nk] = k + (p - kv_start) * D;
                    vals[nk] = v + (p - kv_start) * D;
                    ++nk;
                }
                const size_t off = ((size_t)i * H + h) * D;
                attend_row(q + off, g + off, keys, vals, nk, D, scale, s, out + off);
            }
        }
        free(keys);
        free(vals);
        free(s);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

/*
 * Decode: one new query per sequence.
 *   q, g    [B, H, D]           the new token's query rows and gate logits
 *   ck, cv  [B, nc_cap, D]      per-sequence compressed entries
 *   wk, wv  [B, window, D]      per-sequence ring of the latest raw rows;
 *                               position p lives in slot p % window
 *   pos     [B]                 position t of the new token in each sequence
 *   out     [B, H, D]           double
 * Keys of sequence b: entries 0 .. floor((t+1)/block)-1, then the raw
 * positions max(0, t-window+1) .. t read from their ring slots.
 * Returns ORACLE_ERANGE if a sequence needs more entries than nc_cap.
 */
int hca_oracle_decode(const uint16_t *q, const uint16_t *g, const uint16_t *ck,
                      const uint16_t *cv, int64_t nc_cap, const uint16_t *wk,
                      const uint16_t *wv, const int64_t *pos, int B, int H, int D, int block,
                      int window, double scale, double *out, int nthreads)
{
    if (!q || !g || !wk || !wv || !pos || !out || B < 0 || H <= 0 || D <= 0 || block <= 0 ||
        window <= 0 || nc_cap < 0)
        return ORACLE_EBADARG;
    if (nc_cap > 0 && (!ck || !cv)) return ORACLE_EBADARG;
    for (int b = 0; b < B; ++b) {
        if (pos[b] < 0 || (pos[b] + 1) / block > nc_cap) return ORACLE_ERANGE;
    }
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    int64_t maxkeys = nc_cap + window;
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        const uint16_t **keys = malloc(sizeof(*keys) * (size_t)maxkeys);
        const uint16_t **vals = malloc(sizeof(*vals) * (size_t)maxkeys);
        double *s = malloc(sizeof(*s) * (size_t)maxkeys);
        if (!keys || !vals || !s) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp barrier
        if (!failed) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < (int64_t)B * H; ++r) {
                int b = (int)(r / H);
                int h = (int)(r % H);
                int64_t t = pos[b];
                int64_t nc = (t + 1) / block;
                const uint16_t *ckb = ck ? ck + (size_t)b * nc_cap * D : NULL;
                const uint16_t *cvb = cv ? cv + (size_t)b * nc_cap * D : NULL;
                const uint16_t *wkb = wk + (size_t)b * window * D;
                const uint16_t *wvb = wv + (size_t)b * window * D;
                int64_t nk = 0;
                for (int64_t e = 0; e < nc; ++e) {
                    keys[nk] = ckb + e * D;
                    vals[nk] = cvb + e * D;
                    ++nk;
                }
                int64_t lo = t - window + 1 < 0 ? 0 : t - window + 1;
                for (int64_t p = lo; p <= t; ++p) {
                    keys[nk] = wkb + (p % window) * D;
                    vals[nk] = wvb + (p % window) * D;
                    ++nk;
                }
                const size_t off = ((size_t)b * H + h) * D;
                attend_row(q + off, g + off, keys, vals, nk, D, scale, s, out + off);
            }
        }
        free(keys);
        free(vals);
        free(s);
    }
    return failed ? ORACLE_ENOMEM : 0;
}
