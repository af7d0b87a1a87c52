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

/*
 * Backward pass of prefill attention over a whole sequence (queries at
 * positions 0 .. T-1, raw rows 0 .. T-1, entries of blocks 0 .. Nc-1), for the
 * training step of the layer (blog.derekhsu.net, section 訓練基礎設施: the
 * pages' attention kernel runs both passes).  With, for one (t, h) row,
 *   s_j = scale <q, k_j>,  p = softmax(s),  a = sum_j p_j v_j,
 *   sig = 1 / (1 + exp(-g)),  o = a * sig,
 * and the upstream gradient dO of o, the chain rule gives
 *   dg   = dO * a * sig * (1 - sig)          da  = dO * sig
 *   dp_j = <da, v_j>                         ds_j = p_j (dp_j - sum_i p_i dp_i)
 *   dq   = scale * sum_j ds_j k_j
 *   dk_j += scale * ds_j * q                 dv_j += p_j * da
 * where key j is an entry (into dck, dcv) or a raw row (into dk, dv).  The
 * gradients of the raw rows through the entries (every row of block b gets
 * dck[b] / block, the mean's derivative) are added by the caller, so that this
 * routine only follows the attention itself.
 *   q, g, dout  [T, H, D]   bfloat16 bits
 *   k, v        [T, D]      ck, cv [Nc, D]   bfloat16 bits
 *   dq, dg      [T, H, D]   dk, dv [T, D]    dck, dcv [Nc, D]   double (overwritten)
 * Each thread accumulates its own copy of dk, dv, dck, dcv; the copies are
 * added in thread order at the end.
 */
/*
 * One (t, h) row of the backward (row data at offset off of q, g, dout, dq,
 * dg): gathers the row's keys, recomputes its weights p and ungated output a,
 * writes dq and dg of the row and, when ak, av are given, adds the row's key
 * gradients into them (accumulator row s for raw row s, T + b for entry b).
 * kid, keys, vals, p, dp (Nc + window) and a, da (D) are the caller's scratch.
 */
static void backward_row(const uint16_t *q, const uint16_t *g, const uint16_t *dout, size_t off,
                         int64_t t, int64_t T, const uint16_t *k, const uint16_t *v,
                         const uint16_t *ck, const uint16_t *cv, int64_t Nc, int D, int block,
                         int window, double scale, double *dq, double *dg, double *ak, double *av,
                         int64_t *kid, const uint16_t **keys, const uint16_t **vals, double *p,
                         double *dp, double *a, double *da)
{
    int64_t nk = 0;
    for (int64_t b = 0; b < Nc; ++b) {
        if (b * block + block - 1 <= t) {
            keys[nk] = ck + b * D;
            vals[nk] = cv + b * D;
            kid[nk] = T + b;
            ++nk;
        }
    }
    const int64_t lo = t - window + 1 < 0 ? 0 : t - window + 1;
    for (int64_t s = lo; s <= t; ++s) {
        keys[nk] = k + s * D;
        vals[nk] = v + s * D;
        kid[nk] = s;
        ++nk;
    }
    /* forward: weights and the ungated output */
    double m = -INFINITY;
    for (int64_t j = 0; j < nk; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += widen_bf16(q[off + d]) * widen_bf16(keys[j][d]);
        p[j] = scale * dot;
        if (p[j] > m) m = p[j];
    }
    double z = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        p[j] = exp(p[j] - m);
        z += p[j];
    }
    for (int64_t j = 0; j < nk; ++j) p[j] /= z;
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < nk; ++j) acc += p[j] * widen_bf16(vals[j][d]);
        a[d] = acc;
    }
    /* gate and its gradient */
    for (int d = 0; d < D; ++d) {
        const double sig = 1.0 / (1.0 + exp(-widen_bf16(g[off + d])));
        const double go = widen_bf16(dout[off + d]);
        dg[off + d] = go * a[d] * sig * (1.0 - sig);
        da[d] = go * sig;
    }
    /* softmax backward */
    double dsum = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += da[d] * widen_bf16(vals[j][d]);
        dp[j] = dot;
        dsum += p[j] * dot;
    }
    for (int d = 0; d < D; ++d) dq[off + d] = 0.0;
    for (int64_t j = 0; j < nk; ++j) {
        const double ds = p[j] * (dp[j] - dsum);
        double *akj = ak ? ak + (size_t)kid[j] * D : NULL;
        double *avj = av ? av + (size_t)kid[j] * D : NULL;
        for (int d = 0; d < D; ++d) {
            dq[off + d] += scale * ds * widen_bf16(keys[j][d]);
            if (akj) {
                akj[d] += scale * ds * widen_bf16(q[off + d]);
                avj[d] += p[j] * da[d];
            }
        }
    }
}

int hca_oracle_attn_backward(const uint16_t *q, const uint16_t *g, const uint16_t *dout,
                             int64_t T, const uint16_t *k, const uint16_t *v,
                             const uint16_t *ck, const uint16_t *cv, int64_t Nc, int H, int D,
                             int block, int window, double scale, double *dq, double *dg,
                             double *dk, double *dv, double *dck, double *dcv, int nthreads)
{
    if (!q || !g || !dout || !k || !v || !dq || !dg || !dk || !dv || T < 0 || H <= 0 ||
        D <= 0 || block <= 0 || window <= 0 || Nc < 0 || Nc > T / block)
        return ORACLE_EBADARG;
    if (Nc > 0 && (!ck || !cv || !dck || !dcv)) return ORACLE_EBADARG;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    if (nthreads > 8) nthreads = 8;
    const int64_t maxkeys = Nc + window;
    const size_t acc_n = (size_t)(T + Nc) * D;  /* rows 0..T-1 raw, T..T+Nc-1 entries */
    double *acc_k = calloc((size_t)nthreads * acc_n, sizeof(double));
    double *acc_v = calloc((size_t)nthreads * acc_n, sizeof(double));
    if (!acc_k || !acc_v) {
        free(acc_k);
        free(acc_v);
        return ORACLE_ENOMEM;
    }
    int failed = 0;

#pragma omp parallel num_threads(nthreads)
    {
        const int tid = omp_get_thread_num();
        double *ak = acc_k + (size_t)tid * acc_n, *av = acc_v + (size_t)tid * acc_n;
        int64_t *kid = malloc(sizeof(*kid) * (size_t)maxkeys);   /* accumulator row of key j */
        const uint16_t **keys = malloc(sizeof(*keys) * (size_t)maxkeys);
        const uint16_t **vals = malloc(sizeof(*vals) * (size_t)maxkeys);
        double *p = malloc(sizeof(*p) * (size_t)maxkeys);
        double *dp = malloc(sizeof(*dp) * (size_t)maxkeys);
        double *a = malloc(sizeof(*a) * (size_t)D);
        double *da = malloc(sizeof(*da) * (size_t)D);
        if (!kid || !keys || !vals || !p || !dp || !a || !da) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp barrier
        if (!failed) {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < T * H; ++r)
                backward_row(q, g, dout, (size_t)r * D, r / H, T, k, v, ck, cv, Nc, D, block,
                             window, scale, dq, dg, ak, av, kid, keys, vals, p, dp, a, da);
        }
        free(kid);
        free(keys);
        free(vals);
        free(p);
        free(dp);
        free(a);
        free(da);
    }
    if (!failed) {
        for (size_t i = 0; i < acc_n; ++i) {
            double sk = 0.0, sv = 0.0;
            for (int th = 0; th < nthreads; ++th) {
                sk += acc_k[(size_t)th * acc_n + i];
                sv += acc_v[(size_t)th * acc_n + i];
            }
            const size_t row = i / (size_t)D;
            if (row < (size_t)T) {
                dk[i] = sk;
                dv[i] = sv;
            } else {
                dck[i - (size_t)T * D] = sk;
                dcv[i - (size_t)T * D] = sv;
            }
        }
    }
    free(acc_k);
    free(acc_v);
    return failed ? ORACLE_ENOMEM : 0;
}

/*
 * dq and dg of the rows of chosen query positions only (the same per-row
 * computation as hca_oracle_attn_backward; the key gradients, which need every
 * row, are not formed): q, g, dout, dq, dg are [npos, H, D], row i of them
 * belonging to position pos[i] of the sequence whose raw rows k, v are [T, D]
 * and entries ck, cv [Nc, D].
 */
int hca_oracle_attn_backward_rows(const uint16_t *q, const uint16_t *g, const uint16_t *dout,
                                  const int64_t *pos, int64_t npos, int64_t T, const uint16_t *k,
                                  const uint16_t *v, const uint16_t *ck, const uint16_t *cv,
                                  int64_t Nc, int H, int D, int block, int window, double scale,
                                  double *dq, double *dg, int nthreads)
{
    if (!q || !g || !dout || !pos || !k || !v || !dq || !dg || npos < 0 || T < 0 || H <= 0 ||
        D <= 0 || block <= 0 || window <= 0 || Nc < 0 || Nc > T / block)
        return ORACLE_EBADARG;
    if (Nc > 0 && (!ck || !cv)) return ORACLE_EBADARG;
    for (int64_t i = 0; i < npos; ++i)
        if (pos[i] < 0 || pos[i] >= T) return ORACLE_EBADARG;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const int64_t maxkeys = Nc + window;
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        int64_t *kid = malloc(sizeof(*kid) * (size_t)maxkeys);
        const uint16_t **keys = malloc(sizeof(*keys) * (size_t)maxkeys);
        const uint16_t **vals = malloc(sizeof(*vals) * (size_t)maxkeys);
        double *p = malloc(sizeof(*p) * (size_t)maxkeys);
        double *dp = malloc(sizeof(*dp) * (size_t)maxkeys);
        double *a = malloc(sizeof(*a) * (size_t)D);
        double *da = malloc(sizeof(*da) * (size_t)D);
        if (!kid || !keys || !vals || !p || !dp || !a || !da) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp barrier
        if (!failed) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < npos * H; ++r)
                backward_row(q, g, dout, (size_t)r * D, pos[r / H], T, k, v, ck, cv, Nc, D, block,
                             window, scale, dq, dg, NULL, NULL, kid, keys, vals, p, dp, a, da);
        }
        free(kid);
        free(keys);
        free(vals);
        free(p);
        free(dp);
        free(a);
        free(da);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

/*
 * Log-sum-exp of each row's scores (the statistic the forward keeps for the
 * training pass): lse[i, h] = ln sum_j exp(scale <q[i, h], key_j>) over the keys
 * query position tpos[i] sees (entries, then window rows, as in hca_oracle_attn).
 *   q [n, H, D] bfloat16 bits;  lse [n, H] double
 * The largest score is subtracted before exponentiating and added back.
 */
int hca_oracle_attn_lse(const uint16_t *q, const int64_t *tpos, int64_t n, const uint16_t *k,
                        int64_t Tkv, int64_t kv_start, const uint16_t *ck, int64_t Nc, int H,
                        int D, int block, int window, double scale, double *lse, int nthreads)
{
    if (!q || !tpos || !lse || n < 0 || H <= 0 || D <= 0 || block <= 0 || window <= 0 ||
        Nc < 0 || Tkv < 0)
        return ORACLE_EBADARG;
    if ((Nc > 0 && !ck) || (Tkv > 0 && !k)) return ORACLE_EBADARG;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t t = tpos[i];
        const int64_t first = t - window + 1 < 0 ? 0 : t - window + 1;
        if (t < 0 || first < kv_start || t >= kv_start + Tkv) return ORACLE_ERANGE;
    }
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    const int64_t cap = Nc + window;
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        double *sc = malloc(sizeof(*sc) * (size_t)cap);
        if (!sc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp barrier
        if (!failed) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < n * H; ++r) {
                const int64_t t = tpos[r / H];
                const uint16_t *qr = q + (size_t)r * D;
                int64_t cnt = 0;
                double top = -INFINITY;
                /* entries b with b*block + block - 1 <= t, then raw positions */
                const int64_t first = t - window + 1 < 0 ? 0 : t - window + 1;
                for (int64_t j = 0; j < Nc + (t - first + 1); ++j) {
                    const uint16_t *key;
                    if (j < Nc) {
                        if (j * block + block - 1 > t) continue;
                        key = ck + j * D;
                    } else {
                        key = k + (first + (j - Nc) - kv_start) * D;
                    }
                    double acc = 0.0;
                    for (int d = 0; d < D; ++d) acc += widen_bf16(qr[d]) * widen_bf16(key[d]);
                    sc[cnt] = scale * acc;
                    if (sc[cnt] > top) top = sc[cnt];
                    ++cnt;
                }
                double sum = 0.0;
                for (int64_t j = 0; j < cnt; ++j) sum += exp(sc[j] - top);
                lse[r] = top + log(sum);
            }
        }
        free(sc);
    }
    return failed ? ORACLE_ENOMEM : 0;
}

/*
 * Backward from the forward's saved state, the way training frameworks run it:
 * the caller keeps the gated output o and the per-row log-sum-exp lse of the
 * forward, and for row (t, h)
 *   p_j  = exp(scale <q, k_j> - lse)           (the row's attention weights)
 *   D    = <dO, o>                              (= <dA, a>, since o = a sigmoid(g))
 *   dA   = dO sigmoid(g), rounded to bfloat16 when round_da is set (the operand
 *          the GPU kernels multiply)
 *   ds_j = p_j (<dA, v_j> - D)
 *   dq   = scale sum_j ds_j k_j,   dk_j += scale ds_j q,   dv_j += p_j dA
 *   dg   = dO o (1 - sigmoid(g))               (= dO a s (1 - s))
 * With the exact o and lse (and round_da off) this is the exact gradient of
 * hca_oracle_attn_backward.  Arguments as there, plus o [T, H, D] and
 * lse [T, H] (double).  Entry gradients go to dck, dcv (not pooled).
 */
static void saved_backward_row(const uint16_t *q, const uint16_t *g, const uint16_t *dout,
                               const double *o, double lse, size_t off, int64_t t, int64_t T,
                               const uint16_t *k, const uint16_t *v, const uint16_t *ck,
                               const uint16_t *cv, int64_t Nc, int D, int block, int window,
                               double scale, int round_da, double *dq, double *dg, double *gk,
                               double *gv, double *dA)
{
    double dsum_o = 0.0;
    for (int d = 0; d < D; ++d) {
        const double s_g = 1.0 / (1.0 + exp(-widen_bf16(g[off + d])));
        const double up = widen_bf16(dout[off + d]);
        dsum_o += up * o[off + d];
        dg[off + d] = up * o[off + d] * (1.0 - s_g);
        dA[d] = round_da ? widen_bf16(round_bf16(up * s_g)) : up * s_g;
        dq[off + d] = 0.0;
    }
    const int64_t w0 = t - window + 1 < 0 ? 0 : t - window + 1;
    for (int64_t j = 0; j < Nc + (t - w0 + 1); ++j) {
        const uint16_t *kr, *vr;
        int64_t acc_row;
        if (j < Nc) {
            if (j * block + block - 1 > t) continue;
            kr = ck + j * D;
            vr = cv + j * D;
            acc_row = T + j;
        } else {
            acc_row = w0 + (j - Nc);
            kr = k + acc_row * D;
            vr = v + acc_row * D;
        }
        double qk = 0.0, av = 0.0;
        for (int d = 0; d < D; ++d) {
            qk += widen_bf16(q[off + d]) * widen_bf16(kr[d]);
            av += dA[d] * widen_bf16(vr[d]);
        }
        const double pj = exp(scale * qk - lse);
        const double dsj = pj * (av - dsum_o);
        for (int d = 0; d < D; ++d) {
            dq[off + d] += scale * dsj * widen_bf16(kr[d]);
            gk[(size_t)acc_row * D + d] += scale * dsj * widen_bf16(q[off + d]);
            gv[(size_t)acc_row * D + d] += pj * dA[d];
        }
    }
}

int hca_oracle_attn_backward_saved(const uint16_t *q, const uint16_t *g, const uint16_t *dout,
                                   const double *o, const double *lse, int64_t T,
                                   const uint16_t *k, const uint16_t *v, const uint16_t *ck,
                                   const uint16_t *cv, int64_t Nc, int H, int D, int block,
                                   int window, double scale, int round_da, double *dq,
                                   double *dg, double *dk, double *dv, double *dck, double *dcv,
                                   int nthreads)
{
    if (!q || !g || !dout || !o || !lse || !k || !v || !dq || !dg || !dk || !dv || T < 0 ||
        H <= 0 || D <= 0 || block <= 0 || window <= 0 || Nc < 0 || Nc > T / block)
        return ORACLE_EBADARG;
    if (Nc > 0 && (!ck || !cv || !dck || !dcv)) return ORACLE_EBADARG;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    if (nthreads > 8) nthreads = 8;
    const size_t rows_acc = (size_t)(T + Nc) * D;  /* raw rows, then entries */
    double *all_k = calloc((size_t)nthreads * rows_acc, sizeof(double));
    double *all_v = calloc((size_t)nthreads * rows_acc, sizeof(double));
    if (!all_k || !all_v) {
        free(all_k);
        free(all_v);
        return ORACLE_ENOMEM;
    }
    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        const int me = omp_get_thread_num();
        double *dA = malloc(sizeof(*dA) * (size_t)D);
        if (!dA) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp barrier
        if (!failed) {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < T * H; ++r)
                saved_backward_row(q, g, dout, o, lse[r], (size_t)r * D, r / H, T, k, v, ck, cv,
                                   Nc, D, block, window, scale, round_da, dq, dg,
                                   all_k + (size_t)me * rows_acc, all_v + (size_t)me * rows_acc,
                                   dA);
        }
        free(dA);
    }
    if (!failed) {
        for (size_t i = 0; i < rows_acc; ++i) {
            double tk = 0.0, tv = 0.0;
            for (int th = 0; th < nthreads; ++th) {
                tk += all_k[(size_t)th * rows_acc + i];
                tv += all_v[(size_t)th * rows_acc + i];
            }
            if (i < (size_t)T * D) {
                dk[i] = tk;
                dv[i] = tv;
            } else {
                dck[i - (size_t)T * D] = tk;
                dcv[i - (size_t)T * D] = tv;
            }
        }
    }
    free(all_k);
    free(all_v);
    return failed ? ORACLE_ENOMEM : 0;
}
