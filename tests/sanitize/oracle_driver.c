/* Host driver for the sanitizer build of the fp64 oracle: runs each oracle entry
 * point on small seeded inputs (block 4, window 4, D 8, so every boundary case is
 * reached) and on the real constants, and checks a closed form (constant values
 * give value * sigmoid(gate)).  Returns non-zero on a failed check; AddressSanitizer
 * and UndefinedBehaviorSanitizer abort on any error they see. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int hca_oracle_compress(const uint16_t* x, int64_t T, int64_t ld, int D, int block, uint16_t* out);
int hca_oracle_attn(const uint16_t* q, const uint16_t* g, const int64_t* tpos, int64_t n,
                    const uint16_t* k, const uint16_t* v, int64_t Tkv, int64_t kv_start,
                    const uint16_t* ck, const uint16_t* cv, int64_t Nc, int H, int D, int block,
                    int window, double scale, double* out, int nthreads);
int hca_oracle_decode(const uint16_t* q, const uint16_t* g, const uint16_t* ck,
                      const uint16_t* cv, int64_t nc_cap, const uint16_t* wk, const uint16_t* wv,
                      const int64_t* pos, int B, int H, int D, int block, int window,
                      double scale, double* out, int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint16_t rnd_bf16(void) {  /* small multiples of 1/8, exact in bf16 */
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  int v = (int)((state >> 33) % 33) - 16;
  float f = v / 8.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static void fill(uint16_t* a, size_t n) { for (size_t i = 0; i < n; ++i) a[i] = rnd_bf16(); }

static int run(int T, int H, int D, int block, int window) {
  const size_t n = (size_t)T;
  uint16_t *q = malloc(n * H * D * 2), *g = malloc(n * H * D * 2);
  uint16_t *k = malloc(n * D * 2), *v = malloc(n * D * 2);
  const int Nc = T / block;
  uint16_t *ck = malloc((Nc + 1) * D * 2), *cv = malloc((Nc + 1) * D * 2);
  int64_t* tpos = malloc(n * sizeof(int64_t));
  double* out = malloc(n * H * D * sizeof(double));
  fill(q, n * H * D); fill(g, n * H * D); fill(k, n * D); fill(v, n * D);
  for (int64_t t = 0; t < T; ++t) tpos[t] = t;
  int rc = hca_oracle_compress(k, T, D, D, block, ck) | hca_oracle_compress(v, T, D, D, block, cv);
  rc |= hca_oracle_attn(q, g, tpos, T, k, v, T, 0, ck, cv, Nc, H, D, block, window,
                        1.0 / sqrt((double)D), out, 1);
  if (rc) { fprintf(stderr, "oracle rc %d\n", rc); return 1; }
  /* constant values: every row of v equal to v[0] -> out = v0 * sigmoid(g) */
  for (int64_t t = 1; t < T; ++t) memcpy(v + t * D, v, D * 2);
  rc = hca_oracle_compress(v, T, D, D, block, cv);
  rc |= hca_oracle_attn(q, g, tpos, T, k, v, T, 0, ck, cv, Nc, H, D, block, window,
                        1.0 / sqrt((double)D), out, 1);
  double worst = 0;
  for (int64_t t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        uint32_t uv = (uint32_t)v[d] << 16, ug = (uint32_t)g[(t * H + h) * D + d] << 16;
        float fv, fg;
        memcpy(&fv, &uv, 4); memcpy(&fg, &ug, 4);
        const double want = fv / (1.0 + exp(-(double)fg));
        const double e = fabs(out[(t * H + h) * D + d] - want);
        if (e > worst) worst = e;
      }
  if (rc || worst > 1e-12) { fprintf(stderr, "constant-V check: rc %d err %g\n", rc, worst); return 1; }
  /* decode: B sequences at positions around block ends, ring of `window` slots */
  const int B = 4;
  const int64_t pos[4] = {0, block - 1, block, 3 * block + 1};
  const int nc_cap = 4;
  uint16_t *dq = malloc((size_t)B * H * D * 2), *dg = malloc((size_t)B * H * D * 2);
  uint16_t *dck = malloc((size_t)B * nc_cap * D * 2), *dcv = malloc((size_t)B * nc_cap * D * 2);
  uint16_t *wk = malloc((size_t)B * window * D * 2), *wv = malloc((size_t)B * window * D * 2);
  double* dout = malloc((size_t)B * H * D * sizeof(double));
  fill(dq, (size_t)B * H * D); fill(dg, (size_t)B * H * D); fill(dck, (size_t)B * nc_cap * D);
  fill(dcv, (size_t)B * nc_cap * D); fill(wk, (size_t)B * window * D); fill(wv, (size_t)B * window * D);
  rc = hca_oracle_decode(dq, dg, dck, dcv, nc_cap, wk, wv, pos, B, H, D, block, window,
                         1.0 / sqrt((double)D), dout, 1);
  if (rc) { fprintf(stderr, "decode rc %d\n", rc); return 1; }
  /* invalid arguments are rejected without touching memory */
  if (hca_oracle_attn(q, g, tpos, T, k, v, T, 0, ck, cv, Nc, 0, D, block, window, 0.1, out, 1) == 0)
    return 1;
  free(q); free(g); free(k); free(v); free(ck); free(cv); free(tpos); free(out);
  free(dq); free(dg); free(dck); free(dcv); free(wk); free(wv); free(dout);
  return 0;
}

int main(void) {
  if (run(37, 3, 8, 4, 4)) return 1;
  if (run(300, 2, 512, 128, 128)) return 1;
  puts("oracle sanitizer run ok");
  return 0;
}
