/* Drives every entry point of the two C oracles on small seeded inputs, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds
 * access, use of freed memory or undefined arithmetic aborts with a report.
 * Shapes cover ragged lengths (not multiples of the chunk or block), every chunk
 * length 1..T of the chunked form, nonzero initial states, norm weights and the
 * sparse layer's imposed and computed block choices.  Exit status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void lao_set_threads(int n);
void lao_rmsnorm_row(const double* x, int D, double eps, const float* w, double* out);
void lao_rope_row(const double* x, int D, int64_t pos, double base, double* out);
void lao_prologue(const float* x, int B, int T, int H, int D, int64_t pos0, double base, double eps,
                  const float* w, double* out);
void lao_forward(const float* q, const float* k, const float* v, const float* g, int B, int T, int H, int D,
                 int64_t pos0, double base, double eps, const float* q_w, const float* k_w, double* S, double* o);
void lao_chunked(const float* q, const float* k, const float* v, const float* g, int B, int T, int H, int D,
                 int64_t pos0, double base, double eps, const float* q_w, const float* k_w, int C, double* S,
                 double* o);
void lao_backward(const float* q, const float* k, const float* v, const float* g, const float* dout, int B, int T,
                  int H, int D, int64_t pos0, double base, double eps, const float* q_w, const float* k_w,
                  const double* S_in, const double* dS_out, double* dq, double* dk, double* dv, double* dg,
                  double* dS_in, double* dqw_part, double* dkw_part);
void lso_set_threads(int n);
void lso_sparse_forward(const float* q, const float* k, const float* v, const float* g, int B, int T, int H, int D,
                        int blk, int topk, int32_t* sel, int use_sel, double* scores, double* o);
void lso_sparse_decode(const float* q, const float* kc, const float* vc, const float* g, const int32_t* lens, int B,
                       int Tmax, int H, int D, int blk, int topk, int32_t* sel, int use_sel, double* scores,
                       double* o);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in (-1, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0;
}
static float* randf(size_t n) {
  float* p = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) p[i] = (float)uniform();
  return p;
}
static double* randd(size_t n) {
  double* p = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = 0.1 * uniform();
  return p;
}
static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}
#define CHECK(c) do { if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

static int linear_layer(int B, int T, int H, int D, int64_t pos0, int weights) {
  const size_t act = (size_t)B * T * H * D, st = (size_t)B * H * D * D;
  float *q = randf(act), *k = randf(act), *v = randf(act), *g = randf(act), *dout = randf(act);
  float *qw = weights ? randf(D) : NULL, *kw = weights ? randf(D) : NULL;
  double *S = randd(st), *S2 = malloc(st * sizeof(double)), *o = malloc(act * sizeof(double));
  double *o2 = malloc(act * sizeof(double)), *S_in = randd(st), *dS = randd(st);
  for (size_t i = 0; i < st; ++i) S2[i] = S[i];
  lao_forward(q, k, v, g, B, T, H, D, pos0, 10000.0, 1e-6, qw, kw, S, o);
  CHECK(finite_all(o, act) && finite_all(S, st));
  for (int C = 1; C <= T; ++C) {
    for (size_t i = 0; i < st; ++i) S[i] = S2[i];
    lao_chunked(q, k, v, g, B, T, H, D, pos0, 10000.0, 1e-6, qw, kw, C, S, o2);
    CHECK(finite_all(o2, act) && finite_all(S, st));
    for (size_t i = 0; i < act; ++i) CHECK(fabs(o2[i] - o[i]) <= 1e-9 * (1.0 + fabs(o[i])));
  }
  double *dq = malloc(act * sizeof(double)), *dk = malloc(act * sizeof(double));
  double *dv = malloc(act * sizeof(double)), *dg = malloc(act * sizeof(double)), *dSin = malloc(st * sizeof(double));
  double *dqw = weights ? malloc((size_t)B * H * D * sizeof(double)) : NULL;
  double *dkw = weights ? malloc((size_t)B * H * D * sizeof(double)) : NULL;
  lao_backward(q, k, v, g, dout, B, T, H, D, pos0, 10000.0, 1e-6, qw, kw, S_in, dS, dq, dk, dv, dg, dSin, dqw, dkw);
  CHECK(finite_all(dq, act) && finite_all(dk, act) && finite_all(dv, act) && finite_all(dg, act));
  CHECK(finite_all(dSin, st));
  lao_backward(q, k, v, g, dout, B, T, H, D, pos0, 10000.0, 1e-6, qw, kw, NULL, NULL, dq, dk, dv, dg, dSin, dqw, dkw);
  double *pro = malloc(act * sizeof(double));
  lao_prologue(q, B, T, H, D, pos0, 10000.0, 1e-6, qw, pro);
  CHECK(finite_all(pro, act));
  double row[16], out[16];
  for (int i = 0; i < D && i < 16; ++i) row[i] = uniform();
  if (D <= 16) {
    lao_rmsnorm_row(row, D, 1e-6, qw, out);
    lao_rope_row(row, D, pos0, 10000.0, out);
  }
  free(q); free(k); free(v); free(g); free(dout); free(qw); free(kw); free(S); free(S2); free(o); free(o2);
  free(S_in); free(dS); free(dq); free(dk); free(dv); free(dg); free(dSin); free(dqw); free(dkw); free(pro);
  return 0;
}

static int sparse_layer(int B, int T, int H, int D, int blk, int topk) {
  const size_t act = (size_t)B * T * H * D;
  const int nqb = (T + blk - 1) / blk, nkb = T / blk;
  float *q = randf(act), *k = randf(act), *v = randf(act), *g = randf(act);
  int32_t* sel = malloc((size_t)B * H * nqb * topk * sizeof(int32_t));
  double* scores = malloc((size_t)B * H * nqb * (nkb > 0 ? nkb : 1) * sizeof(double));
  double* o = malloc(act * sizeof(double));
  lso_sparse_forward(q, k, v, g, B, T, H, D, blk, topk, sel, 0, scores, o);
  CHECK(finite_all(o, act));
  lso_sparse_forward(q, k, v, g, B, T, H, D, blk, topk, sel, 1, NULL, o);  /* the choice imposed */
  CHECK(finite_all(o, act));
  /* decode: caches of T tokens, every length 1..T in turn */
  float *qd = randf((size_t)B * H * D), *gd = randf((size_t)B * H * D);
  int32_t* lens = malloc((size_t)B * sizeof(int32_t));
  int32_t* seld = malloc((size_t)B * H * topk * sizeof(int32_t));
  double* sc = malloc((size_t)B * H * (nkb > 0 ? nkb : 1) * sizeof(double));
  double* od = malloc((size_t)B * H * D * sizeof(double));
  for (int len = 1; len <= T; ++len) {
    for (int b = 0; b < B; ++b) lens[b] = 1 + (len + 7 * b) % T;
    lso_sparse_decode(qd, k, v, gd, lens, B, T, H, D, blk, topk, seld, 0, sc, od);
    CHECK(finite_all(od, (size_t)B * H * D));
  }
  free(q); free(k); free(v); free(g); free(sel); free(scores); free(o); free(qd); free(gd); free(lens);
  free(seld); free(sc); free(od);
  return 0;
}

int main(void) {
  lao_set_threads(2);
  lso_set_threads(2);
  const int cases[][6] = {{1, 1, 1, 2, 0, 0}, {1, 7, 2, 4, 5, 1}, {2, 33, 3, 8, 262144, 0}, {1, 70, 1, 16, 1000000, 1}};
  for (unsigned i = 0; i < sizeof(cases) / sizeof(cases[0]); ++i)
    if (linear_layer(cases[i][0], cases[i][1], cases[i][2], cases[i][3], cases[i][4], cases[i][5])) return 1;
  const int sp[][6] = {{1, 5, 1, 4, 2, 1}, {1, 37, 2, 8, 4, 2}, {2, 100, 2, 16, 8, 3}, {1, 64, 1, 8, 16, 4}};
  for (unsigned i = 0; i < sizeof(sp) / sizeof(sp[0]); ++i)
    if (sparse_layer(sp[i][0], sp[i][1], sp[i][2], sp[i][3], sp[i][4], sp[i][5])) return 1;
  printf("oracle driver: clean\n");
  return 0;
}
