/*
 * fp64 CPU oracle of the sparse attention layers of SALA (InfLLM-v2 with NoPE and an
 * output gate).  TEST INFRASTRUCTURE ONLY: called by tests/, smoke() and the bench's
 * CPU-baseline leg, never by the HIP library, with which it shares no code.
 *
 * What the pages fix ("創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型，端側跑通百萬上下文",
 * 04 技術報告 > 02 模型架構 > (2) 稀疏注意力模塊 and (4) 混合位置編碼; "9B端側開源模型跑通百萬上下文，
 * 面壁全新稀疏-線性混合注意力", architecture section):
 *   - a block-selection mechanism lets each query attend to only a few key/value blocks;
 *   - the layer falls back to dense attention at ordinary lengths;
 *   - no position encoding in these layers (NoPE);
 *   - an output gate, as in the linear layers.
 * Everything else is a reading (the pages give one line to the layer):
 *   - softmax attention with scale 1/sqrt(D), causal;
 *   - tokens form blocks of `blk`; a key block is scored by its mean key, a block of
 *     queries by its mean query (a decode step is a query block of one token);
 *   - the candidates of query block i are the key blocks j < i (complete, strictly
 *     earlier); the `topk` best by score (ties: lower block index) are attended, plus
 *     the query's own block up to the query itself;
 *   - with no more than `topk` candidates every earlier block is attended, which is
 *     dense causal attention: the dense fallback;
 *   - o = sigmoid(g) * attention output.
 * All arithmetic is in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <omp.h>

static int g_threads = 0;
void lso_set_threads(int n) { g_threads = n; }

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Mean over tokens [t0, t1) of row-major [T][H][D] data of one (b, h). */
static void mean_rows(const float* x, int64_t row0, int64_t rs, int t0, int t1, int D, double* out) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int t = t0; t < t1; ++t)
    for (int d = 0; d < D; ++d) out[d] += (double)x[row0 + (int64_t)t * rs + d];
  for (int d = 0; d < D; ++d) out[d] /= (double)(t1 - t0);
}

/* The selected blocks: the n = min(topk, ncand) candidates with the highest score,
 * ties to the lower index, written in increasing block order, the rest of sel = -1. */
static void select_top(const double* score, int ncand, int topk, int32_t* sel) {
  char* taken = (char*)calloc((size_t)(ncand > 0 ? ncand : 1), 1);
  int n = ncand < topk ? ncand : topk;
  for (int r = 0; r < n; ++r) {
    int best = -1;
    for (int j = 0; j < ncand; ++j)
      if (!taken[j] && (best < 0 || score[j] > score[best])) best = j;
    taken[best] = 1;
  }
  int m = 0;
  for (int j = 0; j < ncand; ++j)
    if (taken[j]) sel[m++] = j;
  for (; m < topk; ++m) sel[m] = -1;
  free(taken);
}

/* Attention of one query row q (D) over the tokens listed in keys[0..nk) of one
 * (b, h) of k, v; gate g; result in o (D). */
static void attend(const float* q, const float* k, const float* v, const float* g, int64_t row0, int64_t rs,
                   const int* keys, int nk, int D, double* logit, double* o) {
  const double scale = 1.0 / sqrt((double)D);
  double mx = -INFINITY;
  for (int i = 0; i < nk; ++i) {
    const float* kr = k + row0 + (int64_t)keys[i] * rs;
    double a = 0.0;
    for (int d = 0; d < D; ++d) a += (double)q[d] * (double)kr[d];
    logit[i] = a * scale;
    if (logit[i] > mx) mx = logit[i];
  }
  double den = 0.0;
  for (int d = 0; d < D; ++d) o[d] = 0.0;
  for (int i = 0; i < nk; ++i) {
    const double p = exp(logit[i] - mx);
    den += p;
    const float* vr = v + row0 + (int64_t)keys[i] * rs;
    for (int d = 0; d < D; ++d) o[d] += p * (double)vr[d];
  }
  for (int d = 0; d < D; ++d) o[d] = sigmoid((double)g[d]) * o[d] / den;
}

/* Sparse layer over whole sequences from position 0.
 * q, k, v, g: [B][T][H][D]; o: [B][T][H][D].
 * sel: [B][H][nqb][topk] with nqb = ceil(T / blk): written (use_sel = 0) or read
 * (use_sel = 1: the given blocks are attended instead of the computed choice);
 * may be NULL when use_sel = 0.  scores: [B][H][nqb][nkb] (nkb = T / blk; entry j of
 * query block i is its score against key block j for j < i, else 0) or NULL. */
void lso_sparse_forward(const float* q, const float* k, const float* v, const float* g, int B, int T, int H,
                        int D, int blk, int topk, int32_t* sel, int use_sel, double* scores, double* o) {
  const int nqb = (T + blk - 1) / blk, nkb = T / blk;
  const int64_t rs = (int64_t)H * D;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(g_threads > 0 ? g_threads : omp_get_max_threads())
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t row0 = (int64_t)b * T * rs + (int64_t)h * D;
      double* kmean = (double*)malloc(sizeof(double) * (size_t)(nkb > 0 ? nkb : 1) * D);
      double* qmean = (double*)malloc(sizeof(double) * D);
      double* sc = (double*)malloc(sizeof(double) * (size_t)(nkb > 0 ? nkb : 1));
      int32_t* s = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
      int* keys = (int*)malloc(sizeof(int) * (size_t)(topk + 1) * blk);
      double* logit = (double*)malloc(sizeof(double) * (size_t)(topk + 1) * blk);
      for (int j = 0; j < nkb; ++j) mean_rows(k, row0, rs, j * blk, j * blk + blk, D, kmean + (size_t)j * D);
      for (int i = 0; i < nqb; ++i) {
        const int r0 = i * blk, r1 = r0 + blk < T ? r0 + blk : T;
        const int ncand = i < nkb ? i : nkb;
        mean_rows(q, row0, rs, r0, r1, D, qmean);
        for (int j = 0; j < ncand; ++j) {
          double a = 0.0;
          for (int d = 0; d < D; ++d) a += qmean[d] * kmean[(size_t)j * D + d];
          sc[j] = a;
        }
        int32_t* si = sel ? sel + (((size_t)b * H + h) * nqb + i) * topk : NULL;
        if (use_sel)
          memcpy(s, si, sizeof(int32_t) * (size_t)topk);
        else
          select_top(sc, ncand, topk, s);
        if (si && !use_sel) memcpy(si, s, sizeof(int32_t) * (size_t)topk);
        if (scores) {
          double* so = scores + (((size_t)b * H + h) * nqb + i) * (size_t)nkb;
          for (int j = 0; j < nkb; ++j) so[j] = j < ncand ? sc[j] : 0.0;
        }
        int nk = 0;
        for (int m = 0; m < topk; ++m)
          if (s[m] >= 0)
            for (int u = 0; u < blk; ++u) keys[nk++] = s[m] * blk + u;
        for (int t = r0; t < r1; ++t) {
          int n = nk;
          for (int u = r0; u <= t; ++u) keys[n++] = u;
          const int64_t row = row0 + (int64_t)t * rs;
          double ot[1024];
          attend(q + row, k, v, g + row, row0, rs, keys, n, D, logit, ot);
          for (int d = 0; d < D; ++d) o[row + d] = ot[d];
        }
      }
      free(kmean);
      free(qmean);
      free(sc);
      free(s);
      free(keys);
      free(logit);
    }
}

/* One decode step per sequence.  q, g: [B][H][D], the query of the cache's last
 * token; k_cache, v_cache: [B][Tmax][H][D]; lens[b] >= 1 tokens are valid (the
 * query's own token included), the query at position lens[b] - 1.  Key blocks and
 * their means come from the cache.  sel: [B][H][topk] (written or, with use_sel,
 * read), scores: [B][H][Tmax / blk] or NULL; o: [B][H][D]. */
void lso_sparse_decode(const float* q, const float* kc, const float* vc, const float* g, const int32_t* lens,
                       int B, int Tmax, int H, int D, int blk, int topk, int32_t* sel, int use_sel,
                       double* scores, double* o) {
  const int64_t rs = (int64_t)H * D;
  const int nkb_max = Tmax / blk;
#pragma omp parallel for collapse(2) schedule(dynamic) num_threads(g_threads > 0 ? g_threads : omp_get_max_threads())
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t row0 = (int64_t)b * Tmax * rs + (int64_t)h * D;
      const int t = lens[b] - 1;
      const int own = t / blk;  /* the query's block; the candidates are the blocks before it */
      const int ncand = own;
      double* kmean = (double*)malloc(sizeof(double) * D);
      double* sc = (double*)malloc(sizeof(double) * (size_t)(ncand > 0 ? ncand : 1));
      int32_t* s = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
      int* keys = (int*)malloc(sizeof(int) * (size_t)(topk + 1) * blk);
      double* logit = (double*)malloc(sizeof(double) * (size_t)(topk + 1) * blk);
      const float* qb = q + ((int64_t)b * H + h) * D;
      for (int j = 0; j < ncand; ++j) {
        mean_rows(kc, row0, rs, j * blk, j * blk + blk, D, kmean);
        double a = 0.0;
        for (int d = 0; d < D; ++d) a += (double)qb[d] * kmean[d];
        sc[j] = a;
      }
      int32_t* si = sel ? sel + ((size_t)b * H + h) * topk : NULL;
      if (use_sel)
        memcpy(s, si, sizeof(int32_t) * (size_t)topk);
      else
        select_top(sc, ncand, topk, s);
      if (si && !use_sel) memcpy(si, s, sizeof(int32_t) * (size_t)topk);
      if (scores) {
        double* so = scores + ((size_t)b * H + h) * (size_t)nkb_max;
        for (int j = 0; j < nkb_max; ++j) so[j] = j < ncand ? sc[j] : 0.0;
      }
      int nk = 0;
      for (int m = 0; m < topk; ++m)
        if (s[m] >= 0)
          for (int u = 0; u < blk; ++u) keys[nk++] = s[m] * blk + u;
      for (int u = own * blk; u <= t; ++u) keys[nk++] = u;
      double ot[1024];
      attend(qb, kc, vc, g + ((int64_t)b * H + h) * D, row0, rs, keys, nk, D, logit, ot);
      for (int d = 0; d < D; ++d) o[((int64_t)b * H + h) * D + d] = ot[d];
      free(kmean);
      free(sc);
      free(s);
      free(keys);
      free(logit);
    }
}
