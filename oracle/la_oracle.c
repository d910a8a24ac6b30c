/*
 * la_oracle.c -- plain, slow, fp64 CPU oracle for the causal linear-attention
 * (Lightning Attention) layer.  TEST INFRASTRUCTURE ONLY: it exists to check the
 * HIP library.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it; the product path never does.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes, per (batch b, head h), with every value promoted to double:
 *
 *   1. QK-normalization (RMSNorm over the head dimension) of q_t and k_t.
 *      Source: "創新Transformer！面壁基於稀疏-線性混合架構SALA訓練9B模型" (rendering of
 *      the MiniCPM-SALA technical report), 04 技術報告 > 02 模型架構 > (3) 線性注意力模塊:
 *      the linear layers use QK-normalization, GQA-to-MHA and output gating.
 *      Reading: RMSNorm, n_i = w_i * x_i / sqrt(mean_i(x_i^2) + eps).
 *   2. RoPE on the normalized q and k at absolute position p = pos0 + t.
 *      Source: same page, (4) 混合位置編碼 (HyPE keeps RoPE in the linear layers).
 *      Reading: rotate-half pairing (i, i + D/2), theta_i = base^(-2i/D).
 *   3. The state-update recurrence S_t = S_{t-1} + k_t v_t^T.
 *      Source: "MiniCPM-SALA: Hybridizing Sparse and Linear Attention for
 *      Efficient Long-Context Modeling" (paper digest), 前置知识 > 线性注意力.
 *      Readout o_t = q_t S_t with S_t already holding token t (the causal mask
 *      includes the diagonal); no decay, no feature map, no denominator.
 *   4. Output gate: o_t = sigmoid(g_t) (elementwise) * (q_t S_t).
 *      Source: the technical-report page, (3) 線性注意力模塊 (output gating).
 *      Reading: g is a per-element logit tensor of o's shape.
 *
 * Layouts: activations are row-major [B, T, H, D]; the state S is row-major
 * [B, H, D, D] with S[i][j] = sum_t k_t[i] * v_t[j] (row i: key dim, column j:
 * value dim).  Inputs arrive as float (exact images of bf16 or fp32 data).
 *
 * Parallelism: OpenMP over independent (b, h, value-column block) tasks.  Each
 * task runs the recurrence in token order, so the arithmetic of every output
 * element is the same as in a single-threaded run.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0; /* 0 = OpenMP default */

void lao_set_threads(int n) { g_threads = n; }

int lao_get_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/* RMSNorm of one head row: out_i = w_i * x_i / sqrt(mean(x^2) + eps). w may be NULL (= ones). */
void lao_rmsnorm_row(const double* x, int D, double eps, const float* w, double* out) {
  double ss = 0.0;
  for (int i = 0; i < D; ++i) ss += x[i] * x[i];
  double r = sqrt(ss / (double)D + eps);
  for (int i = 0; i < D; ++i) out[i] = (w ? (double)w[i] : 1.0) * x[i] / r;
}

/* RoPE of one head row at absolute position pos, rotate-half pairing:
 *   a = pos * base^(-2i/D),  y_i = x_i cos a - x_{i+D/2} sin a,
 *                            y_{i+D/2} = x_{i+D/2} cos a + x_i sin a.   (D even) */
void lao_rope_row(const double* x, int D, int64_t pos, double base, double* out) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double theta = pow(base, -2.0 * (double)i / (double)D);
    double a = (double)pos * theta;
    double c = cos(a), s = sin(a);
    double x0 = x[i], x1 = x[i + half];
    out[i] = x0 * c - x1 * s;
    out[i + half] = x1 * c + x0 * s;
  }
}

/* QK prologue of one row: RMSNorm then RoPE. x is float, out is double. */
static void prologue_row(const float* x, int D, int64_t pos, double base, double eps,
                         const float* w, double* tmp, double* out) {
  for (int i = 0; i < D; ++i) tmp[i] = (double)x[i];
  lao_rmsnorm_row(tmp, D, eps, w, out);
  for (int i = 0; i < D; ++i) tmp[i] = out[i];
  lao_rope_row(tmp, D, pos, base, out);
}

/* The prologue on a whole [B, T, H, D] tensor (token t is at position pos0 + t). */
void lao_prologue(const float* x, int B, int T, int H, int D, int64_t pos0, double base,
                  double eps, const float* w, double* out) {
  int64_t rows = (int64_t)B * T * H;
#pragma omp parallel for schedule(static) num_threads(lao_get_threads())
  for (int64_t r = 0; r < rows; ++r) {
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
    int t = (int)((r / H) % T);
    prologue_row(x + r * D, D, pos0 + t, base, eps, w, tmp, out + r * D);
    free(tmp);
  }
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static int column_block(int D) { return D >= 16 ? 16 : D; }

/*
 * Token-by-token recurrence from raw inputs (this is the oracle of the prefill
 * call; a decode step is the same call with T = 1 at position pos).
 *
 *   S   : [B, H, D, D] double, holds S_in on entry and S_out on return.
 *   o   : [B, T, H, D] double, gated output.
 *   q_w, k_w : [D] RMSNorm weights or NULL.
 */
void lao_forward(const float* q, const float* k, const float* v, const float* g, int B,
                 int T, int H, int D, int64_t pos0, double base, double eps,
                 const float* q_w, const float* k_w, double* S, double* o) {
  int jb = column_block(D);
  int nblk = (D + jb - 1) / jb;
  int64_t tasks = (int64_t)B * H * nblk;
#pragma omp parallel for schedule(dynamic, 1) num_threads(lao_get_threads())
  for (int64_t task = 0; task < tasks; ++task) {
    int blk = (int)(task % nblk);
    int h = (int)((task / nblk) % H);
    int b = (int)(task / ((int64_t)nblk * H));
    int j0 = blk * jb, j1 = j0 + jb < D ? j0 + jb : D;
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D * 3);
    double* qh = tmp + D;
    double* kh = tmp + 2 * D;
    double* Sbh = S + ((int64_t)b * H + h) * D * D;
    for (int t = 0; t < T; ++t) {
      int64_t row = (((int64_t)b * T + t) * H + h) * D;
      prologue_row(q + row, D, pos0 + t, base, eps, q_w, tmp, qh);
      prologue_row(k + row, D, pos0 + t, base, eps, k_w, tmp, kh);
      /* S_t = S_{t-1} + k_t v_t^T  (columns j0..j1 of this task) */
      for (int i = 0; i < D; ++i)
        for (int j = j0; j < j1; ++j) Sbh[i * D + j] += kh[i] * (double)v[row + j];
      /* o_t = sigmoid(g_t) * (q_t S_t) */
      for (int j = j0; j < j1; ++j) {
        double u = 0.0;
        for (int i = 0; i < D; ++i) u += qh[i] * Sbh[i * D + j];
        o[row + j] = sigmoid((double)g[row + j]) * u;
      }
    }
    free(tmp);
  }
}

/*
 * The same layer evaluated chunk by chunk (chunk length C >= 1; the last chunk
 * may be shorter).  For a chunk c with prefix state S_pre (the state before its
 * first token) and token t inside it:
 *     u_t = sum_{s in c, s <= t} (qh_t . kh_s) v_s  +  qh_t S_pre,
 * then S_pre <- S_pre + sum_{s in c} kh_s v_s^T.
 * This follows from summing the state update over a chunk; it is kept here only
 * so the tests can check that the chunked and recurrent forms agree.
 */
void lao_chunked(const float* q, const float* k, const float* v, const float* g, int B,
                 int T, int H, int D, int64_t pos0, double base, double eps,
                 const float* q_w, const float* k_w, int C, double* S, double* o) {
  if (C < 1) C = 1;
  int64_t tasks = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(lao_get_threads())
  for (int64_t task = 0; task < tasks; ++task) {
    int h = (int)(task % H);
    int b = (int)(task / H);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
    double* qh = (double*)malloc(sizeof(double) * (size_t)C * D);
    double* kh = (double*)malloc(sizeof(double) * (size_t)C * D);
    double* Sbh = S + ((int64_t)b * H + h) * D * D;
    for (int c0 = 0; c0 < T; c0 += C) {
      int n = T - c0 < C ? T - c0 : C;
      for (int r = 0; r < n; ++r) {
        int64_t row = (((int64_t)b * T + c0 + r) * H + h) * D;
        prologue_row(q + row, D, pos0 + c0 + r, base, eps, q_w, tmp, qh + (int64_t)r * D);
        prologue_row(k + row, D, pos0 + c0 + r, base, eps, k_w, tmp, kh + (int64_t)r * D);
      }
      /* outputs of the chunk: intra-chunk causal term + term through S_pre */
      for (int r = 0; r < n; ++r) {
        int64_t row = (((int64_t)b * T + c0 + r) * H + h) * D;
        for (int j = 0; j < D; ++j) {
          double u = 0.0;
          for (int s = 0; s <= r; ++s) {
            double a = 0.0;
            for (int i = 0; i < D; ++i) a += qh[(int64_t)r * D + i] * kh[(int64_t)s * D + i];
            u += a * (double)v[(((int64_t)b * T + c0 + s) * H + h) * D + j];
          }
          for (int i = 0; i < D; ++i) u += qh[(int64_t)r * D + i] * Sbh[i * D + j];
          o[row + j] = sigmoid((double)g[row + j]) * u;
        }
      }
      /* S_pre of the next chunk */
      for (int s = 0; s < n; ++s) {
        int64_t row = (((int64_t)b * T + c0 + s) * H + h) * D;
        for (int i = 0; i < D; ++i)
          for (int j = 0; j < D; ++j) Sbh[i * D + j] += kh[(int64_t)s * D + i] * (double)v[row + j];
      }
    }
    free(tmp);
    free(qh);
    free(kh);
  }
}

/*
 * Gradients of the layer (reverse mode of the recurrence above), for a scalar
 * loss L whose gradients with respect to the gated output o and the final state
 * S_out are do and dS_out.  Per (b, h), with du_t = do_t * sigmoid(g_t):
 *   forward, token by token:  S_t = S_{t-1} + kh_t v_t^T,  u_t = qh_t S_t,
 *       dg_t  = do_t * u_t * sigmoid'(g_t),     dqh_t = S_t du_t;
 *   backward, tokens in reverse:  G_t = G_{t+1} + qh_t du_t^T  (G_T = dS_out),
 *       dkh_t = G_t v_t,   dv_t = G_t^T kh_t,   and dS_in = G_0;
 *   then through RoPE (rotate back by the same angle) and RMSNorm:
 *       n = w x / r,  r = sqrt(mean(x^2) + eps):
 *       dx_i = w_i dn_i / r - x_i (sum_j w_j x_j dn_j) / (D r^3),  dw_i += dn_i x_i / r.
 * Outputs are double.  dS_in may be NULL; dqw_part / dkw_part, when not NULL, get
 * one [D] partial weight gradient per (b, h) task ([B*H][D]), to be summed.
 */
static void rope_back_row(const double* dy, int D, int64_t pos, double base, double* dn) {
  int half = D / 2;
  for (int i = 0; i < half; ++i) {
    double theta = pow(base, -2.0 * (double)i / (double)D);
    double a = (double)pos * theta;
    double c = cos(a), s = sin(a);
    dn[i] = dy[i] * c + dy[i + half] * s;
    dn[i + half] = -dy[i] * s + dy[i + half] * c;
  }
}

static void rmsnorm_back_row(const float* x, int D, double eps, const float* w, const double* dn,
                             double* dx, double* dw) {
  double ss = 0.0;
  for (int i = 0; i < D; ++i) ss += (double)x[i] * (double)x[i];
  double r = sqrt(ss / (double)D + eps);
  double dot = 0.0;
  for (int i = 0; i < D; ++i) dot += (w ? (double)w[i] : 1.0) * (double)x[i] * dn[i];
  for (int i = 0; i < D; ++i) {
    double wi = w ? (double)w[i] : 1.0;
    dx[i] = wi * dn[i] / r - (double)x[i] * dot / ((double)D * r * r * r);
    if (dw) dw[i] += dn[i] * (double)x[i] / r;
  }
}

void lao_backward(const float* q, const float* k, const float* v, const float* g, const float* dout,
                  int B, int T, int H, int D, int64_t pos0, double base, double eps, const float* q_w,
                  const float* k_w, const double* S_in, const double* dS_out, double* dq, double* dk,
                  double* dv, double* dg, double* dS_in, double* dqw_part, double* dkw_part) {
  int64_t tasks = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic, 1) num_threads(lao_get_threads())
  for (int64_t task = 0; task < tasks; ++task) {
    int h = (int)(task % H);
    int b = (int)(task / H);
    size_t DD = (size_t)D * D;
    double* S = (double*)malloc(sizeof(double) * DD);
    double* G = (double*)malloc(sizeof(double) * DD);
    double* qh = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* kh = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* du = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* dqh = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* dkh = (double*)malloc(sizeof(double) * (size_t)T * D);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D * 2);
    double* dn = tmp + D;
    double* dqw = dqw_part ? dqw_part + task * D : NULL;
    double* dkw = dkw_part ? dkw_part + task * D : NULL;
    if (dqw) memset(dqw, 0, sizeof(double) * (size_t)D);
    if (dkw) memset(dkw, 0, sizeof(double) * (size_t)D);
    for (size_t e = 0; e < DD; ++e) S[e] = S_in ? S_in[task * DD + e] : 0.0;
    /* forward: u, dg, du, dqh */
    for (int t = 0; t < T; ++t) {
      int64_t row = (((int64_t)b * T + t) * H + h) * D;
      prologue_row(q + row, D, pos0 + t, base, eps, q_w, tmp, qh + (int64_t)t * D);
      prologue_row(k + row, D, pos0 + t, base, eps, k_w, tmp, kh + (int64_t)t * D);
      for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j) S[(size_t)i * D + j] += kh[(int64_t)t * D + i] * (double)v[row + j];
      for (int j = 0; j < D; ++j) {
        double u = 0.0;
        for (int i = 0; i < D; ++i) u += qh[(int64_t)t * D + i] * S[(size_t)i * D + j];
        double sg = sigmoid((double)g[row + j]);
        dg[row + j] = (double)dout[row + j] * u * sg * (1.0 - sg);
        du[(int64_t)t * D + j] = (double)dout[row + j] * sg;
      }
      for (int i = 0; i < D; ++i) {
        double a = 0.0;
        for (int j = 0; j < D; ++j) a += S[(size_t)i * D + j] * du[(int64_t)t * D + j];
        dqh[(int64_t)t * D + i] = a;
      }
    }
    /* backward over tokens: G, dkh, dv */
    for (size_t e = 0; e < DD; ++e) G[e] = dS_out ? dS_out[task * DD + e] : 0.0;
    for (int t = T - 1; t >= 0; --t) {
      int64_t row = (((int64_t)b * T + t) * H + h) * D;
      for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j) G[(size_t)i * D + j] += qh[(int64_t)t * D + i] * du[(int64_t)t * D + j];
      for (int i = 0; i < D; ++i) {
        double a = 0.0;
        for (int j = 0; j < D; ++j) a += G[(size_t)i * D + j] * (double)v[row + j];
        dkh[(int64_t)t * D + i] = a;
      }
      for (int j = 0; j < D; ++j) {
        double a = 0.0;
        for (int i = 0; i < D; ++i) a += kh[(int64_t)t * D + i] * G[(size_t)i * D + j];
        dv[row + j] = a;
      }
    }
    if (dS_in)
      for (size_t e = 0; e < DD; ++e) dS_in[task * DD + e] = G[e];
    /* through RoPE and RMSNorm */
    for (int t = 0; t < T; ++t) {
      int64_t row = (((int64_t)b * T + t) * H + h) * D;
      rope_back_row(dqh + (int64_t)t * D, D, pos0 + t, base, dn);
      rmsnorm_back_row(q + row, D, eps, q_w, dn, dq + row, dqw);
      rope_back_row(dkh + (int64_t)t * D, D, pos0 + t, base, dn);
      rmsnorm_back_row(k + row, D, eps, k_w, dn, dk + row, dkw);
    }
    free(S);
    free(G);
    free(qh);
    free(kh);
    free(du);
    free(dqh);
    free(dkh);
    free(tmp);
  }
}
