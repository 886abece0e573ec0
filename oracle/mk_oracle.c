/*
 * CPU oracle for one Llama-style decoder step (test infrastructure only).
 *
 * This file is the plain, slow, obviously-correct definition that the HIP
 * path is checked against.  It is used only by the test-suite, by the smoke
 * check and by the benchmark's CPU-baseline leg; no product code links it.
 * It shares no code, header or table with the GPU library.
 *
 * What it computes.  The megakernel page ("2 . Definition et genealogie")
 * names the fused instruction kinds of a decoder pass in section 2.6 (its
 * dispatch example: an RMSNorm+QKV+RoPE instruction, attention, the output
 * projection) and, in section 2.1, the op families a megakernel mixes
 * (normalisation, matrix products, attention); it never writes out the
 * arithmetic.  The arithmetic below is therefore the standard Llama decoder
 * read from the workload shapes (hidden size, q/kv heads, head_dim, SwiGLU
 * MLP, RMSNorm eps, RoPE theta, tied embeddings, greedy decode):
 *
 *   x = E[token]
 *   per layer l:
 *     xn = rmsnorm(x, g_attn[l])                       (eps inside the sqrt)
 *     q, k, v = Wq xn, Wk xn, Wv xn                    (no biases)
 *     rotate-half RoPE on every q and k head at the token's position p
 *     K[l][g][p] = bf16(k_g), V[l][g][p] = bf16(v_g)   (cache is bf16)
 *     per q head h, kv group g = h * n_kv / n_q:
 *        softmax over t in [0, p] of (q_h . K_t) / sqrt(d), weighted sum of V_t
 *     x = x + Wo concat(o_h)
 *     x = x + Wd (silu(Wg xn2) * (Wu xn2)),  xn2 = rmsnorm(x, g_mlp[l])
 *   logits = W_lm rmsnorm(x, g_final)   (W_lm = E when tied)
 *   next   = smallest index of the largest fp32-rounded logit
 *
 * Precision: every activation and every sum is IEEE double, summed
 * sequentially in index order.  Weights are bf16 and are widened exactly.
 * The KV cache holds bf16 (round-to-nearest-even of the double value); a
 * double-precision cache mode exists only so tests can compare the
 * composition against a library implementation without the bf16 storage
 * rounding.  OpenMP splits only independent output rows; no sum is
 * reordered.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  double rms_eps, rope_theta;
  int32_t tied; /* 1: logits use the embedding matrix */
} orc_shape;

/* All weight tensors are bf16 bit patterns, row-major, nn.Linear convention
 * W[out][in].  Per-layer tensors come as arrays of n_layers pointers. */
typedef struct {
  const uint16_t *embed;      /* [V][H] */
  const uint16_t *lm_head;    /* [V][H]; ignored when tied */
  const uint16_t *final_norm; /* [H] */
  const uint16_t *const *attn_norm; /* [H] */
  const uint16_t *const *wq;        /* [n_q*d][H] */
  const uint16_t *const *wk;        /* [n_kv*d][H] */
  const uint16_t *const *wv;        /* [n_kv*d][H] */
  const uint16_t *const *wo;        /* [H][n_q*d] */
  const uint16_t *const *mlp_norm;  /* [H] */
  const uint16_t *const *wg;        /* [I][H] */
  const uint16_t *const *wu;        /* [I][H] */
  const uint16_t *const *wd;        /* [H][I] */
} orc_weights;

enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_TOKEN = -2, ORC_ERR_POS = -3, ORC_ERR_MEM = -4 };
enum { ORC_KV_BF16 = 0, ORC_KV_F64 = 1 };

/* ---------------------------------------------------------------- bf16 */

double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a double to the nearest bf16 (8 significant bits, exponent range of
 * fp32), ties to even, in one rounding step. */
uint16_t orc_f64_to_bf16(double v) {
  if (isnan(v)) return (uint16_t)0x7FC0;
  if (v == 0.0) return signbit(v) ? (uint16_t)0x8000 : (uint16_t)0x0000;
  double a = fabs(v);
  int e;
  frexp(a, &e);          /* a = m * 2^e, m in [0.5, 1) -> leading bit is 2^(e-1) */
  int lead = e - 1;
  if (lead < -126) lead = -126; /* subnormal range keeps a fixed quantum */
  double quantum = ldexp(1.0, lead - 7);
  double r = rint(a / quantum) * quantum; /* rint: round half to even */
  if (r >= ldexp(1.0, 128)) r = INFINITY;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  if (signbit(v)) f = -f;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* --------------------------------------------------------------- pieces */

/* y[r] = sum_c W[r][c] * x[c] for a bf16 row-major W[rows][cols]. */
void orc_matvec(const uint16_t *W, int64_t rows, int64_t cols, const double *x, double *y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t *row = W + r * cols;
    double s = 0.0;
    for (int64_t c = 0; c < cols; ++c) s += orc_bf16_to_f64(row[c]) * x[c];
    y[r] = s;
  }
}

/* RMSNorm with the epsilon inside the square root; gain may be NULL (= 1). */
void orc_rmsnorm(const double *x, const uint16_t *gain, int64_t n, double eps, double *out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double r = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) {
    double g = gain ? orc_bf16_to_f64(gain[i]) : 1.0;
    out[i] = (x[i] * r) * g;
  }
}

/* Rotate-half RoPE of one head vector u[d] at position pos: the pair
 * (u[i], u[i+d/2]) is turned by the angle pos * theta^(-2i/d). */
void orc_rope(double *u, int d, int64_t pos, double theta) {
  int half = d / 2;
  for (int i = 0; i < half; ++i) {
    double ang = (double)pos * pow(theta, -2.0 * (double)i / (double)d);
    double c = cos(ang), s = sin(ang);
    double a = u[i], b = u[i + half];
    u[i] = a * c - b * s;
    u[i + half] = b * c + a * s;
  }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

static double kv_get(const void *kv, int kv_mode, size_t idx) {
  if (kv_mode == ORC_KV_F64) return ((const double *)kv)[idx];
  return orc_bf16_to_f64(((const uint16_t *)kv)[idx]);
}

/* Single-head decode attention over n_pos cached positions.  K and V point at
 * position 0 of one (layer, sequence, kv head) row block, rows of d values
 * with a stride of d.  w_out (optional) receives the n_pos softmax weights. */
void orc_attend(const double *q, const void *K, const void *V, int kv_mode, int64_t n_pos, int d,
                double scale, double *out, double *w_out) {
  double *s = (double *)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
  double m = -INFINITY;
  for (int64_t t = 0; t < n_pos; ++t) {
    double dot = 0.0;
    for (int i = 0; i < d; ++i) dot += q[i] * kv_get(K, kv_mode, (size_t)t * d + i);
    s[t] = dot * scale;
    if (s[t] > m) m = s[t];
  }
  double z = 0.0;
  for (int64_t t = 0; t < n_pos; ++t) {
    s[t] = exp(s[t] - m);
    z += s[t];
  }
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  for (int64_t t = 0; t < n_pos; ++t) {
    double w = s[t] / z;
    if (w_out) w_out[t] = w;
    for (int i = 0; i < d; ++i) out[i] += w * kv_get(V, kv_mode, (size_t)t * d + i);
  }
  free(s);
}

/* Index of the largest value after rounding each to fp32; the smallest index
 * wins a tie. */
int64_t orc_argmax_f32(const double *v, int64_t n) {
  int64_t best = 0;
  float bv = (float)v[0];
  for (int64_t i = 1; i < n; ++i) {
    float f = (float)v[i];
    if (f > bv) {
      bv = f;
      best = i;
    }
  }
  return best;
}

/* Flat element index into the KV cache laid out [L][2][B_max][n_kv][max_ctx][d]
 * (plane 0 = keys, plane 1 = values). */
int64_t orc_kv_index(const orc_shape *sh, int64_t b_max, int64_t max_ctx, int64_t l, int64_t plane,
                     int64_t b, int64_t g, int64_t t) {
  return (((((l * 2 + plane) * b_max + b) * sh->n_kv_heads + g) * max_ctx + t) * sh->head_dim);
}

/* --------------------------------------------------------------- a step */

/* One decode step for `batch` sequences.  Sequence b reads token tokens[b] at
 * position positions[b], appends its keys/values to the cache at that slot of
 * every layer, attends over slots [0, positions[b]] and writes logits[b][V]
 * (double) and, if next_tokens is not NULL, the greedy next token.
 * kv_probe (optional, test instrumentation): receives, for every sequence and
 * layer, the appended keys before and after the rotation and the appended
 * values, all unrounded: double [batch][n_layers][3][n_kv_heads][head_dim]. */
int orc_decode_step(const orc_shape *sh, const orc_weights *w, int32_t batch, const int32_t *tokens,
                    const int32_t *positions, void *kv, int32_t kv_mode, int32_t b_max, int32_t max_ctx,
                    double *logits, int32_t *next_tokens, double *kv_probe) {
  if (!sh || !w || !tokens || !positions || !kv || !logits) return ORC_ERR_ARG;
  const int64_t H = sh->hidden, nq = sh->n_q_heads, nkv = sh->n_kv_heads, d = sh->head_dim;
  const int64_t I = sh->ffn, V = sh->vocab, L = sh->n_layers;
  if (H <= 0 || nq <= 0 || nkv <= 0 || d <= 0 || (d % 2) || I <= 0 || V <= 0 || L < 0) return ORC_ERR_ARG;
  if (nq % nkv) return ORC_ERR_ARG;
  if (batch < 0 || batch > b_max) return ORC_ERR_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    if (tokens[b] < 0 || tokens[b] >= V) return ORC_ERR_TOKEN;
    if (positions[b] < 0 || positions[b] >= max_ctx) return ORC_ERR_POS;
  }
  const double scale = 1.0 / sqrt((double)d);
  const uint16_t *wlm = sh->tied ? w->embed : w->lm_head;

  double *x = (double *)malloc(sizeof(double) * H);
  double *xn = (double *)malloc(sizeof(double) * H);
  double *q = (double *)malloc(sizeof(double) * nq * d);
  double *k = (double *)malloc(sizeof(double) * nkv * d);
  double *v = (double *)malloc(sizeof(double) * nkv * d);
  double *att = (double *)malloc(sizeof(double) * nq * d);
  double *tmp = (double *)malloc(sizeof(double) * (H > I ? H : I));
  double *a = (double *)malloc(sizeof(double) * I);
  double *u = (double *)malloc(sizeof(double) * I);
  if (!x || !xn || !q || !k || !v || !att || !tmp || !a || !u) {
    free(x); free(xn); free(q); free(k); free(v); free(att); free(tmp); free(a); free(u);
    return ORC_ERR_MEM;
  }

  for (int32_t b = 0; b < batch; ++b) {
    const int64_t p = positions[b];
    for (int64_t i = 0; i < H; ++i) x[i] = orc_bf16_to_f64(w->embed[(int64_t)tokens[b] * H + i]);

    for (int64_t l = 0; l < L; ++l) {
      /* attention block */
      orc_rmsnorm(x, w->attn_norm[l], H, sh->rms_eps, xn);
      orc_matvec(w->wq[l], nq * d, H, xn, q);
      orc_matvec(w->wk[l], nkv * d, H, xn, k);
      orc_matvec(w->wv[l], nkv * d, H, xn, v);
      double *probe = kv_probe ? kv_probe + ((size_t)b * L + l) * 3 * nkv * d : NULL;
      if (probe)
        for (int64_t i = 0; i < nkv * d; ++i) {
          probe[i] = k[i];
          probe[2 * nkv * d + i] = v[i];
        }
      for (int64_t h = 0; h < nq; ++h) orc_rope(q + h * d, (int)d, p, sh->rope_theta);
      for (int64_t g = 0; g < nkv; ++g) orc_rope(k + g * d, (int)d, p, sh->rope_theta);
      if (probe)
        for (int64_t i = 0; i < nkv * d; ++i) probe[nkv * d + i] = k[i];
      for (int64_t g = 0; g < nkv; ++g) {
        int64_t ki = orc_kv_index(sh, b_max, max_ctx, l, 0, b, g, p);
        int64_t vi = orc_kv_index(sh, b_max, max_ctx, l, 1, b, g, p);
        for (int64_t i = 0; i < d; ++i) {
          if (kv_mode == ORC_KV_F64) {
            ((double *)kv)[ki + i] = k[g * d + i];
            ((double *)kv)[vi + i] = v[g * d + i];
          } else {
            ((uint16_t *)kv)[ki + i] = orc_f64_to_bf16(k[g * d + i]);
            ((uint16_t *)kv)[vi + i] = orc_f64_to_bf16(v[g * d + i]);
          }
        }
      }
      for (int64_t h = 0; h < nq; ++h) {
        int64_t g = h * nkv / nq;
        size_t esz = kv_mode == ORC_KV_F64 ? sizeof(double) : sizeof(uint16_t);
        const char *K = (const char *)kv + esz * (size_t)orc_kv_index(sh, b_max, max_ctx, l, 0, b, g, 0);
        const char *Vv = (const char *)kv + esz * (size_t)orc_kv_index(sh, b_max, max_ctx, l, 1, b, g, 0);
        orc_attend(q + h * d, K, Vv, kv_mode, p + 1, (int)d, scale, att + h * d, NULL);
      }
      orc_matvec(w->wo[l], H, nq * d, att, tmp);
      for (int64_t i = 0; i < H; ++i) x[i] += tmp[i];

      /* MLP block */
      orc_rmsnorm(x, w->mlp_norm[l], H, sh->rms_eps, xn);
      orc_matvec(w->wg[l], I, H, xn, a);
      orc_matvec(w->wu[l], I, H, xn, u);
      for (int64_t j = 0; j < I; ++j) a[j] = orc_silu(a[j]) * u[j];
      orc_matvec(w->wd[l], H, I, a, tmp);
      for (int64_t i = 0; i < H; ++i) x[i] += tmp[i];
    }

    orc_rmsnorm(x, w->final_norm, H, sh->rms_eps, xn);
    orc_matvec(wlm, V, H, xn, logits + (int64_t)b * V);
    if (next_tokens) next_tokens[b] = (int32_t)orc_argmax_f32(logits + (int64_t)b * V, V);
  }

  free(x); free(xn); free(q); free(k); free(v); free(att); free(tmp); free(a); free(u);
  return ORC_OK;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
