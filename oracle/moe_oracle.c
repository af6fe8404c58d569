/*
 * CPU oracle of the MoE SwiGLU feed-forward forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain definition that the
 * HIP path is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; the product path never does.
 * It shares no code, header, table or helper with the HIP library.
 *
 * Every sum is accumulated in fp64 and no intermediate result is rounded:
 * inputs are read exactly as stored (fp32, or bf16 widened by this file's
 * own converter) and the results are fp64.
 *
 * Sources (page title, section):
 *  - "APEX-1 Mathematical Reference - Part 3", section 12.2 (SwiGLU formula),
 *    12.3 (SiLU), 13.2 (MoE = shared experts + sum_k g_k Expert_{e_k},
 *    router r = x W_router + b, top-K, softmax over the selected scores).
 *  - "A working MoE layer in PyTorch" (moe-from-scratch): fp32 softmax over
 *    all experts, top-K, renormalise; sorted dispatch with bincount.
 *  - "StableLatentMoE and QuantileBalancer": sigmoid scores + bias select
 *    the top-(K+1), the last is dropped, weights are the uncorrected sigmoid
 *    scores (renormalised only on request) times a routed scaling factor;
 *    stable argsort dispatch with counts and cumulative ends; latent
 *    down-projection M->L, routed experts in L, optional RMSNorm in L,
 *    up-projection L->M, output = shared + routed.
 *  - "10 - Mixture of Experts" (APEX-1 docs): shared experts see every token
 *    and are added to the routed sum; an expert with no tokens is skipped.
 *
 * Readings where the pages are silent (listed with the rest in the design
 * notes): equal scores rank the lower expert id first; slots are ordered by
 * descending score; the balance bias enters the softmax-over-selected
 * weights (it is part of the ranked logits) but not the sigmoid weights;
 * RMSNorm is R / sqrt(mean(R^2) + eps) * gamma.
 *
 * The backward pass (or_backward) differentiates the same definition by
 * hand: SiLU' = sigma (1 + x (1 - sigma)), the routing weights' Jacobians of
 * the three rules, no gradient through the (piecewise constant) selection or
 * into the balance bias; weight gradients reach only the experts that some
 * token selected ("StableLatentMoE and QuantileBalancer": inactive experts
 * get no gradient). Its pins are central finite differences of the forward.
 *
 * Parity pins live in the test suite: the SiLU table of section 12.3, the
 * derivable part of the section 12.5 worked example, the router example of
 * section 13.5, the dispatch example of the StableLatentMoE page, closed-form
 * identities and a dense, masked brute force on tiny inputs.
 *
 * Parity unpinned: the RMSNorm formula is pinned only by its properties
 * (invariance to scaling of the routed sum, unit mean square at gamma = 1,
 * gamma applied per element), and the latent workload's eps (1e-6), gamma
 * (ones) and routed scale (1.0) are readings with no value on the pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_F64 2 /* only for the y_rows argument of or_combine */

#define OR_ROUTE_TOPK_SOFTMAX 0  /* rank r = xW + b, softmax over the K picked */
#define OR_ROUTE_SOFTMAX_TOPK 1  /* p = softmax(r) over E, top-K, renormalise  */
#define OR_ROUTE_SIGMOID_BIAS 2  /* s = sigmoid(xW); rank s + b; g = s (raw)   */

typedef struct {
  int64_t T;
  int32_t d, d_ff, E, K, d_shared, latent;
  int32_t act;
  int32_t route;
  int32_t renormalize, has_rmsnorm;
  double routed_scale, rms_eps;
} or_layer;

typedef struct {
  const void *x;          /* [T, d]                act                */
  const float *w_router;  /* [E, d]                fp32               */
  const float *bias;      /* [E] or NULL           fp32               */
  const void *w_gate;     /* [E, d_ff, d_e]        act (out x in)     */
  const void *w_up;       /* [E, d_ff, d_e]        act                */
  const void *w_down;     /* [E, d_e, d_ff]        act                */
  const void *ws_gate;    /* [d_shared, d]         act (may be NULL)  */
  const void *ws_up;      /* [d_shared, d]         act                */
  const void *ws_down;    /* [d, d_shared]         act                */
  const void *w_lat_down; /* [L, d]                act (latent only)  */
  const void *w_lat_up;   /* [d, L]                act                */
  const float *rms_gamma; /* [L]                   fp32               */
} or_tensors;

/* ------------------------------------------------------------ scalars */

double or_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Logistic sigmoid, 1 / (1 + e^-x)   (Math. Reference Part 3, 12.3). */
double or_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^-x)   (Math. Reference Part 3, 12.3). */
double or_silu(double x) { return x / (1.0 + exp(-x)); }

static double ld(const void *p, int act, int64_t i) {
  if (act == OR_BF16) return or_bf16_to_double(((const uint16_t *)p)[i]);
  if (act == OR_F64) return ((const double *)p)[i];
  return (double)((const float *)p)[i];
}

/* sum_i w[off + i] * v[i] over n entries, fp64 accumulation. */
static double dot(const void *w, int act, int64_t off, const double *v, int n) {
  double s = 0.0;
  if (act == OR_BF16) {
    const uint16_t *p = (const uint16_t *)w + off;
    for (int i = 0; i < n; ++i) s += or_bf16_to_double(p[i]) * v[i];
  } else {
    const float *p = (const float *)w + off;
    for (int i = 0; i < n; ++i) s += (double)p[i] * v[i];
  }
  return s;
}

/* ------------------------------------------------------------ routing */

/* Rank by repeatedly taking the largest remaining score; on equal scores the
 * earlier (lower) expert id is taken first. Writes the first n_pick ids. */
static void rank_top(const double *score, int E, int n_pick, int *taken, int32_t *out) {
  for (int e = 0; e < E; ++e) taken[e] = 0;
  for (int r = 0; r < n_pick; ++r) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (!taken[e] && (best < 0 || score[e] > score[best])) best = e;
    taken[best] = 1;
    out[r] = best;
  }
}

/* Route one token (Math. Reference Part 3, 13.2; moe-from-scratch router;
 * StableLatentMoE "FP32 router and training-only QB update").
 * xv: the token's d inputs. Outputs idx[K], g[K], *gap, top[K+1] (may be NULL).
 * If force_idx is given, it replaces the selection (weights still computed
 * from this token's scores). */
static void route_one(const or_layer *L, const or_tensors *W, const double *xv,
                      const int32_t *force_idx, int32_t *idx, double *g, double *gap,
                      double *top) {
  const int E = L->E, K = L->K, d = L->d;
  double *r = (double *)malloc(sizeof(double) * (size_t)E * 3);
  double *rank_score = r + E, *raw = r + 2 * E;
  int *taken = (int *)malloc(sizeof(int) * (size_t)E);
  int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
  for (int e = 0; e < E; ++e) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += (double)W->w_router[(int64_t)e * d + i] * xv[i];
    r[e] = s;
  }
  if (L->route == OR_ROUTE_SIGMOID_BIAS) {
    for (int e = 0; e < E; ++e) {
      raw[e] = or_sigmoid(r[e]);
      rank_score[e] = raw[e] + (W->bias ? (double)W->bias[e] : 0.0);
    }
  } else {
    for (int e = 0; e < E; ++e) rank_score[e] = r[e] + (W->bias ? (double)W->bias[e] : 0.0);
    if (L->route == OR_ROUTE_SOFTMAX_TOPK) {
      double m = rank_score[0], z = 0.0;
      for (int e = 1; e < E; ++e) m = rank_score[e] > m ? rank_score[e] : m;
      for (int e = 0; e < E; ++e) { rank_score[e] = exp(rank_score[e] - m); z += rank_score[e]; }
      for (int e = 0; e < E; ++e) rank_score[e] /= z;
    }
  }
  const int n_pick = K + 1 <= E ? K + 1 : E;
  rank_top(rank_score, E, n_pick, taken, sel);
  if (gap) *gap = (K < E) ? rank_score[sel[K - 1]] - rank_score[sel[K]] : INFINITY;
  if (top)
    for (int r2 = 0; r2 <= K; ++r2) top[r2] = r2 < n_pick ? rank_score[sel[r2]] : -INFINITY;
  if (force_idx)
    for (int k = 0; k < K; ++k) sel[k] = force_idx[k];
  for (int k = 0; k < K; ++k) idx[k] = sel[k];

  if (L->route == OR_ROUTE_TOPK_SOFTMAX) {
    /* softmax over the K selected biased logits */
    double m = rank_score[sel[0]], z = 0.0;
    for (int k = 1; k < K; ++k) m = rank_score[sel[k]] > m ? rank_score[sel[k]] : m;
    for (int k = 0; k < K; ++k) { g[k] = exp(rank_score[sel[k]] - m); z += g[k]; }
    for (int k = 0; k < K; ++k) g[k] /= z;
  } else if (L->route == OR_ROUTE_SOFTMAX_TOPK) {
    /* probabilities of the selected experts, divided by their sum */
    double z = 0.0;
    for (int k = 0; k < K; ++k) { g[k] = rank_score[sel[k]]; z += g[k]; }
    for (int k = 0; k < K; ++k) g[k] /= z;
  } else {
    /* uncorrected sigmoid scores; renormalised only on request */
    double z = 0.0;
    for (int k = 0; k < K; ++k) { g[k] = raw[sel[k]]; z += g[k]; }
    if (L->renormalize)
      for (int k = 0; k < K; ++k) g[k] /= z;
  }
  for (int k = 0; k < K; ++k) g[k] *= L->routed_scale;
  free(sel);
  free(taken);
  free(r);
}

static void load_row(const void *x, int act, int64_t row, int n, double *out) {
  for (int i = 0; i < n; ++i) out[i] = ld(x, act, row * (int64_t)n + i);
}

static int check_layer(const or_layer *L) {
  if (!L || L->T < 0 || L->d <= 0 || L->E <= 0 || L->K <= 0 || L->K > L->E) return -2;
  if (L->route < 0 || L->route > 2 || (L->act != OR_F32 && L->act != OR_BF16)) return -3;
  return 0;
}

int or_route(const or_layer *L, const or_tensors *W, const int64_t *tokens, int64_t n,
             int32_t *idx, double *g, double *gap, double *top_scores) {
  int rc = check_layer(L);
  if (rc) return rc;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < n; ++j) {
    double *xv = (double *)malloc(sizeof(double) * (size_t)L->d);
    load_row(W->x, L->act, tokens ? tokens[j] : j, L->d, xv);
    route_one(L, W, xv, NULL, idx + j * L->K, g + j * L->K, gap ? gap + j : NULL,
              top_scores ? top_scores + j * (L->K + 1) : NULL);
    free(xv);
  }
  return 0;
}

/* ------------------------------------------------------------ SwiGLU */

/* y += scale * W_down (SiLU(W_gate v) * (W_up v))   (Math. Reference Part 3,
 * 12.2), one expert, weights stored out x in: gate/up [f, n], down [n, f]. */
static void swiglu_acc(const void *wg, const void *wu, const void *wd, int act,
                       int64_t base_gu, int64_t base_d, int n, int f, const double *v,
                       double scale, double *y, double *h) {
  for (int j = 0; j < f; ++j) {
    double a = dot(wg, act, base_gu + (int64_t)j * n, v, n);
    double u = dot(wu, act, base_gu + (int64_t)j * n, v, n);
    h[j] = or_silu(a) * u;
  }
  for (int i = 0; i < n; ++i) y[i] += scale * dot(wd, act, base_d + (int64_t)i * f, h, f);
}

/* Whole layer for one token, fp64 (Math. Reference Part 3, 13.2; latent
 * variant per StableLatentMoE "Return to model width"). */
static void forward_one(const or_layer *L, const or_tensors *W, int64_t t,
                        const int32_t *force_idx, double *y, int32_t *idx, double *g,
                        double *gap) {
  const int d = L->d, f = L->d_ff, K = L->K;
  const int de = L->latent ? L->latent : d;
  int hmax = f > L->d_shared ? f : L->d_shared;
  double *xv = (double *)malloc(sizeof(double) * (size_t)d);
  double *zv = (double *)malloc(sizeof(double) * (size_t)de);
  double *rv = (double *)calloc((size_t)de, sizeof(double));
  double *h = (double *)malloc(sizeof(double) * (size_t)(hmax > 0 ? hmax : 1));
  load_row(W->x, L->act, t, d, xv);
  route_one(L, W, xv, force_idx, idx, g, gap, NULL);

  /* routed input: x itself, or its latent projection z = W_lat_down x */
  if (L->latent)
    for (int l = 0; l < de; ++l) zv[l] = dot(W->w_lat_down, L->act, (int64_t)l * d, xv, d);
  else
    memcpy(zv, xv, sizeof(double) * (size_t)d);

  for (int k = 0; k < K; ++k) {
    const int64_t e = idx[k];
    swiglu_acc(W->w_gate, W->w_up, W->w_down, L->act, e * (int64_t)f * de,
               e * (int64_t)de * f, de, f, zv, g[k], rv, h);
  }

  for (int i = 0; i < d; ++i) y[i] = 0.0;
  if (L->latent) {
    if (L->has_rmsnorm) {
      double ms = 0.0;
      for (int l = 0; l < de; ++l) ms += rv[l] * rv[l];
      ms /= de;
      const double inv = 1.0 / sqrt(ms + L->rms_eps);
      for (int l = 0; l < de; ++l)
        rv[l] = rv[l] * inv * (W->rms_gamma ? (double)W->rms_gamma[l] : 1.0);
    }
    for (int i = 0; i < d; ++i) y[i] = dot(W->w_lat_up, L->act, (int64_t)i * de, rv, de);
  } else {
    for (int i = 0; i < d; ++i) y[i] = rv[i];
  }
  if (L->d_shared > 0)
    swiglu_acc(W->ws_gate, W->ws_up, W->ws_down, L->act, 0, 0, d, L->d_shared, xv, 1.0, y, h);
  free(h);
  free(rv);
  free(zv);
  free(xv);
}

int or_forward(const or_layer *L, const or_tensors *W, const int64_t *tokens, int64_t n,
               const int32_t *idx_override, double *out, int32_t *idx, double *g,
               double *gap) {
  int rc = check_layer(L);
  if (rc) return rc;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t j = 0; j < n; ++j) {
    forward_one(L, W, tokens ? tokens[j] : j, idx_override ? idx_override + j * L->K : NULL,
                out + j * L->d, idx + j * L->K, g + j * L->K, gap ? gap + j : NULL);
  }
  return 0;
}

/* Expert FFN on given rows: out[p] = scale[p] * FFN_{expert[p]}(rows[p]), at
 * the routed width d_e. Used to check the grouped expert stage alone. */
int or_expert_rows(const or_layer *L, const or_tensors *W, const void *rows,
                   const int32_t *expert, const float *scale, int64_t n, double *out) {
  int rc = check_layer(L);
  if (rc) return rc;
  const int f = L->d_ff, de = L->latent ? L->latent : L->d;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t p = 0; p < n; ++p) {
    double *v = (double *)malloc(sizeof(double) * (size_t)de);
    double *h = (double *)malloc(sizeof(double) * (size_t)f);
    load_row(rows, L->act, p, de, v);
    for (int i = 0; i < de; ++i) out[p * de + i] = 0.0;
    const int64_t e = expert[p];
    swiglu_acc(W->w_gate, W->w_up, W->w_down, L->act, e * (int64_t)f * de,
               e * (int64_t)de * f, de, f, v, scale ? (double)scale[p] : 1.0, out + p * de, h);
    free(h);
    free(v);
  }
  return 0;
}

/* Combine for given tokens: out[t] = shared(x_t) + routed(t), where the routed
 * part is sum_k y_rows[inv[t*K + k]] (fixed expert-slot order), passed through
 * the latent RMSNorm and up-projection when the layer is latent. y_rows is
 * [T*K, d_e] in y_dtype (OR_F32, OR_BF16 or OR_F64). */
int or_combine(const or_layer *L, const or_tensors *W, const void *y_rows, int y_dtype,
               const int32_t *inv, const int64_t *tokens, int64_t n, double *out) {
  int rc = check_layer(L);
  if (rc) return rc;
  const int d = L->d, K = L->K, de = L->latent ? L->latent : d;
  const int hs = L->d_shared > 0 ? L->d_shared : 1;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t j = 0; j < n; ++j) {
    const int64_t t = tokens ? tokens[j] : j;
    double *rv = (double *)calloc((size_t)de, sizeof(double));
    double *xv = (double *)malloc(sizeof(double) * (size_t)d);
    double *h = (double *)malloc(sizeof(double) * (size_t)hs);
    double *y = out + j * d;
    for (int k = 0; k < K; ++k) {
      const int64_t p = inv[t * K + k];
      for (int l = 0; l < de; ++l) rv[l] += ld(y_rows, y_dtype, p * de + l);
    }
    if (L->latent) {
      if (L->has_rmsnorm) {
        double ms = 0.0;
        for (int l = 0; l < de; ++l) ms += rv[l] * rv[l];
        ms /= de;
        const double s = 1.0 / sqrt(ms + L->rms_eps);
        for (int l = 0; l < de; ++l) rv[l] = rv[l] * s * (W->rms_gamma ? (double)W->rms_gamma[l] : 1.0);
      }
      for (int i = 0; i < d; ++i) y[i] = dot(W->w_lat_up, L->act, (int64_t)i * de, rv, de);
    } else {
      for (int i = 0; i < d; ++i) y[i] = rv[i];
    }
    if (L->d_shared > 0) {
      load_row(W->x, L->act, t, d, xv);
      swiglu_acc(W->ws_gate, W->ws_up, W->ws_down, L->act, 0, 0, d, L->d_shared, xv, 1.0, y, h);
    }
    free(h);
    free(xv);
    free(rv);
  }
  return 0;
}

/* ------------------------------------------------------------ dispatch */

/* Stable counting sort of the T*K (token, slot) assignments by expert id
 * (StableLatentMoE, "Dispatch is a stable permutation"): counts per expert,
 * exclusive offsets (offsets[E] = T*K), then each slot in increasing t*K + k
 * order is placed at offsets[e] + (number of earlier slots with expert e).
 * perm[pos] = t*K + k, sorted_token[pos] = t, inv[t*K + k] = pos,
 * sorted_w[pos] = g[t*K + k]. Any output pointer except counts may be NULL. */
int or_dispatch(int64_t T, int32_t K, int32_t E, const int32_t *idx, const float *g,
                int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *sorted_token,
                int32_t *inv, float *sorted_w) {
  if (T < 0 || K <= 0 || E <= 0 || !counts) return -1;
  const int64_t n = T * K;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t s = 0; s < n; ++s) {
    if (idx[s] < 0 || idx[s] >= E) return -2;
    counts[idx[s]]++;
  }
  int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E + 1));
  next[0] = 0;
  for (int e = 0; e < E; ++e) next[e + 1] = next[e] + counts[e];
  if (offsets)
    for (int e = 0; e <= E; ++e) offsets[e] = next[e];
  for (int64_t s = 0; s < n; ++s) {
    const int32_t pos = next[idx[s]]++;
    if (perm) perm[pos] = (int32_t)s;
    if (sorted_token) sorted_token[pos] = (int32_t)(s / K);
    if (inv) inv[s] = pos;
    if (sorted_w && g) sorted_w[pos] = g[s];
  }
  free(next);
  return 0;
}

/* Bias-based load balancing ("APEX-1 Mathematical Reference - Part 3",
 * section 14.3): after a step with n_tokens tokens, expert e's observed load
 * is f_e = counts[e] / (n_tokens * K) against the target 1/E; its bias moves
 * by alpha * sign(1/E - f_e) and is clamped to [-1, 1] (section 14.4: a
 * balanced expert, f_e = 1/E, does not move). The sign is taken exactly, on
 * the integers n_tokens * K - E * counts[e] (same sign as 1/E - f_e). The new
 * bias is the fp64 value b + alpha * s, clamped, and stored as fp32: b and
 * alpha are fp32 values, so this is the correctly rounded fp32 sum.
 * n_tokens = 0 leaves the bias unchanged (no load was observed). */
int or_balance_bias(int32_t E, int32_t K, int64_t n_tokens, const int32_t *counts, float alpha,
                    float *bias) {
  if (E <= 0 || K <= 0 || n_tokens < 0 || !counts || !bias) return -1;
  if (n_tokens == 0) return 0;
  for (int e = 0; e < E; ++e) {
    const int64_t diff = n_tokens * (int64_t)K - (int64_t)E * counts[e];
    const double s = diff > 0 ? 1.0 : (diff < 0 ? -1.0 : 0.0);
    double b = (double)bias[e] + (double)alpha * s;
    if (b > 1.0) b = 1.0;
    if (b < -1.0) b = -1.0;
    bias[e] = (float)b;
  }
  return 0;
}

static int cmp_double(const void *a, const void *b) {
  const double x = *(const double *)a, y = *(const double *)b;
  return (x > y) - (x < y);
}

/* QuantileBalancer update ("StableLatentMoE and QuantileBalancer",
 * "QuantileBalancer: persistent biases, no gradient update"; sigmoid routing
 * only). For every token t: s[t,e] = sigmoid(x_t . W_router[e]) (raw scores),
 * corrected scores s + b with the current bias b, and the threshold thresh_t =
 * the (K+1)-th largest corrected score. For every expert e the new bias is
 * the p = K/E quantile over tokens of thresh_t - s[t,e] with the "higher"
 * rule (the sorted value at position ceil(p (T-1)), taken exactly as
 * ceil(K (T-1) / E)); the E quantiles are then centred by their mean.
 * Needs K < E and T >= 1; writes new_bias[E] (fp64). */
int or_quantile_balance(const or_layer *L, const or_tensors *W, double *new_bias) {
  int rc = check_layer(L);
  if (rc) return rc;
  if (L->route != OR_ROUTE_SIGMOID_BIAS) return -3;
  const int E = L->E, K = L->K, d = L->d;
  const int64_t T = L->T;
  if (K >= E || T < 1 || !new_bias) return -2;
  double *diff = (double *)malloc(sizeof(double) * (size_t)(T * E)); /* [E][T] */
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    double *xv = (double *)malloc(sizeof(double) * (size_t)d);
    double *raw = (double *)malloc(sizeof(double) * (size_t)E * 2);
    double *corr = raw + E;
    int *taken = (int *)malloc(sizeof(int) * (size_t)E);
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)(K + 1));
    load_row(W->x, L->act, t, d, xv);
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int i = 0; i < d; ++i) s += (double)W->w_router[(int64_t)e * d + i] * xv[i];
      raw[e] = or_sigmoid(s);
      corr[e] = raw[e] + (W->bias ? (double)W->bias[e] : 0.0);
    }
    rank_top(corr, E, K + 1, taken, sel);
    const double thresh = corr[sel[K]];
    for (int e = 0; e < E; ++e) diff[(int64_t)e * T + t] = thresh - raw[e];
    free(sel);
    free(taken);
    free(raw);
    free(xv);
  }
  const int64_t pos = ((int64_t)K * (T - 1) + E - 1) / E; /* ceil(K (T-1) / E) */
  double mean = 0.0;
  for (int e = 0; e < E; ++e) {
    qsort(diff + (int64_t)e * T, (size_t)T, sizeof(double), cmp_double);
    new_bias[e] = diff[(int64_t)e * T + pos];
    mean += new_bias[e];
  }
  mean /= E;
  for (int e = 0; e < E; ++e) new_bias[e] -= mean;
  free(diff);
  return 0;
}

/* Router auxiliary losses over the T tokens of a step, on the router's own
 * logits r_t = x_t . W_router (the balance bias is a non-gradient nudge and
 * is left out):
 *  - load-balancing loss ("A working MoE layer in PyTorch", the Switch
 *    load-balancing loss of MoELayer.forward): alpha * E * sum_e f_e * P_e,
 *    f_e = counts[e] / (T K), P_e = mean over tokens of softmax(r_t)_e;
 *  - router z-loss ("Mixture of Experts (MoE)", transformer book chapter 16,
 *    MoEAuxiliaryLoss.router_z_loss, weight 0.001 there): z_weight * mean
 *    over tokens of logsumexp(r_t)^2.
 * Writes out[0] = load-balancing loss, out[1] = z-loss (fp64). Needs T >= 1. */
int or_router_losses(const or_layer *L, const or_tensors *W, const int32_t *counts, double alpha,
                     double z_weight, double *out) {
  int rc = check_layer(L);
  if (rc) return rc;
  const int E = L->E, d = L->d;
  const int64_t T = L->T;
  if (T < 1 || !counts || !out) return -2;
  double *psum = (double *)calloc((size_t)E, sizeof(double));
  double zsum = 0.0;
  double *xv = (double *)malloc(sizeof(double) * (size_t)d);
  double *r = (double *)malloc(sizeof(double) * (size_t)E);
  for (int64_t t = 0; t < T; ++t) {
    load_row(W->x, L->act, t, d, xv);
    double m = -INFINITY;
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int i = 0; i < d; ++i) s += (double)W->w_router[(int64_t)e * d + i] * xv[i];
      r[e] = s;
      m = s > m ? s : m;
    }
    double z = 0.0;
    for (int e = 0; e < E; ++e) z += exp(r[e] - m);
    for (int e = 0; e < E; ++e) psum[e] += exp(r[e] - m) / z;
    const double lse = m + log(z);
    zsum += lse * lse;
  }
  double aux = 0.0;
  for (int e = 0; e < E; ++e)
    aux += ((double)counts[e] / ((double)T * L->K)) * (psum[e] / (double)T);
  out[0] = alpha * E * aux;
  out[1] = z_weight * zsum / (double)T;
  free(r);
  free(xv);
  free(psum);
  return 0;
}

/* ------------------------------------------------------------ backward */

/* Gradient of the routing weights g[K] of one token with respect to its
 * router logits r = x W_router^T (the balance bias is a fixed input and
 * gets none; the selection is piecewise constant, so it passes no gradient).
 * Weight rules as in route_one:
 *  - softmax over the selected (Math. Reference Part 3, 13.2) and the
 *    moe-from-scratch rule (softmax over all, top-K, renormalised: the same
 *    function of the selected logits): g_k = c q_k, q = softmax over the
 *    selected of r + b, c = routed_scale, so dr_k = q_k (c dg_k - sum_j q_j c dg_j);
 *  - sigmoid rule (StableLatentMoE): g_k = c s_k, or c s_k / sum_j s_j when
 *    renormalised, s = sigmoid(r), ds/dr = s (1 - s).
 * dr[E] is zero outside the selection. */
static void route_grad(const or_layer *L, const or_tensors *W, const double *xv,
                       const int32_t *sel, const double *dg, double *dr) {
  const int E = L->E, K = L->K, d = L->d;
  const double c = L->routed_scale;
  for (int e = 0; e < E; ++e) dr[e] = 0.0;
  double *r = (double *)malloc(sizeof(double) * (size_t)K);
  for (int k = 0; k < K; ++k) {
    double s = 0.0;
    for (int i = 0; i < d; ++i) s += (double)W->w_router[(int64_t)sel[k] * d + i] * xv[i];
    r[k] = s;
  }
  if (L->route == OR_ROUTE_SIGMOID_BIAS) {
    double S = 0.0, sdg = 0.0;
    for (int k = 0; k < K; ++k) {
      const double s = or_sigmoid(r[k]);
      S += s;
      sdg += dg[k] * s;
    }
    for (int k = 0; k < K; ++k) {
      const double s = or_sigmoid(r[k]);
      const double ds = L->renormalize ? c * (dg[k] / S - sdg / (S * S)) : c * dg[k];
      dr[sel[k]] += ds * s * (1.0 - s);
    }
  } else {
    double m = -INFINITY, z = 0.0, qdg = 0.0;
    double *q = (double *)malloc(sizeof(double) * (size_t)K);
    for (int k = 0; k < K; ++k) {
      q[k] = r[k] + (W->bias ? (double)W->bias[sel[k]] : 0.0);
      m = q[k] > m ? q[k] : m;
    }
    for (int k = 0; k < K; ++k) { q[k] = exp(q[k] - m); z += q[k]; }
    for (int k = 0; k < K; ++k) { q[k] /= z; qdg += q[k] * c * dg[k]; }
    for (int k = 0; k < K; ++k) dr[sel[k]] += q[k] * (c * dg[k] - qdg);
    free(q);
  }
  free(r);
}

/* Backward of one SwiGLU FFN (Math. Reference Part 3, 12.2) on input v[n]
 * with output gradient dy[n] scaled by w (the routing weight; 1 for shared
 * experts): y = W_down h, h = SiLU(a) * u, a = W_gate v, u = W_up v,
 * SiLU'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))). Adds the input gradient to
 * dv and the weight gradients to dwg / dwu [f, n] and dwd [n, f] (any may be
 * NULL); returns <dy, y> (the gradient of the routing weight). */
static double swiglu_backward(const void *wg, const void *wu, const void *wd, int act,
                              int64_t base_gu, int64_t base_d, int n, int f, const double *v,
                              const double *dy, double w, double *dv, double *dwg, double *dwu,
                              double *dwd, double *buf) {
  double *a = buf, *u = buf + f, *h = buf + 2 * f, *dh = buf + 3 * f;
  for (int j = 0; j < f; ++j) {
    a[j] = dot(wg, act, base_gu + (int64_t)j * n, v, n);
    u[j] = dot(wu, act, base_gu + (int64_t)j * n, v, n);
    h[j] = or_silu(a[j]) * u[j];
  }
  double dg = 0.0;
  for (int i = 0; i < n; ++i) dg += dy[i] * dot(wd, act, base_d + (int64_t)i * f, h, f);
  for (int j = 0; j < f; ++j) {
    double s = 0.0;
    for (int i = 0; i < n; ++i) s += ld(wd, act, base_d + (int64_t)i * f + j) * w * dy[i];
    dh[j] = s;
  }
  if (dwd)
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < f; ++j) dwd[(int64_t)i * f + j] += w * dy[i] * h[j];
  for (int j = 0; j < f; ++j) {
    const double sg = or_sigmoid(a[j]);
    const double da = dh[j] * u[j] * sg * (1.0 + a[j] * (1.0 - sg));
    const double du = dh[j] * or_silu(a[j]);
    for (int i = 0; i < n; ++i) {
      dv[i] += ld(wg, act, base_gu + (int64_t)j * n + i) * da +
               ld(wu, act, base_gu + (int64_t)j * n + i) * du;
      if (dwg) dwg[(int64_t)j * n + i] += da * v[i];
      if (dwu) dwu[(int64_t)j * n + i] += du * v[i];
    }
  }
  return dg;
}

/* Backward of the layer for the listed tokens (all if NULL)
 * with output gradients d_out[n, d] (row j belongs to token tokens[j]):
 *  - dx[n, d] (may be NULL): input gradients (routed experts, shared
 *    experts, router);
 *  - dw_router[E, d] (may be NULL);
 *  - expert weight gradients summed over the listed tokens: for every
 *    expert if want_expert == -1 (dw_gate / dw_up [E, d_ff, d], dw_down
 *    [E, d, d_ff]), for expert want_expert only (one expert's shape), or
 *    none if want_expert < -1 (the three may also be NULL);
 *  - dws_gate / dws_up [d_shared, d], dws_down [d, d_shared] (may be NULL);
 *  - latent layers: dw_lat_down [L, d], dw_lat_up [d, L], d_rms_gamma [L]
 *    (may be NULL; expert weight gradients are then at the routed width L).
 * Gradient outputs are zeroed first. Experts no listed token selects keep
 * zero gradients. idx_override [n, K] replaces the selection (near ties).
 * Tokens run in parallel when no weight gradient is requested. */
int or_backward(const or_layer *L, const or_tensors *W, const double *d_out,
                const int64_t *tokens, int64_t n, const int32_t *idx_override,
                int32_t want_expert, double *dx, double *dw_router, double *dw_gate,
                double *dw_up, double *dw_down, double *dws_gate, double *dws_up,
                double *dws_down, double *dw_lat_down, double *dw_lat_up,
                double *d_rms_gamma) {
  int rc = check_layer(L);
  if (rc) return rc;
  const int d = L->d, f = L->d_ff, E = L->E, K = L->K, ds = L->d_shared;
  const int de = L->latent ? L->latent : d; /* routed width */
  const int64_t egu = (int64_t)f * de;
  const int want_w = want_expert >= -1 && (dw_gate || dw_up || dw_down);
  const int serial = want_w || dw_router || dws_gate || dws_up || dws_down || dw_lat_down ||
                     dw_lat_up || d_rms_gamma;
  if (dx) memset(dx, 0, sizeof(double) * (size_t)(n * d));
  if (dw_router) memset(dw_router, 0, sizeof(double) * (size_t)E * d);
  const int64_t n_exp = want_expert == -1 ? E : 1;
  if (want_w) {
    if (dw_gate) memset(dw_gate, 0, sizeof(double) * (size_t)(n_exp * egu));
    if (dw_up) memset(dw_up, 0, sizeof(double) * (size_t)(n_exp * egu));
    if (dw_down) memset(dw_down, 0, sizeof(double) * (size_t)(n_exp * egu));
  }
  if (ds > 0) {
    if (dws_gate) memset(dws_gate, 0, sizeof(double) * (size_t)ds * d);
    if (dws_up) memset(dws_up, 0, sizeof(double) * (size_t)ds * d);
    if (dws_down) memset(dws_down, 0, sizeof(double) * (size_t)ds * d);
  }
  if (L->latent) {
    if (dw_lat_down) memset(dw_lat_down, 0, sizeof(double) * (size_t)de * d);
    if (dw_lat_up) memset(dw_lat_up, 0, sizeof(double) * (size_t)de * d);
    if (d_rms_gamma) memset(d_rms_gamma, 0, sizeof(double) * (size_t)de);
  }
#pragma omp parallel for schedule(dynamic, 1) if (!serial)
  for (int64_t j = 0; j < n; ++j) {
    const int64_t t = tokens ? tokens[j] : j;
    const int fm = f > ds ? f : ds;
    double *xv = (double *)malloc(sizeof(double) * (size_t)d);
    double *dv = (double *)calloc((size_t)d, sizeof(double));
    double *buf = (double *)malloc(sizeof(double) * (size_t)(4 * (fm > 0 ? fm : 1)));
    double *g = (double *)malloc(sizeof(double) * (size_t)K * 2);
    double *dg = g + K;
    double *dr = (double *)malloc(sizeof(double) * (size_t)E);
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    /* routed input and its gradient (latent: z = W_lat_down x, else x) */
    double *zv = (double *)malloc(sizeof(double) * (size_t)de);
    double *dz = (double *)calloc((size_t)de, sizeof(double));
    double *dR = (double *)malloc(sizeof(double) * (size_t)de);
    double gap;
    const double *dy = d_out + j * d;
    load_row(W->x, L->act, t, d, xv);
    route_one(L, W, xv, idx_override ? idx_override + j * K : NULL, idx, g, &gap, NULL);
    if (L->latent) {
      /* StableLatentMoE "Return to model width": y = W_lat_up R' + shared,
       * R' = R / sqrt(mean(R^2) + eps) * gamma (or R' = R without the norm),
       * R = sum_k g_k FFN_{e_k}(z), z = W_lat_down x. */
      for (int l = 0; l < de; ++l) zv[l] = dot(W->w_lat_down, L->act, (int64_t)l * d, xv, d);
      double *R = (double *)calloc((size_t)de, sizeof(double));
      double *hb = (double *)malloc(sizeof(double) * (size_t)f);
      for (int k = 0; k < K; ++k) {
        const int64_t e = idx[k];
        swiglu_acc(W->w_gate, W->w_up, W->w_down, L->act, e * egu, e * egu, de, f, zv, g[k], R,
                   hb);
      }
      double inv = 1.0;
      if (L->has_rmsnorm) {
        double ms = 0.0;
        for (int l = 0; l < de; ++l) ms += R[l] * R[l];
        inv = 1.0 / sqrt(ms / de + L->rms_eps);
      }
      /* dR' = W_lat_up^T dy; dW_lat_up += dy R'^T */
      double sR = 0.0;
      for (int l = 0; l < de; ++l) {
        double s2 = 0.0;
        for (int i = 0; i < d; ++i) s2 += ld(W->w_lat_up, L->act, (int64_t)i * de + l) * dy[i];
        const double gam = (L->has_rmsnorm && W->rms_gamma) ? (double)W->rms_gamma[l] : 1.0;
        const double Rn = L->has_rmsnorm ? R[l] * inv * gam : R[l];
        if (dw_lat_up)
          for (int i = 0; i < d; ++i) dw_lat_up[(int64_t)i * de + l] += dy[i] * Rn;
        if (L->has_rmsnorm && d_rms_gamma) d_rms_gamma[l] += s2 * R[l] * inv;
        dR[l] = L->has_rmsnorm ? s2 * gam : s2; /* gamma-weighted dR' for the norm */
        sR += dR[l] * R[l];
      }
      /* RMSNorm: dR = inv (gamma dR') - R inv^3 <gamma dR', R> / L */
      if (L->has_rmsnorm)
        for (int l = 0; l < de; ++l) dR[l] = inv * dR[l] - R[l] * inv * inv * inv * sR / de;
      free(hb);
      free(R);
    } else {
      memcpy(zv, xv, sizeof(double) * (size_t)d);
      memcpy(dR, dy, sizeof(double) * (size_t)d);
    }
    for (int k = 0; k < K; ++k) {
      const int64_t e = idx[k];
      const int mine = want_w && (want_expert == -1 || want_expert == e);
      const int64_t wo = want_expert == -1 ? e * egu : 0;
      dg[k] = swiglu_backward(W->w_gate, W->w_up, W->w_down, L->act, e * egu, e * egu, de, f, zv,
                              dR, g[k], L->latent ? dz : dv,
                              mine && dw_gate ? dw_gate + wo : NULL,
                              mine && dw_up ? dw_up + wo : NULL,
                              mine && dw_down ? dw_down + wo : NULL, buf);
    }
    if (L->latent) { /* dx += W_lat_down^T dz; dW_lat_down += dz x^T */
      for (int l = 0; l < de; ++l) {
        for (int i = 0; i < d; ++i) {
          dv[i] += ld(W->w_lat_down, L->act, (int64_t)l * d + i) * dz[l];
          if (dw_lat_down) dw_lat_down[(int64_t)l * d + i] += dz[l] * xv[i];
        }
      }
    }
    if (ds > 0)
      swiglu_backward(W->ws_gate, W->ws_up, W->ws_down, L->act, 0, 0, d, ds, xv, dy, 1.0, dv,
                      dws_gate, dws_up, dws_down, buf);
    route_grad(L, W, xv, idx, dg, dr);
    for (int e = 0; e < E; ++e) {
      if (dr[e] == 0.0) continue;
      for (int i = 0; i < d; ++i) {
        dv[i] += (double)W->w_router[(int64_t)e * d + i] * dr[e];
        if (dw_router) dw_router[(int64_t)e * d + i] += dr[e] * xv[i];
      }
    }
    if (dx) memcpy(dx + j * d, dv, sizeof(double) * (size_t)d);
    free(dR);
    free(dz);
    free(zv);
    free(idx);
    free(dr);
    free(g);
    free(buf);
    free(dv);
    free(xv);
  }
  return 0;
}
