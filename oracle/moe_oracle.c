/*
 * moe_oracle.c -- plain fp64 CPU reference of the MoE decode layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or its library: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * helper with the HIP library; it reads the same stored bytes and decodes
 * them itself.
 *
 * What it computes (the layer of MoeLayer::forward, forward.rs, and of the
 * token-major N-row decode, forward_token_major.rs, in their step order:
 * router gate product -> top-k -> expert gate+up -> act(gate)*up -> down ->
 * weighted sum + shared expert):
 *
 *   logits[t,e] = sum_i x[t,i] * W[e,i]
 *   softmax scoring: key_e = logits_e; p = softmax over all E;
 *       w_j = p_sel_j / sum_sel p   (norm_topk)   or   p_sel_j
 *   sigmoid scoring: key_e = sigmoid(logits_e) + bias_e (bias selects only);
 *       w_j = s_j / sum_sel s        (norm_topk)   or   s_j,  s_j = sigmoid(l_sel_j)
 *   every w_j is then multiplied by routed_scaling
 *   the k largest keys are selected, ties to the lowest expert index, slots
 *   in descending key order
 *   y(e, v) = Wd_e * ( silu(Wg_e v) .* (Wu_e v) ),  silu(z) = z * sigmoid(z)
 *   out[t] = sum_j w[t,j] * y(idx[t,j], x_t)  +  g_t * y_shared(x_t),
 *       g_t = sigmoid(x_t . gate_vec) with a gate vector, else 1
 *       (the weighted-sum blend described in forward.rs beside
 *        moe_weighted_sum_blend)
 *   zero-computation experts (forward.rs: the zero-expert step of the layer;
 *   forward_token_major.rs: a router wider than num_experts): the router has
 *   E + Z rows, scoring and top-k run over all E + Z logits, and a pick
 *   e >= E computes nothing and passes its input row through:
 *   y(e, v) = v for E <= e < E + Z
 *   hash routing instead of top-k (forward.rs): the experts of row t are
 *   tid2eid[token_id[t]], weighted by sqrt(softplus(logit)) at them,
 *   renormalised if norm_topk, times routed_scaling
 *   optional pre-norms (forward.rs: the router's input and the
 *   pre_expert_norm step): rmsnorm(x)[t,i] = x[t,i] * w[i] / sqrt(mean x_t^2
 *   + eps), one weight vector for the router's input, another for the
 *   experts' input; the shared-expert gate keeps the layer's own input
 *
 * Every stored value is decoded exactly to double; all sums run in double in
 * index order.  Weight bytes are stored in tiles of 16 rows x 64 bytes (see
 * tiled_at); scales are row-major.  Formats:
 *   F32, BF16            plain IEEE / bfloat16 (top 16 bits of an fp32)
 *   FP8_B128             OCP E4M3 'fn' codes; value = code * s[r/128][c/128]
 *                        with fp32 scales, row-major [ceil(R/128), ceil(C/128)]
 *   MXFP4                OCP MX v1.0: e2m1 codes, two per byte, element 2i in
 *                        the low nibble; value = code * 2^(E-127), E the u8
 *                        scale of the 32-element block, scales [R, C/32]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_B128 = 2, ORC_MXFP4 = 3 };
enum { ORC_SOFTMAX = 0, ORC_SIGMOID = 1 };

typedef struct {
  int hidden, num_experts, top_k, inter, shared_inter;
  int scoring, norm_topk;
  double routed_scaling;
  int act_fmt;    /* ORC_F32 or ORC_BF16: x, router, gate vector */
  int expert_fmt; /* ORC_F32 .. ORC_MXFP4 */
  int zero_experts; /* Z: ids E .. E+Z-1 are zero-computation experts */
} orc_cfg;

/* ---------------------------------------------------------------- decode */

double orc_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP 8-bit floating point spec, E4M3: bias 7, no infinities,
 * S.1111.111 is NaN, exponent field 0 is subnormal. */
double orc_fp8_e4m3(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, 1 - 7);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

/* OCP MX v1.0, E2M1: bias 1, exponent field 0 is subnormal (0 or 0.5). */
double orc_e2m1(uint8_t nib) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double v;
  if (e == 0)
    v = 0.5 * (double)m;
  else
    v = ldexp(1.0 + 0.5 * (double)m, e - 1);
  return s ? -v : v;
}

/* OCP MX v1.0, E8M0 scale: 2^(E-127), 0xFF is NaN. */
double orc_e8m0(uint8_t b) {
  if (b == 255) return NAN;
  return ldexp(1.0, (int)b - 127);
}

static double act_at(int fmt, const void *p, size_t i) {
  if (fmt == ORC_F32) return (double)((const float *)p)[i];
  return orc_bf16(((const uint16_t *)p)[i]);
}

/* Where byte b of row r of a matrix with rb bytes per row lives in the
 * storage layout of expert weights: tiles of 16 rows x 64 bytes.  Rows come
 * in groups of 16, each group 16 rb contiguous bytes; inside a group, tile
 * column t holds bytes [64 t, 64 t + 64) of the 16 rows, row after row,
 * tile columns in order; a last tile column narrower than 64 bytes (rb % 64)
 * holds its 16 rows the same way.  (Rows a multiple of 16, rb of 16.) */
static size_t tiled_at(int r, size_t b, size_t rb) {
  const size_t full = rb / 64, t = b / 64;
  const size_t width = t < full ? 64 : rb % 64;
  return (size_t)(r / 16) * 16 * rb + t * 16 * 64 + (size_t)(r % 16) * width + b % 64;
}

/* element (r, c) of an R x C weight matrix in storage format fmt (weights
 * tiled, scales row-major) */
static double weight_at(int fmt, const void *w, const void *s, int R, int C,
                        int r, int c) {
  (void)R;
  const uint8_t *wb = (const uint8_t *)w;
  switch (fmt) {
    case ORC_F32: {
      float f;
      memcpy(&f, wb + tiled_at(r, (size_t)c * 4, (size_t)C * 4), 4);
      return (double)f;
    }
    case ORC_BF16: {
      uint16_t h;
      memcpy(&h, wb + tiled_at(r, (size_t)c * 2, (size_t)C * 2), 2);
      return orc_bf16(h);
    }
    case ORC_FP8_B128: {
      int bc = (C + 127) / 128;
      double q = orc_fp8_e4m3(wb[tiled_at(r, (size_t)c, (size_t)C)]);
      return q * (double)((const float *)s)[(size_t)(r / 128) * bc + c / 128];
    }
    case ORC_MXFP4: {
      uint8_t byte = wb[tiled_at(r, (size_t)c / 2, (size_t)C / 2)];
      uint8_t nib = (c & 1) ? (byte >> 4) : (byte & 15);
      return orc_e2m1(nib) * orc_e8m0(((const uint8_t *)s)[(size_t)r * (C / 32) + c / 32]);
    }
  }
  return NAN;
}

/* Decode a whole R x C matrix to double (row-major). */
int orc_dequant(int fmt, int R, int C, const void *w, const void *s, double *out) {
  if (fmt == ORC_MXFP4 && C % 32) return -1;
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int r = 0; r < R; r++)
    for (int c = 0; c < C; c++) out[(size_t)r * C + c] = weight_at(fmt, w, s, R, C, r, c);
  return 0;
}

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ---------------------------------------------------------------- router */

/* logits[N,E] = x[N,h] . W[E,h]^T */
void orc_router_logits(int act_fmt, int N, int h, int E, const void *x, const void *W,
                       double *logits) {
  for (int t = 0; t < N; t++)
    for (int e = 0; e < E; e++) {
      double acc = 0.0;
      for (int i = 0; i < h; i++)
        acc += act_at(act_fmt, x, (size_t)t * h + i) * act_at(act_fmt, W, (size_t)e * h + i);
      logits[(size_t)t * E + e] = acc;
    }
}

/* Selection keys of one row: the logit (softmax) or sigmoid(logit) + bias. */
void orc_keys(int E, int scoring, const double *logits, const float *bias, double *keys) {
  for (int e = 0; e < E; e++)
    keys[e] = scoring == ORC_SIGMOID
                  ? sigmoid(logits[e]) + (bias ? (double)bias[e] : 0.0)
                  : logits[e];
}

/* Routing weights of k given picks of one row (the weight half of the
 * scored top-k, forward_token_major.rs: moe_topk_softmax_batched /
 * moe_topk_sigmoid_batched):
 *   softmax: p_e = exp(l_e - max l) / sum over all E of exp(l - max l)
 *   sigmoid: p_e = sigmoid(l_e)          (no correction bias in the weight)
 *   w_j = p_{idx_j} / sum_j p_{idx_j} if norm, else p_{idx_j}; then w_j *= rsf.
 * The picks need not be the top-k: this also weights a near-tie pick that
 * differs from this oracle's own selection.  -1 if a pick is outside [0, E). */
int orc_route_weights(int E, int k, int scoring, int norm, double rsf, const double *logits,
                      const int *idx, double *w) {
  if (k < 1 || k > E) return -1;
  for (int j = 0; j < k; j++)
    if (idx[j] < 0 || idx[j] >= E) return -1;
  if (scoring == ORC_SOFTMAX) {
    double m = logits[0];
    for (int e = 1; e < E; e++)
      if (logits[e] > m) m = logits[e];
    double z = 0.0;
    for (int e = 0; e < E; e++) z += exp(logits[e] - m);
    for (int j = 0; j < k; j++) w[j] = exp(logits[idx[j]] - m) / z;
  } else {
    for (int j = 0; j < k; j++) w[j] = sigmoid(logits[idx[j]]);
  }
  if (norm) {
    double s = 0.0;
    for (int j = 0; j < k; j++) s += w[j];
    for (int j = 0; j < k; j++) w[j] /= s;
  }
  for (int j = 0; j < k; j++) w[j] *= rsf;
  return 0;
}

/* Top-k of one row plus its weights.  Slot j holds the largest key not yet
 * taken; a later index replaces the current best only with a strictly larger
 * key, so equal keys go to the lowest index.  The weights are those of
 * orc_route_weights at the picks. */
int orc_topk_row(int E, int k, int scoring, int norm, double rsf, const double *logits,
                 const float *bias, int *idx, double *w) {
  double *keys = (double *)malloc(sizeof(double) * E);
  char *taken = (char *)calloc(E, 1);
  if (!keys || !taken || k < 1 || k > E) {
    free(keys);
    free(taken);
    return -1;
  }
  orc_keys(E, scoring, logits, bias, keys);
  for (int j = 0; j < k; j++) {
    int best = -1;
    for (int e = 0; e < E; e++) {
      if (taken[e]) continue;
      if (best < 0 || keys[e] > keys[best]) best = e;
    }
    idx[j] = best;
    taken[best] = 1;
  }
  free(keys);
  free(taken);
  return orc_route_weights(E, k, scoring, norm, rsf, logits, idx, w);
}

/* ---------------------------------------------------------------- experts */

/* One expert's three matrices decoded to double: Wg, Wu (I x h) and
 * Wd (h x I), row-major.  Returns 0, or -1 if memory runs out. */
typedef struct {
  double *g, *u, *d;
} orc_mats;

static void free_mats(orc_mats *m) {
  free(m->g);
  free(m->u);
  free(m->d);
  m->g = m->u = m->d = NULL;
}

/* room for the matrices of an expert of width up to I */
static int alloc_mats(int h, int I, orc_mats *m) {
  m->g = (double *)malloc(sizeof(double) * (size_t)I * h);
  m->u = (double *)malloc(sizeof(double) * (size_t)I * h);
  m->d = (double *)malloc(sizeof(double) * (size_t)h * I);
  if (!m->g || !m->u || !m->d) {
    free_mats(m);
    return -1;
  }
  return 0;
}

static int load_mats(int fmt, int h, int I, const void *wg, const void *sg, const void *wu,
                     const void *su, const void *wd, const void *sd, orc_mats *m) {
  if (orc_dequant(fmt, I, h, wg, sg, m->g) || orc_dequant(fmt, I, h, wu, su, m->u) ||
      orc_dequant(fmt, h, I, wd, sd, m->d))
    return -1;
  return 0;
}

/* y[h] = Wd (silu(Wg v) .* (Wu v)) for one input row v[h], on decoded
 * matrices; a[I] is scratch.  Every dot product sums in index order (the
 * threads split output elements, never a sum). */
static void mlp64(int h, int I, const orc_mats *m, const double *v, double *a, double *y) {
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int i = 0; i < I; i++) {
    const double *gr = m->g + (size_t)i * h, *ur = m->u + (size_t)i * h;
    double g = 0.0, u = 0.0;
    for (int c = 0; c < h; c++) {
      g += gr[c] * v[c];
      u += ur[c] * v[c];
    }
    a[i] = g * sigmoid(g) * u;
  }
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
  for (int r = 0; r < h; r++) {
    const double *dr = m->d + (size_t)r * I;
    double acc = 0.0;
    for (int i = 0; i < I; i++) acc += dr[i] * a[i];
    y[r] = acc;
  }
}

/* y[h] = Wd (silu(Wg v) .* (Wu v)) for one input row v[h] (double).
 * Wg, Wu: I x h; Wd: h x I; all in format fmt with their scales. */
int orc_expert_mlp(int fmt, int h, int I, const double *v, const void *wg, const void *sg,
                   const void *wu, const void *su, const void *wd, const void *sd,
                   double *y) {
  orc_mats m;
  double *a = (double *)malloc(sizeof(double) * I);
  if (!a || alloc_mats(h, I, &m)) {
    free(a);
    return -1;
  }
  if (load_mats(fmt, h, I, wg, sg, wu, su, wd, sd, &m)) {
    free_mats(&m);
    free(a);
    return -1;
  }
  mlp64(h, I, &m, v, a, y);
  free_mats(&m);
  free(a);
  return 0;
}

/* Hash routing of one row (forward.rs, the hash-routing branch of the top-k
 * step: a row's experts are the static table row of its token id, weighted
 * by the gate's sqrtsoftplus scores): for j < k, e_j = eids[j];
 *   s_j = sqrt(softplus(logit[e_j])),  softplus(z) = log(1 + exp(z)),
 * an entry outside [0, E) is dropped (s_j = 0);
 *   w_j = s_j / sum_j s_j (norm_topk; 0 if every entry is dropped) or s_j,
 * then w_j *= routed_scaling. */
int orc_hash_route_row(int E, int k, int norm, double rsf, const double *logits, const int *eids,
                       double *w) {
  if (k < 1) return -1;
  double sum = 0.0;
  for (int j = 0; j < k; j++) {
    const int e = eids[j];
    double sj = 0.0;
    if (e >= 0 && e < E) {
      const double z = logits[e];
      const double sp = z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));
      sj = sqrt(sp);
    }
    w[j] = sj;
    sum += sj;
  }
  for (int j = 0; j < k; j++) {
    if (norm) w[j] = sum > 0.0 ? w[j] / sum : 0.0;
    w[j] *= rsf;
  }
  return 0;
}

/* RMSNorm of N rows of h values (x and w in act format), unrounded:
 *   out[t,i] = x[t,i] * w[i] / sqrt((1/h) sum_i x[t,i]^2 + eps)
 * (forward.rs: the pre_expert_norm step runs rms_norm with the layer's
 * rms_norm_eps over the layer input; the router's pre-norm is the same
 * operation with its own weights). */
int orc_rmsnorm(int act_fmt, int N, int h, const void *x, const void *w, double eps,
                double *out) {
  if (N < 1 || h < 1 || !(eps >= 0.0)) return -1;
  for (int t = 0; t < N; t++) {
    double ss = 0.0;
    for (int i = 0; i < h; i++) {
      const double v = act_at(act_fmt, x, (size_t)t * h + i);
      ss += v * v;
    }
    const double r = 1.0 / sqrt(ss / h + eps);
    for (int i = 0; i < h; i++)
      out[(size_t)t * h + i] = act_at(act_fmt, x, (size_t)t * h + i) * r * act_at(act_fmt, w, i);
  }
  return 0;
}

/* Routed + shared experts for N rows under a given routing.
 * gate/up/down(_s): host arrays of E host pointers (entries of experts no row
 * selects may be NULL).  sh_*: the shared expert (sh_gate NULL = none).
 * gate_vec: optional [h] in act format; gate_x: the rows the shared-expert
 * gate reads ([N,h] act format), NULL = x.  out[N,h] double. */
int orc_experts(const orc_cfg *c, int N, const void *x, const void *const *gate,
                const void *const *gate_s, const void *const *up, const void *const *up_s,
                const void *const *down, const void *const *down_s, const void *sh_gate,
                const void *sh_gate_s, const void *sh_up, const void *sh_up_s,
                const void *sh_down, const void *sh_down_s, const void *gate_vec,
                const void *gate_x, const int *idx, const double *w, double *out,
                int nthreads) {
  const int h = c->hidden, k = c->top_k, nr = N * k;
  const int has_sh = sh_gate != NULL && c->shared_inter > 0;
  const int amax = c->inter > c->shared_inter ? c->inter : c->shared_inter;
  double *xv = (double *)malloc(sizeof(double) * (size_t)N * h);
  double *yr = (double *)malloc(sizeof(double) * (size_t)nr * h);
  double *ys = has_sh ? (double *)malloc(sizeof(double) * (size_t)N * h) : NULL;
  double *a = (double *)malloc(sizeof(double) * (size_t)amax);
  orc_mats m;
  int err = 0;
  if (!xv || !yr || !a || (has_sh && !ys) || alloc_mats(h, amax, &m)) {
    free(xv); free(yr); free(ys); free(a);
    return -1;
  }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  for (size_t i = 0; i < (size_t)N * h; i++) xv[i] = act_at(c->act_fmt, x, i);
  for (int r = 0; r < nr; r++) {
    int e = idx[r];
    if (e >= c->num_experts && e < c->num_experts + c->zero_experts) {
      /* a zero-computation expert: no weights, its output is its input row */
      memcpy(yr + (size_t)r * h, xv + (size_t)(r / k) * h, sizeof(double) * h);
      continue;
    }
    if (e < 0 || e >= c->num_experts || !gate[e] || !up[e] || !down[e]) err = -2;
  }
  /* every selected expert is decoded once, then runs each of its routes */
  for (int e = 0; e < c->num_experts && !err; e++) {
    int used = 0;
    for (int r = 0; r < nr && !used; r++) used = idx[r] == e;
    if (!used) continue;
    if (load_mats(c->expert_fmt, h, c->inter, gate[e], gate_s ? gate_s[e] : NULL, up[e],
                  up_s ? up_s[e] : NULL, down[e], down_s ? down_s[e] : NULL, &m)) {
      err = -1;
      break;
    }
    for (int r = 0; r < nr; r++)
      if (idx[r] == e) mlp64(h, c->inter, &m, xv + (size_t)(r / k) * h, a, yr + (size_t)r * h);
  }
  if (has_sh && !err) {
    if (load_mats(c->expert_fmt, h, c->shared_inter, sh_gate, sh_gate_s, sh_up, sh_up_s, sh_down,
                  sh_down_s, &m)) {
      err = -1;
    } else {
      for (int t = 0; t < N; t++)
        mlp64(h, c->shared_inter, &m, xv + (size_t)t * h, a, ys + (size_t)t * h);
    }
  }
  free_mats(&m);
  if (err) {
    free(xv); free(yr); free(ys); free(a);
    return err;
  }
  for (int t = 0; t < N; t++) {
    double g = 1.0;
    if (has_sh && gate_vec) {
      double d = 0.0;
      for (int i = 0; i < h; i++)
        d += (gate_x ? act_at(c->act_fmt, gate_x, (size_t)t * h + i) : xv[(size_t)t * h + i]) *
             act_at(c->act_fmt, gate_vec, i);
      g = sigmoid(d);
    }
    for (int i = 0; i < h; i++) {
      double acc = 0.0;
      for (int j = 0; j < k; j++) acc += w[t * k + j] * yr[((size_t)t * k + j) * h + i];
      if (has_sh) acc += g * ys[(size_t)t * h + i];
      out[(size_t)t * h + i] = acc;
    }
  }
  free(xv); free(yr); free(ys); free(a);
  return 0;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
