/* Plain float64 CPU oracle of the routed Mixture-of-Experts FFN forward, in C.
 *
 * TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's cpu_baseline
 * leg load it; the GPU library never does. Contracts are in moe_ref.h.
 *
 * Every function is the plain definition of its step, written from the pages cited in
 * moe_ref.h: loops over tokens, experts and elements in float64, sums taken in index
 * order, values rounded to a storage format only where the pages put a rounding
 * (selection compares float32 keys; the gated activation is stored in the operand dtype
 * before the down projection; outputs are stored in their dtype). Where the pages leave
 * a point open the reading is the one stated at the function. Threads split independent
 * tokens or rows; no sum is split.
 */
#include "moe_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static __thread char g_err[256];
static int g_threads = 1;

const char* moe_ref_last_error(void) { return g_err; }

static int fail(const char* msg) {
  snprintf(g_err, sizeof g_err, "%s", msg);
  return -1;
}

int moe_ref_set_threads(int n) {
  if (n >= 1) g_threads = n;
  return g_threads;
}

/* ------------------------------------------------------------------ parallel loop */
typedef void (*item_fn)(void* ctx, int64_t i, double* scratch);
typedef struct {
  item_fn fn;
  void* ctx;
  int64_t n, next;
  size_t scratch_doubles;
  int failed;
} loop_t;

static void* worker(void* p) {
  loop_t* L = (loop_t*)p;
  double* scratch = L->scratch_doubles ? malloc(L->scratch_doubles * sizeof(double)) : NULL;
  if (L->scratch_doubles && !scratch) {
    __atomic_store_n(&L->failed, 1, __ATOMIC_SEQ_CST);
    return NULL;
  }
  for (;;) {
    const int64_t i = __atomic_fetch_add(&L->next, 1, __ATOMIC_SEQ_CST);
    if (i >= L->n) break;
    L->fn(L->ctx, i, scratch);
  }
  free(scratch);
  return NULL;
}

/* Calls fn(ctx, i, scratch) for i in [0, n) on g_threads threads; each thread owns a
 * scratch of scratch_doubles doubles. */
static int parallel_for(int64_t n, item_fn fn, void* ctx, size_t scratch_doubles) {
  loop_t L = {fn, ctx, n, 0, scratch_doubles, 0};
  int nt = g_threads;
  if (nt > n) nt = n > 0 ? (int)n : 1;
  pthread_t th[256];
  if (nt > 256) nt = 256;
  int started = 0;
  for (int k = 1; k < nt; ++k)
    if (pthread_create(&th[started], NULL, worker, &L) == 0) ++started;
  worker(&L);
  for (int k = 0; k < started; ++k) pthread_join(th[k], NULL);
  return L.failed ? fail("out of host memory") : 0;
}

/* ------------------------------------------------------------------ storage formats */
/* float16 bits to value: sign, 5-bit exponent (bias 15), 10-bit fraction; exponent 0
 * holds the subnormals f / 1024 * 2^-14, exponent 31 infinities and NaN. */
static double f16_value(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp(1024.0 + f, e - 25);
  return s ? -v : v;
}

/* bfloat16 bits are the upper half of a float32. */
static double bf16_value(uint16_t h) {
  const uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, sizeof f);
  return (double)f;
}

static inline double widen1(const void* p, int32_t fmt, int64_t i) {
  switch (fmt) {
    case MOE_REF_F64: return ((const double*)p)[i];
    case MOE_REF_F32: return (double)((const float*)p)[i];
    case MOE_REF_BF16: return bf16_value(((const uint16_t*)p)[i]);
    case MOE_REF_F16: return f16_value(((const uint16_t*)p)[i]);
  }
  return NAN;
}

void moe_ref_widen(const void* x, int32_t fmt, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen1(x, fmt, i);
}

static int fmt_ok(int32_t f) { return f >= MOE_REF_F64 && f <= MOE_REF_F16; }

/* Round to p significant bits (the implicit one included), smallest normal exponent
 * emin, largest exponent emax: scale so that the last kept bit is the units digit, round
 * to an integer with ties to even (nearbyint in the default rounding mode), scale back;
 * both scalings are exact. Subnormals keep the spacing of the smallest normal binade. */
double moe_ref_round(double x, int32_t fmt) {
  int p, emin, emax;
  switch (fmt) {
    case MOE_REF_F32: p = 24; emin = -126; emax = 127; break;
    case MOE_REF_BF16: p = 8; emin = -126; emax = 127; break;
    case MOE_REF_F16: p = 11; emin = -14; emax = 15; break;
    default: return x;
  }
  if (!isfinite(x) || x == 0.0) return x;
  int e;
  frexp(x, &e);                 /* |x| in [2^(e-1), 2^e) */
  int q = e - p;                /* weight of the last kept bit */
  if (q < emin - p + 1) q = emin - p + 1;
  const double r = ldexp(nearbyint(ldexp(x, -q)), q);
  const double maxv = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
  return fabs(r) > maxv ? copysign(INFINITY, r) : r;
}

void moe_ref_round_array(const double* x, int64_t n, int32_t fmt, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = moe_ref_round(x[i], fmt);
}

/* ------------------------------------------------------------------ scoring */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* [MR] MoERouter scoring of one row of E logits.
 * softmax: exp(z_e - max) / sum_j exp(z_j - max); sigmoid: 1 / (1 + exp(-z));
 * sqrt_softplus (the page only names it; reading: the square root of softplus):
 * sqrt(max(z, 0) + log1p(exp(-|z|))). */
static void score_row(const void* logits, int32_t fmt, int64_t row, int64_t E, int32_t scoring,
                      double* s) {
  const int64_t base = row * E;
  if (scoring == MOE_REF_SOFTMAX) {
    double mx = -INFINITY;
    for (int64_t e = 0; e < E; ++e) {
      const double z = widen1(logits, fmt, base + e);
      if (z > mx) mx = z;
    }
    double sum = 0.0;
    for (int64_t e = 0; e < E; ++e) {
      s[e] = exp(widen1(logits, fmt, base + e) - mx);
      sum += s[e];
    }
    for (int64_t e = 0; e < E; ++e) s[e] /= sum;
  } else if (scoring == MOE_REF_SIGMOID) {
    for (int64_t e = 0; e < E; ++e) s[e] = sigmoid(widen1(logits, fmt, base + e));
  } else {
    for (int64_t e = 0; e < E; ++e) {
      const double z = widen1(logits, fmt, base + e);
      s[e] = sqrt(fmax(z, 0.0) + log1p(exp(-fabs(z))));
    }
  }
}

int moe_ref_scores(const void* logits, int32_t logits_fmt, int64_t T, int64_t E,
                   int32_t scoring, double* scores) {
  if (!fmt_ok(logits_fmt) || scoring < 0 || scoring > 2 || E < 1) return fail("bad scores args");
  for (int64_t t = 0; t < T; ++t) score_row(logits, logits_fmt, t, E, scoring, scores + t * E);
  return 0;
}

/* a ranks before b: larger value, or equal value and lower index ([MR]: ties go to the
 * lower expert index; [TO] FusedTopKFwdOp: ties between groups to the lower group). */
static int before(double va, int64_t a, double vb, int64_t b) {
  return va > vb || (va == vb && a < b);
}

void moe_ref_ranked(const double* v, int64_t n, int64_t* order) {
  /* selection order: position j takes the best of the values not yet placed */
  char* used = calloc((size_t)(n > 0 ? n : 1), 1);
  for (int64_t j = 0; j < n; ++j) {
    int64_t best = -1;
    for (int64_t i = 0; i < n; ++i)
      if (!used[i] && (best < 0 || before(v[i], i, v[best], best))) best = i;
    used[best] = 1;
    order[j] = best;
  }
  free(used);
}

/* ------------------------------------------------------------------ router */
typedef struct {
  const moe_ref_route_cfg* c;
  const void* logits;
  int32_t fmt;
  const double* bias;   /* E values rounded to float32, or NULL */
  const int64_t* ids;   /* hash routing, or NULL */
  const double* given;  /* scores given instead of logits, or NULL */
  double *scores, *wn, *w, *keys, *gscores, *gap_sel, *gap_group;
  int64_t* topk_ids;
} route_ctx;

/* Route row `row` of the logits into the outputs at row `slot`. Scratch: 3E + 2G doubles.
 * [MR] MoERouter (selection topk / noaux_tc), [TO] FusedTopKFwdOp and FusedMoEFwdOp
 * (DeepSeek-V3 grouped routing):
 *   u_e = f32(s_e), or f32(f32(s_e) + f32(bias_e)) with a bias;
 *   group g (E/G consecutive experts) scores f32(best u + second best u) with a bias
 *   (its single u for groups of one), its best u without;
 *   the topk_group best groups stay eligible; the K best eligible keys are chosen, in
 *   (key descending, index ascending) order;
 *   weights: the unbiased scores of the chosen experts, divided by their sum when
 *   renormalize is set (no epsilon: the pages give none), then times
 *   routed_scaling_factor (once), stored as float32. */
static int route_row(const route_ctx* x, int64_t row, int64_t slot, double* scratch) {
  const moe_ref_route_cfg* c = x->c;
  const int64_t E = c->E, K = c->K, G = c->num_expert_group > 1 ? c->num_expert_group : 1;
  const int64_t TG = c->topk_group, gsz = E / G;
  double* s = scratch;
  double* u = s + E;
  double* elig = u + E;        /* 1 for eligible experts */
  double* gs = elig + E;       /* G group scores */
  double* gtaken = gs + G;
  if (x->given) memcpy(s, x->given + row * E, (size_t)E * sizeof(double));
  else score_row(x->logits, x->fmt, row, E, c->scoring, s);
  for (int64_t e = 0; e < E; ++e) {
    const double s32 = moe_ref_round(s[e], MOE_REF_F32);
    u[e] = x->bias ? moe_ref_round(s32 + x->bias[e], MOE_REF_F32) : s32;
  }
  if (x->scores) memcpy(x->scores + slot * E, s, (size_t)E * sizeof(double));
  if (x->keys) memcpy(x->keys + slot * E, u, (size_t)E * sizeof(double));
  int64_t* ids = x->topk_ids + slot * K;
  double gap_sel = INFINITY, gap_group = INFINITY;

  for (int64_t g = 0; g < G; ++g) {
    const double* ug = u + g * gsz;
    if (x->bias && gsz >= 2) {
      int64_t b1 = 0;
      for (int64_t i = 1; i < gsz; ++i) if (ug[i] > ug[b1]) b1 = i;
      int64_t b2 = b1 == 0 ? 1 : 0;
      for (int64_t i = 0; i < gsz; ++i) if (i != b1 && ug[i] > ug[b2]) b2 = i;
      gs[g] = moe_ref_round(ug[b1] + ug[b2], MOE_REF_F32);
    } else {
      double m = ug[0];
      for (int64_t i = 1; i < gsz; ++i) if (ug[i] > m) m = ug[i];
      gs[g] = m;
    }
    gtaken[g] = 0.0;
  }
  if (x->gscores && G > 1) memcpy(x->gscores + slot * G, gs, (size_t)G * sizeof(double));

  if (x->ids) {
    for (int64_t k = 0; k < K; ++k) {
      ids[k] = x->ids[row * K + k];
      if (ids[k] < 0 || ids[k] >= E) return -1;
    }
  } else {
    for (int64_t e = 0; e < E; ++e) elig[e] = G > 1 ? 0.0 : 1.0;
    if (G > 1) {
      int64_t last = -1;
      for (int64_t j = 0; j <= TG && j < G; ++j) {
        int64_t best = -1;
        for (int64_t g = 0; g < G; ++g)
          if (gtaken[g] == 0.0 && (best < 0 || before(gs[g], g, gs[best], best))) best = g;
        if (j == TG) {          /* the first group left out */
          gap_group = gs[last] - gs[best];
          break;
        }
        gtaken[best] = 1.0;
        last = best;
        for (int64_t i = 0; i < gsz; ++i) elig[best * gsz + i] = 1.0;
      }
    }
    double prev = 0.0;
    for (int64_t j = 0; j <= K; ++j) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; ++e)
        if (elig[e] == 1.0 && (best < 0 || before(u[e], e, u[best], best))) best = e;
      if (best < 0) {
        if (j < K) return -2;   /* fewer eligible experts than top_k */
        break;
      }
      if (j > 0 && prev - u[best] < gap_sel) gap_sel = prev - u[best];
      prev = u[best];
      if (j == K) break;
      ids[j] = best;
      elig[best] = 2.0;         /* taken */
    }
  }
  double sum = 0.0;
  for (int64_t k = 0; k < K; ++k) sum += s[ids[k]];
  for (int64_t k = 0; k < K; ++k) {
    const double wn = c->renormalize ? s[ids[k]] / sum : s[ids[k]];
    if (x->wn) x->wn[slot * K + k] = wn;
    x->w[slot * K + k] = moe_ref_round(wn * c->routed_scaling_factor, MOE_REF_F32);
  }
  if (x->gap_sel) x->gap_sel[slot] = gap_sel;
  if (x->gap_group) x->gap_group[slot] = gap_group;
  return 0;
}

static int route_cfg_ok(const moe_ref_route_cfg* c) {
  const int64_t G = c->num_expert_group > 1 ? c->num_expert_group : 1;
  if (c->E < 1 || c->K < 1 || c->scoring < 0 || c->scoring > 2) return 0;
  if (c->E % G) return 0;
  if (G > 1 && (c->topk_group < 1 || c->topk_group > G || c->topk_group * (c->E / G) < c->K))
    return 0;
  return c->K <= c->E;
}

static size_t route_scratch(const moe_ref_route_cfg* c) {
  const int64_t G = c->num_expert_group > 1 ? c->num_expert_group : 1;
  return (size_t)(3 * c->E + 2 * G);
}

static double* rounded_bias(const double* bias, int64_t E) {
  if (!bias) return NULL;
  double* b = malloc((size_t)E * sizeof(double));
  if (b) for (int64_t e = 0; e < E; ++e) b[e] = moe_ref_round(bias[e], MOE_REF_F32);
  return b;
}

int moe_ref_route(const moe_ref_route_cfg* c, const void* logits, int32_t logits_fmt,
                  int64_t T, const double* correction_bias, const int64_t* expert_ids,
                  double* scores, int64_t* topk_ids, double* wn, double* w, double* keys,
                  double* group_scores, double* gap_sel, double* gap_group) {
  if (!route_cfg_ok(c) || !fmt_ok(logits_fmt) || T < 0) return fail("bad route config");
  double* b = rounded_bias(correction_bias, c->E);
  double* scratch = malloc(route_scratch(c) * sizeof(double));
  route_ctx x = {c, logits, logits_fmt, b, expert_ids, NULL, scores, wn, w,
                 keys, group_scores, gap_sel, gap_group, topk_ids};
  int rc = scratch ? 0 : fail("out of host memory");
  for (int64_t t = 0; t < T && rc == 0; ++t)
    if (route_row(&x, t, t, scratch)) rc = fail("expert id out of range or too few eligible");
  free(scratch);
  free(b);
  return rc;
}

int moe_ref_select_experts(const moe_ref_route_cfg* c, const double* scores, int64_t T,
                           const double* correction_bias, int64_t* topk_ids, double* gap_sel,
                           double* gap_group) {
  if (!route_cfg_ok(c) || T < 0) return fail("bad route config");
  double* b = rounded_bias(correction_bias, c->E);
  double* scratch = malloc(route_scratch(c) * sizeof(double));
  double* w = malloc((size_t)(T * c->K > 0 ? T * c->K : 1) * sizeof(double));
  int rc = scratch && w ? 0 : fail("out of host memory");
  for (int64_t t = 0; t < T && rc == 0; ++t) {
    route_ctx x = {c, NULL, MOE_REF_F64, b, NULL, scores, NULL, NULL, w, NULL, NULL,
                   gap_sel, gap_group, topk_ids};
    if (route_row(&x, t, t, scratch)) rc = fail("too few eligible experts");
  }
  free(w);
  free(scratch);
  free(b);
  return rc;
}

int moe_ref_ep_outputs(const int64_t* topk_ids, const double* wn, int64_t T, int64_t K,
                       double routed_scaling_factor, int64_t start, int64_t count,
                       int32_t fmt, double* router_probs, double* weight_scale) {
  if (!fmt_ok(fmt) || count < 0) return fail("bad ep args");
  const double fill = fmt == MOE_REF_F16 ? -1.0e4 : -1.0e30;
  for (int64_t t = 0; t < T; ++t) {
    double* row = router_probs + t * count;
    for (int64_t j = 0; j < count; ++j) row[j] = fill;
    double local = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t e = topk_ids[t * K + k];
      if (e >= start && e < start + count) {
        row[e - start] = log(wn[t * K + k]);
        local += wn[t * K + k];
      }
    }
    for (int64_t j = 0; j < count; ++j) row[j] = moe_ref_round(row[j], fmt);
    weight_scale[t] = moe_ref_round(routed_scaling_factor * local, fmt);
  }
  return 0;
}

/* ------------------------------------------------------------------ gated activation */
/* swiglu: G sigmoid(alpha G) (L + beta) with G = min(g, limit), L = clamp(l, -limit,
 * limit); limit <= 0 turns both clamps off. gelu: gelu(g) l with the exact GELU
 * x Phi(x) = x (1 + erf(x / sqrt 2)) / 2 (the page names gelu_and_mul only; the exact
 * form is the reading taken). */
double moe_ref_gated(const moe_ref_act* a, double g, double l) {
  if (a->kind == MOE_REF_GELU) return 0.5 * g * (1.0 + erf(g / sqrt(2.0))) * l;
  if (a->limit > 0.0) {
    if (g > a->limit) g = a->limit;
    if (l > a->limit) l = a->limit;
    if (l < -a->limit) l = -a->limit;
  }
  return g * sigmoid(a->alpha * g) * (l + a->beta);
}

void moe_ref_gated_array(const moe_ref_act* a, const double* g, const double* l, int64_t n,
                         double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = moe_ref_gated(a, g[i], l[i]);
}

/* Gate and up halves of output j of a [2F] product: [TO] MoEGroupedGemmFwdOp and [SPEC]
 * Fusion Behavior (stacked: j and F + j; interleaved: 2j and 2j + 1). */
static void gate_up_at(int32_t layout, int64_t F, int64_t j, int64_t* gi, int64_t* ui) {
  if (layout == MOE_REF_INTERLEAVED) { *gi = 2 * j; *ui = 2 * j + 1; }
  else { *gi = j; *ui = F + j; }
}

/* One expert on one row: h = Wgu x (+ b_gu) over 2F rows of H, a = act(h) rounded to
 * act_fmt, y = Wd a (+ b_d) over N rows of F. Scratch h: 2F doubles. */
static void expert_row(const void* x, int64_t xrow, int64_t H, int64_t F, int64_t N,
                       const void* wgu, const void* wd, const void* bgu, const void* bd,
                       int64_t e, int32_t fmt, const moe_ref_act* act, int32_t act_fmt,
                       double* h, double* a, double* y) {
  const int64_t wgu0 = e * 2 * F * H, wd0 = e * N * F;
  for (int64_t j = 0; j < 2 * F; ++j) {
    double acc = 0.0;
    for (int64_t i = 0; i < H; ++i)
      acc += widen1(wgu, fmt, wgu0 + j * H + i) * widen1(x, fmt, xrow * H + i);
    h[j] = bgu ? acc + widen1(bgu, fmt, e * 2 * F + j) : acc;
  }
  for (int64_t j = 0; j < F; ++j) {
    int64_t gi, ui;
    gate_up_at(act->layout, F, j, &gi, &ui);
    a[j] = moe_ref_round(moe_ref_gated(act, h[gi], h[ui]), act_fmt);
  }
  for (int64_t o = 0; o < N; ++o) {
    double acc = 0.0;
    for (int64_t j = 0; j < F; ++j) acc += widen1(wd, fmt, wd0 + o * F + j) * a[j];
    y[o] = bd ? acc + widen1(bd, fmt, e * N + o) : acc;
  }
}

typedef struct {
  const void *x, *wgu, *wd, *bgu, *bd;
  int64_t H, F, N;
  int32_t fmt, act_fmt;
  const moe_ref_act* act;
  double *a, *y;
} mlp_ctx;

static void mlp_item(void* p, int64_t m, double* h) {
  const mlp_ctx* c = (const mlp_ctx*)p;
  expert_row(c->x, m, c->H, c->F, c->N, c->wgu, c->wd, c->bgu, c->bd, 0, c->fmt, c->act,
             c->act_fmt, h, c->a + m * c->F, c->y + m * c->N);
}

int moe_ref_expert_mlp(const void* x, int64_t M, int64_t H, int64_t F, int64_t N,
                       const void* w_gate_up, const void* w_down, const void* b_gate_up,
                       const void* b_down, int32_t fmt, const moe_ref_act* act,
                       int32_t act_fmt, double* a, double* y) {
  if (!fmt_ok(fmt) || !fmt_ok(act_fmt) || H < 1 || F < 1 || N < 1 || M < 0)
    return fail("bad mlp args");
  mlp_ctx c = {x, w_gate_up, w_down, b_gate_up, b_down, H, F, N, fmt, act_fmt, act, a, y};
  return parallel_for(M, mlp_item, &c, (size_t)(2 * F));
}

/* ------------------------------------------------------------------ grouped GEMM */
typedef struct {
  const void *a, *b, *bias;
  int64_t K, N, E;
  const int64_t* offsets;
  int32_t fmt, out_fmt;
  const moe_ref_act* act;
  double* out;
} gg_ctx;

static void gg_item(void* p, int64_t m, double* h) {
  const gg_ctx* c = (const gg_ctx*)p;
  const int64_t No = c->act ? c->N / 2 : c->N;
  double* o = c->out + m * No;
  int64_t e = -1;
  for (int64_t g = 0; g < c->E; ++g)
    if (m >= c->offsets[g] && m < c->offsets[g + 1]) { e = g; break; }
  if (e < 0) {
    for (int64_t n = 0; n < No; ++n) o[n] = 0.0;
    return;
  }
  for (int64_t n = 0; n < c->N; ++n) {
    double acc = 0.0;
    for (int64_t k = 0; k < c->K; ++k)
      acc += widen1(c->a, c->fmt, m * c->K + k) * widen1(c->b, c->fmt, (e * c->N + n) * c->K + k);
    h[n] = c->bias ? acc + widen1(c->bias, c->fmt, e * c->N + n) : acc;
  }
  for (int64_t n = 0; n < No; ++n) {
    double v = h[n];
    if (c->act) {
      int64_t gi, ui;
      gate_up_at(c->act->layout, No, n, &gi, &ui);
      v = moe_ref_gated(c->act, h[gi], h[ui]);
    }
    o[n] = moe_ref_round(v, c->out_fmt);
  }
}

int moe_ref_grouped_gemm(const void* a, int64_t M, int64_t K, const void* b, const void* bias,
                         int64_t E, int64_t N, const int64_t* offsets, int32_t fmt,
                         const moe_ref_act* act, int32_t out_fmt, double* out) {
  if (!fmt_ok(fmt) || !fmt_ok(out_fmt) || M < 0 || K < 1 || N < 1 || E < 1 || (act && N % 2))
    return fail("bad grouped gemm args");
  gg_ctx c = {a, b, bias, K, N, E, offsets, fmt, out_fmt, act, out};
  return parallel_for(M, gg_item, &c, (size_t)N);
}

/* ------------------------------------------------------------------ permute, combine */
/* Counting sort of the routes r = t K + k by expert, routes of one expert in ascending r
 * ([TO] MoEPermuteAlignFwdOp leaves that order open; this is the order taken). */
int moe_ref_permute(const int64_t* topk_ids, int64_t T, int64_t K, int64_t E,
                    int64_t* offsets, int64_t* sorted_route, int64_t* route_pos) {
  const int64_t R = T * K;
  for (int64_t e = 0; e <= E; ++e) offsets[e] = 0;
  for (int64_t r = 0; r < R; ++r) {
    if (topk_ids[r] < 0 || topk_ids[r] >= E) return fail("expert id out of range");
    offsets[topk_ids[r] + 1] += 1;
  }
  for (int64_t e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  int64_t* fill = malloc((size_t)(E > 0 ? E : 1) * sizeof(int64_t));
  if (!fill) return fail("out of host memory");
  for (int64_t e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int64_t r = 0; r < R; ++r) {
    const int64_t p = fill[topk_ids[r]]++;
    sorted_route[p] = r;
    route_pos[r] = p;
  }
  free(fill);
  return 0;
}

int moe_ref_combine(const void* y, int32_t fmt, int64_t rows, const double* topk_weights,
                    const int64_t* route_pos, int64_t T, int64_t K, int64_t H, double scale,
                    int32_t out_fmt, double* out) {
  if (!fmt_ok(fmt) || !fmt_ok(out_fmt)) return fail("bad combine args");
  for (int64_t t = 0; t < T; ++t)
    for (int64_t h = 0; h < H; ++h) {
      double acc = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t p = route_pos[t * K + k];
        if (p < 0) continue;
        if (p >= rows) return fail("route position past y");
        acc += topk_weights[t * K + k] * widen1(y, fmt, p * H + h);
      }
      out[t * H + h] = moe_ref_round(scale * acc, out_fmt);
    }
  return 0;
}

/* ------------------------------------------------------------------ shared expert */
/* [TO] SharedExpertMLPFwdOp: a = silu(x G^T) (x U^T) stored in out_fmt, then a D^T stored
 * in out_fmt. Scratch: 2S + S + H doubles. */
static void shared_row(const void* x, int64_t row, int64_t H, int64_t S, const void* wgu,
                       const void* wd, int32_t fmt, int32_t out_fmt, double* scratch,
                       double* out) {
  double* h = scratch;
  double* a = h + 2 * S;
  for (int64_t j = 0; j < 2 * S; ++j) {
    double acc = 0.0;
    for (int64_t i = 0; i < H; ++i) acc += widen1(wgu, fmt, j * H + i) * widen1(x, fmt, row * H + i);
    h[j] = acc;
  }
  for (int64_t j = 0; j < S; ++j)
    a[j] = moe_ref_round(h[j] * sigmoid(h[j]) * h[S + j], out_fmt);
  for (int64_t o = 0; o < H; ++o) {
    double acc = 0.0;
    for (int64_t j = 0; j < S; ++j) acc += widen1(wd, fmt, o * S + j) * a[j];
    out[o] = moe_ref_round(acc, out_fmt);
  }
}

typedef struct {
  const void *x, *wgu, *wd;
  int64_t H, S;
  int32_t fmt, out_fmt;
  double* out;
} shared_ctx;

static void shared_item(void* p, int64_t m, double* scratch) {
  const shared_ctx* c = (const shared_ctx*)p;
  shared_row(c->x, m, c->H, c->S, c->wgu, c->wd, c->fmt, c->out_fmt, scratch, c->out + m * c->H);
}

int moe_ref_shared_expert(const void* x, int64_t M, int64_t H, int64_t S,
                          const void* w_gate_up, const void* w_down, int32_t fmt,
                          int32_t out_fmt, double* out) {
  if (!fmt_ok(fmt) || !fmt_ok(out_fmt) || S < 1 || H < 1) return fail("bad shared args");
  shared_ctx c = {x, w_gate_up, w_down, H, S, fmt, out_fmt, out};
  return parallel_for(M, shared_item, &c, (size_t)(3 * S));
}

/* ------------------------------------------------------------------ the layer */
typedef struct {
  const moe_ref_ffn_cfg* c;
  route_ctx r;
  const void *hidden, *wgu, *wd, *bgu, *bd, *swgu, *swd;
  const int64_t* tokens;
  double *out, *shared_out;
  int failed;
} ffn_ctx;

/* One token of [TO] FusedMoEFwdOp: out[t] = sum_k w[t,k] (Wd_k act(Wgu_k x_t + bgu_k) +
 * bd_k), k ascending, with the activation stored in dtype; then the cast to dtype. */
static void ffn_item(void* p, int64_t i, double* scratch) {
  ffn_ctx* x = (ffn_ctx*)p;
  const moe_ref_ffn_cfg* c = x->c;
  const int64_t H = c->H, F = c->F, K = c->route.K;
  const int64_t t = x->tokens ? x->tokens[i] : i;
  if (route_row(&x->r, t, i, scratch)) {
    __atomic_store_n(&x->failed, 1, __ATOMIC_SEQ_CST);
    return;
  }
  double* h = scratch + route_scratch(&c->route);
  double* a = h + 2 * F;
  double* y = a + F;
  double* acc = y + H;
  for (int64_t o = 0; o < H; ++o) acc[o] = 0.0;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t e = x->r.topk_ids[i * K + k];
    expert_row(x->hidden, t, H, F, H, x->wgu, x->wd, x->bgu, x->bd, e, c->fmt, &c->act,
               c->dtype, h, a, y);
    const double w = x->r.w[i * K + k];
    for (int64_t o = 0; o < H; ++o) acc[o] += w * y[o];
  }
  for (int64_t o = 0; o < H; ++o) x->out[i * H + o] = moe_ref_round(acc[o], c->dtype);
  if (c->S > 0 && x->shared_out)
    shared_row(x->hidden, t, H, c->S, x->swgu, x->swd, c->fmt, c->dtype, h,
               x->shared_out + i * H);
}

int moe_ref_ffn_forward(const moe_ref_ffn_cfg* c, const void* hidden, int64_t T,
                        const void* logits, int32_t logits_fmt, const double* correction_bias,
                        const int64_t* expert_ids, const void* w_gate_up, const void* w_down,
                        const void* b_gate_up, const void* b_down, const void* shared_w_gate_up,
                        const void* shared_w_down, const int64_t* tokens, int64_t n_tokens,
                        int64_t* topk_ids, double* topk_weights, double* out, double* shared_out) {
  if (!route_cfg_ok(&c->route) || !fmt_ok(c->fmt) || !fmt_ok(c->dtype) || !fmt_ok(logits_fmt) ||
      c->H < 1 || c->F < 1 || c->S < 0 || (c->S > 0 && (!shared_w_gate_up || !shared_w_down)))
    return fail("bad layer config");
  const int64_t n = tokens ? n_tokens : T;
  for (int64_t i = 0; tokens && i < n; ++i)
    if (tokens[i] < 0 || tokens[i] >= T) return fail("token index out of range");
  double* b = rounded_bias(correction_bias, c->route.E);
  ffn_ctx x = {c, {&c->route, logits, logits_fmt, b, expert_ids, NULL, NULL, NULL,
                   topk_weights, NULL, NULL, NULL, NULL, topk_ids},
               hidden, w_gate_up, w_down, b_gate_up, b_down, shared_w_gate_up, shared_w_down,
               tokens, out, shared_out, 0};
  size_t need = 2 * (size_t)c->F + (size_t)c->F + 2 * (size_t)c->H;
  if (c->S > 0 && 3 * (size_t)c->S > need) need = 3 * (size_t)c->S;
  int rc = parallel_for(n, ffn_item, &x, route_scratch(&c->route) + need);
  free(b);
  if (rc == 0 && x.failed) rc = fail("expert id out of range or too few eligible");
  return rc;
}

/* ------------------------------------------------------------------ FP8 */
/* [TO] MoEGroupedGemmFP8FwdOp types both operands float8_e4m3fn (the OCP E4M3 encoding):
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds m/8 2^-6; no
 * infinities; only exponent 15 with mantissa 7 is NaN (largest value 1.75 2^8 = 448). */
void moe_ref_decode_e4m3fn(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) {
    const int c = codes[i], e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, e - 10);
    out[i] = (c & 0x80) ? -v : v;
  }
}

typedef struct {
  const uint8_t *a, *b;
  const double *sa, *sb;
  const int64_t* counts;
  int64_t max_m, N, K;
  double* out;
} fp8_ctx;

/* One row (g, m) of the masked FP8 GEMM; scratch: 2K doubles (decoded a row, b row). */
static void fp8_item(void* p, int64_t gm, double* scratch) {
  const fp8_ctx* c = (const fp8_ctx*)p;
  const int64_t g = gm / c->max_m, m = gm % c->max_m, K = c->K, N = c->N, nkb = K / 128;
  int64_t cnt = c->counts[g];
  if (cnt < 0) cnt = 0;
  if (cnt > c->max_m) cnt = c->max_m;
  double* o = c->out + gm * N;
  if (m >= cnt) {
    for (int64_t n = 0; n < N; ++n) o[n] = NAN;
    return;
  }
  double* av = scratch;
  double* bv = scratch + K;
  moe_ref_decode_e4m3fn(c->a + gm * K, K, av);
  for (int64_t n = 0; n < N; ++n) {
    moe_ref_decode_e4m3fn(c->b + (g * N + n) * K, K, bv);
    double acc = 0.0;
    for (int64_t kb = 0; kb < nkb; ++kb) {
      double blk = 0.0;
      for (int64_t k = 128 * kb; k < 128 * (kb + 1); ++k) blk += av[k] * bv[k];
      acc += blk * c->sa[gm * nkb + kb] * c->sb[(g * (N / 128) + n / 128) * nkb + kb];
    }
    o[n] = moe_ref_round(acc, MOE_REF_BF16);
  }
}

int moe_ref_grouped_gemm_fp8_masked(const uint8_t* a, const double* a_scale, const uint8_t* b,
                                    const double* b_scale, const int64_t* counts, int64_t E,
                                    int64_t max_m, int64_t N, int64_t K, double* out) {
  if (E < 1 || max_m < 0 || N < 128 || K < 128 || N % 128 || K % 128)
    return fail("bad fp8 args");
  fp8_ctx c = {a, b, a_scale, b_scale, counts, max_m, N, K, out};
  return parallel_for(E * max_m, fp8_item, &c, (size_t)(2 * K));
}
