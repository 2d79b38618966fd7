/*
 * Plain CPU oracle for Psi-Spec lossless block verification.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct
 * reference that the GPU library is checked against. Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark load it; the GPU
 * library never links, includes or calls it, and it shares no code, header,
 * table or constant with the GPU library.
 *
 * Everything is scalar C in IEEE double, in the order the method states it.
 * Sources (web pages on Uno, a diffusion-augmented LLM):
 *   [UnoX §3.2]  "Uno" research explainer, §3.2 Diffusion Distillation: one
 *                forward gives frozen-teacher and student logits; the TV term
 *                minimises the total-variation distance of the two token
 *                distributions (it governs the expected acceptance).
 *   [UnoX §3.3]  "Uno" research explainer, §3.3 Psi-Spec: drafts x_i ~ q_i in
 *                parallel; acceptance probability a_i = min(1, p(x_i)/q(x_i));
 *                the longest accepted prefix is kept; at the first rejection one
 *                token is drawn from the normalised positive part of p - q; if
 *                every draft is accepted one more token is drawn from the last
 *                target row. Same section: 1 <= tokens per forward <= (B+1)/2.
 *   [UnoX §3.4]  same page, §3.4: Linear sampler (one candidate per position)
 *                and Tree sampler (several candidate prefixes verified at once).
 *   [UnoX §7]    same page, §7: "lossless" means the output law is the AR law;
 *                same-seed equality with plain AR decoding is not promised.
 *   [UnoR inf]   Uno repository README, inference section: sampling controls
 *                temperature, top-p, top-k.
 *   [Philox]     Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
 *                as 1, 2, 3", SC'11 (counter-based generator Philox4x32-10);
 *                not on the pages, it fixes the random numbers both sides use.
 * Readings where the pages are silent (one fixed choice each, so that GPU and
 * oracle can be compared decision by decision):
 *   - temperature divides both target and draft logits; filters run in the
 *     order temperature -> top-k -> top-p -> renormalise, ties to the lower id;
 *   - the accept test is strict: accept iff u * q(x) < p(x), u in [0, 1);
 *   - every draw is an inverse-CDF draw in token-id order with one uniform;
 *   - the residual that sums to zero falls back to the target row;
 *   - greedy (temperature 0): accept iff the draft equals the target argmax
 *     (lowest id on ties), final token = target argmax;
 *   - tree: candidates at a node are i.i.d. draws from that node's draft row,
 *     tested in ascending node id with the recursive residual update;
 *   - NaN, +inf, an all -inf row or an out-of-range token makes the whole
 *     request an error (length -1, tokens -1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_DRAFT_DRAW 0x40000000u
#define PSI_MAXK_ORACLE_PLUS1 257 /* the oracle accepts K <= 256 */

/* ------------------------------------------------------------------------ */
/* [Philox] Philox4x32-10: ten rounds of two 32x32->64 multiplies with the
 * multipliers 0xD2511F53 and 0xCD9E8D57; the key is bumped between rounds by
 * the Weyl constants 0x9E3779B9 and 0xBB67AE85. */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t prod0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
    uint64_t prod1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* Uniform U(seed, step, b, r, d) = first Philox word / 2^32, key =
 * (lo32 seed, hi32 seed), counter = (d, r, b, step). */
double orc_uniform(uint64_t seed, uint32_t step, uint32_t b, uint32_t r, uint32_t d) {
  uint32_t ctr[4] = {d, r, b, step};
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  orc_philox4x32_10(ctr, key, out);
  return (double)out[0] / 4294967296.0;
}

/* ------------------------------------------------------------------------ */
/* Decoding: a bfloat16 is the upper half of a binary32, so it converts to
 * double exactly; binary32 converts to double exactly. */
static double decode_one(const void* base, int dtype, size_t idx) {
  float f;
  if (dtype == ORC_F32) {
    memcpy(&f, (const char*)base + 4 * idx, 4);
  } else {
    uint16_t h;
    memcpy(&h, (const char*)base + 2 * idx, 2);
    uint32_t u = (uint32_t)h << 16;
    memcpy(&f, &u, 4);
  }
  return (double)f;
}

/* Decodes row `row` (V values) into out[]; returns 1 if the row holds a NaN
 * or +inf or is entirely -inf (a request error), else 0. */
int orc_decode_row(const void* base, int dtype, int64_t row, int V, double* out) {
  int finite_or_minf_only = 1, any_not_minf = 0;
  for (int j = 0; j < V; ++j) {
    double a = decode_one(base, dtype, (size_t)row * (size_t)V + (size_t)j);
    out[j] = a;
    if (isnan(a) || (isinf(a) && a > 0)) finite_or_minf_only = 0;
    if (!(isinf(a) && a < 0)) any_not_minf = 1;
  }
  return (finite_or_minf_only && any_not_minf) ? 0 : 1;
}

/* ------------------------------------------------------------------------ */
/* [UnoR inf] filters. Sorting helper: (key desc, index asc). */
typedef struct {
  double key;
  int idx;
} keyed;

static int cmp_desc_then_idx(const void* pa, const void* pb) {
  const keyed* a = (const keyed*)pa;
  const keyed* b = (const keyed*)pb;
  if (a->key > b->key) return -1;
  if (a->key < b->key) return 1;
  return (a->idx < b->idx) ? -1 : (a->idx > b->idx);
}

/* Top-k: keep the top_k largest z (ties: lower id first), the rest -> -inf.
 * top_k <= 0 or top_k >= V disables it. */
static void filter_top_k(double* z, int V, int top_k, keyed* buf) {
  if (top_k <= 0 || top_k >= V) return;
  for (int j = 0; j < V; ++j) {
    buf[j].key = z[j];
    buf[j].idx = j;
  }
  qsort(buf, (size_t)V, sizeof(keyed), cmp_desc_then_idx);
  for (int t = top_k; t < V; ++t) z[buf[t].idx] = -INFINITY;
}

/* Top-p over the surviving tokens: softmax over them (sum in id order), sort
 * by probability (desc, ties lower id), keep the shortest prefix whose running
 * sum reaches top_p (at least one token). top_p >= 1 disables it.
 * *margin (may be NULL) = how far the cut decision is from going the other
 * way: the distance of top_p to the running sum on either side of the cut,
 * min(cum_t - top_p, top_p - cum_{t-1}) with cum_{-1} = 0 (probabilities sum
 * to 1, so this is a fraction of the kept mass); +inf when nothing is cut. */
static void filter_top_p(double* z, int V, double top_p, keyed* buf, double* margin) {
  if (margin) *margin = INFINITY;
  if (!(top_p < 1.0)) return;
  double m = -INFINITY;
  for (int j = 0; j < V; ++j)
    if (z[j] > m) m = z[j];
  if (isinf(m) && m < 0) return;
  double s = 0.0;
  for (int j = 0; j < V; ++j)
    if (!(isinf(z[j]) && z[j] < 0)) s += exp(z[j] - m);
  int n = 0;
  for (int j = 0; j < V; ++j) {
    if (isinf(z[j]) && z[j] < 0) continue;
    buf[n].key = exp(z[j] - m) / s;
    buf[n].idx = j;
    ++n;
  }
  qsort(buf, (size_t)n, sizeof(keyed), cmp_desc_then_idx);
  double cum = 0.0, prev = 0.0;
  int keep = n;
  for (int t = 0; t < n; ++t) {
    prev = cum;
    cum += buf[t].key;
    if (cum >= top_p) {
      keep = t + 1;
      break;
    }
  }
  if (margin) *margin = fmin(fabs(cum - top_p), top_p - prev);
  for (int t = keep; t < n; ++t) z[buf[t].idx] = -INFINITY;
}

/* Temperature then filters, in place: z = a / T, top-k, top-p. *margin (may
 * be NULL): the top-p cut's margin (+inf without a top-p cut). */
static void filter_row_buf(double* z, int V, double temperature, int top_k, double top_p, keyed* buf,
                           double* margin) {
  for (int j = 0; j < V; ++j) z[j] = z[j] / temperature;
  filter_top_k(z, V, top_k, buf);
  filter_top_p(z, V, top_p, buf, margin);
}

void orc_filter_row(double* z, int V, double temperature, int top_k, double top_p, double* margin) {
  keyed* buf = (keyed*)malloc(sizeof(keyed) * (size_t)V);
  filter_row_buf(z, V, temperature, top_k, top_p, buf, margin);
  free(buf);
}

/* ------------------------------------------------------------------------ */
/* Log-normaliser L = m + log sum_j exp(z_j - m), m = max z, summed in id
 * order. All -inf gives -inf. */
double orc_logsumexp(const double* z, int V) {
  double m = -INFINITY;
  for (int j = 0; j < V; ++j)
    if (z[j] > m) m = z[j];
  if (isinf(m) && m < 0) return -INFINITY;
  double s = 0.0;
  for (int j = 0; j < V; ++j) s += exp(z[j] - m);
  return m + log(s);
}

/* Inverse-CDF draw with one uniform u in [0, 1): W = sum w (id order), return
 * the smallest j with C_j = w_0 + ... + w_j > u * W; if rounding leaves none,
 * the largest j with w_j > 0. Returns -1 when W is not positive.
 * *margin (may be NULL) = distance of u*W to the nearer edge of the chosen
 * interval [C_{j-1}, C_j), divided by W; *alt (may be NULL) = the token a draw
 * lands on when that edge moves past u*W: below a lower edge the previous
 * index with positive weight, beyond an upper edge the next one (-1 if there
 * is none). The rounding fallback gives margin 0 and alt = j. */
int orc_sample(const double* w, int V, double u, double* margin, int* alt) {
  double W = 0.0;
  for (int j = 0; j < V; ++j) W += w[j];
  if (margin) *margin = 0.0;
  if (alt) *alt = -1;
  if (!(W > 0.0)) return -1;
  double t = u * W, c = 0.0;
  for (int j = 0; j < V; ++j) {
    double prev = c;
    c += w[j];
    if (c > t) {
      const double lo = t - prev, hi = c - t;
      if (margin) *margin = fmin(lo, hi) / W;
      if (alt) {
        if (lo <= hi) {
          for (int k = j - 1; k >= 0; --k)
            if (w[k] > 0.0) {
              *alt = k;
              break;
            }
        } else {
          for (int k = j + 1; k < V; ++k)
            if (w[k] > 0.0) {
              *alt = k;
              break;
            }
        }
      }
      return j;
    }
  }
  for (int j = V - 1; j >= 0; --j)
    if (w[j] > 0.0) {
      if (alt) *alt = j;
      return j;
    }
  return -1;
}

/* Lowest index of the maximum (raw logits; ties to the lowest id). */
static int argmax_row(const double* a, int V) {
  int best = 0;
  for (int j = 1; j < V; ++j)
    if (a[j] > a[best]) best = j;
  return best;
}

/* ------------------------------------------------------------------------ */
typedef struct {
  double temperature;
  int top_k;
  double top_p;
  uint64_t seed;
  uint32_t step;
} orc_params;

/* Uniform for (b, r, d), from the override table when one is given. The
 * override slot is chosen by the caller-specific `slot` index. */
static double uni(const orc_params* pr, int64_t b, int r, uint32_t d, const double* ovr, size_t slot) {
  if (ovr) return ovr[slot];
  return orc_uniform(pr->seed, pr->step, (uint32_t)b, (uint32_t)r, d);
}

/* ------------------------------------------------------------------------ */
/* Draft sampling [UnoX §3.3]: x_i drawn from softmax(filter(q_i / T)) by an
 * inverse-CDF draw over exp(z - max z) with U(seed, step, b, i, 0x40000000);
 * greedy: argmax q_i. Per draft: the draw's margin and alternative token (see
 * orc_sample) and the margin of its row's top-p cut (+inf where there is no
 * such decision). */
typedef struct {
  const void* q;
  int dtype;
  int K, V;
  orc_params pr;
  int32_t* out;
  double* out_margin;
  int32_t* out_alt;
  double* out_margin_filter;
  const double* ovr; /* [B][K] */
  int64_t b0, b1;
} draft_job;

static void* draft_worker(void* arg) {
  draft_job* J = (draft_job*)arg;
  int V = J->V, K = J->K;
  double* z = (double*)malloc(sizeof(double) * (size_t)V);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  keyed* buf = (keyed*)malloc(sizeof(keyed) * (size_t)V);
  for (int64_t b = J->b0; b < J->b1; ++b) {
    int bad = 0;
    for (int i = 0; i < K; ++i) bad |= orc_decode_row(J->q, J->dtype, b * K + i, V, z);
    for (int i = 0; i < K; ++i) {
      double margin = INFINITY, fmargin = INFINITY;
      int x = -1, alt = -1;
      if (!bad) {
        orc_decode_row(J->q, J->dtype, b * K + i, V, z);
        if (J->pr.temperature == 0.0) {
          x = argmax_row(z, V);
        } else {
          filter_row_buf(z, V, J->pr.temperature, J->pr.top_k, J->pr.top_p, buf, &fmargin);
          double m = -INFINITY;
          for (int j = 0; j < V; ++j)
            if (z[j] > m) m = z[j];
          for (int j = 0; j < V; ++j) w[j] = exp(z[j] - m);
          double u = uni(&J->pr, b, i, ORC_DRAFT_DRAW, J->ovr, J->ovr ? (size_t)(b * K + i) : 0);
          x = orc_sample(w, V, u, &margin, &alt);
        }
      }
      J->out[b * K + i] = x;
      if (J->out_margin) J->out_margin[b * K + i] = margin;
      if (J->out_alt) J->out_alt[b * K + i] = alt;
      if (J->out_margin_filter) J->out_margin_filter[b * K + i] = fmargin;
    }
  }
  free(z);
  free(w);
  free(buf);
  return NULL;
}

static void run_jobs(void* jobs, size_t job_size, int n, void* (*fn)(void*)) {
  if (n == 1) {
    fn(jobs);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n);
  for (int t = 0; t < n; ++t) pthread_create(&th[t], NULL, fn, (char*)jobs + job_size * (size_t)t);
  for (int t = 0; t < n; ++t) pthread_join(th[t], NULL);
  free(th);
}

static int clamp_threads(int nthreads, int64_t B) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > B) nthreads = (int)B;
  if (nthreads > 256) nthreads = 256;
  return nthreads;
}

int orc_draft_sample(const void* q, int dtype, int64_t B, int K, int V, double temperature, int top_k,
                     double top_p, uint64_t seed, uint32_t step, int32_t* out, double* out_margin, int32_t* out_alt,
                     double* out_margin_filter, const double* u_override, int nthreads) {
  if (!q || !out || B <= 0 || K <= 0 || V <= 0 || !(temperature >= 0.0)) return -1;
  nthreads = clamp_threads(nthreads, B);
  draft_job* jobs = (draft_job*)calloc((size_t)nthreads, sizeof(draft_job));
  for (int t = 0; t < nthreads; ++t) {
    draft_job* J = &jobs[t];
    J->q = q;
    J->dtype = dtype;
    J->K = K;
    J->V = V;
    J->pr.temperature = temperature;
    J->pr.top_k = top_k;
    J->pr.top_p = top_p;
    J->pr.seed = seed;
    J->pr.step = step;
    J->out = out;
    J->out_margin = out_margin;
    J->out_alt = out_alt;
    J->out_margin_filter = out_margin_filter;
    J->ovr = u_override;
    J->b0 = B * t / nthreads;
    J->b1 = B * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(draft_job), nthreads, draft_worker);
  free(jobs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Linear verification [UnoX §3.3, §3.4 Linear Sampler]. */

/* Margins of the decisions of one verification, so that a comparison with a
 * finite-precision implementation can tell which decision parted first and
 * how close it was (any pointer may be NULL):
 *   acc [B][K]        |u - min(1, P/Q)| of each accept test taken; +inf at
 *                     positions never tested, for Q(x) = 0, and in greedy mode;
 *   draft [B][K]      inverse-CDF margin of each draft drawn inside the call
 *                     (+inf when drafts are given or greedy), draft_alt the
 *                     token across its nearer edge (orc_sample);
 *   fin [B], fin_alt  the same for the final (residual or bonus) draw;
 *   filter [B]        the smallest top-p cut margin over the request's
 *                     2K + 1 rows (+inf without a top-p cut). */
typedef struct {
  double *acc, *draft, *fin, *filter;
  int32_t *draft_alt, *fin_alt;
} orc_lin_margins;

typedef struct {
  const void *p, *q;
  int dtype, K, V, fused;
  orc_params pr;
  int32_t* draft;
  int32_t* out_tokens;
  int32_t* out_len;
  double* out_probs;
  double* out_resid;
  orc_lin_margins mg;
  const double* ovr; /* [B][K+1][3]: final (d=0), accept (d=1), draft (d=0x40000000) */
  int64_t b0, b1;
} linear_job;

static void linear_one(linear_job* J, int64_t b, double* zp, double* zq, double* w, keyed* buf) {
  const int K = J->K, V = J->V;
  const orc_params* pr = &J->pr;
  const orc_lin_margins* M = &J->mg;
  int32_t* toks = J->out_tokens + b * (K + 1);
  for (int i = 0; i <= K; ++i) toks[i] = -1;
  if (J->out_resid) J->out_resid[b] = 0.0;
  for (int i = 0; i < K; ++i) {
    if (M->acc) M->acc[b * K + i] = INFINITY;
    if (M->draft) M->draft[b * K + i] = INFINITY;
    if (M->draft_alt) M->draft_alt[b * K + i] = -1;
  }
  if (M->fin) M->fin[b] = INFINITY;
  if (M->fin_alt) M->fin_alt[b] = -1;
  if (M->filter) M->filter[b] = INFINITY;
  if (J->out_probs)
    for (int i = 0; i < 2 * K; ++i) J->out_probs[b * 2 * K + i] = 0.0;

  /* validity of every row of the request */
  int bad = 0;
  for (int i = 0; i <= K; ++i) bad |= orc_decode_row(J->p, J->dtype, b * (K + 1) + i, V, zp + (size_t)i * V);
  for (int i = 0; i < K; ++i) bad |= orc_decode_row(J->q, J->dtype, b * K + i, V, zq + (size_t)i * V);
  if (!J->fused)
    for (int i = 0; i < K; ++i) {
      int32_t x = J->draft[b * K + i];
      if (x < 0 || x >= V) bad = 1;
    }
  if (bad) {
    if (J->fused)
      for (int i = 0; i < K; ++i) J->draft[b * K + i] = -1;
    J->out_len[b] = -1;
    return;
  }

  int n = K, y = -1;
  if (pr->temperature == 0.0) {
    /* greedy */
    int g[PSI_MAXK_ORACLE_PLUS1];
    for (int i = 0; i <= K; ++i) g[i] = argmax_row(zp + (size_t)i * V, V);
    for (int i = 0; i < K; ++i) {
      int gq = argmax_row(zq + (size_t)i * V, V);
      if (J->fused) J->draft[b * K + i] = gq;
      int x = J->draft[b * K + i];
      if (J->out_probs) {
        J->out_probs[(b * K + i) * 2 + 0] = (x == g[i]) ? 1.0 : 0.0;
        J->out_probs[(b * K + i) * 2 + 1] = (x == gq) ? 1.0 : 0.0;
      }
    }
    for (int i = 0; i < K; ++i)
      if (J->draft[b * K + i] != g[i]) {
        n = i;
        break;
      }
    y = g[n];
  } else {
    double Lp[PSI_MAXK_ORACLE_PLUS1], Lq[PSI_MAXK_ORACLE_PLUS1];
    double fmin_all = INFINITY, fm;
    for (int i = 0; i <= K; ++i) {
      filter_row_buf(zp + (size_t)i * V, V, pr->temperature, pr->top_k, pr->top_p, buf, &fm);
      fmin_all = fmin(fmin_all, fm);
      Lp[i] = orc_logsumexp(zp + (size_t)i * V, V);
    }
    for (int i = 0; i < K; ++i) {
      filter_row_buf(zq + (size_t)i * V, V, pr->temperature, pr->top_k, pr->top_p, buf, &fm);
      fmin_all = fmin(fmin_all, fm);
      Lq[i] = orc_logsumexp(zq + (size_t)i * V, V);
    }
    if (M->filter) M->filter[b] = fmin_all;
    if (J->fused) {
      for (int i = 0; i < K; ++i) {
        const double* z = zq + (size_t)i * V;
        double m = -INFINITY;
        for (int j = 0; j < V; ++j)
          if (z[j] > m) m = z[j];
        for (int j = 0; j < V; ++j) w[j] = exp(z[j] - m);
        double u = uni(pr, b, i, ORC_DRAFT_DRAW, J->ovr, J->ovr ? (size_t)((b * (K + 1) + i) * 3 + 2) : 0);
        double mg;
        int alt;
        J->draft[b * K + i] = orc_sample(w, V, u, &mg, &alt);
        if (M->draft) M->draft[b * K + i] = mg;
        if (M->draft_alt) M->draft_alt[b * K + i] = alt;
      }
    }
    /* per-position target and draft probability of the draft token */
    double P[PSI_MAXK_ORACLE_PLUS1], Q[PSI_MAXK_ORACLE_PLUS1];
    for (int i = 0; i < K; ++i) {
      int x = J->draft[b * K + i];
      P[i] = exp(zp[(size_t)i * V + x] - Lp[i]);
      Q[i] = exp(zq[(size_t)i * V + x] - Lq[i]);
      if (J->out_probs) {
        J->out_probs[(b * K + i) * 2 + 0] = P[i];
        J->out_probs[(b * K + i) * 2 + 1] = Q[i];
      }
    }
    /* accept tests in order; the first rejection ends the prefix. Each
       position has its own uniform, so testing in parallel and taking the
       first failure gives the same n. */
    for (int i = 0; i < K; ++i) {
      double u = uni(pr, b, i, 1u, J->ovr, J->ovr ? (size_t)((b * (K + 1) + i) * 3 + 1) : 0);
      int acc = u * Q[i] < P[i];
      if (M->acc && Q[i] > 0.0) M->acc[b * K + i] = fabs(u - fmin(1.0, P[i] / Q[i]));
      if (!acc) {
        n = i;
        break;
      }
    }
    double mg;
    int alt;
    if (n < K) {
      /* residual max(0, p_n - q_n), falling back to p_n when it sums to 0 */
      const double* a = zp + (size_t)n * V;
      const double* d = zq + (size_t)n * V;
      double W = 0.0;
      for (int j = 0; j < V; ++j) {
        double pj = exp(a[j] - Lp[n]);
        double qj = exp(d[j] - Lq[n]);
        w[j] = fmax(0.0, pj - qj);
        W += w[j];
      }
      if (J->out_resid) J->out_resid[b] = W;
      if (!(W > 0.0))
        for (int j = 0; j < V; ++j) w[j] = exp(a[j] - Lp[n]);
      double u = uni(pr, b, n, 0u, J->ovr, J->ovr ? (size_t)((b * (K + 1) + n) * 3 + 0) : 0);
      y = orc_sample(w, V, u, &mg, &alt);
    } else {
      /* bonus token from the last target row */
      const double* a = zp + (size_t)K * V;
      for (int j = 0; j < V; ++j) w[j] = exp(a[j] - Lp[K]);
      double u = uni(pr, b, K, 0u, J->ovr, J->ovr ? (size_t)((b * (K + 1) + K) * 3 + 0) : 0);
      y = orc_sample(w, V, u, &mg, &alt);
    }
    if (M->fin) M->fin[b] = mg;
    if (M->fin_alt) M->fin_alt[b] = alt;
  }
  for (int i = 0; i < n; ++i) toks[i] = J->draft[b * K + i];
  toks[n] = y;
  J->out_len[b] = n;
}

static void* linear_worker(void* arg) {
  linear_job* J = (linear_job*)arg;
  size_t V = (size_t)J->V, K = (size_t)J->K;
  double* zp = (double*)malloc(sizeof(double) * (K + 1) * V);
  double* zq = (double*)malloc(sizeof(double) * K * V);
  double* w = (double*)malloc(sizeof(double) * V);
  keyed* buf = (keyed*)malloc(sizeof(keyed) * V);
  for (int64_t b = J->b0; b < J->b1; ++b) linear_one(J, b, zp, zq, w, buf);
  free(zp);
  free(zq);
  free(w);
  free(buf);
  return NULL;
}

int orc_verify_linear(const void* p, const void* q, int dtype, int64_t B, int K, int V, int32_t* draft_tokens,
                      double temperature, int top_k, double top_p, uint64_t seed, uint32_t step, int fused,
                      int32_t* out_tokens, int32_t* out_len, double* out_probs, double* out_resid,
                      const orc_lin_margins* margins, const double* u_override, int nthreads) {
  if (!p || !q || !draft_tokens || !out_tokens || !out_len) return -1;
  if (B <= 0 || K <= 0 || K >= PSI_MAXK_ORACLE_PLUS1 || V <= 0 || !(temperature >= 0.0)) return -1;
  nthreads = clamp_threads(nthreads, B);
  linear_job* jobs = (linear_job*)calloc((size_t)nthreads, sizeof(linear_job));
  for (int t = 0; t < nthreads; ++t) {
    linear_job* J = &jobs[t];
    J->p = p;
    J->q = q;
    J->dtype = dtype;
    J->K = K;
    J->V = V;
    J->fused = fused;
    J->pr.temperature = temperature;
    J->pr.top_k = top_k;
    J->pr.top_p = top_p;
    J->pr.seed = seed;
    J->pr.step = step;
    J->draft = draft_tokens;
    J->out_tokens = out_tokens;
    J->out_len = out_len;
    J->out_probs = out_probs;
    J->out_resid = out_resid;
    if (margins) J->mg = *margins;
    J->ovr = u_override;
    J->b0 = B * t / nthreads;
    J->b1 = B * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(linear_job), nthreads, linear_worker);
  free(jobs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Tree verification [UnoX §3.4 Tree Sampler]; per-node rule: candidates are
 * i.i.d. draws from the node's draft row Q, tested in ascending node id
 * against a running target r (starting at P): accept iff u * Q(tok) < r(tok);
 * after a rejection r <- norm(max(0, r - Q)) (kept when that sums to 0). */
/* Margins of a tree verification (any pointer may be NULL): acc [B][N] the
 * accept test of node n at its parent row, |u - min(1, r(tok)/Q(tok))| with r
 * the running target (+inf for nodes never tested, Q(tok) = 0, greedy);
 * fin [B] and fin_alt [B] the final draw (orc_sample); filter [B] the smallest
 * top-p cut margin over the rows the walk filtered (+inf without top-p). */
typedef struct {
  double *acc, *fin, *filter;
  int32_t* fin_alt;
} orc_tree_margins;

typedef struct {
  const void *p, *q;
  int dtype, N, V, maxC;
  const int32_t* parent;
  const int32_t* tokens;
  orc_params pr;
  int32_t *out_tokens, *out_path, *out_len;
  orc_tree_margins mg;
  const double* ovr; /* [B][N+1][1+maxC]: slot 0 = d=0, slot 1+j = d=1+j */
  int D;
  int64_t b0, b1;
} tree_job;

static void tree_one(tree_job* J, int64_t b, double* zp, double* zq, double* rt, double* Qv, double* w,
                     keyed* buf) {
  const int N = J->N, V = J->V, R = J->N + 1, D = J->D;
  const orc_params* pr = &J->pr;
  const orc_tree_margins* M = &J->mg;
  int32_t* toks = J->out_tokens + b * (D + 1);
  int32_t* path = J->out_path + b * D;
  for (int i = 0; i <= D; ++i) toks[i] = -1;
  for (int i = 0; i < D; ++i) path[i] = -1;
  if (M->acc)
    for (int n = 0; n < N; ++n) M->acc[b * N + n] = INFINITY;
  if (M->fin) M->fin[b] = INFINITY;
  if (M->fin_alt) M->fin_alt[b] = -1;
  if (M->filter) M->filter[b] = INFINITY;
  int bad = 0;
  for (int r = 0; r < R; ++r) {
    bad |= orc_decode_row(J->p, J->dtype, b * R + r, V, zp + (size_t)r * V);
    bad |= orc_decode_row(J->q, J->dtype, b * R + r, V, zq + (size_t)r * V);
  }
  for (int n = 0; n < N; ++n) {
    int32_t t = J->tokens[b * N + n];
    if (t < 0 || t >= V) bad = 1;
  }
  if (bad) {
    J->out_len[b] = -1;
    return;
  }
  double fmin_all = INFINITY;
  int greedy = pr->temperature == 0.0;
  int row = 0, len = 0, y = -1;
  for (;;) {
    const double* a = zp + (size_t)row * V;
    const double* d = zq + (size_t)row * V;
    /* children of this row: nodes whose parent is row-1, ascending id */
    int accepted = -1, j = 0;
    if (greedy) {
      int g = argmax_row(a, V);
      for (int c = 0; c < N; ++c) {
        if (J->parent[c] != row - 1) continue;
        if (J->tokens[b * N + c] == g) {
          accepted = c;
          break;
        }
      }
      if (accepted < 0) {
        y = g;
        break;
      }
    } else {
      /* target and draft distributions of this row, after filtering */
      memcpy(rt, a, sizeof(double) * (size_t)V);
      memcpy(Qv, d, sizeof(double) * (size_t)V);
      double fm;
      filter_row_buf(rt, V, pr->temperature, pr->top_k, pr->top_p, buf, &fm);
      fmin_all = fmin(fmin_all, fm);
      filter_row_buf(Qv, V, pr->temperature, pr->top_k, pr->top_p, buf, &fm);
      fmin_all = fmin(fmin_all, fm);
      double Lp = orc_logsumexp(rt, V), Lq = orc_logsumexp(Qv, V);
      for (int t = 0; t < V; ++t) {
        rt[t] = exp(rt[t] - Lp);
        Qv[t] = exp(Qv[t] - Lq);
      }
      for (int c = 0; c < N; ++c) {
        if (J->parent[c] != row - 1) continue;
        int tok = J->tokens[b * N + c];
        double u = uni(pr, b, row, 1u + (uint32_t)j, J->ovr,
                       J->ovr ? (size_t)((b * R + row) * (1 + J->maxC) + 1 + j) : 0);
        if (M->acc && Qv[tok] > 0.0) M->acc[b * N + c] = fabs(u - fmin(1.0, rt[tok] / Qv[tok]));
        if (u * Qv[tok] < rt[tok]) {
          accepted = c;
          break;
        }
        double S = 0.0;
        for (int t = 0; t < V; ++t) {
          w[t] = fmax(0.0, rt[t] - Qv[t]);
          S += w[t];
        }
        if (S > 0.0)
          for (int t = 0; t < V; ++t) rt[t] = w[t] / S;
        ++j;
      }
      if (accepted < 0) {
        double u = uni(pr, b, row, 0u, J->ovr, J->ovr ? (size_t)((b * R + row) * (1 + J->maxC)) : 0);
        double mg;
        int alt;
        y = orc_sample(rt, V, u, &mg, &alt);
        if (M->fin) M->fin[b] = mg;
        if (M->fin_alt) M->fin_alt[b] = alt;
        break;
      }
    }
    path[len] = accepted;
    toks[len] = J->tokens[b * N + accepted];
    ++len;
    row = accepted + 1;
  }
  toks[len] = y;
  J->out_len[b] = len;
  if (M->filter) M->filter[b] = fmin_all;
}

static void* tree_worker(void* arg) {
  tree_job* J = (tree_job*)arg;
  size_t V = (size_t)J->V, R = (size_t)J->N + 1;
  double* zp = (double*)malloc(sizeof(double) * R * V);
  double* zq = (double*)malloc(sizeof(double) * R * V);
  double* rt = (double*)malloc(sizeof(double) * V);
  double* Qv = (double*)malloc(sizeof(double) * V);
  double* w = (double*)malloc(sizeof(double) * V);
  keyed* buf = (keyed*)malloc(sizeof(keyed) * V);
  for (int64_t b = J->b0; b < J->b1; ++b) tree_one(J, b, zp, zq, rt, Qv, w, buf);
  free(zp);
  free(zq);
  free(rt);
  free(Qv);
  free(w);
  free(buf);
  return NULL;
}

/* Depth of the tree (children of the root have depth 1); -1 if malformed. */
int orc_tree_depth(const int32_t* parent, int N) {
  int depth[1024];
  if (N <= 0 || N > 1024) return -1;
  int D = 0;
  for (int n = 0; n < N; ++n) {
    if (parent[n] < -1 || parent[n] >= n) return -1;
    depth[n] = parent[n] < 0 ? 1 : depth[parent[n]] + 1;
    if (depth[n] > D) D = depth[n];
  }
  return D;
}

/* Tree drafts [UnoX §3.4 Tree Sampler; the rule above is lossless only when
 * the children of a row are i.i.d. draws from that row's draft distribution]:
 * node n, the j-th child (ascending id) of row r = parent[n] + 1, is an
 * inverse-CDF draw from softmax(filter(q_r / T)) with
 * U(seed, step, b, r, 0x40000000 + j); greedy: argmax q_r. A request with an
 * invalid draft row gets -1 for every node. Per node (any may be NULL): the
 * draw's margin and alternative token (orc_sample) and the top-p cut margin
 * of its row (+inf where there is no such decision). */
typedef struct {
  const void* q;
  int dtype, N, V;
  const int32_t* parent;
  orc_params pr;
  int32_t* out;
  double *out_margin, *out_margin_filter;
  int32_t* out_alt;
  int64_t b0, b1;
} tree_draft_job;

static void* tree_draft_worker(void* arg) {
  tree_draft_job* J = (tree_draft_job*)arg;
  const int N = J->N, V = J->V, R = J->N + 1;
  double* z = (double*)malloc(sizeof(double) * (size_t)V);
  double* w = (double*)malloc(sizeof(double) * (size_t)V);
  keyed* buf = (keyed*)malloc(sizeof(keyed) * (size_t)V);
  for (int64_t b = J->b0; b < J->b1; ++b) {
    for (int n = 0; n < N; ++n) {
      if (J->out_margin) J->out_margin[b * N + n] = INFINITY;
      if (J->out_margin_filter) J->out_margin_filter[b * N + n] = INFINITY;
      if (J->out_alt) J->out_alt[b * N + n] = -1;
    }
    int bad = 0;
    for (int r = 0; r < R; ++r) bad |= orc_decode_row(J->q, J->dtype, b * R + r, V, z);
    for (int r = 0; r < R && !bad; ++r) {
      int j = 0; /* sibling index within row r */
      for (int n = 0; n < N; ++n) {
        if (J->parent[n] != r - 1) continue;
        orc_decode_row(J->q, J->dtype, b * R + r, V, z);
        int x;
        if (J->pr.temperature == 0.0) {
          x = argmax_row(z, V);
        } else {
          double fm, mg;
          int alt;
          filter_row_buf(z, V, J->pr.temperature, J->pr.top_k, J->pr.top_p, buf, &fm);
          double m = -INFINITY;
          for (int t = 0; t < V; ++t)
            if (z[t] > m) m = z[t];
          for (int t = 0; t < V; ++t) w[t] = exp(z[t] - m);
          x = orc_sample(w, V, uni(&J->pr, b, r, ORC_DRAFT_DRAW + (uint32_t)j, NULL, 0), &mg, &alt);
          if (J->out_margin) J->out_margin[b * N + n] = mg;
          if (J->out_margin_filter) J->out_margin_filter[b * N + n] = fm;
          if (J->out_alt) J->out_alt[b * N + n] = alt;
        }
        J->out[b * N + n] = x;
        ++j;
      }
    }
    if (bad)
      for (int n = 0; n < N; ++n) J->out[b * N + n] = -1;
  }
  free(z);
  free(w);
  free(buf);
  return NULL;
}

int orc_tree_draft(const void* q, int dtype, int64_t B, int N, int V, const int32_t* parent, double temperature,
                   int top_k, double top_p, uint64_t seed, uint32_t step, int32_t* out, double* out_margin,
                   int32_t* out_alt, double* out_margin_filter, int nthreads) {
  if (!q || !parent || !out || B <= 0 || V <= 0 || !(temperature >= 0.0)) return -1;
  if (orc_tree_depth(parent, N) < 0) return -1;
  nthreads = clamp_threads(nthreads, B);
  tree_draft_job* jobs = (tree_draft_job*)calloc((size_t)nthreads, sizeof(tree_draft_job));
  for (int t = 0; t < nthreads; ++t) {
    tree_draft_job* J = &jobs[t];
    J->q = q;
    J->dtype = dtype;
    J->N = N;
    J->V = V;
    J->parent = parent;
    J->pr.temperature = temperature;
    J->pr.top_k = top_k;
    J->pr.top_p = top_p;
    J->pr.seed = seed;
    J->pr.step = step;
    J->out = out;
    J->out_margin = out_margin;
    J->out_alt = out_alt;
    J->out_margin_filter = out_margin_filter;
    J->b0 = B * t / nthreads;
    J->b1 = B * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(tree_draft_job), nthreads, tree_draft_worker);
  free(jobs);
  return 0;
}


int orc_verify_tree(const void* p, const void* q, int dtype, int64_t B, int N, int V, const int32_t* parent,
                    const int32_t* node_tokens, double temperature, int top_k, double top_p, uint64_t seed,
                    uint32_t step, int32_t* out_tokens, int32_t* out_path, int32_t* out_len,
                    const orc_tree_margins* margins, const double* u_override, int maxC, int nthreads) {
  if (!p || !q || !parent || !node_tokens || !out_tokens || !out_path || !out_len) return -1;
  if (B <= 0 || V <= 0 || !(temperature >= 0.0)) return -1;
  int D = orc_tree_depth(parent, N);
  if (D < 0) return -1;
  if (u_override) {
    /* every row's child count must fit the override table */
    for (int r = 0; r <= N; ++r) {
      int nc = 0;
      for (int c = 0; c < N; ++c) nc += parent[c] == r - 1;
      if (nc > maxC) return -1;
    }
  }
  nthreads = clamp_threads(nthreads, B);
  tree_job* jobs = (tree_job*)calloc((size_t)nthreads, sizeof(tree_job));
  for (int t = 0; t < nthreads; ++t) {
    tree_job* J = &jobs[t];
    J->p = p;
    J->q = q;
    J->dtype = dtype;
    J->N = N;
    J->V = V;
    J->maxC = maxC;
    J->parent = parent;
    J->tokens = node_tokens;
    J->pr.temperature = temperature;
    J->pr.top_k = top_k;
    J->pr.top_p = top_p;
    J->pr.seed = seed;
    J->pr.step = step;
    J->out_tokens = out_tokens;
    J->out_path = out_path;
    J->out_len = out_len;
    if (margins) J->mg = *margins;
    J->ovr = u_override;
    J->D = D;
    J->b0 = B * t / nthreads;
    J->b1 = B * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(tree_job), nthreads, tree_worker);
  free(jobs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Tree Sampler candidates [UnoX §3.4 Tree Sampler: each position keeps its
 * top-K tokens, then the V most probable prefixes are kept and verified in
 * one pass; UnoX §6.3 uses (block, K, V) = (16, 32, 32)]. Reading of the
 * construction (the pages give no formula):
 *   q_i = softmax(d_i / T) for draft position i (full row, fp64);
 *   C_i = the `cands` tokens with the largest q_i, ties to the lower id, in
 *         that order (rank 0 first);
 *   a prefix (t_0 .. t_{l-1}), t_i in C_i, has log score
 *         sum_i (z_i(t_i) - L_i), z = d / T, L_i = log sum exp z_i;
 *   the kept prefixes are the first `nodes` ones in the order
 *         log score descending, then length ascending, then the position of
 *         the parent prefix in this order ascending (the empty prefix first),
 *         then the rank of the last token in C ascending.
 * A parent's score is at least its child's and comes first on a tie, so the
 * kept set is closed under taking prefixes. Node n is the n-th kept prefix,
 * parent[n] the node of its parent (-1 for length 1), tokens[n] its last
 * token, so parent[n] < n. Enumerated best first: at each step every kept
 * prefix (and the empty one) offers its best child not yet kept, and the best
 * offer in the order is kept; a prefix of probability zero is never kept
 * (nodes past the last prefix of positive probability get -1).
 * out_margin [B][nodes] (may be NULL): for the step that keeps node n, the
 * smallest log-score gap between the kept offer and any other offer of that
 * step (0 for exact ties across parents; +inf when no other offer has positive
 * probability, or for nodes never kept). A request with an invalid draft row
 * gets -1 in every parent and token. */
typedef struct {
  const void* q;
  int dtype, K, V, cands, nodes;
  double temperature;
  int32_t *out_parent, *out_tokens;
  double* out_margin;
  int64_t b0, b1;
} cand_job;

static void* cand_worker(void* arg) {
  cand_job* J = (cand_job*)arg;
  const int K = J->K, V = J->V, C = J->cands, NN = J->nodes;
  double* z = (double*)malloc(sizeof(double) * (size_t)V);
  keyed* buf = (keyed*)malloc(sizeof(keyed) * (size_t)V);
  int32_t* ctok = (int32_t*)malloc(sizeof(int32_t) * (size_t)K * C);
  double* clq = (double*)malloc(sizeof(double) * (size_t)K * C);
  double* ls = (double*)malloc(sizeof(double) * (size_t)(NN + 1));
  int* depth = (int*)malloc(sizeof(int) * (size_t)(NN + 1));
  int* next = (int*)malloc(sizeof(int) * (size_t)(NN + 1));
  for (int64_t b = J->b0; b < J->b1; ++b) {
    int32_t* par = J->out_parent + b * NN;
    int32_t* tok = J->out_tokens + b * NN;
    int bad = 0;
    for (int i = 0; i < K && !bad; ++i) {
      bad |= orc_decode_row(J->q, J->dtype, b * K + i, V, z);
      if (bad) break;
      for (int j = 0; j < V; ++j) z[j] /= J->temperature;
      const double L = orc_logsumexp(z, V);
      for (int j = 0; j < V; ++j) {
        buf[j].key = z[j];
        buf[j].idx = j;
      }
      qsort(buf, (size_t)V, sizeof(keyed), cmp_desc_then_idx);
      for (int r = 0; r < C; ++r) {
        ctok[i * C + r] = buf[r].idx;
        clq[i * C + r] = buf[r].key - L;
      }
    }
    if (J->out_margin)
      for (int n = 0; n < NN; ++n) J->out_margin[b * NN + n] = INFINITY;
    if (bad) {
      for (int n = 0; n < NN; ++n) par[n] = tok[n] = -1;
      continue;
    }
    /* slot 0 is the empty prefix; slot n + 1 is node n */
    ls[0] = 0.0;
    depth[0] = 0;
    next[0] = 0;
    for (int n = 0; n < NN; ++n) {
      int best = -1;
      double bls = 0.0;
      for (int s = 0; s <= n; ++s) {
        if (depth[s] >= K || next[s] >= C) continue; /* nothing to offer */
        const double o = ls[s] + clq[depth[s] * C + next[s]];
        if (isinf(o)) continue; /* zero probability: never kept (later ranks are no better) */
        int better;
        if (best < 0) better = 1;
        else if (o != bls) better = o > bls;
        else if (depth[s] != depth[best]) better = depth[s] < depth[best];
        else better = 0; /* same score and length: the earlier parent (smaller slot) wins */
        if (better) {
          best = s;
          bls = o;
        }
      }
      if (best < 0) { /* fewer prefixes than nodes */
        for (int m = n; m < NN; ++m) par[m] = tok[m] = -1;
        break;
      }
      double margin = INFINITY;
      for (int s = 0; s <= n; ++s) {
        if (s == best || depth[s] >= K || next[s] >= C) continue;
        const double gap = bls - (ls[s] + clq[depth[s] * C + next[s]]);
        if (gap < margin) margin = gap; /* an offer of zero probability gives +inf */
      }
      if (J->out_margin) J->out_margin[b * NN + n] = margin;
      par[n] = best - 1;
      tok[n] = ctok[depth[best] * C + next[best]];
      ls[n + 1] = bls;
      depth[n + 1] = depth[best] + 1;
      next[n + 1] = 0;
      ++next[best];
    }
  }
  free(z);
  free(buf);
  free(ctok);
  free(clq);
  free(ls);
  free(depth);
  free(next);
  return NULL;
}

int orc_tree_candidates(const void* q, int dtype, int64_t B, int K, int V, double temperature, int cands,
                        int nodes, int32_t* out_parent, int32_t* out_tokens, double* out_margin, int nthreads) {
  if (!q || !out_parent || !out_tokens || B <= 0 || K <= 0 || V <= 0 || !(temperature > 0.0)) return -1;
  if (cands < 1 || cands > V || nodes < 1) return -1;
  nthreads = clamp_threads(nthreads, B);
  cand_job* jobs = (cand_job*)calloc((size_t)nthreads, sizeof(cand_job));
  for (int t = 0; t < nthreads; ++t) {
    cand_job* J = &jobs[t];
    J->q = q;
    J->dtype = dtype;
    J->K = K;
    J->V = V;
    J->cands = cands;
    J->nodes = nodes;
    J->temperature = temperature;
    J->out_parent = out_parent;
    J->out_tokens = out_tokens;
    J->out_margin = out_margin;
    J->b0 = B * t / nthreads;
    J->b1 = B * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(cand_job), nthreads, cand_worker);
  free(jobs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Verification of deterministic candidates (the Tree Sampler's candidates of
 * [UnoX §3.4] are chosen, not drawn; the pages state no rule for them, and
 * this is the plain lossless one). Per request, with its own tree (parent,
 * tokens [N], parent[n] < n): the walk starts at row 0 (row n + 1 follows node
 * n); at a row, r = P = softmax(a / T) and E = 0; its children are tested in
 * ascending node id, the j-th with u = U(seed, step, b, row, 1 + j): a point
 * mass proposal at tok is accepted with probability r(tok), i.e. iff
 * u * (1 - E) < P(tok) when tok is not yet removed (never when it is); on a
 * rejection tok is removed from r (E += P(tok)) and r renormalised. The walk
 * descends into the first accepted child; at a leaf or once every child is
 * rejected, the final token is an inverse-CDF draw from P without the removed
 * tokens, U(seed, step, b, row, 0) (from P itself if nothing remains).
 * Temperature 0: accept iff tok is the target argmax (lowest id on ties);
 * final token = the argmax. Any malformed parent, token out of range or
 * invalid target row makes the request an error. Outputs [N + 1] tokens and
 * [N] path entries per request, -1 past the end. Margins (orc_tree_margins,
 * any pointer may be NULL): acc [B][N] |u - r(tok)| of each test taken, r(tok)
 * = P(tok) / (1 - E) the running target's mass at tok (+inf for nodes never
 * tested, removed tokens and greedy); fin / fin_alt the final draw; filter is
 * +inf (no filters here). */
typedef struct {
  const void* p;
  int dtype, N, V;
  const int32_t *parent, *tokens;
  orc_params pr;
  int32_t *out_tokens, *out_path, *out_len;
  orc_tree_margins mg; /* acc: |u - r(tok)| with r the running target */
  const double* ovr;   /* [B][N+1][1+maxC]: slot 0 = d=0, slot 1+j = d=1+j */
  int maxC;
  int64_t b0, b1;
} dtree_job;

static void dtree_one(dtree_job* J, int64_t b, double* z, double* P, double* w, unsigned char* removed) {
  const int N = J->N, V = J->V, R = N + 1;
  const orc_params* pr = &J->pr;
  const int32_t* par = J->parent + b * N;
  const int32_t* ntk = J->tokens + b * N;
  int32_t* toks = J->out_tokens + b * R;
  int32_t* path = J->out_path + b * N;
  const orc_tree_margins* M = &J->mg;
  for (int i = 0; i < R; ++i) toks[i] = -1;
  for (int i = 0; i < N; ++i) path[i] = -1;
  if (M->acc)
    for (int n = 0; n < N; ++n) M->acc[b * N + n] = INFINITY;
  if (M->fin) M->fin[b] = INFINITY;
  if (M->fin_alt) M->fin_alt[b] = -1;
  if (M->filter) M->filter[b] = INFINITY;
  int bad = 0;
  for (int n = 0; n < N; ++n) {
    if (par[n] < -1 || par[n] >= n) bad = 1;
    if (ntk[n] < 0 || ntk[n] >= V) bad = 1;
  }
  for (int r = 0; r < R && !bad; ++r) bad |= orc_decode_row(J->p, J->dtype, b * R + r, V, z);
  if (bad) {
    J->out_len[b] = -1;
    return;
  }
  const int greedy = pr->temperature == 0.0;
  int row = 0, len = 0, y = -1;
  for (;;) {
    orc_decode_row(J->p, J->dtype, b * R + row, V, z);
    int accepted = -1;
    if (greedy) {
      const int g = argmax_row(z, V);
      for (int c = 0; c < N && accepted < 0; ++c)
        if (par[c] == row - 1 && ntk[c] == g) accepted = c;
      if (accepted < 0) {
        y = g;
        break;
      }
    } else {
      for (int t = 0; t < V; ++t) z[t] /= pr->temperature;
      const double L = orc_logsumexp(z, V);
      for (int t = 0; t < V; ++t) {
        P[t] = exp(z[t] - L);
        removed[t] = 0;
      }
      double E = 0.0;
      int j = 0;
      for (int c = 0; c < N; ++c) {
        if (par[c] != row - 1) continue;
        const int tk = ntk[c];
        const double u = uni(pr, b, row, 1u + (uint32_t)j, J->ovr,
                             J->ovr ? (size_t)((b * R + row) * (1 + J->maxC) + 1 + j) : 0);
        const double pt = removed[tk] ? 0.0 : P[tk];
        if (M->acc && 1.0 - E > 0.0 && pt > 0.0) M->acc[b * N + c] = fabs(u - pt / (1.0 - E));
        if (u * (1.0 - E) < pt) {
          accepted = c;
          break;
        }
        if (!removed[tk]) {
          removed[tk] = 1;
          E += P[tk];
        }
        ++j;
      }
      if (accepted < 0) {
        double S = 0.0;
        for (int t = 0; t < V; ++t) {
          w[t] = removed[t] ? 0.0 : P[t];
          S += w[t];
        }
        const double u = uni(pr, b, row, 0u, J->ovr, J->ovr ? (size_t)((b * R + row) * (1 + J->maxC)) : 0);
        double mg;
        int alt;
        y = orc_sample(S > 0.0 ? w : P, V, u, &mg, &alt);
        if (M->fin) M->fin[b] = mg;
        if (M->fin_alt) M->fin_alt[b] = alt;
        break;
      }
    }
    path[len] = accepted;
    toks[len] = ntk[accepted];
    ++len;
    row = accepted + 1;
  }
  toks[len] = y;
  J->out_len[b] = len;
}

static void* dtree_worker(void* arg) {
  dtree_job* J = (dtree_job*)arg;
  const size_t V = (size_t)J->V;
  double* z = (double*)malloc(sizeof(double) * V);
  double* P = (double*)malloc(sizeof(double) * V);
  double* w = (double*)malloc(sizeof(double) * V);
  unsigned char* removed = (unsigned char*)malloc(V);
  for (int64_t b = J->b0; b < J->b1; ++b) dtree_one(J, b, z, P, w, removed);
  free(z);
  free(P);
  free(w);
  free(removed);
  return NULL;
}

int orc_verify_tree_det(const void* p, int dtype, int64_t B, int N, int V, const int32_t* parent,
                        const int32_t* node_tokens, double temperature, uint64_t seed, uint32_t step,
                        int32_t* out_tokens, int32_t* out_path, int32_t* out_len,
                        const orc_tree_margins* margins, const double* u_override, int maxC, int nthreads) {
  if (!p || !parent || !node_tokens || !out_tokens || !out_path || !out_len) return -1;
  if (B <= 0 || N <= 0 || V <= 0 || !(temperature >= 0.0)) return -1;
  if (u_override) {
    /* every row's child count must fit the override table */
    for (int64_t b = 0; b < B; ++b)
      for (int r = 0; r <= N; ++r) {
        int nc = 0;
        for (int c = 0; c < N; ++c) nc += parent[b * N + c] == r - 1;
        if (nc > maxC) return -1;
      }
  }
  nthreads = clamp_threads(nthreads, B);
  dtree_job* jobs = (dtree_job*)calloc((size_t)nthreads, sizeof(dtree_job));
  for (int t = 0; t < nthreads; ++t) {
    dtree_job* J = &jobs[t];
    J->p = p;
    J->dtype = dtype;
    J->N = N;
    J->V = V;
    J->parent = parent;
    J->tokens = node_tokens;
    J->pr.temperature = temperature;
    J->pr.seed = seed;
    J->pr.step = step;
    J->out_tokens = out_tokens;
    J->out_path = out_path;
    J->out_len = out_len;
    if (margins) J->mg = *margins;
    J->ovr = u_override;
    J->maxC = maxC;
    J->b0 = B * t / nthreads;
    J->b1 = B * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(dtree_job), nthreads, dtree_worker);
  free(jobs);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Total-variation distillation loss [UnoX §3.2 Diffusion Distillation: one
 * forward gives the frozen AR teacher's logits and the diffusion student's;
 * the TV term minimises the total-variation distance between the two token
 * distributions of a position]. Per row r (a position):
 *   p = softmax(a_r / T) (teacher), q = softmax(d_r / T) (student),
 *   loss_r = 1/2 sum_v |p_v - q_v|.
 * Gradient with respect to the student logits, scaled by the row weight w_r
 * (the upstream gradient of loss_r; the teacher is frozen, so it gets none):
 *   dloss/dq_v = g_v = sign(q_v - p_v) / 2 (0 where q_v == p_v),
 *   dq_v/dd_j  = q_v (delta_vj - q_j) / T,
 *   grad_j     = w_r q_j (g_j - sum_v g_v q_v) / T.
 * A row with a NaN or +inf logit, or entirely -inf, gets a NaN loss and a NaN
 * gradient row. out_grad may be NULL (forward only); row_w NULL means w_r = 1. */
typedef struct {
  const void *p, *q;
  int dtype, V;
  double T;
  const double* w;
  double *loss, *grad;
  int64_t r0, r1;
} tv_job;

static void* tv_worker(void* arg) {
  tv_job* J = (tv_job*)arg;
  const int V = J->V;
  double* a = (double*)malloc(sizeof(double) * (size_t)V);
  double* d = (double*)malloc(sizeof(double) * (size_t)V);
  for (int64_t r = J->r0; r < J->r1; ++r) {
    double* gr = J->grad ? J->grad + r * (int64_t)V : NULL;
    const int bad = orc_decode_row(J->p, J->dtype, r, V, a) | orc_decode_row(J->q, J->dtype, r, V, d);
    if (bad) {
      J->loss[r] = NAN;
      if (gr)
        for (int j = 0; j < V; ++j) gr[j] = NAN;
      continue;
    }
    for (int j = 0; j < V; ++j) {
      a[j] /= J->T;
      d[j] /= J->T;
    }
    const double La = orc_logsumexp(a, V), Ld = orc_logsumexp(d, V);
    double l1 = 0.0, gbar = 0.0;
    for (int j = 0; j < V; ++j) {
      const double P = exp(a[j] - La), Q = exp(d[j] - Ld);
      const double g = Q > P ? 0.5 : (Q < P ? -0.5 : 0.0);
      l1 += fabs(P - Q);
      gbar += g * Q;
      a[j] = P; /* keep P and Q for the gradient */
      d[j] = Q;
    }
    J->loss[r] = 0.5 * l1;
    if (gr) {
      const double w = J->w ? J->w[r] : 1.0;
      for (int j = 0; j < V; ++j) {
        const double g = d[j] > a[j] ? 0.5 : (d[j] < a[j] ? -0.5 : 0.0);
        gr[j] = w * d[j] * (g - gbar) / J->T;
      }
    }
  }
  free(a);
  free(d);
  return NULL;
}

int orc_tv_loss(const void* p, const void* q, int dtype, int64_t R, int V, double temperature, const double* row_w,
                double* out_loss, double* out_grad, int nthreads) {
  if (!p || !q || !out_loss || R <= 0 || V <= 0 || !(temperature > 0.0)) return -1;
  nthreads = clamp_threads(nthreads, R);
  tv_job* jobs = (tv_job*)calloc((size_t)nthreads, sizeof(tv_job));
  for (int t = 0; t < nthreads; ++t) {
    tv_job* J = &jobs[t];
    J->p = p;
    J->q = q;
    J->dtype = dtype;
    J->V = V;
    J->T = temperature;
    J->w = row_w;
    J->loss = out_loss;
    J->grad = out_grad;
    J->r0 = R * t / nthreads;
    J->r1 = R * (t + 1) / nthreads;
  }
  run_jobs(jobs, sizeof(tv_job), nthreads, tv_worker);
  free(jobs);
  return 0;
}
