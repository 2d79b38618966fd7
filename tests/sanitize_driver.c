/*
 * Drives every entry point of the CPU oracle (oracle/oracle.c) and of the
 * synthetic-input generator (synth/synth.c) on small inputs, for a build under
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py).
 * Test infrastructure: it checks memory and arithmetic safety, not values.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* synth/synth.c */
int syn_pair(uint64_t seed, int64_t B, int Rp, int Rq, int V, float sd_a, int n_heavy, float boost, int mode,
             float rho, float sd_noise, int bf16, void* p, void* q, int nthreads);
int syn_randint(uint64_t seed, uint64_t stream, int64_t count, int64_t n, int32_t* out);
int syn_normal(uint64_t seed, uint64_t stream, int64_t count, double* out);
int syn_toy_logits(uint64_t seed, int64_t rows, int V, const int32_t* ctx, const int32_t* pos, int kind, float sd,
                   int n_heavy, float boost, float rho, float noise, int bf16, void* out);

/* oracle/oracle.c (the margin structs repeat the oracle's layouts) */
typedef struct {
  double *acc, *draft, *fin, *filter;
  int32_t *draft_alt, *fin_alt;
} lin_margins;
typedef struct {
  double *acc, *fin, *filter;
  int32_t* fin_alt;
} tree_margins;
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
double orc_uniform(uint64_t seed, uint32_t step, uint32_t b, uint32_t r, uint32_t d);
int orc_decode_row(const void* base, int dtype, int64_t row, int V, double* out);
void orc_filter_row(double* z, int V, double temperature, int top_k, double top_p, double* margin);
double orc_logsumexp(const double* z, int V);
int orc_sample(const double* w, int V, double u, double* margin, int* alt);
int orc_draft_sample(const void* q, int dtype, int64_t B, int K, int V, double temperature, int top_k, double top_p,
                     uint64_t seed, uint32_t step, int32_t* out, double* out_margin, int32_t* out_alt,
                     double* out_margin_filter, const double* u_override, int nthreads);
int orc_verify_linear(const void* p, const void* q, int dtype, int64_t B, int K, int V, int32_t* draft_tokens,
                      double temperature, int top_k, double top_p, uint64_t seed, uint32_t step, int fused,
                      int32_t* out_tokens, int32_t* out_len, double* out_probs, double* out_resid,
                      const lin_margins* margins, const double* u_override, int nthreads);
int orc_tree_depth(const int32_t* parent, int N);
int orc_tree_draft(const void* q, int dtype, int64_t B, int N, int V, const int32_t* parent, double temperature,
                   int top_k, double top_p, uint64_t seed, uint32_t step, int32_t* out, double* out_margin,
                   int32_t* out_alt, double* out_margin_filter, int nthreads);
int orc_verify_tree(const void* p, const void* q, int dtype, int64_t B, int N, int V, const int32_t* parent,
                    const int32_t* node_tokens, double temperature, int top_k, double top_p, uint64_t seed,
                    uint32_t step, int32_t* out_tokens, int32_t* out_path, int32_t* out_len,
                    const tree_margins* margins, const double* u_override, int maxC, int nthreads);
int orc_tree_candidates(const void* q, int dtype, int64_t B, int K, int V, double temperature, int cands, int nodes,
                        int32_t* out_parent, int32_t* out_tokens, double* out_margin, int nthreads);
int orc_verify_tree_det(const void* p, int dtype, int64_t B, int N, int V, const int32_t* parent,
                        const int32_t* node_tokens, double temperature, uint64_t seed, uint32_t step,
                        int32_t* out_tokens, int32_t* out_path, int32_t* out_len, const tree_margins* margins,
                        const double* u_override, int maxC, int nthreads);
int orc_tv_loss(const void* p, const void* q, int dtype, int64_t R, int V, double temperature, const double* row_w,
                double* out_loss, double* out_grad, int nthreads);

#define CHECK(x)                                             \
  do {                                                       \
    if (!(x)) {                                              \
      fprintf(stderr, "check failed: %s (line %d)\n", #x, __LINE__); \
      return 1;                                              \
    }                                                        \
  } while (0)

static int run(int dtype, int nthreads) {
  const int B = 5, K = 3, V = 1001, esz = dtype ? 2 : 4;
  char* p = malloc((size_t)B * (K + 1) * V * esz);
  char* q = malloc((size_t)B * K * V * esz);
  CHECK(syn_pair(7, B, K + 1, K, V, 2.0f, 4, 6.0f, 1, 0.8f, 1.0f, dtype, p, q, nthreads) == 0);
  /* one invalid request: a NaN logit (fp32 only; bfloat16 NaN bits likewise) */
  if (dtype == 0) ((float*)p)[(size_t)(2 * (K + 1) + 1) * V + 9] = NAN;
  else ((uint16_t*)p)[(size_t)(2 * (K + 1) + 1) * V + 9] = 0x7fc0u;

  int32_t draft[5 * 3], toks[5 * 4], len[5], dalt[5 * 3], falt[5];
  double probs[5 * 3 * 2], resid[5], macc[5 * 3], mdr[5 * 3], mfin[5], mflt[5], dm[5 * 3], dmf[5 * 3];
  lin_margins lm = {macc, mdr, mfin, mflt, dalt, falt};
  CHECK(orc_draft_sample(q, dtype, B, K, V, 0.9, 0, 1.0, 3, 1, draft, dm, dalt, dmf, NULL, nthreads) == 0);
  CHECK(orc_draft_sample(q, dtype, B, K, V, 0.9, 20, 0.9, 3, 1, draft, dm, dalt, dmf, NULL, nthreads) == 0);
  CHECK(orc_draft_sample(q, dtype, B, K, V, 0.0, 0, 1.0, 3, 1, draft, NULL, NULL, NULL, NULL, nthreads) == 0);
  for (int i = 0; i < B * K; ++i) draft[i] = (draft[i] < 0 ? 0 : draft[i]);
  CHECK(orc_verify_linear(p, q, dtype, B, K, V, draft, 1.0, 0, 1.0, 3, 2, 0, toks, len, probs, resid, &lm, NULL,
                          nthreads) == 0);
  CHECK(orc_verify_linear(p, q, dtype, B, K, V, draft, 0.7, 30, 0.8, 3, 2, 1, toks, len, probs, resid, &lm, NULL,
                          nthreads) == 0);
  CHECK(orc_verify_linear(p, q, dtype, B, K, V, draft, 0.0, 0, 1.0, 3, 2, 1, toks, len, NULL, NULL, NULL, NULL,
                          nthreads) == 0);
  double ovr[5 * 4 * 3];
  for (int i = 0; i < B * (K + 1) * 3; ++i) ovr[i] = (double)((i * 37) % 100) / 100.0;
  CHECK(orc_verify_linear(p, q, dtype, B, K, V, draft, 1.3, 0, 0.5, 3, 2, 1, toks, len, probs, resid, &lm, ovr,
                          nthreads) == 0);

  /* tree: a root with two children, each heading a chain of two */
  const int32_t parent[6] = {-1, -1, 0, 1, 2, 3};
  const int N = 6, R = N + 1;
  CHECK(orc_tree_depth(parent, N) == 3);
  char* tp = malloc((size_t)B * R * V * esz);
  char* tq = malloc((size_t)B * R * V * esz);
  CHECK(syn_pair(9, B, R, R, V, 2.0f, 0, 0.0f, 0, 0.0f, 1.0f, dtype, tp, tq, nthreads) == 0);
  int32_t nodes[5 * 6], nalt[5 * 6], ttok[5 * 4], tpath[5 * 3], tlen[5], talt[5];
  double nm[5 * 6], nmf[5 * 6], tacc[5 * 6], tfin[5], tflt[5];
  tree_margins tm = {tacc, tfin, tflt, talt};
  CHECK(orc_tree_draft(tq, dtype, B, N, V, parent, 1.0, 25, 0.9, 4, 0, nodes, nm, nalt, nmf, nthreads) == 0);
  for (int i = 0; i < B * N; ++i) nodes[i] = nodes[i] < 0 ? 0 : nodes[i];
  CHECK(orc_verify_tree(tp, tq, dtype, B, N, V, parent, nodes, 1.0, 25, 0.9, 4, 0, ttok, tpath, tlen, &tm, NULL, 0,
                        nthreads) == 0);
  CHECK(orc_verify_tree(tp, tq, dtype, B, N, V, parent, nodes, 0.0, 0, 1.0, 4, 0, ttok, tpath, tlen, NULL, NULL, 0,
                        nthreads) == 0);

  /* Tree Sampler candidates and their verification (per-request trees) */
  const int C = 4, NN = 9;
  int32_t cpar[5 * 9], ctok[5 * 9], dtok[5 * 10], dpath[5 * 9], dlen[5];
  double cgap[5 * 9];
  CHECK(orc_tree_candidates(q, dtype, B, K, V, 1.0, C, NN, cpar, ctok, cgap, nthreads) == 0);
  for (int i = 0; i < B * NN; ++i) {
    if (cpar[i] < -1) cpar[i] = -1;
    if (ctok[i] < 0) ctok[i] = 0;
  }
  char* dp = malloc((size_t)B * (NN + 1) * V * esz);
  CHECK(syn_pair(11, B, NN + 1, 0, V, 2.0f, 3, 8.0f, 0, 0.0f, 1.0f, dtype, dp, NULL, nthreads) == 0);
  double dacc[5 * 9], dfin[5], dflt[5];
  int32_t dalt2[5];
  tree_margins dm2 = {dacc, dfin, dflt, dalt2};
  CHECK(orc_verify_tree_det(dp, dtype, B, NN, V, cpar, ctok, 1.0, 5, 1, dtok, dpath, dlen, &dm2, NULL, 0, nthreads) ==
        0);
  CHECK(orc_verify_tree_det(dp, dtype, B, NN, V, cpar, ctok, 0.0, 5, 1, dtok, dpath, dlen, NULL, NULL, 0, nthreads) ==
        0);

  /* TV loss, forward and backward */
  double loss[5 * 3], *grad = malloc(sizeof(double) * (size_t)B * K * V), rw[5 * 3];
  for (int i = 0; i < B * K; ++i) rw[i] = 1.0 / (i + 1);
  CHECK(orc_tv_loss(p, q, dtype, (int64_t)B * K, V, 1.0, rw, loss, grad, nthreads) == 0);
  CHECK(orc_tv_loss(p, q, dtype, (int64_t)B * K, V, 0.5, NULL, loss, NULL, nthreads) == 0);

  /* helpers */
  double z[1001], w[1001], mg;
  int alt;
  CHECK(orc_decode_row(p, dtype, 0, V, z) == 0);
  orc_filter_row(z, V, 0.8, 10, 0.7, &mg);
  CHECK(isfinite(orc_logsumexp(z, V)));
  for (int j = 0; j < V; ++j) w[j] = isinf(z[j]) ? 0.0 : exp(z[j]);
  CHECK(orc_sample(w, V, 0.5, &mg, &alt) >= 0);
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
  orc_philox4x32_10(ctr, key, out);
  CHECK(orc_uniform(1, 2, 3, 4, 5) < 1.0);

  /* generators */
  int32_t ri[64], ctx[2 * 8], pos[8];
  double nr[64];
  CHECK(syn_randint(1, 2, 64, 1000, ri) == 0);
  CHECK(syn_normal(1, 2, 64, nr) == 0);
  for (int i = 0; i < 8; ++i) {
    ctx[2 * i] = ri[i];
    ctx[2 * i + 1] = ri[i + 8];
    pos[i] = i;
  }
  char* tl = malloc((size_t)8 * 777 * esz);
  CHECK(syn_toy_logits(3, 8, 777, ctx, NULL, 0, 2.0f, 4, 6.0f, 0.8f, 1.5f, dtype, tl) == 0);
  CHECK(syn_toy_logits(3, 8, 777, ctx, pos, 1, 2.0f, 4, 6.0f, 0.8f, 1.5f, dtype, tl) == 0);

  free(p);
  free(q);
  free(tp);
  free(tq);
  free(dp);
  free(grad);
  free(tl);
  return 0;
}

int main(void) {
  for (int dtype = 0; dtype < 2; ++dtype)
    for (int nt = 1; nt <= 3; nt += 2)
      if (run(dtype, nt)) return 1;
  puts("sanitize driver: every entry point ran");
  return 0;
}
