/*
 * Seeded synthetic logits for the verification workloads.
 *
 * This module only makes input data; it holds none of the verification
 * arithmetic (no normalisation, ratio, sampling or Philox). Both the GPU tests
 * and the oracle read the arrays it fills, bit for bit.
 *
 * Random numbers: SplitMix64 (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) applied to a counter built
 * from (seed, stream, index), so every element depends only on its own index
 * and the result does not depend on the thread count. Normals come from the
 * Box-Muller transform in double, then round to binary32, then (for bf16
 * output) round-to-nearest-even to bfloat16.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static inline uint64_t splitmix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

/* 64 random bits for (seed, stream, index). */
static inline uint64_t bits64(uint64_t seed, uint64_t stream, uint64_t index) {
  uint64_t k = splitmix64(seed ^ splitmix64(stream * 0x632BE59BD9B4E019ull + 0x2545F4914F6CDD1Dull));
  return splitmix64(k ^ (index * 0xD1B54A32D192ED03ull));
}

/* Uniform in (0, 1] with 53 bits. */
static inline double unit_open0(uint64_t r) { return ((double)(r >> 11) + 1.0) * (1.0 / 9007199254740992.0); }

/* Standard normal for element `index` of (seed, stream): Box-Muller on the
 * pair index/2, cosine branch for even and sine branch for odd indices. */
static inline double normal_at(uint64_t seed, uint64_t stream, uint64_t index) {
  uint64_t pair = index >> 1;
  double u1 = unit_open0(bits64(seed, stream, 2 * pair));
  double u2 = unit_open0(bits64(seed, stream, 2 * pair + 1));
  double rad = sqrt(-2.0 * log(u1));
  double ang = 6.283185307179586 * u2;
  return (index & 1) ? rad * sin(ang) : rad * cos(ang);
}

static inline uint16_t to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40); /* keep NaN a NaN */
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline void store(void* out, int bf16, size_t idx, float v) {
  if (bf16)
    ((uint16_t*)out)[idx] = to_bf16_rne(v);
  else
    ((float*)out)[idx] = v;
}

/* ------------------------------------------------------------------------ */
typedef struct {
  uint64_t seed;
  int64_t B;
  int Rp, Rq, V;
  float sd_a;
  int n_heavy;
  float boost;
  int mode; /* 0: d = a + sd_noise*eps;  1: d = rho*a + sqrt(1-rho^2)*sd_noise*eps */
  float rho, sd_noise;
  int bf16;
  void *p, *q;
  int64_t row0, row1; /* range of request-rows (b, i) with i < Rp handled by this worker */
} pair_job;

/* Heavy ids of target row (b, i): n_heavy distinct ids, uniform over [0, V). */
static int heavy_ids(const pair_job* J, int64_t prow, int* ids) {
  int n = 0;
  uint64_t ctr = 0;
  while (n < J->n_heavy && n < J->V) {
    uint64_t r = bits64(J->seed, 2, (uint64_t)prow * 4096u + ctr++);
    int id = (int)(r % (uint64_t)J->V);
    int dup = 0;
    for (int t = 0; t < n; ++t) dup |= ids[t] == id;
    if (!dup) ids[n++] = id;
  }
  return n;
}

static void* pair_worker(void* arg) {
  pair_job* J = (pair_job*)arg;
  const size_t V = (size_t)J->V;
  float* a = (float*)malloc(sizeof(float) * V);
  int ids[1024];
  const double cnoise = J->mode == 1 ? sqrt(fmax(0.0, 1.0 - (double)J->rho * J->rho)) * J->sd_noise : J->sd_noise;
  for (int64_t rr = J->row0; rr < J->row1; ++rr) {
    int64_t b = rr / J->Rp;
    int i = (int)(rr % J->Rp);
    int64_t prow = b * J->Rp + i;
    for (size_t j = 0; j < V; ++j) a[j] = (float)(J->sd_a * normal_at(J->seed, 0, (uint64_t)prow * V + j));
    int nh = heavy_ids(J, prow, ids);
    for (int t = 0; t < nh; ++t) a[ids[t]] = a[ids[t]] + J->boost;
    for (size_t j = 0; j < V; ++j) store(J->p, J->bf16, (size_t)prow * V + j, a[j]);
    if (i < J->Rq) {
      int64_t qrow = b * J->Rq + i;
      for (size_t j = 0; j < V; ++j) {
        double eps = normal_at(J->seed, 1, (uint64_t)qrow * V + j);
        double d = J->mode == 1 ? (double)J->rho * a[j] + cnoise * eps : (double)a[j] + cnoise * eps;
        store(J->q, J->bf16, (size_t)qrow * V + j, (float)d);
      }
    }
  }
  free(a);
  return NULL;
}

/*
 * Fills target logits p [B, Rp, V] and draft logits q [B, Rq, V] (Rq <= Rp;
 * draft row (b, i) pairs with target row (b, i)):
 *   a = sd_a * N(0,1) per element, then + boost on n_heavy distinct ids per row;
 *   mode 0: d = a + sd_noise * N(0,1)
 *   mode 1: d = rho * a + sqrt(1 - rho^2) * sd_noise * N(0,1)
 * Output is binary32, or bfloat16 bits (round to nearest even) if bf16 != 0.
 */
int syn_pair(uint64_t seed, int64_t B, int Rp, int Rq, int V, float sd_a, int n_heavy, float boost, int mode,
             float rho, float sd_noise, int bf16, void* p, void* q, int nthreads) {
  if (B <= 0 || Rp <= 0 || Rq < 0 || Rq > Rp || V <= 0 || !p || (Rq > 0 && !q) || n_heavy < 0 || n_heavy > 1024)
    return -1;
  if (nthreads < 1) nthreads = 1;
  int64_t rows = B * Rp;
  if (nthreads > rows) nthreads = (int)rows;
  pair_job* jobs = (pair_job*)calloc((size_t)nthreads, sizeof(pair_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  for (int t = 0; t < nthreads; ++t) {
    pair_job* J = &jobs[t];
    J->seed = seed;
    J->B = B;
    J->Rp = Rp;
    J->Rq = Rq;
    J->V = V;
    J->sd_a = sd_a;
    J->n_heavy = n_heavy;
    J->boost = boost;
    J->mode = mode;
    J->rho = rho;
    J->sd_noise = sd_noise;
    J->bf16 = bf16;
    J->p = p;
    J->q = q;
    J->row0 = rows * t / nthreads;
    J->row1 = rows * (t + 1) / nthreads;
    pthread_create(&th[t], NULL, pair_worker, J);
  }
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  free(jobs);
  free(th);
  return 0;
}

/* Uniform integers in [0, n) for index i of (seed, stream): out[i], i < count. */
int syn_randint(uint64_t seed, uint64_t stream, int64_t count, int64_t n, int32_t* out) {
  if (count < 0 || n <= 0 || !out) return -1;
  for (int64_t i = 0; i < count; ++i) out[i] = (int32_t)(bits64(seed, stream, (uint64_t)i) % (uint64_t)n);
  return 0;
}

/* Standard normals for index i of (seed, stream), as double. */
int syn_normal(uint64_t seed, uint64_t stream, int64_t count, double* out) {
  if (count < 0 || !out) return -1;
  for (int64_t i = 0; i < count; ++i) out[i] = normal_at(seed, stream, (uint64_t)i);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Toy order-2 language model, a synthetic stand-in for the AR target and the
 * diffusion drafter of a multi-round generation loop. Integer mixing and
 * fixed-order double arithmetic only, so that a GPU implementation written
 * from this definition gives the same bits:
 *   ctx  = (uint32 t1 << 32) | uint32 t2   (the last two tokens)
 *   r    = bits64(seed, ctx, v)            (SplitMix64 construction above)
 *   z(r) = ((sum of the four 16-bit fields of r) / 65536 - 2) * sqrt(3)
 *          (an Irwin-Hall approximation of a standard normal)
 *   target a(v | ctx) = float(sd * z(r) + (top 10 bits of splitmix64(r) < n_heavy ? boost : 0))
 *   draft  d(v | ctx, i) = float(rho * a + noise * z(bits64(seed ^ K_DRAFT, ctx * 64 + i, v)))
 * with every double operation rounded on its own (no fused multiply-add),
 * then bfloat16 by round-to-nearest-even (or float32 kept). */
#define TOY_DRAFT_KEY 0xA5A5A5A55A5A5A5Aull
static inline double toy_z(uint64_t r) {
  const uint64_t s = (r & 0xffffull) + ((r >> 16) & 0xffffull) + ((r >> 32) & 0xffffull) + (r >> 48);
  const double u = (double)s / 65536.0 - 2.0;
  return u * 1.7320508075688772;
}

static inline float toy_target(uint64_t seed, uint64_t ctx, int v, double sd, int n_heavy, double boost) {
  const uint64_t r = bits64(seed, ctx, (uint64_t)v);
  double a = sd * toy_z(r);
  if ((int)(splitmix64(r) >> 54) < n_heavy) a = a + boost;
  return (float)a;
}

/* Logits of `rows` rows: row k has context ctx[2k], ctx[2k+1] (t1, t2); kind 0
 * gives the target, kind 1 the draft at position pos[k]. */
int syn_toy_logits(uint64_t seed, int64_t rows, int V, const int32_t* ctx, const int32_t* pos, int kind, float sd,
                   int n_heavy, float boost, float rho, float noise, int bf16, void* out) {
  if (rows <= 0 || V <= 0 || !ctx || !out || (kind == 1 && !pos)) return -1;
  for (int64_t k = 0; k < rows; ++k) {
    const uint64_t c = ((uint64_t)(uint32_t)ctx[2 * k] << 32) | (uint64_t)(uint32_t)ctx[2 * k + 1];
    for (int v = 0; v < V; ++v) {
      const float a = toy_target(seed, c, v, (double)sd, n_heavy, (double)boost);
      float x = a;
      if (kind == 1) {
        const double zn = toy_z(bits64(seed ^ TOY_DRAFT_KEY, c * 64u + (uint64_t)(uint32_t)pos[k], (uint64_t)v));
        const double t1 = (double)rho * (double)a;
        const double t2 = (double)noise * zn;
        x = (float)(t1 + t2);
      }
      store(out, bf16, (size_t)k * (size_t)V + (size_t)v, x);
    }
  }
  return 0;
}
