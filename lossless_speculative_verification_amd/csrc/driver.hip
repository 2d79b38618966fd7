// Multi-round Psi-Spec generation on gfx950 ("Uno" research explainer, §3.3:
// every round runs one draft pass and one verify pass; the block's first
// position comes from the AR weights and is always kept, the other block - 1
// positions are proposed in parallel by the drafter, the verifier keeps the
// longest accepted prefix and adds the residual or bonus token; tokens per
// forward pass lie in [1, (block + 1) / 2]).
//
// The model is a synthetic order-2 language model (toy target and drafter
// logits computed from the last two tokens), a stand-in for the AR and
// diffusion passes; it is defined by integer mixing (SplitMix64: Steele, Lea,
// Flood, OOPSLA 2014) and fixed-order double arithmetic so that any
// implementation of the definition gives the same bits:
//   ctx  = (uint32 t1 << 32) | uint32 t2
//   bits(s, stream, i) = mix(mix(s ^ mix(stream * C1 + C2)) ^ (i * C3)), mix = SplitMix64
//   z(r) = ((sum of the four 16-bit fields of r) / 65536 - 2) * sqrt(3)
//   target a(v | ctx) = float(sd * z(r) + (top 10 bits of mix(r) < n_heavy ? boost : 0)),
//                       r = bits(seed, ctx, v)
//   draft  d(v | ctx, i) = float(rho * a + noise * z(bits(seed ^ K_DRAFT, ctx * 64 + i, v)))
// then bfloat16 by round-to-nearest-even (or float32 kept).
//
// Per round, on the caller's stream: contexts -> toy target row -> draft
// sample (first token) -> contexts -> toy drafter rows -> draft sample ->
// contexts -> toy target rows -> linear verification -> commit.
#include "rowops.hpp"

// The toy model's double arithmetic rounds every operation on its own.
#pragma clang fp contract(off)

namespace psi {

namespace {

constexpr uint64_t kToyDraftKey = 0xA5A5A5A55A5A5A5Aull;

__device__ __forceinline__ uint64_t mix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}
// The per-(seed, stream) key of bits(); bits(s, stream, i) = mix(key ^ (i * C3)).
__device__ __forceinline__ uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(seed ^ mix64(stream * 0x632BE59BD9B4E019ull + 0x2545F4914F6CDD1Dull));
}
__device__ __forceinline__ uint64_t keyed_bits(uint64_t key, uint64_t i) { return mix64(key ^ (i * 0xD1B54A32D192ED03ull)); }

__device__ __forceinline__ double toy_z(uint64_t r) {
  const uint64_t s = (r & 0xffffull) + ((r >> 16) & 0xffffull) + ((r >> 32) & 0xffffull) + (r >> 48);
  const double u = (double)s / 65536.0 - 2.0;
  return u * 1.7320508075688772;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace

// Toy logits of `rows` rows, 8 consecutive tokens per thread. ctx [rows, 2],
// pos [rows] (drafter only).
template <int DT>
__global__ __launch_bounds__(kWG) void k_toy_logits(int64_t rows, int V, const int32_t* ctx, const int32_t* pos,
                                                    int kind, psispec_toy_model m, void* out) {
  const int64_t k = blockIdx.y;
  const int64_t v0 = ((int64_t)blockIdx.x * kWG + threadIdx.x) * 8;
  if (v0 >= V) return;
  const uint64_t c = ((uint64_t)(uint32_t)ctx[2 * k] << 32) | (uint64_t)(uint32_t)ctx[2 * k + 1];
  const uint64_t kt = stream_key(m.seed, c);
  const uint64_t kd = kind == 1 ? stream_key(m.seed ^ kToyDraftKey, c * 64u + (uint64_t)(uint32_t)pos[k]) : 0;
  const double sd = m.sd, boost = m.boost, rho = m.rho, noise = m.noise;
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint64_t v = (uint64_t)(v0 + e);
    const uint64_t r = keyed_bits(kt, v);
    double a = sd * toy_z(r);
    if ((int)(mix64(r) >> 54) < m.n_heavy) a = a + boost;
    float y = (float)a;
    if (kind == 1) {
      const double t1 = rho * (double)y;
      const double t2 = noise * toy_z(keyed_bits(kd, v));
      y = (float)(t1 + t2);
    }
    x[e] = y;
  }
  const int64_t base = k * (int64_t)V + v0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (v0 + e >= V) break;
    if constexpr (DT == kBF16) ((uint16_t*)out)[base + e] = bf16_rne(x[e]);
    else ((float*)out)[base + e] = x[e];
  }
}

// Contexts of the rows of one pass: 0 = the first position (t1, t2); 1 = the
// drafter rows (t2, x0) at positions 1 .. K; 2 = the target rows
// (h_i, h_{i+1}), h = (t2, x0, d_0 .. d_{K-1}), i = 0 .. K.
__global__ __launch_bounds__(kWG) void k_round_ctx(int64_t B, int K, int kind, GenState g) {
  const int64_t idx = (int64_t)blockIdx.x * kWG + threadIdx.x;
  if (kind == 0) {
    if (idx >= B) return;
    g.ctx[2 * idx] = g.t12[2 * idx];
    g.ctx[2 * idx + 1] = g.t12[2 * idx + 1];
  } else if (kind == 1) {
    if (idx >= B * K) return;
    const int64_t b = idx / K;
    const int i = (int)(idx - b * K);
    g.ctx[2 * idx] = g.t12[2 * b + 1];
    g.ctx[2 * idx + 1] = g.x0[b];
    g.pos[idx] = i + 1;
  } else {
    if (idx >= B * (K + 1)) return;
    const int64_t b = idx / (K + 1);
    const int i = (int)(idx - b * (K + 1));
    auto h = [&](int j) { return j == 0 ? g.t12[2 * b + 1] : (j == 1 ? g.x0[b] : g.drafts[b * K + (j - 2)]); };
    g.ctx[2 * idx] = h(i);
    g.ctx[2 * idx + 1] = h(i + 1);
  }
}

// Commit of round r: the first token, the accepted drafts and the final token
// are appended (the rejected drafts are dropped), the round's count recorded
// and the context advanced. A request with a verification error (len < 0)
// commits nothing more and its length turns negative.
__global__ __launch_bounds__(kWG) void k_commit(int64_t B, int K, int r, int rounds, int max_len, GenState g,
                                                int32_t* seq, int32_t* len, int32_t* round_tokens) {
  const int64_t b = (int64_t)blockIdx.x * kWG + threadIdx.x;
  if (b >= B) return;
  int L = len[b];
  const int n = g.vlen[b];
  if (L < 0 || n < 0) {
    len[b] = -1;
    round_tokens[b * rounds + r] = 0;
    return;
  }
  int32_t* s = seq + b * (int64_t)max_len;
  int cnt = 0;
  auto put = [&](int32_t x) {
    if (L < max_len) s[L] = x;
    ++L;
    ++cnt;
  };
  put(g.x0[b]);
  for (int i = 0; i <= n; ++i) put(g.vtok[b * (K + 1) + i]);
  round_tokens[b * rounds + r] = cnt;
  len[b] = L;
  // the last two committed tokens: (second to last, last)
  g.t12[2 * b] = n >= 1 ? g.vtok[b * (K + 1) + n - 1] : g.x0[b];
  g.t12[2 * b + 1] = g.vtok[b * (K + 1) + n];
}

__global__ __launch_bounds__(kWG) void k_gen_init(int64_t B, const int32_t* prompt, GenState g, int32_t* len,
                                                  int32_t* seq, int max_len) {
  const int64_t idx = (int64_t)blockIdx.x * kWG + threadIdx.x;
  if (idx < B) {
    g.t12[2 * idx] = prompt[2 * idx];
    g.t12[2 * idx + 1] = prompt[2 * idx + 1];
    len[idx] = 0;
  }
  for (int64_t j = idx; j < B * (int64_t)max_len; j += (int64_t)gridDim.x * kWG) seq[j] = -1;
}

namespace {
inline size_t al256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

// Workspace of a generation call: the three logit buffers, the verifier's
// workspace, then the driver state.
GenLayout gen_layout(int64_t B, int K, int V, int esz, size_t inner_bytes) {
  GenLayout L;
  size_t off = 0;
  L.first = off;
  off = al256(off + (size_t)B * V * esz);
  L.q = off;
  off = al256(off + (size_t)B * K * V * esz);
  L.p = off;
  off = al256(off + (size_t)B * (K + 1) * V * esz);
  L.inner = off;
  L.inner_bytes = inner_bytes;
  off = al256(off + inner_bytes);
  L.st = off;
  const size_t ints = (size_t)B * (2 + 1 + K + (K + 1) + 1 + 2 * (K + 1) + K);
  off = al256(off + ints * sizeof(int32_t));
  L.total = off;
  return L;
}

GenState gen_state(void* ws, const GenLayout& L, int64_t B, int K) {
  int32_t* w = (int32_t*)((char*)ws + L.st);
  GenState g;
  g.t12 = w;
  w += 2 * B;
  g.x0 = w;
  w += B;
  g.drafts = w;
  w += B * K;
  g.vtok = w;
  w += B * (K + 1);
  g.vlen = w;
  w += B;
  g.ctx = w;
  w += 2 * B * (K + 1);
  g.pos = w;
  return g;
}

hipError_t launch_gen_init(int64_t B, const int32_t* prompt, const GenState& g, int32_t* len, int32_t* seq,
                           int max_len, hipStream_t s) {
  const unsigned grid = (unsigned)((B * (int64_t)max_len + kWG - 1) / kWG);
  PSI_LAUNCH(s, k_gen_init, dim3(grid < 1024u ? grid : 1024u), dim3(kWG), B, prompt, g, len, seq, max_len);
  return hipGetLastError();
}
hipError_t launch_round_ctx(int64_t B, int K, int kind, const GenState& g, hipStream_t s) {
  const int64_t n = kind == 0 ? B : (kind == 1 ? B * K : B * (K + 1));
  PSI_LAUNCH(s, k_round_ctx, dim3((unsigned)((n + kWG - 1) / kWG)), dim3(kWG), B, K, kind, g);
  return hipGetLastError();
}
hipError_t launch_commit(int64_t B, int K, int r, int rounds, int max_len, const GenState& g, int32_t* seq,
                         int32_t* len, int32_t* round_tokens, hipStream_t s) {
  PSI_LAUNCH(s, k_commit, dim3((unsigned)((B + kWG - 1) / kWG)), dim3(kWG), B, K, r, rounds, max_len, g, seq, len,
             round_tokens);
  return hipGetLastError();
}

hipError_t launch_toy_logits(int64_t rows, int V, const int32_t* ctx, const int32_t* pos, int kind,
                             const psispec_toy_model& m, int dtype, void* out, hipStream_t s) {
  const dim3 grid((unsigned)((V + kWG * 8 - 1) / (kWG * 8)), (unsigned)rows);
  if (dtype == kBF16) PSI_LAUNCH(s, k_toy_logits<kBF16>, grid, dim3(kWG), rows, V, ctx, pos, kind, m, out);
  else PSI_LAUNCH(s, k_toy_logits<kF32>, grid, dim3(kWG), rows, V, ctx, pos, kind, m, out);
  return hipGetLastError();
}

}  // namespace psi
