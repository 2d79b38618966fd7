// Total-variation distillation loss on gfx950 ("Uno" research explainer,
// §3.2 Diffusion Distillation: the TV term minimises the total-variation
// distance between the frozen AR teacher's token distribution p and the
// diffusion student's q at every position; it governs the acceptance of the
// verifier, since sum min(p, q) = 1 - TV).
//
// Per row r: loss_r = 1/2 sum_v |p_v - q_v|, and the gradient with respect to
// the student logits, scaled by the row weight w_r:
//   grad_j = w_r q_j (g_j - gbar) / T,  g_v = sign(q_v - p_v) / 2 (0 on ties),
//   gbar = sum_v g_v q_v.
// Pipeline on the caller's stream (streaming the rows in chunks that fit the
// last-level cache between the passes measured slower than whole passes):
//   k_stats32   maxima and binary32-grade sums of every teacher and student row;
//   k_tv_rows   a wave per teacher or student row: its maximum and normaliser
//               from the chunk records, once;
//   k_tv_pass   (sub-block, row): sum |p - q| and sum g q per 1,024 logits,
//               and (with a gradient) the sign of q - p of every logit, two
//               bits each, 16 bits per 16-byte vector;
//   k_tv_grad   (sub-block, row): the row's loss and gbar from those records,
//               then the gradient from q and the stored signs (p is not read
//               again), written in the logits' dtype.
// p and q are evaluated as 2^((a - m) c) / S in binary32 from the same
// statistics in both passes, so the signs g_v of the two passes agree.
#include "rowops.hpp"

// No contraction in this file: P and Q are rounded before they are compared
// or subtracted.
#pragma clang fp contract(off)

namespace psi {

namespace {

// Row maximum and normaliser of one row from its statistics records, by one
// wave (lane i holds record i, i < nch <= 64 per round). Returns false for an
// invalid row (NaN or +inf, or entirely -inf).
__device__ __forceinline__ bool wave_row_norm(const StatRec* rec, int nch, float c32, float* m_out, double* S_out) {
  const int lane = threadIdx.x & (kWave - 1);
  float m = -INFINITY;
  int bad = 0;
  for (int i = lane; i < nch; i += kWave) {
    const StatRec r = rec[i];
    m = fmaxnan(m, r.m);
    bad |= isnan(r.s) ? 1 : 0;
  }
  m = wave_max(m);
  double S = 0.0;
  if (!isnan(m) && !isinf(m))
    for (int i = lane; i < nch; i += kWave) {
      const StatRec r = rec[i];
      if (!is_neg_inf(r.m)) S += r.s * ::exp2(((double)r.m - (double)m) * (double)c32);
    }
  S = wave_sum(S);
  bad = wave_or(bad);
  *m_out = m;
  *S_out = S;
  return !(bad || isnan(m) || isinf(m) || !(S > 0.0));
}

struct TvRow {
  float mp, mq;     // row maxima
  float mcp, mcq;   // m * c
  float ip, iq;     // 1 / S
  bool ok;
};

__device__ __forceinline__ TvRow tv_row(const LinCfg& c, const RowStat* rn, int64_t r) {
  TvRow t;
  const RowStat a = rn[2 * r], d = rn[2 * r + 1];
  t.mp = a.m;
  t.mq = d.m;
  const double Sp = a.s, Sq = d.s;
  t.ok = !a.bad && !d.bad;
  t.mcp = t.mp * c.c32;
  t.mcq = t.mq * c.c32;
  t.ip = (float)(1.0 / Sp);
  t.iq = (float)(1.0 / Sq);
  return t;
}

// Teacher and student probabilities of one logit pair (binary32). Equal logit
// rows give equal P and Q, and |P - Q| is 0 there.
__device__ __forceinline__ void tv_probs(const TvRow& t, float c32, float a, float d, float& P, float& Q) {
  P = __builtin_amdgcn_exp2f(__builtin_fmaf(a, c32, -t.mcp)) * t.ip;
  Q = __builtin_amdgcn_exp2f(__builtin_fmaf(d, c32, -t.mcq)) * t.iq;
}


// sub-blocks per wave (the row normalisers are read once per wave): the
// first pass holds two rows' vectors per sub-block, the second one row's and
// keeps the next sub-block's loads in flight
constexpr int kTvSpwPass = 4;
constexpr int kTvSpwGrad = 8;

}  // namespace

// Maximum and normaliser of every teacher and student row (rn[2 r], rn[2 r + 1]),
// a wave per row.
__global__ __launch_bounds__(kWG) void k_tv_rows(LinCfg c, RowStat* rn, int64_t rows) {
  const int64_t sr = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  if (sr >= rows) return;
  float m;
  double S;
  const bool ok = wave_row_norm(c.st + sr * (int64_t)c.nch32, c.nch32, c.c32, &m, &S);
  if ((threadIdx.x & (kWave - 1)) == 0) rn[sr] = RowStat{m, ok ? 0 : 1, S};
}

// c.rows: np = 1 teacher row and nq = 1 student row per "request" (= row of
// the loss); row blockIdx.y.
// Sign code of q - p: 0 tie, 1 positive (g = +1/2), 2 negative (g = -1/2).
__device__ __forceinline__ float tv_code_g(uint32_t code) { return code == 1u ? 0.5f : (code == 2u ? -0.5f : 0.0f); }

template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_tv_pass(LinCfg c, const RowStat* rn, uint16_t* sgn) {
  constexpr int EPV = Elem<DT>::kPerVec;
  constexpr int VPL = kSB / (kWave * EPV);
  const int64_t r = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int sb0 = (blockIdx.x * kWaves + wave) * kTvSpwPass;
  if (sb0 >= c.nsb) return;
  const int64_t nv = ((int64_t)c.V + EPV - 1) / EPV;  // sign words per row
  const TvRow t = tv_row(c, rn, r);
  const char* prow = c.rows.p + (r * (int64_t)c.V) * c.rows.esz;
  const char* qrow = c.rows.q + (r * (int64_t)c.V) * c.rows.esz;
  for (int sb = sb0; sb < sb0 + kTvSpwPass && sb < c.nsb; ++sb) {
    const int64_t vfirst = (int64_t)sb * (kSB / EPV) + lane;
    float xa[VPL][EPV], xd[VPL][EPV];
    load_vecs<DT, AL, VPL, kWave>(prow, c.V, c.nvec, vfirst, xa);
    load_vecs<DT, AL, VPL, kWave>(qrow, c.V, c.nvec, vfirst, xd);
    float l1 = 0.0f, gq = 0.0f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      uint32_t code = 0;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        float P, Q;
        tv_probs(t, c.c32, xa[v][e], xd[v][e], P, Q);
        l1 += fabsf(P - Q);
        const bool gt = Q > P, lt = Q < P;  // the sign and its code share the compares
        gq = __builtin_fmaf(gt ? 0.5f : (lt ? -0.5f : 0.0f), Q, gq);
        code |= ((gt ? 1u : 0u) | (lt ? 2u : 0u)) << (2 * e);
      }
      const int64_t vec = vfirst + (int64_t)v * kWave;
      if (sgn != nullptr && vec < nv) sgn[r * nv + vec] = (uint16_t)code;
    }
    const double L1 = wave_sum((double)l1), GQ = wave_sum((double)gq);
    if (lane == 0) c.res[r * c.nsb + sb] = ResRec{L1, GQ, 0.0, 0.0};
  }
}

template <int DT>
__device__ __forceinline__ void store_grad(void* g, int64_t j, float x);
template <>
__device__ __forceinline__ void store_grad<kF32>(void* g, int64_t j, float x) {
  ((float*)g)[j] = x;
}
template <>
__device__ __forceinline__ void store_grad<kBF16>(void* g, int64_t j, float x) {
  // round to nearest even (NaN kept quiet)
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = isnan(x) ? (u | 0x00400000u) : u + 0x7fffu + ((u >> 16) & 1u);
  ((uint16_t*)g)[j] = (uint16_t)(r >> 16);
}

// Packs EPV binary32 values into one 16-byte vector of the logits' dtype.
template <int DT>
__device__ __forceinline__ uint4 pack_grad(const float (&x)[Elem<DT>::kPerVec]);
template <>
__device__ __forceinline__ uint4 pack_grad<kF32>(const float (&x)[4]) {
  return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3]));
}
template <>
__device__ __forceinline__ uint4 pack_grad<kBF16>(const float (&x)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t h[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float f = x[2 * k + s];
      const uint32_t u = __float_as_uint(f);
      h[s] = (isnan(f) ? (u | 0x00400000u) : u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    }
    w[k] = h[0] | (h[1] << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The row's loss and gbar from its sub-block records (every wave of the row
// computes them), then the gradient of one sub-block per wave from q and the
// sign codes of the first pass. With grad == nullptr only the loss is written
// (grid x = 1).
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_tv_grad(LinCfg c, const RowStat* rn, const uint16_t* sgn, const float* w_row,
                                                 double* loss, void* grad, double T) {
  constexpr int EPV = Elem<DT>::kPerVec;
  constexpr int VPL = kSB / (kWave * EPV);
  const int64_t r = blockIdx.y;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int sb0 = (blockIdx.x * kWaves + wave) * kTvSpwGrad;
  if (sb0 >= c.nsb) return;
  const int64_t nv = ((int64_t)c.V + EPV - 1) / EPV;
  const TvRow t = tv_row(c, rn, r);
  double L1 = 0.0, GQ = 0.0;
  for (int i = lane; i < c.nsb; i += kWave) {
    const ResRec x = c.res[r * c.nsb + i];
    L1 += x.sp;
    GQ += x.sq;
  }
  L1 = wave_sum(L1);
  GQ = wave_sum(GQ);
  if (sb0 == 0 && lane == 0) loss[r] = t.ok ? 0.5 * L1 : NAN;
  if (grad == nullptr) return;
  const float gbar = (float)GQ;
  const float scale = t.ok ? (float)((w_row ? (double)w_row[r] : 1.0) / T) : NAN;
  const char* qrow = c.rows.q + (r * (int64_t)c.V) * c.rows.esz;
  // the loads of sub-block sb + 1 are issued before sub-block sb is written
  const int sbe = min(sb0 + kTvSpwGrad, c.nsb);
  auto load_codes = [&](int64_t vfirst, uint32_t (&codes)[VPL]) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int64_t vec = vfirst + (int64_t)v * kWave;
      codes[v] = vec < nv ? (uint32_t)sgn[r * nv + vec] : 0u;
    }
  };
  float yd[VPL][EPV];
  uint32_t ycodes[VPL];
  load_codes((int64_t)sb0 * (kSB / EPV) + lane, ycodes);
  load_vecs<DT, AL, VPL, kWave>(qrow, c.V, c.nvec, (int64_t)sb0 * (kSB / EPV) + lane, yd);
  for (int sb = sb0; sb < sbe; ++sb) {
    const int64_t vfirst = (int64_t)sb * (kSB / EPV) + lane;
    float xd[VPL][EPV];
    uint32_t codes[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      codes[v] = ycodes[v];
#pragma unroll
      for (int e = 0; e < EPV; ++e) xd[v][e] = yd[v][e];
    }
    if (sb + 1 < sbe) {
      load_codes(vfirst + kSB / EPV, ycodes);
      load_vecs<DT, AL, VPL, kWave>(qrow, c.V, c.nvec, vfirst + kSB / EPV, yd);
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      float gout[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float Q = __builtin_amdgcn_exp2f(__builtin_fmaf(xd[v][e], c.c32, -t.mcq)) * t.iq;
        gout[e] = scale * Q * (tv_code_g((codes[v] >> (2 * e)) & 3u) - gbar);
      }
      const int64_t vec = vfirst + (int64_t)v * kWave;
      if constexpr (AL) {
        if (vec < c.nvec) ((uint4*)grad)[r * (int64_t)c.nvec + vec] = pack_grad<DT>(gout);
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int64_t j = vec * EPV + e;
          if (j < c.V) store_grad<DT>(grad, r * (int64_t)c.V + j, gout[e]);
        }
      }
    }
  }
}

template <int DT, bool AL>
static hipError_t tv_t(const LinCfg& c, RowStat* rn, uint16_t* sgn, const float* w_row, double* loss, void* grad,
                       double T, hipStream_t s) {
  const unsigned gxp = (unsigned)((c.nsb + kWaves * kTvSpwPass - 1) / (kWaves * kTvSpwPass));
  const unsigned gxg = (unsigned)((c.nsb + kWaves * kTvSpwGrad - 1) / (kWaves * kTvSpwGrad));
  hipError_t e = launch_stats32(c, 2 * c.B, DT, s);
  if (e != hipSuccess) return e;
  PSI_LAUNCH(s, k_tv_rows, dim3((unsigned)((2 * c.B + kWaves - 1) / kWaves)), dim3(kWG), c, rn, 2 * c.B);
  PSI_LAUNCH(s, (k_tv_pass<DT, AL>), dim3(gxp, (unsigned)c.B), dim3(kWG), c, (const RowStat*)rn, grad ? sgn : nullptr);
  PSI_LAUNCH(s, (k_tv_grad<DT, AL>), dim3(grad ? gxg : 1u, (unsigned)c.B), dim3(kWG), c, (const RowStat*)rn,
             (const uint16_t*)sgn, w_row,
             loss, grad, T);
  return hipGetLastError();
}

hipError_t launch_tv_loss(const LinCfg& c, RowStat* rn, uint16_t* sgn, const float* w_row, double* loss, void* grad,
                          double T, int dtype, hipStream_t s) {
  return PSI_DISPATCH(tv_t, dtype, c.aligned, c, rn, sgn, w_row, loss, grad, T, s);
}

}  // namespace psi
