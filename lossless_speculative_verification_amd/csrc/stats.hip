// Statistics pass of linear verification on gfx950: one workgroup per
// (row, chunk) reads every logit of the target and draft rows once and writes
// the chunk maximum and the sum of 2^((a - m) * c), c = log2(e) / T (binary32
// exp2, fp64 accumulation). The per-row log-normalisers that follow are good
// to ~1e-7, which is what the accept test min(1, p(x) / q(x)) needs ("Uno"
// research explainer, §3.3 Psi-Spec). This pass streams every logit of a
// verification call and bounds its speed, so it lives alone in this file.
#include "rowload.hpp"

namespace psi {

// ------------------------------------------------------ statistics pass --
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_stats32(LinCfg c) {
  constexpr int EPV = Elem<DT>::kPerVec;
  const int64_t item = blockIdx.x;
  const int chunk = (int)(item % c.nch32);
  const int64_t sr = item / c.nch32;
  const char* row = c.rows.row(sr);
  __shared__ float shf[kWaves];
  __shared__ double shd[kWaves];
  float x[kStatNV][EPV];
  load_vecs<DT, AL, kStatNV, kWG>(row, c.V, c.nvec, (int64_t)chunk * kWG * kStatNV + threadIdx.x, x);
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < kStatNV; ++k)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxnan(m, x[k][e]);
  m = block_max(m, shf);
  double s = 0.0;
  if (!is_neg_inf(m)) {
    // exp2(x*c - round(m*c)) = 2^((x-m)c) * 2^(mc_lo); the common factor
    // 2^(mc_lo) is removed once per chunk in fp64.
    const float mc_hi = m * c.c32;
    const float mc_lo = fmaf(m, c.c32, -mc_hi);
#pragma unroll
    for (int k = 0; k < kStatNV; ++k) {
      float e[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(x[k][j], c.c32, -mc_hi));
      s += (double)pairwise_sum(e);
    }
    s = block_sum(s, shd);
    s *= ::exp2(-(double)mc_lo);
  }
  if (threadIdx.x == 0) {
    StatRec r;
    r.m = m;
    r.pad = 0;
    r.s = s;
    c.st[item] = r;
  }
}

template <int DT, bool AL>
static hipError_t stats32_t(const LinCfg& c, int64_t rows, hipStream_t s) {
  PSI_LAUNCH(s, (k_stats32<DT, AL>), dim3((unsigned)(rows * c.nch32)), dim3(kWG), c);
  return hipGetLastError();
}

hipError_t launch_stats32(const LinCfg& c, int64_t rows, int dtype, hipStream_t s) {
  return PSI_DISPATCH(stats32_t, dtype, c.aligned, c, rows, s);
}

}  // namespace psi
