// Filtered sampling on gfx950: temperature -> top-k -> top-p -> renormalise
// (Uno repository README, inference controls temperature / top-p / top-k),
// applied identically to every target and draft row, then Psi-Spec verification
// ("Uno" research explainer, §3.3) on the filtered distributions.
//
//   k_filter_row   one workgroup per row: streams the row once, keeping an exact
//                  running top-k in LDS (an element enters only if it exceeds the
//                  current k-th value; rows are streamed in index order, so ties
//                  go to the lower id), compacts with a bitonic sort when the
//                  buffer fills, then applies top-p and the log-normaliser in
//                  fp64 over the kept set, in the same order as the plain
//                  definition (sums in token-id order, cumulative sum in
//                  probability order).
//   k_filt_decide  one workgroup per request: fused draft draws, p(x)/q(x),
//                  accept tests, first rejection, residual or bonus draw over the
//                  (at most top_k entry) supports, outputs.
//   k_filt_draft   one workgroup per draft row: draft draw only.
#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kSortCap = 4096;  // LDS sort capacity (power of two)

struct KeyIdx {
  float v;
  int32_t i;
};

// (value desc, index asc): true if a comes first.
__device__ __forceinline__ bool before(const KeyIdx& a, const KeyIdx& b) {
  return a.v > b.v || (a.v == b.v && a.i < b.i);
}

// In-LDS bitonic sort of n (power of two, <= kSortCap) entries in "before" order.
__device__ void bitonic_sort(KeyIdx* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < n; t += blockDim.x) {
        const int p = t ^ j;
        if (p > t) {
          const bool up = (t & k) == 0;
          const KeyIdx x = a[t], y = a[p];
          if (up ? before(y, x) : before(x, y)) {
            a[t] = y;
            a[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Sorts the first `cnt` candidates and keeps the best `kk`; returns the new count.
__device__ int compact(KeyIdx* cand, int cnt, int kk) {
  const int n = pow2_at_least(cnt < 2 ? 2 : cnt);
  for (int t = cnt + threadIdx.x; t < n; t += blockDim.x) cand[t] = KeyIdx{-INFINITY, 0x7fffffff};
  __syncthreads();
  bitonic_sort(cand, n);
  return cnt < kk ? cnt : kk;
}

// Double-precision entries of a filtered row, sorted by token id.
struct DEnt {
  double z;
  int32_t i;
  int32_t pad;
};

}  // namespace

// -------------------------------------------------------------- row filter --
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_filter_row(LinCfg c, FiltCfg f) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int NV = 4;  // 16-byte vectors per thread per tile
  const int64_t sr = blockIdx.x;
  const char* row = c.rows.row(sr);
  const int kk = f.kk;
  const int cap = kSortCap;
  __shared__ KeyIdx cand[kSortCap];
  __shared__ int s_cnt, s_bad, s_any;
  __shared__ float s_tau;
  if (threadIdx.x == 0) {
    s_cnt = 0;
    s_bad = 0;
    s_any = 0;
    s_tau = -INFINITY;
  }
  __syncthreads();
  const int64_t nvec = (c.V + EPV - 1) / EPV;
  const int64_t tile_vec = (int64_t)kWG * NV;
  const int64_t ntiles = (nvec + tile_vec - 1) / tile_vec;
  int bad = 0, any = 0;
  for (int64_t tl = 0; tl < ntiles; ++tl) {
    uint4 v[NV];
    load_raw<DT, AL, NV, kWG>(row, c.V, c.nvec, tl * tile_vec + threadIdx.x, v);
    // sub-tile k = vectors [k*kWG, (k+1)*kWG) of the tile: sub-tiles are in token
    // order, so a value equal to the current threshold always loses its tie
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float x[EPV];
      E::unpack(v[k], x);
      const float tau = s_tau;
      const int64_t j0 = (tl * tile_vec + (int64_t)k * kWG + threadIdx.x) * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xe = x[e];
        bad |= isnan(xe) || (isinf(xe) && xe > 0.0f);
        any |= xe > -INFINITY;
        if (xe > tau) {
          const int slot = atomicAdd(&s_cnt, 1);
          if (slot < cap) cand[slot] = KeyIdx{xe, (int32_t)(j0 + e)};
        }
      }
      __syncthreads();
      if (s_cnt > cap - kWG * EPV) {
        const int kept = compact(cand, s_cnt < cap ? s_cnt : cap, kk);
        if (threadIdx.x == 0) {
          s_cnt = kept;
          if (kept >= kk) s_tau = cand[kk - 1].v;
        }
      }
      __syncthreads();
    }
  }
  if (bad) atomicOr(&s_bad, 1);
  if (any) atomicOr(&s_any, 1);
  __syncthreads();
  int cnt = compact(cand, s_cnt, kk);
  __syncthreads();
  // ---- fp64 filter over the kept set ----
  // cand[0..cnt) is sorted by (value desc, id asc), which is also the order of
  // probability desc / id asc because z = a / T is strictly increasing in a.
  __shared__ DEnt ent[kMaxTopK];
  __shared__ KeyIdx byid[kMaxTopK];
  __shared__ int s_keep;
  const double T = f.T;
  const int n2 = pow2_at_least(cnt < 2 ? 2 : cnt);
  for (int t = threadIdx.x; t < n2; t += kWG) byid[t] = t < cnt ? KeyIdx{0.0f, cand[t].i} : KeyIdx{-INFINITY, 0x7fffffff};
  __syncthreads();
  bitonic_sort(byid, n2);  // equal keys -> ascending token id
  for (int t = threadIdx.x; t < cnt; t += kWG) {
    const int id = byid[t].i;
    float val = 0.0f;
    for (int u = 0; u < cnt; ++u)
      if (cand[u].i == id) val = cand[u].v;
    ent[t].z = (double)val / T;
    ent[t].i = id;
    ent[t].pad = 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int keep = cnt;
    if (f.top_p < 1.0 && cnt > 0) {
      double m = -INFINITY;
      for (int t = 0; t < cnt; ++t) m = fmax(m, ent[t].z);
      double S = 0.0;
      for (int t = 0; t < cnt; ++t) S += ::exp(ent[t].z - m);  // id order
      double cum = 0.0;
      for (int t = 0; t < cnt; ++t) {  // probability order
        cum += ::exp((double)cand[t].v / T - m) / S;
        if (cum >= f.top_p) {
          keep = t + 1;
          break;
        }
      }
    }
    // final set: the first `keep` candidates, listed in id order
    int w = 0;
    if (keep < cnt) {
      const KeyIdx last = cand[keep - 1];
      for (int t = 0; t < cnt; ++t) {
        const int id = ent[t].i;
        float val = 0.0f;
        for (int u = 0; u < cnt; ++u)
          if (cand[u].i == id) val = cand[u].v;
        const KeyIdx me = KeyIdx{val, id};
        if (!before(last, me)) ent[w++] = ent[t];
      }
    } else {
      w = cnt;
    }
    s_keep = w;
  }
  __syncthreads();
  cnt = s_keep;
  // log-normaliser over the final set (id order)
  if (threadIdx.x == 0) {
    double m = -INFINITY;
    for (int t = 0; t < cnt; ++t) m = fmax(m, ent[t].z);
    double S = 0.0;
    for (int t = 0; t < cnt; ++t) S += ::exp(ent[t].z - m);
    FiltRow h;
    h.cnt = cnt;
    h.bad = s_bad || !s_any;
    h.m = m;
    h.L = cnt > 0 ? m + ::log(S) : -INFINITY;
    f.hdr[sr] = h;
  }
  __syncthreads();
  FiltEnt* out = f.ent + sr * (int64_t)f.stride;
  for (int t = threadIdx.x; t < cnt; t += kWG) {
    FiltEnt e;
    e.i = ent[t].i;
    e.pad = 0;
    e.z = ent[t].z;
    out[t] = e;
  }
}

// --------------------------------------------------- per-request decision --
__global__ __launch_bounds__(kWG) void k_filt_decide(LinCfg c, FiltCfg f) {
  const int64_t b = blockIdx.x;
  const int K = c.K, R = 2 * K + 1, t = threadIdx.x;
  const FiltRow* H = f.hdr + b * R;
  const FiltEnt* Ent = f.ent + b * R * (int64_t)f.stride;
  __shared__ int s_bad, s_n;
  __shared__ int s_x[kMaxK];
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < R; i += kWG)
    if (H[i].bad || H[i].cnt <= 0) atomicOr(&s_bad, 1);
  if (t < K) {
    int x;
    if (c.fused) {
      const FiltRow hq = H[K + 1 + t];
      const FiltEnt* eq = Ent + (K + 1 + t) * (int64_t)f.stride;
      const double u = c.rng.u((uint32_t)b, (uint32_t)t, kDrawDraft);
      x = hq.cnt > 0 ? draw_list(hq.cnt, u, [&](int k) { return ::exp(eq[k].z - hq.m); }, eq) : -1;
    } else {
      x = c.draft[b * K + t];
    }
    if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
    s_x[t] = x;
  }
  __syncthreads();
  int acc = 1;
  double P = 0.0, Q = 0.0;
  if (t < K && !s_bad) {
    const int x = s_x[t];
    P = filt_prob(H[t], Ent + t * (int64_t)f.stride, x);
    Q = filt_prob(H[K + 1 + t], Ent + (K + 1 + t) * (int64_t)f.stride, x);
    const double u = c.rng.u((uint32_t)b, (uint32_t)t, kDrawAccept);
    acc = u * Q < P;
  }
  if (t < kWave) {
    const unsigned long long rej = __ballot(t < K && !acc);
    if (t == 0) s_n = rej ? (__ffsll((long long)rej) - 1) : K;
  }
  __syncthreads();
  if (s_bad) {
    for (int i = t; i <= K; i += kWG) c.out_tokens[b * (K + 1) + i] = -1;
    if (c.out_probs)
      for (int i = t; i < 2 * K; i += kWG) c.out_probs[b * 2 * K + i] = 0.0f;
    if (c.fused)
      for (int i = t; i < K; i += kWG) c.draft[b * K + i] = -1;
    if (t == 0) {
      c.out_len[b] = -1;
      if (c.out_resid) c.out_resid[b] = 0.0;
    }
    return;
  }
  const int n = s_n;
  if (t < K) {
    if (c.fused) c.draft[b * K + t] = s_x[t];
    if (c.out_probs) {
      c.out_probs[(b * K + t) * 2 + 0] = (float)P;
      c.out_probs[(b * K + t) * 2 + 1] = (float)Q;
    }
  }
  if (t == 0) {
    const double u = c.rng.u((uint32_t)b, (uint32_t)n, kDrawFinal);
    const FiltRow hp = H[n];
    const FiltEnt* ep = Ent + n * (int64_t)f.stride;
    int y;
    double resid = 0.0;
    if (n < K) {
      const FiltRow hq = H[K + 1 + n];
      const FiltEnt* eq = Ent + (K + 1 + n) * (int64_t)f.stride;
      auto w = [&](int k) {
        const double pj = ::exp(ep[k].z - hp.L);
        const double qj = filt_prob(hq, eq, ep[k].i);
        return fmax(0.0, pj - qj);
      };
      for (int k = 0; k < hp.cnt; ++k) resid += w(k);
      if (resid > 0.0) y = draw_list(hp.cnt, u, w, ep);
      else y = draw_list(hp.cnt, u, [&](int k) { return ::exp(ep[k].z - hp.L); }, ep);
    } else {
      y = draw_list(hp.cnt, u, [&](int k) { return ::exp(ep[k].z - hp.L); }, ep);
    }
    for (int i = 0; i <= K; ++i) c.out_tokens[b * (K + 1) + i] = i < n ? s_x[i] : (i == n ? y : -1);
    c.out_len[b] = n;
    if (c.out_resid) c.out_resid[b] = resid;
  }
}

__global__ __launch_bounds__(kWG) void k_filt_draft(LinCfg c, FiltCfg f) {
  const int64_t b = blockIdx.x;
  const int K = c.K, t = threadIdx.x;
  const FiltRow* H = f.hdr + b * K;
  __shared__ int s_bad;
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < K; i += kWG)
    if (H[i].bad || H[i].cnt <= 0) atomicOr(&s_bad, 1);
  __syncthreads();
  for (int i = t; i < K; i += kWG) {
    int x = -1;
    if (!s_bad) {
      const FiltRow hq = H[i];
      const FiltEnt* eq = f.ent + (b * K + i) * (int64_t)f.stride;
      const double u = c.rng.u((uint32_t)b, (uint32_t)i, kDrawDraft);
      x = draw_list(hq.cnt, u, [&](int k) { return ::exp(eq[k].z - hq.m); }, eq);
    }
    c.draft[b * K + i] = x;
  }
}

// ------------------------------------------------------------ launchers --
template <int DT, bool AL>
static hipError_t filtered_t(const LinCfg& c, const FiltCfg& f, bool draft_only, hipStream_t s) {
  const int64_t rows = c.B * (c.rows.np + c.rows.nq);
  PSI_LAUNCH(s, (k_filter_row<DT, AL>), dim3((unsigned)rows), dim3(kWG), c, f);
  if (draft_only) PSI_LAUNCH(s, k_filt_draft, dim3((unsigned)c.B), dim3(kWG), c, f);
  else PSI_LAUNCH(s, k_filt_decide, dim3((unsigned)c.B), dim3(kWG), c, f);
  return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t filter_rows_t(const LinCfg& c, const FiltCfg& f, int64_t rows, hipStream_t s) {
  PSI_LAUNCH(s, (k_filter_row<DT, AL>), dim3((unsigned)rows), dim3(kWG), c, f);
  return hipGetLastError();
}

hipError_t launch_filter_rows(const LinCfg& c, const FiltCfg& f, int64_t rows, int dtype, hipStream_t s) {
  if (dtype == kBF16)
    return c.aligned ? filter_rows_t<kBF16, true>(c, f, rows, s) : filter_rows_t<kBF16, false>(c, f, rows, s);
  return c.aligned ? filter_rows_t<kF32, true>(c, f, rows, s) : filter_rows_t<kF32, false>(c, f, rows, s);
}

hipError_t launch_filtered(const LinCfg& c, const FiltCfg& f, int dtype, bool draft_only, hipStream_t s) {
  if (dtype == kBF16)
    return c.aligned ? filtered_t<kBF16, true>(c, f, draft_only, s) : filtered_t<kBF16, false>(c, f, draft_only, s);
  return c.aligned ? filtered_t<kF32, true>(c, f, draft_only, s) : filtered_t<kF32, false>(c, f, draft_only, s);
}

}  // namespace psi
