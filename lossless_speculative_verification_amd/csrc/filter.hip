// Filtered sampling on gfx950: temperature -> top-k -> top-p -> renormalise
// (Uno repository README, inference controls temperature / top-p / top-k),
// applied identically to every target and draft row, then Psi-Spec verification
// ("Uno" research explainer, §3.3) on the filtered distributions.
//
//   k_filt_chunk   one workgroup per (row, 16384-logit chunk), logits kept in
//                  registers: a lower bound tau of the chunk's k-th largest
//                  logit (each wave's ceil(k/4)-th largest per-thread maximum,
//                  the smallest of the four: at least k logits are >= tau),
//                  then every finite logit >= tau is a candidate (with too
//                  many, tau is raised by bisection). Every logit of the
//                  chunk's exact top-k, ties included, is one.
//   k_filt_mergew  one wave per row: the row bound is the largest chunk
//                  bound; the candidates >= it (a chunk with too many stored
//                  none and is read again) are cut again by the same bound
//                  over the candidates, then each survivor's position in
//                  (logit desc, id asc) order, the plain definition's order,
//                  is counted and the first k kept; then top-p over that
//                  order and the log-normaliser, in fp64, and the kept set in
//                  id order. Rows that do not fit a wave go to
//   k_filt_fallback  the same merge by a whole workgroup, which reads chunks
//                  again and, beyond LDS, streams the row with a running
//                  exact top-k.
//   k_filt_decide  one workgroup per request: fused draft draws (one wave per
//                  row), p(x)/q(x), accept tests, first rejection, residual or
//                  bonus draw over the kept set staged in LDS, outputs.
//   k_filt_draft   draft draws only.
#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kSortCap = 4096;  // LDS candidate capacity of the row merge (power of two)
constexpr int kMaxOvf = 64;     // chunks read again per row before the whole row is

// (value desc, index asc): true if a comes first.
__device__ __forceinline__ bool before(const FiltCand& a, const FiltCand& b) {
  return a.v > b.v || (a.v == b.v && a.i < b.i);
}

// Branch-free form of before() for counting loops.
__device__ __forceinline__ int before_i(const FiltCand& a, const FiltCand& b) {
  return (int)(a.v > b.v) | ((int)(a.v == b.v) & (int)(a.i < b.i));
}

// In-LDS bitonic sort of n (power of two, <= kSortCap) entries in "before" order.
__device__ void bitonic_sort(FiltCand* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < n; t += blockDim.x) {
        const int p = t ^ j;
        if (p > t) {
          const bool up = (t & k) == 0;
          const FiltCand x = a[t], y = a[p];
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

// Pads cand[cnt .. pow2) with entries that sort last, sorts, and returns the
// number kept (at most kk).
__device__ int sort_keep(FiltCand* cand, int cnt, int kk) {
  const int n = pow2_at_least(cnt < 2 ? 2 : cnt);
  for (int t = cnt + threadIdx.x; t < n; t += blockDim.x) cand[t] = FiltCand{-INFINITY, 0x7fffffff};
  __syncthreads();
  bitonic_sort(cand, n);
  return cnt < kk ? cnt : kk;
}

// Exclusive scan of one int per thread over the workgroup, in thread order;
// writes the total. `sh` needs kWaves slots.
__device__ int block_scan_int(int v, int* sh, int* total) {
  const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  __syncthreads();
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  int before_ = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int x = sh[i];
    if (i < w) before_ += x;
    all += x;
  }
  *total = all;
  return before_ + incl - v;
}

// Unsigned keys in the order of the float values (-0 before +0) and back.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// The k-th largest of the R * 64 values a wave holds (R per lane; 1 <= k;
// not NaN; -inf allowed): bisection over the order keys of the floats, each
// step counting with ballots. If fewer than k values are finite, -inf.
template <int R>
__device__ __forceinline__ float wave_kth_largest(const float (&x)[R], int k) {
  uint32_t lo = 0x007fffffu;  // key of -inf: every value is >= it
  uint32_t hi = 0xff800001u;  // one past the key of +inf: no value is >= it
  while (hi - lo > 1u) {
    const uint32_t mid = lo + ((hi - lo) >> 1);
    const float t = from_order_key(mid);
    int n = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) n += __popcll(__ballot(x[r] >= t));
    if (n >= k) lo = mid;
    else hi = mid;
  }
  return from_order_key(lo);
}
__device__ __forceinline__ float wave_kth_largest(float x, int k) {
  const float v[1] = {x};
  return wave_kth_largest<1>(v, k);
}

// Appends one entry for every lane of the (converged) wave whose pred is set:
// one LDS atomic per wave. Returns this lane's slot (meaningful where pred).
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
  const int lane = threadIdx.x & (kWave - 1);
  const unsigned long long m = __ballot(pred);
  int base = 0;
  if (m) {
    const int leader = __ffsll((long long)m) - 1;
    if (lane == leader) base = atomicAdd(counter, __popcll(m));
    base = __shfl(base, leader);
  }
  return base + __popcll(m & ((1ull << lane) - 1ull));
}

// Running exact top-k of a whole row streamed in token order: an element
// enters the LDS buffer only if it exceeds the current k-th value (so a later
// equal element loses its tie), and a full buffer is sorted and cut back to k.
// Leaves the kept entries sorted in cand[0 .. returned count).
template <int DT, bool AL>
__device__ int stream_topk(const LinCfg& c, const char* row, int kk, FiltCand* cand, int* s_cnt, float* s_tau) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int NV = 4;
  if (threadIdx.x == 0) {
    *s_cnt = 0;
    *s_tau = -INFINITY;
  }
  __syncthreads();
  const int64_t nvec = (c.V + EPV - 1) / EPV;
  const int64_t tile_vec = (int64_t)kWG * NV;
  const int64_t ntiles = (nvec + tile_vec - 1) / tile_vec;
  for (int64_t tl = 0; tl < ntiles; ++tl) {
    uint4 v[NV];
    load_raw<DT, AL, NV, kWG>(row, c.V, c.nvec, tl * tile_vec + threadIdx.x, v);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float x[EPV];
      E::unpack(v[k], x);
      const float tau = *s_tau;
      const int64_t j0 = (tl * tile_vec + (int64_t)k * kWG + threadIdx.x) * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        if (x[e] > tau) {
          const int slot = atomicAdd(s_cnt, 1);
          if (slot < kSortCap) cand[slot] = FiltCand{x[e], (int32_t)(j0 + e)};
        }
      }
      __syncthreads();
      if (*s_cnt > kSortCap - kWG * EPV) {
        const int kept = sort_keep(cand, *s_cnt < kSortCap ? *s_cnt : kSortCap, kk);
        if (threadIdx.x == 0) {
          *s_cnt = kept;
          if (kept >= kk) *s_tau = cand[kk - 1].v;
        }
      }
      __syncthreads();
    }
  }
  const int cnt = *s_cnt;
  __syncthreads();
  return sort_keep(cand, cnt, kk);
}

}  // namespace

// ------------------------------------------------------- chunk candidates --
// With STATS the chunk's maximum and fp32-grade sum of 2^((a - m) c) are
// stored too (f.cst), for the full-row log-normaliser of the Tree Sampler.
template <int DT, bool AL, bool STATS = false>
__device__ __forceinline__ void filt_chunk(const LinCfg& c, const FiltCfg& f) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec, NV = kFiltVals / EPV;
  const int64_t item = blockIdx.x;
  const int64_t sr = item / f.nchf;
  const int ch = (int)(item - sr * f.nchf);
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const char* row = c.rows.row(sr);
  const int64_t v0 = (int64_t)ch * kWG * NV + t;
  float x[NV][EPV];
  load_vecs<DT, AL, NV, kWG>(row, c.V, c.nvec, v0, x);
  bool tbad = false, tany = false;
  float mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float xe = x[k][e];
      tbad |= isnan(xe) || xe == INFINITY;
      tany |= xe > -INFINITY;
      mx = fmaxf(mx, xe);
    }
  // Each wave has kq threads whose maximum is >= its kq-th largest thread
  // maximum, so the smallest of the four wave values bounds the chunk's
  // (4 kq >= kk)-th largest logit from below.
  __shared__ float s_w[kWaves];
  __shared__ int s_f[kWaves];
  __shared__ int s_sc[kWaves];
  __shared__ int s_cnt;
  __shared__ FiltCand s_out[kFiltChunkCap];
  const int kq = (f.kk + kWaves - 1) / kWaves;
  const float wq = wave_kth_largest(mx, kq);
  const int wf = (__ballot(tbad) ? 1 : 0) | (__ballot(tany) ? 2 : 0);
  __shared__ float s_sm[kWaves];
  __shared__ double s_ss[kWaves];
  if constexpr (STATS) {
    double st = 0.0;
    if (mx > -INFINITY)
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        float y[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) y[e] = exp2f((x[k][e] - mx) * c.c32);
        st += (double)pairwise_sum<EPV>(y);  // one vector in binary32, then fp64
      }
    const float mw = wave_max(mx);
    double sw = mx > -INFINITY ? st * (double)exp2f((mx - mw) * c.c32) : 0.0;
    sw = wave_sum(sw);
    if (lane == 0) {
      s_sm[wave] = mw;
      s_ss[wave] = sw;
    }
  }
  if (lane == 0) {
    s_w[wave] = wq;
    s_f[wave] = wf;
  }
  if (t == 0) s_cnt = 0;
  __syncthreads();
  if constexpr (STATS) {
    if (t == 0) {
      float m = s_sm[0];
#pragma unroll
      for (int i = 1; i < kWaves; ++i) m = fmaxf(m, s_sm[i]);
      double sum = 0.0;
      if (m > -INFINITY)
#pragma unroll
        for (int i = 0; i < kWaves; ++i)
          if (s_sm[i] > -INFINITY) sum += s_ss[i] * ::exp2(((double)s_sm[i] - (double)m) * (double)c.c32);
      bool bad = false;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) bad |= s_f[i] & 1;
      f.cst[item] = bad ? StatRec{NAN, 0u, NAN} : StatRec{m, 0u, sum};
    }
  }
  float tau = s_w[0];
  int flags = s_f[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) {
    tau = fminf(tau, s_w[i]);
    flags |= s_f[i];
  }
  // Candidates (finite logits >= tau) staged in LDS: a thread that has some
  // reserves its slots with one LDS atomic (candidates are sparse), and each
  // 16-byte vector is tested once before its logits are.
  auto stage = [&](float th) {
    int n = 0;
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < EPV; ++e) n += (x[k][e] >= th && x[k][e] > -INFINITY) ? 1 : 0;
    int w = n > 0 ? atomicAdd(&s_cnt, n) : 0;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      bool anyk = false;
#pragma unroll
      for (int e = 0; e < EPV; ++e) anyk |= x[k][e] >= th && x[k][e] > -INFINITY;
      if (anyk) {
#pragma unroll
        for (int e = 0; e < EPV; ++e)
          if (x[k][e] >= th && x[k][e] > -INFINITY) {
            if (w < kFiltChunkCap) s_out[w] = FiltCand{x[k][e], (int32_t)((v0 + (int64_t)k * kWG) * EPV + e)};
            ++w;
          }
      }
    }
    __syncthreads();
  };
  stage(tau);
  int total = s_cnt;
  if (total > kFiltChunkCap && !(flags & 1) && 2 * f.kk <= kFiltChunkCap) {
    // Too many candidates: raise tau by bisection over the order of the
    // logits while at least kk logits stay >= it, until at most
    // kFiltChunkCap do (many equal logits can keep the count above it).
    __shared__ float shm[kWaves];
    uint32_t lo = order_key(tau), hi = order_key(block_max(mx, shm)) + 1u;
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      const float fm = from_order_key(mid);
      int cm = 0;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < EPV; ++e) cm += (x[k][e] >= fm && x[k][e] > -INFINITY) ? 1 : 0;
      int all;
      block_scan_int(cm, s_sc, &all);
      if (all >= f.kk) {
        lo = mid;
        if (all <= kFiltChunkCap) break;
      } else {
        hi = mid;
      }
    }
    tau = from_order_key(lo);
    if (t == 0) s_cnt = 0;
    __syncthreads();
    stage(tau);
    total = s_cnt;
  }
  if (total <= kFiltChunkCap && t < total) f.fc[item * kFiltChunkCap + t] = s_out[t];
  const bool bad = flags & 1, any = flags & 2;
  if (t == 0) f.chk[item] = FiltChunk{tau, total, (bad ? 1 : 0) | (any ? 2 : 0), 0};
  if (item == 0 && t == 0) *f.nfall = 0;
}

template <int DT, bool AL, bool STATS>
__global__ __launch_bounds__(kWG) void k_filt_chunk(LinCfg c, FiltCfg f) {
  filt_chunk<DT, AL, STATS>(c, f);
}
// Aligned fp32 rows: held to 96 registers (five waves per SIMD), which it
// meets without spilling.
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(5))) void k_filt_chunk_f32(LinCfg c, FiltCfg f) {
  filt_chunk<kF32, true>(c, f);
}

// ------------------------------------------------- row merge, workgroup --
// The merge of one row by a whole workgroup: any number of chunks read again,
// up to kSortCap candidates in LDS, else the row streamed again.
template <int DT, bool AL>
__device__ void merge_row_wg(const LinCfg& c, const FiltCfg& f, int64_t sr) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec, NV = kFiltVals / EPV;
  constexpr int PER = kSortCap / kWG;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int kk = f.kk;
  __shared__ FiltCand cand[kSortCap];
  __shared__ FiltCand kept[kMaxTopK];
  __shared__ int s_cnt, s_novf, s_first;
  __shared__ float s_tau;
  __shared__ int s_ovf[kMaxOvf];
  __shared__ float shf[kWaves];
  __shared__ double shd[kWG + kWaves];
  const FiltChunk* rec = f.chk + sr * f.nchf;
  FiltRow* hdr = f.hdr + sr;
  if (t == 0) {
    s_cnt = 0;
    s_novf = 0;
  }
  // row bound and validity from the chunk records
  float tl = -INFINITY;
  int fl = 0;
  for (int ch = t; ch < f.nchf; ch += kWG) {
    const FiltChunk r = rec[ch];
    tl = fmaxf(tl, r.tau);
    fl |= r.flags;
  }
  const float tau = block_max(tl, shf);
  const int bad = __syncthreads_or(fl & 1);
  const int any = __syncthreads_or(fl & 2);
  if (bad || !any) {
    if (t == 0) *hdr = FiltRow{0, 1, -INFINITY, -INFINITY};
    __syncthreads();
    return;
  }
  // gather every stored candidate >= tau; note the chunks that stored none
  const FiltCand* src = f.fc + sr * f.nchf * (int64_t)kFiltChunkCap;
  const int nslot = f.nchf * kFiltChunkCap;
  for (int s0 = 0; s0 < nslot; s0 += kWG) {
    const int s = s0 + t;
    FiltCand e = {-INFINITY, 0};
    bool take = false;
    if (s < nslot) {
      const int ch = s / kFiltChunkCap, i = s - ch * kFiltChunkCap;
      const int n = rec[ch].cnt;
      if (n <= kFiltChunkCap) {
        if (i < n) {
          e = src[s];
          take = e.v >= tau;
        }
      } else if (i == 0) {
        const int k = atomicAdd(&s_novf, 1);
        if (k < kMaxOvf) s_ovf[k] = ch;
      }
    }
    const int slot = wave_append(take, &s_cnt);
    if (take && slot < kSortCap) cand[slot] = e;
  }
  __syncthreads();
  const int novf = s_novf;
  const char* row = c.rows.row(sr);
  if (novf <= kMaxOvf) {
    for (int k = 0; k < novf; ++k) {
      const int ch = s_ovf[k];
      const int64_t v0 = (int64_t)ch * kWG * NV + t;
      float x[NV][EPV];
      load_vecs<DT, AL, NV, kWG>(row, c.V, c.nvec, v0, x);
#pragma unroll
      for (int q = 0; q < NV; ++q)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const bool take = x[q][e] >= tau && x[q][e] > -INFINITY;
          const int slot = wave_append(take, &s_cnt);
          if (take && slot < kSortCap) cand[slot] = FiltCand{x[q][e], (int32_t)((v0 + (int64_t)q * kWG) * EPV + e)};
        }
    }
  }
  __syncthreads();
  const int total = s_cnt;
  __syncthreads();
  int cnt;
  if (novf > kMaxOvf || total > kSortCap) {
    cnt = stream_topk<DT, AL>(c, row, kk, cand, &s_cnt, &s_tau);
    if (t < cnt) kept[t] = cand[t];
  } else {
    // Second bound over the candidates (same argument as in the chunks): at
    // least kk candidates are >= tau2.
    FiltCand mine[PER];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = t + r * kWG;
      mine[r] = i < total ? cand[i] : FiltCand{-INFINITY, 0x7fffffff};
      tmax = fmaxf(tmax, mine[r].v);
    }
    const int kq = (kk + kWaves - 1) / kWaves;
    const float wq = wave_kth_largest(tmax, kq);
    if (lane == 0) shf[wave] = wq;
    if (t == 0) s_cnt = 0;
    __syncthreads();
    float tau2 = shf[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) tau2 = fminf(tau2, shf[i]);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const bool take = mine[r].v >= tau2 && mine[r].v > -INFINITY;
      const int slot = wave_append(take, &s_cnt);
      if (take) cand[slot] = mine[r];
    }
    __syncthreads();
    const int n2 = s_cnt;
    __syncthreads();
    if (n2 <= 4 * kWG) {
      // exact position of each survivor in (logit desc, id asc) order
      for (int i = t; i < n2; i += kWG) {
        const FiltCand me = cand[i];
        int rank = 0;
        for (int j = 0; j < n2; ++j) rank += before(cand[j], me) ? 1 : 0;
        if (rank < kk) kept[rank] = me;
      }
      cnt = n2 < kk ? n2 : kk;
    } else {
      cnt = sort_keep(cand, n2, kk);
      if (t < cnt) kept[t] = cand[t];
    }
  }
  __syncthreads();
  // ---- fp64 filter over kept[0 .. cnt), ordered by (logit desc, id asc),
  // which is the order of probability desc / id asc since z = a / T is
  // increasing in a. One entry per thread (cnt <= kMaxTopK = kWG).
  const double T = f.T;
  const double m = (double)kept[0].v / T;
  const bool own = t < cnt;
  double z = 0.0, e = 0.0;
  if (own) {
    z = (double)kept[t].v / T;
    e = ::exp(z - m);
  }
  int keep = cnt;
  if (f.top_p < 1.0) {
    const double S = block_sum(e, shd);
    const double p = own ? e / S : 0.0;
    double tot;
    const double incl = block_exclusive_scan(p, shd, &tot) + p;
    if (t == 0) s_first = 0x7fffffff;
    __syncthreads();
    if (own && incl >= f.top_p) atomicMin(&s_first, t);
    __syncthreads();
    if (s_first < cnt) keep = s_first + 1;
  }
  const double S = block_sum(t < keep ? e : 0.0, shd);
  if (t == 0) *hdr = FiltRow{keep, 0, m, m + ::log(S)};
  if (t < keep) {
    // position in token-id order (or the rank order of kept)
    const int id = kept[t].i;
    int rank = t;
    if (!f.by_rank) {
      rank = 0;
      for (int s = 0; s < keep; ++s) rank += kept[s].i < id ? 1 : 0;
    }
    FiltEnt* out = f.ent + sr * (int64_t)f.stride;
    out[rank] = FiltEnt{id, 0, z};
  }
  __syncthreads();
}

// ------------------------------------------------------ row merge, wave --
namespace {

constexpr int kWCap = 512;    // candidates one wave merges in LDS
constexpr int kFastCh = 12;   // chunks per row whose candidates a wave holds in registers
constexpr int kFallWgs = 64;  // workgroups of the fallback merge

// The four largest values seen (a multiset, largest first).
struct Top4 {
  float t0 = -INFINITY, t1 = -INFINITY, t2 = -INFINITY, t3 = -INFINITY;
  // inserts v and drops the smallest (a min/max network, no branches)
  __device__ __forceinline__ void add(float v) {
    const float v1 = fminf(t0, v);
    t0 = fmaxf(t0, v);
    const float v2 = fminf(t1, v1);
    t1 = fmaxf(t1, v1);
    const float v3 = fminf(t2, v2);
    t2 = fmaxf(t2, v2);
    t3 = fmaxf(t3, v3);
  }
  // the j-th largest, 1 <= j <= 4
  __device__ __forceinline__ float nth(int j) const { return j == 1 ? t0 : j == 2 ? t1 : j == 3 ? t2 : t3; }
};


// The top kk of cand[0 .. n) (n > kk, n <= R * 64) under (logit desc, id
// asc), written unordered to out[0 .. kk): ts = the kk-th largest logit;
// every entry above ts, then the entries equal to ts in id order.
template <int R>
__device__ void select_topk(const FiltCand* cand, int n, int kk, FiltCand* out) {
  const int lane = threadIdx.x & (kWave - 1);
  const unsigned long long lt = (1ull << lane) - 1ull;
  FiltCand e[R];
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = lane + r * kWave;
    e[r] = i < n ? cand[i] : FiltCand{-INFINITY, 0x7fffffff};
    v[r] = e[r].v;
  }
  const float ts = wave_kth_largest<R>(v, kk);
  int above = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) above += __popcll(__ballot(e[r].v > ts));
  const int need = kk - above;  // >= 1 entries equal to ts
  // rank of each entry equal to ts among those, by id
  int trank[R];
#pragma unroll
  for (int r = 0; r < R; ++r) trank[r] = 0;
#pragma unroll
  for (int r2 = 0; r2 < R; ++r2) {
    unsigned long long m = __ballot(e[r2].v == ts);
    while (m) {
      const int src = __ffsll((long long)m) - 1;
      m &= m - 1ull;
      const int oid = __builtin_amdgcn_readlane(e[r2].i, src);
#pragma unroll
      for (int r = 0; r < R; ++r) trank[r] += (e[r].v == ts && oid < e[r].i) ? 1 : 0;
    }
  }
  int w = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool take = e[r].v > ts || (e[r].v == ts && trank[r] < need);
    const unsigned long long m = __ballot(take);
    if (take) out[w + __popcll(m & lt)] = e[r];
    w += __popcll(m);
  }
}

// fp64 top-p and log-normaliser over kept[0 .. cnt) (sorted by logit desc,
// id asc) by one wave, lane l owning kept[4l .. 4l+3]; writes the row header
// and the kept set in token-id order.
__device__ void finish_row_wave(const FiltCfg& f, int64_t sr, FiltCand* kept, int cnt) {
  const int lane = threadIdx.x & (kWave - 1);
  const double T = f.T;
  const double m = (double)kept[0].v / T;
  double z[4], e[4], loc = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = lane * 4 + q;
    z[q] = j < cnt ? (double)kept[j].v / T : 0.0;
    e[q] = j < cnt ? ::exp(z[q] - m) : 0.0;
    loc += e[q];
  }
  int keep = cnt;
  if (f.top_p < 1.0) {
    const double S = wave_sum(loc);
    double p[4], lp = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      p[q] = e[q] / S;
      lp += p[q];
    }
    double acc = wave_incl_scan(lp) - lp;
    int first = -1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += p[q];
      const int j = lane * 4 + q;
      if (first < 0 && j < cnt && acc >= f.top_p) first = j;
    }
    const unsigned long long hit = __ballot(first >= 0);
    if (hit) keep = __shfl(first, __ffsll((long long)hit) - 1) + 1;
  }
  double ls = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) ls += lane * 4 + q < keep ? e[q] : 0.0;
  const double S = wave_sum(ls);
  if (lane == 0) f.hdr[sr] = FiltRow{keep, 0, m, m + ::log(S)};
  // position in token-id order, counted over kept[0 .. keep) padded to a
  // multiple of 8 with ids that count for nobody (kept has room for them)
  int id[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) id[q] = lane * 4 + q < keep ? kept[lane * 4 + q].i : 0;
  FiltEnt* out = f.ent + sr * (int64_t)f.stride;
  if (f.by_rank) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (lane * 4 + q < keep) out[lane * 4 + q] = FiltEnt{id[q], 0, z[q]};
    return;
  }
  wave_sync();
  const int keep8 = (keep + 7) & ~7;
  if (lane < keep8 - keep) kept[keep + lane].i = 0x7fffffff;
  wave_sync();
  int rank[4] = {0, 0, 0, 0};
#pragma unroll 8
  for (int s = 0; s < keep8; ++s) {
    const int o = kept[s].i;
#pragma unroll
    for (int q = 0; q < 4; ++q) rank[q] += o < id[q] ? 1 : 0;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (lane * 4 + q < keep) out[rank[q]] = FiltEnt{id[q], 0, z[q]};
}

}  // namespace

// One wave per row: the row bound and validity from the chunk records, a
// second bound from the stored candidates >= it, the candidates >= both
// gathered into the wave's LDS buffer, the exact top k cut by bisection on
// the k-th largest logit, its order by counting (LDS broadcast reads), then
// the fp64 finish.
// Rows with a chunk whose candidates overflowed its store, more than kWCap
// candidates >= both bounds, or more than 64 chunks are listed for the
// workgroup merge.
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_filt_mergew(LinCfg c, FiltCfg f, int64_t rows) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int64_t sr = blockIdx.x * (int64_t)kWaves + wave;
  if (sr >= rows) return;  // the whole wave; no workgroup barrier below
  __shared__ FiltCand s_cand[kWaves][kWCap + 8];
  __shared__ FiltCand s_kept[kWaves][kMaxTopK + 8];
  FiltCand* cand = s_cand[wave];
  FiltCand* kept = s_kept[wave];
  const FiltChunk* rec = f.chk + sr * f.nchf;
  const int kk = f.kk;
  const unsigned long long lt = (1ull << lane) - 1ull;
  float tl = -INFINITY;
  int fl = 0, mycnt = 0;
  for (int ch = lane; ch < f.nchf; ch += kWave) {
    const FiltChunk r = rec[ch];
    tl = fmaxf(tl, r.tau);
    fl |= r.flags;
    mycnt = r.cnt;
  }
  const float tau = wave_max(tl);
  fl = wave_or(fl);
  if ((fl & 1) || !(fl & 2)) {
    if (lane == 0) f.hdr[sr] = FiltRow{0, 1, -INFINITY, -INFINITY};
    return;
  }
  bool fall = f.nchf > kWave || __ballot(mycnt > kFiltChunkCap) != 0;
  // Pass 1 over the stored candidates >= tau: each lane keeps its jj largest
  // (jj = ceil(kk / 64) <= 4); ceil(kk / jj) lanes then hold jj candidates
  // each >= tau2, the ceil(kk / jj)-th largest of the lanes' jj-th values.
  const int jj = (kk + kWave - 1) / kWave, ll = (kk + jj - 1) / jj;
  float tau2 = tau;
  int n2 = 0;
  if (!fall && f.nchf <= kFastCh) {
    // the logits of every stored candidate loaded at once: lane l holds slots
    // l and l + 64 of each chunk (ids are read again for the survivors)
    float bv[2 * kFastCh];
    const FiltCand* src = f.fc + sr * f.nchf * (int64_t)kFiltChunkCap;
#pragma unroll
    for (int r = 0; r < 2 * kFastCh; ++r) {
      const int ch = r >> 1, i = (r & 1) * kWave + lane;
      const int cc = ch < f.nchf ? __shfl(mycnt, ch) : 0;
      bv[r] = i < cc ? src[ch * kFiltChunkCap + i].v : -INFINITY;
    }
    Top4 top;
#pragma unroll
    for (int r = 0; r < 2 * kFastCh; ++r) top.add(bv[r] >= tau ? bv[r] : -INFINITY);
    tau2 = fmaxf(tau, wave_kth_largest(top.nth(jj), ll));
#pragma unroll
    for (int r = 0; r < 2 * kFastCh; ++r) {
      const bool take = bv[r] >= tau2 && bv[r] > -INFINITY;
      const unsigned long long m = __ballot(take);
      const int slot = n2 + __popcll(m & lt);
      if (take && slot < kWCap) {
        const int ch = r >> 1, i = (r & 1) * kWave + lane;
        cand[slot] = FiltCand{bv[r], src[ch * kFiltChunkCap + i].i};
      }
      n2 += __popcll(m);
    }
    fall = n2 > kWCap;
  } else if (!fall) {
    Top4 top;
    for (int ch = 0; ch < f.nchf; ++ch) {
      const int cc = __shfl(mycnt, ch);
      const FiltCand* src = f.fc + (sr * f.nchf + ch) * kFiltChunkCap;
      for (int i = lane; i < cc; i += kWave) {
        const float v = src[i].v;
        top.add(v >= tau ? v : -INFINITY);
      }
    }
    tau2 = fmaxf(tau, wave_kth_largest(top.nth(jj), ll));
    // Pass 2: gather the candidates >= tau2.
    for (int ch = 0; ch < f.nchf; ++ch) {
      const int cc = __shfl(mycnt, ch);
      const FiltCand* src = f.fc + (sr * f.nchf + ch) * kFiltChunkCap;
      for (int i0 = 0; i0 < cc; i0 += kWave) {
        const int i = i0 + lane;
        FiltCand e = {-INFINITY, 0};
        if (i < cc) e = src[i];
        const bool take = i < cc && e.v >= tau2;
        const unsigned long long m = __ballot(take);
        const int slot = n2 + __popcll(m & lt);
        if (take && slot < kWCap) cand[slot] = e;
        n2 += __popcll(m);
      }
    }
    fall = n2 > kWCap;
  }
  if (fall) {
    if (lane == 0) f.fall[atomicAdd(f.nfall, 1)] = (int32_t)sr;
    return;
  }
  wave_sync();
  FiltCand* sel = cand;  // the kept set, unordered
  FiltCand* ord = kept;  // the kept set in (logit desc, id asc) order
  int cnt = n2;
  if (n2 > kk && n2 <= 2 * kWave) {
    cnt = kk;
    select_topk<2>(cand, n2, kk, kept);
    sel = kept;
    ord = cand;
  } else if (n2 > kk) {
    // a cut among more than 128: every survivor's position, by counting
    const int n28 = (n2 + 7) & ~7;
    if (lane < n28 - n2) cand[n2 + lane] = FiltCand{-INFINITY, 0x7fffffff};
    wave_sync();
    for (int i0 = 0; i0 < n2; i0 += kWave) {
      const int i = i0 + lane;
      const FiltCand me = i < n2 ? cand[i] : FiltCand{-INFINITY, 0x7fffffff};
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < n28; ++j) rank += before_i(cand[j], me);
      if (i < n2 && rank < kk) kept[rank] = me;
    }
    wave_sync();
    finish_row_wave(f, sr, kept, kk);
    return;
  }
  // exact position of each kept entry in (logit desc, id asc) order, counted
  // over sel[0 .. cnt) padded to a multiple of 8 with entries that come last
  const int c8 = (cnt + 7) & ~7;
  if (lane < c8 - cnt) sel[cnt + lane] = FiltCand{-INFINITY, 0x7fffffff};
  wave_sync();
  for (int i0 = 0; i0 < cnt; i0 += kWave) {
    const int i = i0 + lane;
    const FiltCand me = i < cnt ? sel[i] : FiltCand{-INFINITY, 0x7fffffff};
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < c8; ++j) rank += before_i(sel[j], me);
    if (i < cnt) ord[rank] = me;
  }
  wave_sync();
  finish_row_wave(f, sr, ord, cnt);
}

// The listed rows, one workgroup each.
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_filt_fallback(LinCfg c, FiltCfg f) {
  const int n = *f.nfall;
  for (int i = blockIdx.x; i < n; i += gridDim.x) merge_row_wg<DT, AL>(c, f, f.fall[i]);
}

// --------------------------------------------------- per-request decision --
namespace {

// Inverse-CDF draw over a kept list (cnt <= 4 * 64 entries in token-id order)
// by one whole wave, lane l owning entries 4l .. 4l+3: the smallest entry
// whose running sum exceeds u * W, else the last positive one; -1 if W is not
// positive. Returns the entry's position on every lane.
template <class W>
__device__ int wave_draw(int cnt, double u, W w) {
  const int lane = threadIdx.x & (kWave - 1);
  double wl[4], loc = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = lane * 4 + j;
    wl[j] = k < cnt ? w(k) : 0.0;
    loc += wl[j];
  }
  const double incl = wave_incl_scan(loc);
  const double tot = __shfl(incl, kWave - 1);
  if (!(tot > 0.0)) return -1;
  const double target = u * tot;
  double acc = incl - loc;
  int jj = -1, jl = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (wl[j] > 0.0) {
      if (jj < 0 && acc + wl[j] > target) jj = lane * 4 + j;
      jl = lane * 4 + j;
    }
    acc += wl[j];
  }
  unsigned long long m = __ballot(jj >= 0);
  if (m) return __shfl(jj, __ffsll((long long)m) - 1);
  m = __ballot(jl >= 0);
  return m ? __shfl(jl, 63 - __clzll((long long)m)) : -1;
}

// Probability of token x under a kept set held in LDS (id order).
__device__ __forceinline__ double lds_prob(const FiltEnt* e, int cnt, double L, int x) {
  int lo = 0, hi = cnt - 1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int id = e[mid].i;
    if (id == x) return ::exp(e[mid].z - L);
    if (id < x) lo = mid + 1;
    else hi = mid - 1;
  }
  return 0.0;
}

// Draft draws of request b by the workgroup's waves, one draft row per wave
// at a time; writes s_x[i] (-1 for an invalid row).
__device__ void filt_drafts(const LinCfg& c, const FiltCfg& f, int64_t b, const FiltRow* Hq, const FiltEnt* Eq,
                            int K, int* s_x) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  for (int i = wave; i < K; i += kWaves) {
    const FiltRow hq = Hq[i];
    const FiltEnt* eq = Eq + i * (int64_t)f.stride;
    int x = -1;
    if (!hq.bad && hq.cnt > 0) {
      const double u = c.rng.u((uint32_t)b, (uint32_t)i, kDrawDraft);
      const int k = wave_draw(hq.cnt, u, [&](int j) { return ::exp(eq[j].z - hq.m); });
      x = k >= 0 ? eq[k].i : -1;
    }
    if (lane == 0) s_x[i] = x;
  }
}

}  // namespace

__global__ __launch_bounds__(kWG) void k_filt_decide(LinCfg c, FiltCfg f) {
  const int64_t b = blockIdx.x;
  const int K = c.K, R = 2 * K + 1, t = threadIdx.x;
  const FiltRow* H = f.hdr + b * R;
  const FiltEnt* Ent = f.ent + b * R * (int64_t)f.stride;
  __shared__ int s_bad, s_n, s_sel;
  __shared__ int s_x[kMaxK];
  __shared__ FiltEnt s_ep[kMaxTopK], s_eq[kMaxTopK];
  __shared__ double shd[kWG + kWaves];
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < R; i += kWG)
    if (H[i].bad || H[i].cnt <= 0) atomicOr(&s_bad, 1);
  if (c.fused) {
    filt_drafts(c, f, b, H + K + 1, Ent + (K + 1) * (int64_t)f.stride, K, s_x);
  } else {
    for (int i = t; i < K; i += kWG) s_x[i] = c.draft[b * K + i];
  }
  __syncthreads();
  for (int i = t; i < K; i += kWG)
    if (s_x[i] < 0 || s_x[i] >= c.V) atomicOr(&s_bad, 1);
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
  // ---- final draw over the kept set of target row n (one entry per thread)
  const bool resid = n < K;
  const FiltRow hp = H[n];
  const FiltRow hq = resid ? H[K + 1 + n] : FiltRow{0, 0, 0.0, 0.0};
  if (t < hp.cnt) s_ep[t] = Ent[n * (int64_t)f.stride + t];
  if (resid && t < hq.cnt) s_eq[t] = Ent[(K + 1 + n) * (int64_t)f.stride + t];
  __syncthreads();
  const bool mine = t < hp.cnt;
  const double pj = mine ? ::exp(s_ep[t].z - hp.L) : 0.0;
  double w = pj, mass = 0.0;
  if (resid) {
    w = mine ? fmax(0.0, pj - lds_prob(s_eq, hq.cnt, hq.L, s_ep[t].i)) : 0.0;
    mass = block_sum(w, shd);
    if (!(mass > 0.0)) w = pj;  // the residual vanished: draw from the target
  }
  const double u = c.rng.u((uint32_t)b, (uint32_t)n, kDrawFinal);
  double tot;
  const double excl = block_exclusive_scan(w, shd, &tot);
  const double target = u * tot;
  if (t == 0) s_sel = 0x7fffffff;
  __syncthreads();
  if (w > 0.0 && excl + w > target) atomicMin(&s_sel, t);
  __syncthreads();
  if (s_sel == 0x7fffffff) {  // rounding left no crossing: the last positive weight
    __syncthreads();
    if (t == 0) s_sel = -1;
    __syncthreads();
    if (w > 0.0) atomicMax(&s_sel, t);
    __syncthreads();
  }
  if (t == 0) {
    const int y = s_sel >= 0 ? s_ep[s_sel].i : -1;
    for (int i = 0; i <= K; ++i) c.out_tokens[b * (K + 1) + i] = i < n ? s_x[i] : (i == n ? y : -1);
    c.out_len[b] = n;
    if (c.out_resid) c.out_resid[b] = mass;
  }
}

__global__ __launch_bounds__(kWG) void k_filt_draft(LinCfg c, FiltCfg f) {
  const int64_t b = blockIdx.x;
  const int K = c.K, t = threadIdx.x;
  const FiltRow* H = f.hdr + b * K;
  __shared__ int s_bad;
  __shared__ int s_x[kMaxK];
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < K; i += kWG)
    if (H[i].bad || H[i].cnt <= 0) atomicOr(&s_bad, 1);
  filt_drafts(c, f, b, H, f.ent + b * K * (int64_t)f.stride, K, s_x);
  __syncthreads();
  for (int i = t; i < K; i += kWG) c.draft[b * K + i] = s_bad ? -1 : s_x[i];
}

// ------------------------------------------------------------ launchers --
template <int DT, bool AL>
static hipError_t filter_rows_t(const LinCfg& c, const FiltCfg& f, int64_t rows, hipStream_t s) {
  if constexpr (DT == kF32 && AL) {
    if (f.cst) PSI_LAUNCH(s, (k_filt_chunk<DT, AL, true>), dim3((unsigned)(rows * f.nchf)), dim3(kWG), c, f);
    else PSI_LAUNCH(s, k_filt_chunk_f32, dim3((unsigned)(rows * f.nchf)), dim3(kWG), c, f);
  }
  else if (f.cst) PSI_LAUNCH(s, (k_filt_chunk<DT, AL, true>), dim3((unsigned)(rows * f.nchf)), dim3(kWG), c, f);
  else PSI_LAUNCH(s, (k_filt_chunk<DT, AL, false>), dim3((unsigned)(rows * f.nchf)), dim3(kWG), c, f);
  PSI_LAUNCH(s, (k_filt_mergew<DT, AL>), dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kWG), c, f, rows);
  PSI_LAUNCH(s, (k_filt_fallback<DT, AL>), dim3((unsigned)kFallWgs), dim3(kWG), c, f);
  return hipGetLastError();
}

hipError_t launch_filter_rows(const LinCfg& c, const FiltCfg& f, int64_t rows, int dtype, hipStream_t s) {
  return PSI_DISPATCH(filter_rows_t, dtype, c.aligned, c, f, rows, s);
}

hipError_t launch_filtered(const LinCfg& c, const FiltCfg& f, int dtype, bool draft_only, hipStream_t s) {
  const hipError_t e = launch_filter_rows(c, f, c.B * (c.rows.np + c.rows.nq), dtype, s);
  if (e != hipSuccess) return e;
  if (draft_only) PSI_LAUNCH(s, k_filt_draft, dim3((unsigned)c.B), dim3(kWG), c, f);
  else PSI_LAUNCH(s, k_filt_decide, dim3((unsigned)c.B), dim3(kWG), c, f);
  return hipGetLastError();
}

}  // namespace psi
