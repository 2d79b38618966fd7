// Filters with no small bound on the kept set, on gfx950: top-p without a
// top-k, or a top-k above the kept-set capacity of the candidate path
// (filter.hip). Controls: temperature -> top-k -> top-p -> renormalise (Uno
// repository README, inference section), then Psi-Spec verification ("Uno"
// research explainer, §3.3) on the filtered distributions.
//
// Both filters keep a prefix of the order (logit descending, token id
// ascending): top-k its first k tokens, top-p, within those, the shortest
// prefix whose probability reaches top_p. So a filtered row is described by
// one cut, the last kept token's (order key, id): token j is kept iff
// key(a_j) > key_cut, or key(a_j) == key_cut and j <= id_cut, with key the
// order key of the logit (-0 counted as +0). Temperature does not change this
// order.
//
//   k_wcut      one 1024-thread workgroup per row: row maximum and validity;
//               the top-k cut by radix selection over the keys (12, 12 and 8
//               bits, exact integer counts in LDS); the fp64 mass S of the
//               kept set; the top-p crossing located by the same selection
//               over fixed-point masses (integer atomics, deterministic), then
//               confirmed on exact fp64 sums and moved to a neighbouring key
//               when the fixed-point rounding chose the wrong one; ties at the
//               cut resolved by the rank of the token id. Writes the cut and
//               the kept set's fp64 mass.
//   k_wdraft    one workgroup per draft row: fp64 sub-block sums of the kept
//               weights in LDS, then the inverse-CDF draw (wave_select and a
//               rescan of one sub-block).
//   k_wresolve  one workgroup per request: p(x) and q(x) from the cuts, accept
//               tests, first rejection, then fp64 sub-block sums of the final
//               row's kept weights (target alone, or max(0, p - q)) and the
//               final draw.
//   k_wtdraft   tree node drafts, one workgroup per node, as k_wdraft.
//   k_wtree     tree walk, one workgroup per request: child tests with the
//               recursive residual kept as one coefficient, one fp64 pass over
//               the row pair per rejection, and the final draw.
#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kWT = 1024;          // threads of a resolve workgroup
constexpr int kWTW = kWT / kWave;  // waves of one
constexpr int kDWT = 512;          // threads of a draft-row workgroup
constexpr int kTT = 512;           // threads of a tree-walk workgroup (registers for the fp64 passes)
constexpr int kTTW = kTT / kWave;
constexpr int kHist = 4096;        // bins of the widest radix level (12 bits)
constexpr uint32_t kKeyNegInf = 0x007fffffu;  // order key of -inf

// Order key of a logit: unsigned, increasing with the value; -0 and +0 share
// the key of +0 (they are equal logits).
__device__ __forceinline__ uint32_t wkey(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float wkey_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ bool kept_by(uint32_t key, int64_t j, uint32_t ckey, int32_t cid) {
  return key > ckey || (key == ckey && j <= (int64_t)cid);
}

// fp64 weight 2^((a - m) c) of a logit (0 for -inf).
__device__ __forceinline__ double wweight(float a, double c64, double mc) {
  return exp2_fast(__builtin_fma((double)a, c64, -mc));
}

// The EPV logits of 16-byte vector v of a row (-inf past V). Rows are read
// several times by the cut search, so these are ordinary cached loads.
template <int DT, bool AL>
__device__ __forceinline__ void wvec(const char* row, int V, int nvec, int64_t v, float (&x)[Elem<DT>::kPerVec]) {
  using E = Elem<DT>;
  if constexpr (AL) {
    const uint4 w = v < nvec ? ((const uint4*)row)[v]
                             : make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
    E::unpack(w, x);
  } else {
#pragma unroll
    for (int e = 0; e < E::kPerVec; ++e) {
      const int64_t j = v * E::kPerVec + e;
      x[e] = j < V ? E::load1(row, j) : -INFINITY;
    }
  }
}

// Workgroup sums of integers, in a fixed order.
template <int NT>
__device__ __forceinline__ long long block_sum_ll(long long v, long long* sh) {
  constexpr int NW = NT / kWave;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) sh[w] = v;
  __syncthreads();
  long long r = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += sh[i];
  return r;
}

// Exclusive scan of one integer per thread in thread order, and the total.
template <int NT>
__device__ __forceinline__ long long block_scan_ll(long long v, long long* sh, long long* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  long long incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long up = __shfl_up(incl, o);
    if (lane >= o) incl += up;
  }
  __syncthreads();
  if (lane == kWave - 1) sh[w] = incl;
  __syncthreads();
  long long before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    if (i < w) before += sh[i];
    all += sh[i];
  }
  *total = all;
  return before + incl - v;
}

// From the top bin down, the first bin d at which above + (sum of bins >= d)
// reaches need; returns d and sets *above to the sum of the bins above d
// added to it. If no bin reaches need, the lowest non-empty bin. `val` holds
// nb <= kHist bins; of NT threads, thread t owns the ceil(nb / NT) bins of
// descending rank from t * ceil(nb / NT). `shl` needs NT / kWave + 1 slots.
template <int NT, class T>
__device__ int select_bin(const T* val, int nb, unsigned long long need, unsigned long long* above, long long* shl,
                          int* shi) {
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x;
  const int per = (nb + NT - 1) / NT;
  // thread t owns bins of descending rank [t * per, t * per + per)
  long long mine = 0;
  for (int r = t * per; r < t * per + per && r < nb; ++r) mine += (long long)val[nb - 1 - r];
  long long tot;
  const long long excl = block_scan_ll<NT>(mine, shl, &tot);
  if (t == 0) {
    shi[0] = -1;
    shi[1] = -1;
  }
  __syncthreads();
  const unsigned long long base = *above;
  {
    unsigned long long acc = base + (unsigned long long)excl;
    for (int r = t * per; r < t * per + per && r < nb; ++r) {
      const unsigned long long v = (unsigned long long)val[nb - 1 - r];
      if (v > 0 && acc + v >= need) {
        atomicMin((unsigned int*)&shi[0], (unsigned int)r);  // shi[0] starts at -1 = UINT_MAX
        break;
      }
      acc += v;
    }
    for (int r = t * per; r < t * per + per && r < nb; ++r)
      if (val[nb - 1 - r] > 0) atomicMax(&shi[1], r);
  }
  __syncthreads();
  int rsel = shi[0];
  if (rsel < 0) rsel = shi[1];  // rounding left no crossing: the lowest non-empty bin
  __syncthreads();
  // the exact sum of the bins above the chosen one, by the thread that owns it
  if (rsel >= 0 && rsel >= t * per && rsel < t * per + per) {
    unsigned long long acc = base + (unsigned long long)excl;
    for (int r = t * per; r < rsel; ++r) acc += (unsigned long long)val[nb - 1 - r];
    shl[NW] = (long long)acc;
  }
  __syncthreads();
  if (rsel >= 0) *above = (unsigned long long)shl[NW];
  __syncthreads();
  return rsel < 0 ? -1 : nb - 1 - rsel;
}

}  // namespace

// ------------------------------------------------------------------ cut --
constexpr int kCT = 512;             // threads of a cut workgroup
constexpr int kCTW = kCT / kWave;
constexpr int kCutNV = 4;            // 16-byte vectors in flight per thread in the cut passes

// Calls f(j, a_j) for every logit of a row: thread t takes vectors t, t + NT,
// ... in groups of NV whose loads are all issued before any is used.
template <int DT, bool AL, int NT, int NV, class F>
__device__ __forceinline__ void row_each(const char* row, int V, int nvec, F&& f) {
  constexpr int EPV = Elem<DT>::kPerVec;
  const int nv = (V + EPV - 1) / EPV;
  for (int v0 = threadIdx.x; v0 < nv; v0 += NT * NV) {
    float x[NV][EPV];
#pragma unroll
    for (int k = 0; k < NV; ++k) wvec<DT, AL>(row, V, nvec, (int64_t)v0 + k * NT, x[k]);
#pragma unroll
    for (int k = 0; k < NV; ++k)
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t j = ((int64_t)v0 + k * NT) * EPV + e;
        if (j < V) f(j, x[k][e]);
      }
  }
}

template <int DT, bool AL>
__global__ __launch_bounds__(kCT) void k_wcut(LinCfg c, WideCfg wc) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int NV = kCutNV;
  const int64_t sr = blockIdx.x;
  const char* row = c.rows.row(sr);
  const int V = c.V, t = threadIdx.x;
  const int nv = (V + EPV - 1) / EPV;
  __shared__ uint32_t s_cnt[kHist];
  __shared__ unsigned long long s_mass[kHist];
  __shared__ long long shl[kCTW + 1];
  __shared__ float shf[kCTW];
  __shared__ double shd[kCTW];
  __shared__ int shi[4];
  // radix levels: key bits [20, 32), [8, 20), [0, 8)
  auto kShift = [](int L) { return L == 0 ? 20 : (L == 1 ? 8 : 0); };
  auto kBits = [](int L) { return L == 2 ? 8 : 12; };
  for (int i = t; i < kHist; i += kCT) {
    s_cnt[i] = 0;
    s_mass[i] = 0;
  }
  __syncthreads();

  // ---- pass 0: maximum, validity, finite count, and the first count level
  // of the top-k selection (it needs no maximum)
  const bool kwant = wc.top_k > 0;
  float m = -INFINITY;
  long long nf = 0, bad = 0;
  row_each<DT, AL, kCT, NV>(row, V, c.nvec, [&](int64_t, float a) {
    m = fmaxnan(m, a);
    if (isnan(a) || (isinf(a) && a > 0.0f)) bad = 1;
    if (!is_neg_inf(a)) {
      ++nf;
      if (kwant) atomicAdd(&s_cnt[wkey(a) >> kShift(0)], 1u);
    }
  });
  m = block_max<kCT>(m, shf);
  bad = block_sum_ll<kCT>(bad, shl);
  nf = block_sum_ll<kCT>(nf, shl);
  CutRec* out = wc.cut + sr;
  if (bad || nf == 0 || isnan(m) || isinf(m)) {
    if (t == 0) *out = CutRec{m, kKeyNegInf, -1, 1, 0.0, 0.0};
    return;
  }
  const double c64 = c.c64, mc = (double)m * c64;
  // Fixed-point masses of the top-p guess: 2^((a - m) c) in binary32 (at
  // most 1 + 2^-23) scaled so that V of them stay below 2^63. The guess only
  // picks the first key to try; exact fp64 sums decide.
  const float c32 = c.c32, mc32 = m * c.c32;
  const int lg = 64 - __clzll((unsigned long long)V);
  const double fx_scale = ldexp(1.0, 62 - lg);
  auto fxw = [&](float a) {
    return (unsigned long long)((double)__builtin_amdgcn_exp2f(__builtin_fmaf(a, c32, -mc32)) * fx_scale);
  };

  // tokens kept by the top-k stage: kept_by(key, j, kkey, kid) (every finite
  // token until a top-k cut is set)
  uint32_t kkey = kKeyNegInf;
  int32_t kid = -1;

  // id of the r-th smallest kept token (1-based) whose key is `key`: rounds of
  // kCT * NV vectors in id order (thread t takes NV consecutive vectors), each
  // counted and scanned in thread order
  auto id_select = [&](uint32_t key, long long r) -> int32_t {
    long long base = 0;
    if (t == 0) shi[2] = -1;
    __syncthreads();
    for (int v0 = 0; v0 < nv; v0 += kCT * NV) {
      const int vt = v0 + t * NV;
      float x[NV][EPV];
#pragma unroll
      for (int k = 0; k < NV; ++k) wvec<DT, AL>(row, V, c.nvec, (int64_t)vt + k, x[k]);
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < NV; ++k)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int64_t j = ((int64_t)vt + k) * EPV + e;
          cnt += (j < V && wkey(x[k][e]) == key && kept_by(key, j, kkey, kid)) ? 1 : 0;
        }
      long long tot;
      const long long excl = block_scan_ll<kCT>(cnt, shl, &tot);
      if (base + excl < r && r <= base + excl + cnt) {
        long long n = base + excl;
#pragma unroll
        for (int k = 0; k < NV; ++k)
#pragma unroll
          for (int e = 0; e < EPV; ++e) {
            const int64_t j = ((int64_t)vt + k) * EPV + e;
            if (j < V && wkey(x[k][e]) == key && kept_by(key, j, kkey, kid) && ++n == r) shi[2] = (int)j;
          }
      }
      __syncthreads();
      const int found = shi[2];
      __syncthreads();
      if (found >= 0) return found;
      base += tot;
    }
    return -1;
  };

  // radix level L > 0 over the kept tokens whose key matches (key & pmask) ==
  // prefix: counts, or fixed-point masses when `mass`, per value of the
  // kBits(L) key bits below kShift(L)
  auto level = [&](int L, uint32_t prefix, uint32_t pmask, bool mass) {
    const int nb = 1 << kBits(L);
    for (int i = t; i < nb; i += kCT) {
      s_cnt[i] = 0;
      s_mass[i] = 0;
    }
    __syncthreads();
    row_each<DT, AL, kCT, NV>(row, V, c.nvec, [&](int64_t j, float a) {
      const uint32_t key = wkey(a);
      if (!kept_by(key, j, kkey, kid) || (key & pmask) != prefix) return;
      const int d = (int)((key >> kShift(L)) & (uint32_t)(nb - 1));
      if (mass) atomicAdd(&s_mass[d], fxw(a));
      else atomicAdd(&s_cnt[d], 1u);
    });
    __syncthreads();
  };

  // ---- top-k: the top_k-th token of the order
  const bool kact = kwant && (long long)wc.top_k < nf;
  if (kact) {
    uint32_t prefix = 0, pmask = 0;
    unsigned long long above = 0;
    for (int L = 0; L < 3; ++L) {
      if (L > 0) level(L, prefix, pmask, false);
      const int d = select_bin<kCT>(s_cnt, 1 << kBits(L), (unsigned long long)wc.top_k, &above, shl, shi);
      prefix |= (uint32_t)d << kShift(L);
      pmask |= (uint32_t)((1u << kBits(L)) - 1u) << kShift(L);
    }
    const long long r = (long long)wc.top_k - (long long)above;  // ties of that key taken, in id order
    const int32_t id = id_select(prefix, r);
    kkey = prefix;
    kid = id;
  }

  // ---- mass of the kept-by-top-k tokens (fp64, fixed order), and with a
  // top-p the first mass level of the guess and the total fixed-point mass
  const bool pact = wc.top_p < 1.0;
  if (pact) {
    for (int i = t; i < kHist; i += kCT) s_mass[i] = 0;
    __syncthreads();
  }
  double S = 0.0;
  long long M = 0;
  row_each<DT, AL, kCT, NV>(row, V, c.nvec, [&](int64_t j, float a) {
    const uint32_t key = wkey(a);
    if (!kept_by(key, j, kkey, kid)) return;
    S += wweight(a, c64, mc);
    if (pact) {
      const unsigned long long f = fxw(a);
      M += (long long)f;
      atomicAdd(&s_mass[key >> kShift(0)], f);
    }
  });
  S = block_sum<kCT>(S, shd);
  if (!pact) {
    if (t == 0) *out = CutRec{m, kkey, kid, 0, S, 0.0};
    return;
  }
  M = block_sum_ll<kCT>(M, shl);

  // ---- top-p: the crossing key of the fixed-point masses
  const double target = wc.top_p * S;
  uint32_t prefix = 0, pmask = 0;
  {
    unsigned long long above = 0;
    const unsigned long long need = (unsigned long long)(wc.top_p * (double)M);
    for (int L = 0; L < 3; ++L) {
      if (L > 0) level(L, prefix, pmask, true);
      const int d = select_bin<kCT>(s_mass, 1 << kBits(L), need > 0 ? need : 1ull, &above, shl, shi);
      prefix |= (uint32_t)d << kShift(L);
      pmask |= (uint32_t)((1u << kBits(L)) - 1u) << kShift(L);
    }
  }
  // ---- confirm on exact fp64 sums. For a probe key k: ma = the mass of the
  // kept tokens above k, cn = the kept tokens at k (all of weight wk). The
  // crossing is at k iff ma < target <= ma + cn wk; then r = the smallest count
  // of them reaching target. Otherwise the crossing key lies above k (ma >=
  // target) or below it, and the bracket [lo, hi] of kept keys that may hold
  // it shrinks past k. Probes: the fixed-point guess, up to two neighbouring
  // keys, then bisection of the bracket in key space (at most 32 more).
  uint32_t lo = 0u, hi = 0xffffffffu, key_p = prefix;
  double mass_above = 0.0;
  long long r = 0, cnt_p = 0;
  bool found = false, have_fb = false;
  uint32_t fb_key = 0u;  // a key whose whole group falls short of target by rounding
  double fb_ma = 0.0;
  long long fb_cn = 0;
  for (int it = 0; it < 48; ++it) {
    double ma = 0.0;
    long long cn = 0;
    uint32_t up = 0xffffffffu, down = 0u;  // nearest kept keys above and below key_p
    row_each<DT, AL, kCT, NV>(row, V, c.nvec, [&](int64_t j, float a) {
      const uint32_t key = wkey(a);
      if (!kept_by(key, j, kkey, kid)) return;
      if (key > key_p) {
        ma += wweight(a, c64, mc);
        up = min(up, key);
      } else if (key == key_p) {
        ++cn;
      } else {
        down = max(down, key);
      }
    });
    ma = block_sum<kCT>(ma, shd);
    cn = block_sum_ll<kCT>(cn, shl);
    // nearest keys: wave minimum and maximum, then across the waves
    up = ~wave_max_u32(~up);
    down = wave_max_u32(down);
    if (t == 0) {
      shi[0] = -1;  // 0xffffffff as unsigned
      shi[1] = 0;
    }
    __syncthreads();
    if ((t & (kWave - 1)) == 0) {
      atomicMin((unsigned int*)&shi[0], up);
      atomicMax((unsigned int*)&shi[1], down);
    }
    __syncthreads();
    up = (uint32_t)shi[0];
    down = (uint32_t)shi[1];
    __syncthreads();
    bool go_up;
    if (ma >= target) {
      go_up = true;
      lo = up;
    } else {
      if (cn > 0) {
        const double wk = wweight(wkey_value(key_p), c64, mc);
        long long rr = cn + 1;
        if (wk > 0.0) {
          const double need = ceil((target - ma) / wk);
          rr = need < 1.0 ? 1 : (need > (double)cn ? cn + 1 : (long long)need);
          while (rr > 1 && ma + (double)(rr - 1) * wk >= target) --rr;
          while (rr <= cn && ma + (double)rr * wk < target) ++rr;
        }
        if (rr <= cn) {
          found = true;
          mass_above = ma;
          cnt_p = cn;
          r = rr;
          break;
        }
        have_fb = true;
        fb_key = key_p;
        fb_ma = ma;
        fb_cn = cn;
      }
      go_up = false;
      hi = down;
    }
    if (lo > hi) break;
    key_p = it < 2 ? (go_up ? lo : hi) : lo + (hi - lo) / 2;
  }
  if (!found) {
    if (!have_fb) {  // no probe reached a decision (not expected): report the row as invalid
      if (t == 0) *out = CutRec{m, kKeyNegInf, -1, 1, 0.0, 0.0};
      return;
    }
    key_p = fb_key;  // the crossing fell between keys by rounding: keep the whole group
    mass_above = fb_ma;
    cnt_p = fb_cn;
    r = fb_cn;
  }
  const int32_t id_p = id_select(key_p, r);
  const double wp = wweight(wkey_value(key_p), c64, mc);
  if (t == 0) *out = CutRec{m, key_p, id_p, 0, mass_above + (double)r * wp, (double)cnt_p};
}

// ------------------------------------------------------------ draft row --
// Inverse-CDF draw in token-id order from softmax of the kept set of one row
// (cut cr), with uniform u, by a workgroup of NT threads: fp64 sub-block sums
// of the kept weights into s_sb[nsb], then wave 0 picks. Returns the token on
// the lanes of wave 0 (other waves return -2 and must do nothing more).
template <int DT, bool AL, int NT>
__device__ int wide_draw(const LinCfg& c, const CutRec& cr, const char* row, double u, double* s_sb) {
  constexpr int EPV = Elem<DT>::kPerVec;
  constexpr int EPL = kSB / kWave;
  const int t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1);
  const double c64 = c.c64, mc = (double)cr.m * c64;
  auto weights = [&](int64_t j0, double (&w)[EPL]) {
#pragma unroll
    for (int v = 0; v < EPL / EPV; ++v) {
      float x[EPV];
      wvec<DT, AL>(row, c.V, c.nvec, j0 / EPV + v, x);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t j = j0 + v * EPV + e;
        w[v * EPV + e] = (j < c.V && kept_by(wkey(x[e]), j, cr.key, cr.id)) ? wweight(x[e], c64, mc) : 0.0;
      }
    }
  };
  const int nsb = c.nsb;
  for (int sb = wave; sb < nsb; sb += NT / kWave) {
    double w[EPL];
    weights((int64_t)sb * kSB + (int64_t)lane * EPL, w);
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) s += w[k];
    s = wave_sum(s);
    if (lane == 0) s_sb[sb] = s;
  }
  __syncthreads();
  if (wave != 0) return -2;
  double mine = 0.0;
  for (int sb = lane; sb < nsb; sb += kWave) mine += s_sb[sb];
  const double W = wave_sum(mine);
  return wave_pick(nsb, c.V, u * W, [&](int sb) { return s_sb[sb]; },
                   [&](int64_t j0, double(&w)[EPL]) { weights(j0, w); });
}

// One workgroup per draft row: x ~ softmax(filter(q / T)) by inverse CDF in
// token-id order with U(seed, step, b, i, 0x40000000) ("Uno" research
// explainer, §3.3: drafts are drawn from the draft distributions); -1 for an
// invalid row.
template <int DT, bool AL>
__global__ __launch_bounds__(kDWT) void k_wdraft(LinCfg c, WideCfg wc) {
  extern __shared__ double s_sb[];  // one fp64 sum per sub-block
  const int64_t qr = blockIdx.x;    // draft row in [0, B * K)
  const int K = c.K;
  const int64_t b = qr / K;
  const int i = (int)(qr - b * K);
  const int64_t sr = b * (c.rows.np + c.rows.nq) + c.rows.np + i;
  const CutRec cr = wc.cut[sr];
  if (cr.bad) {
    if (threadIdx.x == 0) c.draft[qr] = -1;
    return;
  }
  const int x = wide_draw<DT, AL, kDWT>(c, cr, c.rows.row(sr), c.rng.u((uint32_t)b, (uint32_t)i, kDrawDraft), s_sb);
  if (threadIdx.x == 0) c.draft[qr] = x;
}

// Tree node drafts: node n is the sib[n]-th child of row r = prow[n] and is
// drawn from draft row r with U(seed, step, b, r, 0x40000000 + sib[n]) ("Uno"
// research explainer, §3.4: the Tree Sampler's candidates come from the draft
// distributions); -1 for an invalid row.
template <int DT, bool AL>
__global__ __launch_bounds__(kDWT) void k_wtdraft(LinCfg c, WideCfg wc, TreeTopo tp, TreeCfg tc) {
  extern __shared__ double s_sb[];
  const int N = tc.N;
  const int64_t b = blockIdx.x / N;
  const int n = (int)(blockIdx.x - b * N);
  const int r = tp.prow[n];
  const int64_t sr = b * 2 * (N + 1) + (N + 1) + r;
  const CutRec cr = wc.cut[sr];
  if (cr.bad) {
    if (threadIdx.x == 0) tc.tokens[b * N + n] = -1;
    return;
  }
  const double u = c.rng.u((uint32_t)b, (uint32_t)r, kDrawDraft + (uint32_t)tp.sib[n]);
  const int x = wide_draw<DT, AL, kDWT>(c, cr, c.rows.row(sr), u, s_sb);
  if (threadIdx.x == 0) tc.tokens[b * N + n] = x;
}

// --------------------------------------------------------------- resolve --
template <int DT, bool AL>
__global__ __launch_bounds__(kWT) void k_wresolve(LinCfg c, WideCfg wc) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int EPL = kSB / kWave;
  extern __shared__ double s_rec[];  // per sub-block: target mass, residual mass
  const int64_t b = blockIdx.x;
  const int K = c.K, R = 2 * K + 1, t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1);
  const CutRec* cut = wc.cut + b * R;
  __shared__ int s_bad, s_n;
  __shared__ int s_x[kMaxK];
  if (t == 0) s_bad = 0;
  __syncthreads();
  if (t < R && cut[t].bad) atomicOr(&s_bad, 1);
  if (t < K) {
    const int x = c.draft[b * K + t];
    s_x[t] = x;
    if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  const double c64 = c.c64;
  // probability of token x under filtered row r (its cut and kept mass)
  auto prob = [&](int r, int x) -> double {
    const CutRec cr = cut[r];
    const char* row = c.rows.row(b * R + r);
    const float a = E::load1(row, x);
    return kept_by(wkey(a), x, cr.key, cr.id) ? wweight(a, c64, (double)cr.m * c64) / cr.S : 0.0;
  };
  int acc = 1;
  double P = 0.0, Q = 0.0;
  if (t < K && !s_bad) {
    P = prob(t, s_x[t]);
    Q = prob(K + 1 + t, s_x[t]);
    acc = c.rng.u((uint32_t)b, (uint32_t)t, kDrawAccept) * Q < P;
  }
  if (t < kWave) {
    const unsigned long long rej = __ballot(t < K && !acc);
    if (t == 0) s_n = rej ? (__ffsll((long long)rej) - 1) : K;
  }
  __syncthreads();
  if (s_bad) {
    for (int i = t; i <= K; i += kWT) c.out_tokens[b * (K + 1) + i] = -1;
    if (c.out_probs)
      for (int i = t; i < 2 * K; i += kWT) c.out_probs[b * 2 * K + i] = 0.0f;
    if (c.fused)
      for (int i = t; i < K; i += kWT) c.draft[b * K + i] = -1;
    if (t == 0) {
      c.out_len[b] = -1;
      if (c.out_resid) c.out_resid[b] = 0.0;
    }
    return;
  }
  const int n = s_n;
  if (t < K && c.out_probs) {
    c.out_probs[(b * K + t) * 2 + 0] = (float)P;
    c.out_probs[(b * K + t) * 2 + 1] = (float)Q;
  }
  // ---- final row: target row n and, at a rejection, draft row n
  const bool resid = n < K;
  const CutRec cp = cut[n], cq = resid ? cut[K + 1 + n] : cut[n];
  const char* prow = c.rows.row(b * R + n);
  const char* qrow = c.rows.row(b * R + (resid ? K + 1 + n : n));
  const double mcp = (double)cp.m * c64, mcq = (double)cq.m * c64;
  // target and residual weights of the 16 tokens from j0 (0 past V)
  auto weights = [&](int64_t j0, double (&wp)[EPL], double (&wr)[EPL]) {
#pragma unroll
    for (int v = 0; v < EPL / EPV; ++v) {
      float xp[EPV], xq[EPV];
      wvec<DT, AL>(prow, c.V, c.nvec, j0 / EPV + v, xp);
      if (resid) wvec<DT, AL>(qrow, c.V, c.nvec, j0 / EPV + v, xq);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t j = j0 + v * EPV + e;
        double p = 0.0, q = 0.0;
        if (j < c.V) {
          if (kept_by(wkey(xp[e]), j, cp.key, cp.id)) p = wweight(xp[e], c64, mcp) / cp.S;
          if (resid && kept_by(wkey(xq[e]), j, cq.key, cq.id)) q = wweight(xq[e], c64, mcq) / cq.S;
        }
        wp[v * EPV + e] = p;
        wr[v * EPV + e] = fmax(0.0, p - q);
      }
    }
  };
  const int nsb = c.nsb;
  for (int sb = wave; sb < nsb; sb += kWTW) {
    double wp[EPL], wr[EPL];
    weights((int64_t)sb * kSB + (int64_t)lane * EPL, wp, wr);
    double sp = 0.0, sr_ = 0.0;
#pragma unroll
    for (int k = 0; k < EPL; ++k) {
      sp += wp[k];
      sr_ += wr[k];
    }
    sp = wave_sum(sp);
    sr_ = wave_sum(sr_);
    if (lane == 0) {
      s_rec[2 * sb] = sp;
      s_rec[2 * sb + 1] = sr_;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  const double u = c.rng.u((uint32_t)b, (uint32_t)n, kDrawFinal);
  double mine = 0.0;
  for (int sb = lane; sb < nsb; sb += kWave) mine += s_rec[2 * sb + 1];
  const double resid_mass = resid ? wave_sum(mine) : 0.0;
  const bool rmode = resid && resid_mass > 0.0;  // else the target row (bonus, or a vanished residual)
  mine = 0.0;
  for (int sb = lane; sb < nsb; sb += kWave) mine += s_rec[2 * sb];
  const double W = rmode ? resid_mass : wave_sum(mine);
  const int y = wave_pick(nsb, c.V, u * W, [&](int sb) { return s_rec[2 * sb + (rmode ? 1 : 0)]; },
                          [&](int64_t j0, double(&w)[EPL]) {
                            double wp[EPL], wr[EPL];
                            weights(j0, wp, wr);
#pragma unroll
                            for (int k = 0; k < EPL; ++k) w[k] = rmode ? wr[k] : wp[k];
                          });
  for (int i = lane; i <= K; i += kWave) c.out_tokens[b * (K + 1) + i] = i < n ? s_x[i] : (i == n ? y : -1);
  if (lane == 0) {
    c.out_len[b] = n;
    if (c.out_resid) c.out_resid[b] = resid_mass;
  }
}

// ------------------------------------------------------------------ tree --
// Tree verification on filtered rows ("Uno" research explainer, §3.4;
// recursive rejection over the children of a node, in ascending node id), one
// workgroup per request. At a row with children the running target after j
// rejections is (P - c_j Q)+ / G_j with c_0 = 0, G_0 = 1, c_{j+1} = c_j + G_j
// and G_j = sum_t max(0, P(t) - c_j Q(t)), which equals the normalised
// max(0, r_j - Q) of the recursive update; one fp64 pass over the row pair
// gives each new G. A vanished residual (G = 0) leaves the target as it was.
// The final draw (all children rejected, or a row without children) is an
// fp64 inverse-CDF draw from the running target with U(..., row, 0).
template <int DT, bool AL>
__global__ __launch_bounds__(kTT) void k_wtree(LinCfg c, WideCfg wc, TreeTopo tp, TreeCfg tc) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int EPL = kSB / kWave;
  extern __shared__ double s_sb[];  // per sub-block sums of the final draw's weights
  const int64_t b = blockIdx.x;
  const int N = tc.N, D = tc.D, R = N + 1, t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1);
  const CutRec* cut = wc.cut + b * 2 * R;
  __shared__ int s_bad;
  __shared__ int s_tok[kMaxNodes];
  __shared__ double shd[kTTW];
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < 2 * R; i += kTT)
    if (cut[i].bad) atomicOr(&s_bad, 1);
  for (int n = t; n < N; n += kTT) {
    const int x = tc.tokens[b * N + n];
    s_tok[n] = x;
    if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
  }
  for (int i = t; i <= D; i += kTT) c.out_tokens[b * (D + 1) + i] = -1;
  for (int i = t; i < D; i += kTT) tc.out_path[b * D + i] = -1;
  __syncthreads();
  if (s_bad) {
    if (t == 0) c.out_len[b] = -1;
    return;
  }
  const double c64 = c.c64;
  int row = 0, len = 0;  // uniform across the workgroup
  for (;;) {
    const CutRec cp = cut[row], cq = cut[R + row];
    const char* prow = c.rows.row(b * 2 * R + row);
    const char* qrow = c.rows.row(b * 2 * R + R + row);
    const double mcp = (double)cp.m * c64, mcq = (double)cq.m * c64;
    const double isp = 1.0 / cp.S, isq = 1.0 / cq.S;
    auto probs = [&](int x, double& P, double& Q) {
      const float ap = E::load1(prow, x), aq = E::load1(qrow, x);
      P = kept_by(wkey(ap), x, cp.key, cp.id) ? wweight(ap, c64, mcp) * isp : 0.0;
      Q = kept_by(wkey(aq), x, cq.key, cq.id) ? wweight(aq, c64, mcq) * isq : 0.0;
    };
    // max(0, P - cc Q) of the 16 tokens from j0 (0 past V)
    auto resid16 = [&](int64_t j0, double cc, double (&w)[EPL]) {
#pragma unroll
      for (int v = 0; v < EPL / EPV; ++v) {
        float xp[EPV], xq[EPV];
        wvec<DT, AL>(prow, c.V, c.nvec, j0 / EPV + v, xp);
        if (cc != 0.0) wvec<DT, AL>(qrow, c.V, c.nvec, j0 / EPV + v, xq);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int64_t j = j0 + v * EPV + e;
          double pp = 0.0, qq = 0.0;
          if (j < c.V) {
            if (kept_by(wkey(xp[e]), j, cp.key, cp.id)) pp = wweight(xp[e], c64, mcp) * isp;
            if (cc != 0.0 && kept_by(wkey(xq[e]), j, cq.key, cq.id)) qq = wweight(xq[e], c64, mcq) * isq;
          }
          w[v * EPV + e] = cc != 0.0 ? fmax(0.0, pp - cc * qq) : pp;
        }
      }
    };
    // sum of max(0, P - cc Q) over the 16 tokens from j0, one vector at a time
    auto rsum16 = [&](int64_t j0, double cc) {
      double acc = 0.0;
      for (int v = 0; v < EPL / EPV; ++v) {
        float xp[EPV], xq[EPV];
        wvec<DT, AL>(prow, c.V, c.nvec, j0 / EPV + v, xp);
        wvec<DT, AL>(qrow, c.V, c.nvec, j0 / EPV + v, xq);
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const int64_t j = j0 + v * EPV + e;
          double pp = 0.0, qq = 0.0;
          if (j < c.V) {
            if (kept_by(wkey(xp[e]), j, cp.key, cp.id)) pp = wweight(xp[e], c64, mcp) * isp;
            if (kept_by(wkey(xq[e]), j, cq.key, cq.id)) qq = wweight(xq[e], c64, mcq) * isq;
          }
          acc += fmax(0.0, pp - cc * qq);
        }
      }
      return acc;
    };
    const int k0 = tp.off[row], nk = tp.off[row + 1] - k0;
    double cc = 0.0, G = 1.0;
    int next = -1;
    for (int j = 0; j < nk; ++j) {
      const int child = tp.kids[k0 + j];
      double P, Q;
      probs(s_tok[child], P, Q);
      const double rt = fmax(0.0, P - cc * Q) / G;
      if (c.rng.u((uint32_t)b, (uint32_t)row, kDrawAccept + (uint32_t)j) * Q < rt) {
        next = child;
        break;
      }
      // rejected: G(c + G) over the row pair
      const double cn = cc + G;
      double part = 0.0;
      for (int sb = wave; sb < c.nsb; sb += kTTW) part += rsum16((int64_t)sb * kSB + (int64_t)lane * EPL, cn);
      const double Gn = block_sum<kTT>(part, shd);
      if (Gn > 0.0) {
        cc = cn;
        G = Gn;
      }
    }
    if (next >= 0) {
      if (t == 0) {
        tc.out_path[b * D + len] = next;
        c.out_tokens[b * (D + 1) + len] = s_tok[next];
      }
      ++len;
      row = next + 1;
      continue;
    }
    // final draw from the running target
    for (int sb = wave; sb < c.nsb; sb += kTTW) {
      const double s = wave_sum(rsum16((int64_t)sb * kSB + (int64_t)lane * EPL, cc));
      if (lane == 0) s_sb[sb] = s;
    }
    __syncthreads();
    if (wave != 0) return;
    double mine = 0.0;
    for (int sb = lane; sb < c.nsb; sb += kWave) mine += s_sb[sb];
    const double W = wave_sum(mine);
    const double u = c.rng.u((uint32_t)b, (uint32_t)row, kDrawFinal);
    const int y = wave_pick(c.nsb, c.V, u * W, [&](int sb) { return s_sb[sb]; },
                            [&](int64_t j0, double(&w)[EPL]) { resid16(j0, cc, w); });
    if (lane == 0) {
      c.out_tokens[b * (D + 1) + len] = y;
      c.out_len[b] = len;
    }
    return;
  }
}

// ------------------------------------------------------------ launchers --
template <int DT, bool AL>
static hipError_t wide_t(const LinCfg& c, const WideCfg& wc, bool draft_only, hipStream_t s) {
  const int64_t rows = c.B * (c.rows.np + c.rows.nq);
  PSI_LAUNCH(s, (k_wcut<DT, AL>), dim3((unsigned)rows), dim3(kCT), c, wc);
  if (c.fused || draft_only)
    PSI_LAUNCH_LDS(s, (k_wdraft<DT, AL>), dim3((unsigned)(c.B * c.K)), dim3(kDWT), (size_t)c.nsb * sizeof(double), c,
                   wc);
  if (draft_only) PSI_LAUNCH(s, k_draft_fix, dim3((unsigned)c.B), dim3(kWave), c);
  else PSI_LAUNCH_LDS(s, (k_wresolve<DT, AL>), dim3((unsigned)c.B), dim3(kWT), (size_t)c.nsb * 2 * sizeof(double), c, wc);
  return hipGetLastError();
}

hipError_t launch_wide(const LinCfg& c, const WideCfg& wc, int dtype, bool draft_only, hipStream_t s) {
  return PSI_DISPATCH(wide_t, dtype, c.aligned, c, wc, draft_only, s);
}

template <int DT, bool AL>
static hipError_t wide_tree_t(const LinCfg& c, const WideCfg& wc, const TreeTopo& tp, const TreeCfg& tc,
                              hipStream_t s) {
  const int64_t rows = c.B * 2 * (int64_t)(tc.N + 1);
  const size_t lds = (size_t)c.nsb * sizeof(double);
  PSI_LAUNCH(s, (k_wcut<DT, AL>), dim3((unsigned)rows), dim3(kCT), c, wc);
  if (c.fused) PSI_LAUNCH_LDS(s, (k_wtdraft<DT, AL>), dim3((unsigned)(c.B * tc.N)), dim3(kDWT), lds, c, wc, tp, tc);
  PSI_LAUNCH_LDS(s, (k_wtree<DT, AL>), dim3((unsigned)c.B), dim3(kTT), lds, c, wc, tp, tc);
  return hipGetLastError();
}

hipError_t launch_tree_wide(const LinCfg& c, const WideCfg& wc, const TreeTopo& tp, const TreeCfg& tc, int dtype,
                            hipStream_t s) {
  return PSI_DISPATCH(wide_tree_t, dtype, c.aligned, c, wc, tp, tc, s);
}

}  // namespace psi
