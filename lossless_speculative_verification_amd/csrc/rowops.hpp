// Row access and inverse-CDF helpers shared by the verification kernels.
#pragma once

#include "rowload.hpp"

namespace psi {

// ------------------------------------------------ final-row weights --
// fp64 weight 2^((a - m) c) of one logit a of a row with maximum m (c =
// log2(e) / T). For bfloat16 rows with m < 64 and (m + 64) c >= 100 (WRow.tab)
// the weights come from a per-call table of 2^(a c) over the magnitude window
// [2^-26, 63.25], times scale = 2^(-m c):
//   |a| in the window  tab(a) * scale, tab(a) = exp2_fast(a * c);
//   |a| below 2^-26    scale * (1 + t + t^2/2), t = a c ln 2 (exact to 1e-21);
//   a < -63.25 or -inf 0 (such a weight is below 2^-100 of the row maximum).
// Every other row takes exp2_fast(a c - m c). The rule depends only on a and
// the row, so sub-block sums and rescans of the same elements agree bit for
// bit, whether the (pre-scaled) table entry is read from LDS or recomputed.
//
// Table slot of the 16-bit code h (layout next to kTabLo): codes outside the
// window read the zero slot of their sign.
__device__ __forceinline__ uint32_t tab_idx(uint32_t h) {
  return min((h & 0x7fffu) - kTabLo, (uint32_t)kTabW);  // below or above the window -> kTabW
}
__device__ __forceinline__ uint32_t tab_slot(uint32_t h) { return tab_idx(h) + (h >> 15) * (uint32_t)kTabNeg; }
__device__ __forceinline__ bool tab_tiny(uint32_t h) { return (h & 0x7fffu) < kTabLo; }

// Byte offsets (8 * slot) of the two codes packed in a 32-bit word, in the
// matching 16-bit halves, computed two at a time with packed 16-bit ops. Also
// ORs the wrapped differences into `low`: bit 15 of a half is set iff that
// code lies below the window.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t tab_offsets2(uint32_t w, uint32_t& low) {
  const u16x2_t code = __builtin_bit_cast(u16x2_t, w);
  const u16x2_t d = (code & (u16x2_t)0x7fff) - (u16x2_t)kTabLo;
  low |= __builtin_bit_cast(uint32_t, d);
  const u16x2_t idx = __builtin_elementwise_min(d, (u16x2_t)kTabW);
  static_assert(8 * kTabNeg == 0x8000 && 8 * kTabW < 0x8000, "sign must be bit 15 of the byte offset");
  return (w & 0x80008000u) | __builtin_bit_cast(uint32_t, idx << (u16x2_t)3);
}

// Packed differences t = code - kTabLo of the two codes of w (16-bit halves,
// wrapping). For a code whose magnitude lies in [kTabLo, kTabLo + kTabNeg) a
// half of t holds the sign in bit 15 and the slot within its half in bits
// 0..11; for every other code (below the window: the difference wraps; above
// it; NaN and infinities) bits 12..14 of the half are not all zero. Callers
// test that on all the codes of a vector before tab_fast_off2.
__device__ __forceinline__ uint32_t tab_t2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, w) - (u16x2_t)kTabLo);
}
constexpr uint32_t kTabOutside = 0x70007000u;  // bits of t that flag a code outside the window
// Byte offsets (8 * slot) of the two codes from t = tab_t2(w), for codes
// inside the window, in a table of kTabAlloc slots: slot kTabW and kTabW + 1
// of a half are zero slots, so codes just above the window (magnitude codes
// kTabLo + kTabW, + 1) read zero as tab_offsets2 gives them.
__device__ __forceinline__ uint32_t tab_fast_off2(uint32_t t) {
  static_assert(kTabNeg == 4096 && kTabW + 2 == kTabNeg, "sign in bit 15, slot in bits 3..14");
  return (t & 0x80008000u) | __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, t) << (u16x2_t)3);
}

// tab_offsets2, and also ORs into `high` a value whose bit 15 in a half is
// set when that code lies above the window (or, for codes below it, may be).
__device__ __forceinline__ uint32_t tab_offsets2_chk(uint32_t w, uint32_t& low, uint32_t& high) {
  const u16x2_t code = __builtin_bit_cast(u16x2_t, w);
  const u16x2_t d = (code & (u16x2_t)0x7fff) - (u16x2_t)kTabLo;
  high |= __builtin_bit_cast(uint32_t, d + (u16x2_t)(0x8000 - kTabW));
  return tab_offsets2(w, low);
}

struct WRow {
  double mc, scale;
  bool tab;
};

__device__ __forceinline__ WRow wrow(bool bf16_tab, float m, double c64) {
  WRow w;
  w.mc = (double)m * c64;
  w.tab = bf16_tab && m <= (float)kTabMaxAbs && ((double)m + kTabMaxAbs) * c64 >= 100.0;
  w.scale = w.tab ? exp2_fast(-w.mc) : 0.0;
  return w;
}

// Weights of the row pair a final draw reads: the target row alone (bonus),
// or target and draft rows together, which use the table only if both rows
// qualify, so that the pair is evaluated under one rule.
__device__ __forceinline__ void wpair(bool bf16_tab, float mp, float mq, bool resid, double c64, WRow& wp,
                                      WRow& wq) {
  wp = wrow(bf16_tab, mp, c64);
  wq = wrow(bf16_tab && resid, mq, c64);
  if (resid && !(wp.tab && wq.tab)) {
    wp = wrow(false, mp, c64);
    wq = wrow(false, mq, c64);
  }
}

// The final draw of a linear block divides the pre-scale of a table row pair
// by the rows' normaliser estimates, so that the scaled weights are estimates
// of the probabilities themselves and compare directly.
__device__ __forceinline__ void norm_pair(WRow& wp, WRow& wq, bool resid, double sph, double sqh) {
  if (wp.tab) {
    wp.scale = wp.scale / sph;
    if (resid) wq.scale = wq.scale / sqh;
  }
}

__device__ __forceinline__ double tab_entry(uint32_t code, double c64) {
  return exp2_fast((double)__uint_as_float(code << 16) * c64);
}

__device__ __forceinline__ double tiny_weight(float a, double c64, double scale) {
  const double t = (double)a * (c64 * 0.69314718055994530942);
  return scale * __builtin_fma(t, __builtin_fma(t, 0.5, 1.0), 1.0);
}

// Fills the unscaled kTabSize-entry table with the workgroup's NT threads.
template <int NT>
__device__ __forceinline__ void fill_tab(double* tab, double c64) {
  for (int i = threadIdx.x; i < kTabSize; i += NT) {
    const int half = i >= kTabNeg, j = i - half * kTabNeg;
    tab[i] = j < kTabW ? tab_entry(((uint32_t)half << 15) | (kTabLo + (uint32_t)j), c64) : 0.0;
  }
}

// fp64 weight of one logit under the row rule above, reading a table already
// multiplied by w.scale when given (nullptr: recompute the entry); the two
// agree bit for bit.
template <int DT>
__device__ __forceinline__ double fweight(float a, const WRow& w, double c64, const double* tab_scaled) {
  if constexpr (DT == kBF16) {
    if (w.tab) {
      const uint32_t h = __float_as_uint(a) >> 16;
      if (tab_tiny(h)) return tiny_weight(a, c64, w.scale);
      if (tab_idx(h) == (uint32_t)kTabW) return 0.0;
      return tab_scaled ? tab_scaled[tab_slot(h)] : tab_entry(h, c64) * w.scale;
    }
  }
  return exp2_fast(__builtin_fma((double)a, c64, -w.mc));
}

// 32-bit word i of a 16-byte vector.
__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The 16 consecutive logits j0 .. j0+15 of one row as raw 16-byte vectors
// (the aligned path; elements past V read as -inf), so that their loads can be
// issued before their weights are needed.
template <int DT>
struct Raw16 {
  uint4 v[16 / Elem<DT>::kPerVec];
};
template <int DT, bool AL>
__device__ __forceinline__ void raw16(const LinCfg& c, const char* row, int64_t j0, Raw16<DT>& r) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int NV = 16 / EPV;
  if constexpr (AL) {
    // unconditional loads (indices clamped into the row; weights16 zeroes
    // elements past V), so that no branch makes the compiler wait for them
    const uint4* rp = (const uint4*)row;
#pragma unroll
    for (int v = 0; v < NV; ++v) r.v[v] = rp[min(j0 / EPV + v, (int64_t)c.nvec - 1)];
  } else {
    load_raw<DT, false, NV, 1>(row, c.V, c.nvec, j0 / EPV, r.v);
  }
}
// Weights of the 16 logits held in r (0 past V), under the rule of fweight;
// bfloat16 rows with the pre-scaled table read it without branches, and the
// rare logits below its window are redone out of line.
template <int DT>
__device__ __forceinline__ void weights16(const LinCfg& c, const Raw16<DT>& r, int64_t j0, const WRow& w,
                                          const double* tab_scaled, double (&out)[16]) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  if constexpr (DT == kBF16) {
    if (w.tab && tab_scaled) {
      uint32_t low = 0;
      const char* const tb = (const char*)tab_scaled;
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t o = tab_offsets2(word_of(r.v[v], i), low);
          out[v * 8 + 2 * i] = *(const double*)(tb + (o & 0xffffu));
          out[v * 8 + 2 * i + 1] = *(const double*)(tb + (o >> 16));
        }
      if (__ballot((low & 0x80008000u) != 0u)) {
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          float x[EPV];
          E::unpack(r.v[v], x);
#pragma unroll
          for (int e = 0; e < EPV; ++e)
            if (tab_tiny(__float_as_uint(x[e]) >> 16)) out[v * EPV + e] = tiny_weight(x[e], c.c64, w.scale);
        }
      }
#pragma unroll
      for (int k = 0; k < 16; ++k)
        if (j0 + k >= c.V) out[k] = 0.0;
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < 16 / EPV; ++v) {
    float x[EPV];
    E::unpack(r.v[v], x);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const int k = v * EPV + e;
      out[k] = j0 + k < c.V ? fweight<DT>(x[e], w, c.c64, tab_scaled) : 0.0;
    }
  }
}

// --------------------------------------------- inverse-CDF pick helper --
// Picks the smallest index j with (sum of weights up to and including j) >
// target, given per-sub-block weights wsb(sb) and per-element weights w(j)
// (fp64, index order), with a workgroup of NT threads. Sub-blocks are 1024
// elements. Rounding differences between the sub-block sums and the rescan are
// handled by falling back to the last positive weight. Returns -1 only if
// every weight is zero. `sh` needs NT / kWave doubles.
template <int NT = kWG, class WSB, class WEL>
__device__ int pick_index(int nsb, int V, double target, WSB wsb, WEL wel, double* sh) {
  static_assert(kSB % NT == 0, "a sub-block must split evenly over the workgroup");
  __shared__ int s_sel;
  __shared__ double s_pref;
  const int t = threadIdx.x;
  const int per = (nsb + NT - 1) / NT;
  const int s0 = min(nsb, t * per), s1 = min(nsb, s0 + per);
  double mine = 0.0;
  for (int sb = s0; sb < s1; ++sb) mine += wsb(sb);
  double total;
  const double excl = block_exclusive_scan<NT>(mine, sh, &total);
  if (t == 0) s_sel = 0x7fffffff;
  __syncthreads();
  {
    double acc = excl;
    for (int sb = s0; sb < s1; ++sb) {
      const double w = wsb(sb);
      if (w > 0.0 && acc + w > target) {
        atomicMin(&s_sel, sb);
        break;
      }
      acc += w;
    }
  }
  __syncthreads();
  if (s_sel == 0x7fffffff) {
    // rounding left no crossing: take the last sub-block with positive weight
    __syncthreads();
    if (t == 0) s_sel = -1;
    __syncthreads();
    for (int sb = s0; sb < s1; ++sb)
      if (wsb(sb) > 0.0) atomicMax(&s_sel, sb);
    __syncthreads();
    if (s_sel < 0) return -1;
  }
  const int sel = s_sel;
  // exact prefix before the chosen sub-block, recomputed in one fixed order
  if (sel >= s0 && sel < s1) {
    double acc = excl;
    for (int sb = s0; sb < sel; ++sb) acc += wsb(sb);
    s_pref = acc;
  }
  __syncthreads();
  const double tin = target - s_pref;
  // rescan: thread t owns elements [sel*1024 + EPT*t, +EPT)
  constexpr int EPT = kSB / NT;
  const int64_t j0 = (int64_t)sel * kSB + (int64_t)t * EPT;
  double w[EPT];
  double mine2 = 0.0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    w[k] = (j0 + k < V) ? wel(j0 + k) : 0.0;
    mine2 += w[k];
  }
  double tot2;
  const double excl2 = block_exclusive_scan<NT>(mine2, sh, &tot2);
  if (t == 0) s_sel = 0x7fffffff;
  __syncthreads();
  {
    double acc = excl2;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      if (w[k] > 0.0 && acc + w[k] > tin) {
        atomicMin(&s_sel, (int)(j0 + k));
        break;
      }
      acc += w[k];
    }
  }
  __syncthreads();
  int j = s_sel;
  if (j == 0x7fffffff) {
    __syncthreads();
    if (t == 0) s_sel = -1;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (w[k] > 0.0) atomicMax(&s_sel, (int)(j0 + k));
    __syncthreads();
    j = s_sel;
  }
  __syncthreads();
  return j;
}

// Sub-block selection of an inverse-CDF pick by one whole wave (all 64 lanes
// active), with no workgroup barrier: lane l owns a run of consecutive
// sub-blocks, whose weights wsb(sb) it reads. Returns, on every lane, the
// smallest sub-block whose running weight exceeds target, or the last one with
// positive weight if rounding leaves none (-1 if every weight is zero), and in
// pref the running weight before it.
template <class WSB>
__device__ int wave_select(int nsb, double target, WSB wsb, double& pref) {
  const int lane = threadIdx.x & (kWave - 1);
  const int per = (nsb + kWave - 1) / kWave;
  const int s0 = min(nsb, lane * per), s1 = min(nsb, s0 + per);
  double mine = 0.0;
  for (int sb = s0; sb < s1; ++sb) mine += wsb(sb);
  const double excl = wave_incl_scan(mine) - mine;
  int sel = -1, last = -1;
  double p0 = 0.0, lp = 0.0;
  {
    double acc = excl;
    for (int sb = s0; sb < s1; ++sb) {
      const double w = wsb(sb);
      if (w > 0.0) {
        if (sel < 0 && acc + w > target) {
          sel = sb;
          p0 = acc;
        }
        last = sb;
        lp = acc;
      }
      acc += w;
    }
  }
  unsigned long long m = __ballot(sel >= 0);
  int src;
  if (m) {
    src = __ffsll((long long)m) - 1;
  } else {  // rounding left no crossing: the last sub-block with positive weight
    m = __ballot(last >= 0);
    if (!m) {
      pref = 0.0;
      return -1;
    }
    src = 63 - __clzll((long long)m);
    sel = last;
    p0 = lp;
  }
  pref = __shfl(p0, src);
  return __shfl(sel, src);
}

// wave_select over weights held in registers: lane l owns sub-blocks
// [l * PER, l * PER + PER) (nsb <= 64 * PER) and v[k] is the weight of its
// k-th (0 past nsb). Same result as wave_select on the same weights.
template <int PER>
__device__ int wave_select_reg(int nsb, double target, const double (&v)[PER], double& pref) {
  const int lane = threadIdx.x & (kWave - 1);
  const int s0 = lane * PER;
  double mine = 0.0;
#pragma unroll
  for (int k = 0; k < PER; ++k) mine += v[k];
  const double excl = wave_incl_scan(mine) - mine;
  int sel = -1, last = -1;
  double p0 = 0.0, lp = 0.0, acc = excl;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (s0 + k < nsb && v[k] > 0.0) {
      if (sel < 0 && acc + v[k] > target) {
        sel = s0 + k;
        p0 = acc;
      }
      last = s0 + k;
      lp = acc;
    }
    acc += v[k];
  }
  unsigned long long m = __ballot(sel >= 0);
  int src;
  if (m) {
    src = __ffsll((long long)m) - 1;
  } else {  // rounding left no crossing: the last sub-block with positive weight
    m = __ballot(last >= 0);
    if (!m) {
      pref = 0.0;
      return -1;
    }
    src = 63 - __clzll((long long)m);
    sel = last;
    p0 = lp;
  }
  pref = __shfl(p0, src);
  return __shfl(sel, src);
}

// The element pick inside sub-block sbsel by one whole wave: lane l owns the 16
// consecutive elements from sbsel * kSB + 16 l, whose weights w[16] it holds
// (0 past the end of the row). Returns, on every lane, the smallest element
// whose running weight (from the sub-block's start) exceeds tin, or the last
// positive one if rounding leaves none (-1 if none is positive).
__device__ __forceinline__ int wave_rescan(int sbsel, double tin, const double (&w)[kSB / kWave]) {
  constexpr int EPL = kSB / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t j0 = (int64_t)sbsel * kSB + (int64_t)lane * EPL;
  double loc = 0.0;
#pragma unroll
  for (int k = 0; k < EPL; ++k) loc += w[k];
  double acc = wave_incl_scan(loc) - loc;
  int jj = -1, jl = -1;
#pragma unroll
  for (int k = 0; k < EPL; ++k) {
    if (w[k] > 0.0) {
      if (jj < 0 && acc + w[k] > tin) jj = (int)(j0 + k);
      jl = (int)(j0 + k);
    }
    acc += w[k];
  }
  unsigned long long m = __ballot(jj >= 0);
  if (m) return __shfl(jj, __ffsll((long long)m) - 1);
  m = __ballot(jl >= 0);
  return m ? __shfl(jl, 63 - __clzll((long long)m)) : -1;
}

// The pick of pick_index done by one whole wave: wave_select, then
// wave_rescan over the weights welb(j0, w) writes (w[k] = weight of element
// j0 + k, 0 past the end of the row). Same contract as pick_index; returns j
// on every lane.
template <class WSB, class WELB>
__device__ int wave_pick(int nsb, int V, double target, WSB wsb, WELB welb) {
  double pref;
  const int sbsel = wave_select(nsb, target, wsb, pref);
  if (sbsel < 0) return -1;
  constexpr int EPL = kSB / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  double w[EPL];
  welb((int64_t)sbsel * kSB + (int64_t)lane * EPL, w);
  return wave_rescan(sbsel, target - pref, w);
}

// ------------------------------------------------------- draft pick --
// Inverse-CDF draw (fp64, token-id order) from softmax(a / T) of one draft row
// given its per-sub-block records (maximum, sum of exp((a - m_sb) / T)).
template <int DT>
__device__ int draft_pick(const LinCfg& c, const char* row, const DraftRec* rec, double u, float* shf, double* sh) {
  using E = Elem<DT>;
  const int nsb = c.nsb, t = threadIdx.x;
  float m = -INFINITY;
  for (int sb = t; sb < nsb; sb += kWG) m = fmaxnan(m, rec[sb].m);
  m = block_max(m, shf);
  const double md = m, c64 = c.c64;
  auto wsb = [&](int sb) {
    const DraftRec r = rec[sb];
    return is_neg_inf(r.m) ? 0.0 : r.s * exp2_fast(((double)r.m - md) * c64);
  };
  double W;
  {
    double mine = 0.0;
    for (int sb = t; sb < nsb; sb += kWG) mine += wsb(sb);
    W = block_sum(mine, sh);
  }
  return pick_index(
      nsb, c.V, u * W, wsb,
      [&](int64_t j) {
        const DraftRec r = rec[j / kSB];
        const double f = exp2_fast(((double)r.m - md) * c64);
        return exp2_fast(((double)E::load1(row, j) - (double)r.m) * c64) * f;
      },
      sh);
}

// ------------------------------------------------------------ greedy --
// combine the chunk records of one row: argmax (lowest index on ties), bad flag
__device__ inline int row_argmax(const ArgRec* rec, int nch, int* bad) {
  float v = -INFINITY;
  int idx = 0x7fffffff, bd = 0;
  for (int ch = 0; ch < nch; ++ch) {
    const ArgRec r = rec[ch];
    bd |= r.bad;
    if (r.v > v || (r.v == v && r.idx < idx)) {
      v = r.v;
      idx = r.idx;
    }
  }
  if (is_neg_inf(v)) bd = 1;  // entirely -inf
  *bad = bd;
  return idx;
}

// ------------------------------------------------ filtered supports --
// Probability of token x in a filtered row (0 when filtered out).
__device__ inline double filt_prob(const FiltRow& h, const FiltEnt* e, int x) {
  int lo = 0, hi = h.cnt - 1;
  while (lo <= hi) {
    const int mid = (lo + hi) >> 1;
    const int id = e[mid].i;
    if (id == x) return ::exp(e[mid].z - h.L);
    if (id < x) lo = mid + 1;
    else hi = mid - 1;
  }
  return 0.0;
}

// Inverse-CDF draw over a list of weights in id order: smallest entry whose
// running sum exceeds u * W, else the last positive one; -1 if W is not positive.
template <class W>
__device__ inline int draw_list(int cnt, double u, W w, const FiltEnt* e) {
  double tot = 0.0;
  for (int t = 0; t < cnt; ++t) tot += w(t);
  if (!(tot > 0.0)) return -1;
  const double target = u * tot;
  double acc = 0.0;
  int last = -1;
  for (int t = 0; t < cnt; ++t) {
    const double wt = w(t);
    acc += wt;
    if (wt > 0.0) last = t;
    if (acc > target) return e[t].i;
  }
  return last >= 0 ? e[last].i : -1;
}

// Row normaliser of one row from its statistics records, by one thread: the
// exact maximum m and S = sum over the chunks, in chunk order, of
// s 2^((m_chunk - m) c) in fp64. Returns false for an invalid row (a NaN or
// +inf, or nothing finite). The records are loaded in batches before their
// values are used, so that a row costs a few memory latencies rather than one
// per chunk; the order of the sum is still the chunks' (results are the same
// bit for bit as a plain loop's).
__device__ __forceinline__ bool row_norm(const StatRec* rec, int nch, float c32, float* m_out, double* S_out) {
  constexpr int kB = 8;
  float m = -INFINITY;
  for (int c0 = 0; c0 < nch; c0 += kB) {
    float mm[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) mm[u] = c0 + u < nch ? rec[c0 + u].m : -INFINITY;
#pragma unroll
    for (int u = 0; u < kB; ++u) m = fmaxnan(m, mm[u]);
  }
  double S = 0.0;
  bool bad = isnan(m) || isinf(m);
  if (!bad)
    for (int c0 = 0; c0 < nch; c0 += kB) {
      float mm[kB];
      double ss[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const bool in = c0 + u < nch;
        mm[u] = in ? rec[c0 + u].m : -INFINITY;
        ss[u] = in ? rec[c0 + u].s : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (c0 + u >= nch) break;
        if (isnan(ss[u])) bad = true;
        else if (!is_neg_inf(mm[u])) S += ss[u] * ::exp2(((double)mm[u] - (double)m) * (double)c32);
      }
    }
  if (!(S > 0.0)) bad = true;
  *m_out = m;
  *S_out = S;
  return !bad;
}

}  // namespace psi
