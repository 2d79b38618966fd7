// Linear Psi-Spec verification, draft sampling and greedy mode on gfx950.
//
// Method ("Uno" research explainer, §3.3 Psi-Spec and §3.4 Linear Sampler):
// draft x_i ~ q_i for every block position; accept x_i with probability
// min(1, p_i(x_i) / q_i(x_i)); keep the longest accepted prefix; at the first
// rejection draw from the normalised positive part of p - q; when every draft
// survives draw one more token from the last target row.
//
// Pipeline (every kernel enqueued on the caller's stream, nothing allocated):
//   k_stats32   (stats.hip) chunk maxima and sums of every target and draft
//               row -> log-normalisers good to ~1e-7, enough for the accept
//               test.
//   k_draftrow  with drafts drawn inside the call: per draft row, fp64
//               sub-block sums under the final-draw weight rule and the
//               inverse-CDF pick of the draft.
//   k_resolve   per request (16 waves): row normalisers, p(x_i), q(x_i),
//               Philox accept tests and a wave ballot for the first rejection
//               n; then fp64 sums per 1024-element sub-block over the one row
//               pair the final draw needs (p_n and q_n, or the bonus row p_K);
//               then, when one workgroup owns the request, the inverse-CDF
//               pick from those sums and an fp64 rescan of one sub-block.
//   k_final     the pick, when several workgroups shared a request's sums.
// Draft sampling alone runs k_stats32 over the draft rows, then k_draftrow.
// Greedy mode (temperature 0) uses k_argmax and
// k_greedy_decide. The final draws are done in fp64 because an inverse-CDF
// pick over 151936 tokens must agree with an fp64 reference to ~1e-12 of the
// total mass to give the same token; the accept test only needs ~1e-7.
#include <algorithm>

#include "rowops.hpp"

namespace psi {

// Resolve launch shape: one workgroup per request from this many requests on
// (256 CUs), else about this many workgroups in total.
constexpr int64_t kResolveOneWgMinB = 192;
constexpr int64_t kResolveTargetWgs = 256;
// Sub-block records a one-workgroup resolve keeps in LDS at most: the
// workgroup also holds the two 64 KB weight tables, within 160 KB.
constexpr size_t kResolveMaxLds = 24 * 1024;

// Threads of a draft-row workgroup (k_draftrow, k_qrow, k_tqrow).
constexpr int kDT = 512;
constexpr int kDWaves = kDT / kWave;

// The unscaled 2^(a c) table (kTabAlloc slots), filled by kDT threads
// with one exp2 pair per 16 slots: thread t takes the 16 codes that share
// sign, exponent and the top 3 mantissa bits, A = 2^(a_0 c) for the first of
// them and r = 2^(u c) for the code step u, and slot k gets A * r^k with r^k
// a running product (relative error below 2e-15, far inside what the draws
// need). The draft-row pass and its draw (k_qrow), and the resolve step
// (scaled copies) read this table.
__device__ __forceinline__ void fill_tab_steps(double* tab, double c64) {
  const int t = threadIdx.x;  // kDT = 2 halves x 256 groups of 16 slots
  static_assert(kDT == 512 && kTabW <= 4096 && kTabNeg == 4096, "one group of 16 slots per thread");
  const int half = t >> 8, j0 = (t & 255) * 16;
  const uint32_t code0 = ((uint32_t)half << 15) | (kTabLo + (uint32_t)j0);
  const float a0 = __uint_as_float(code0 << 16);
  const float a1 = __uint_as_float((code0 + 1u) << 16);  // same exponent: j0 + 1 < next multiple of 128
  const double A = exp2_fast((double)a0 * c64);
  const double r = exp2_fast(((double)a1 - (double)a0) * c64);
  double rk = 1.0;
  double* const out = tab + half * kTabNeg + j0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    out[k] = j0 + k < kTabW ? A * rk : 0.0;  // the zero slots of this half
    rk *= r;
  }
}

// ------------------------------------------------------------ resolve --
// Threads of a resolve workgroup: 16 waves, so that one workgroup per request
// keeps every SIMD of a CU busy through the fp64 final-row pass.
constexpr int kRT = 1024;
constexpr int kRWaves = kRT / kWave;


// Corrections for one 16-byte bfloat16 vector pair holding logits whose
// magnitude is below the table window: the pass read a zero slot for them and
// classified the element by the slot values. Returns, in the layout of ResRec
// (sp, sq, and the parts where the target part exceeds the draft part), what
// the exact weights add minus what the slot values added.
__device__ __attribute__((noinline)) ResRec tiny_fixup(uint4 rp, uint4 rq, bool resid, double c64, double scp,
                                                       double scq, const double* tp, const double* tq) {
  float xp[8], xq[8];
  Elem<kBF16>::unpack(rp, xp);
  Elem<kBF16>::unpack(rq, xq);
  ResRec f = {0.0, 0.0, 0.0, 0.0};
  for (int e = 0; e < 8; ++e) {
    const uint32_t hp = __float_as_uint(xp[e]) >> 16, hq = __float_as_uint(xq[e]) >> 16;
    const bool tp_ = tab_tiny(hp), tq_ = resid && tab_tiny(hq);
    if (!tp_ && !tq_) continue;
    const double ep_s = tp[tab_slot(hp)];
    const double ep = tp_ ? tiny_weight(xp[e], c64, scp) : ep_s;
    if (tp_) f.sp += ep;
    if (resid) {
      const double eq_s = tq[tab_slot(hq)];
      const double eq = tq_ ? tiny_weight(xq[e], c64, scq) : eq_s;
      if (tq_) f.sq += eq;
      const bool in = ep > eq, in_s = ep_s > eq_s;
      f.a += (in ? ep : 0.0) - (in_s ? ep_s : 0.0);
      f.bq += (in ? eq : 0.0) - (in_s ? eq_s : 0.0);
    }
  }
  return f;
}

// fp64 sums of this workgroup's sub-blocks [sb0, sb1) of the final row pair
// (RESID) or the target row alone, one wave per sub-block (sb0 + wave, then
// every NW-th, by the first NW waves of the workgroup; every wave runs pre()). Software-pipelined over NBUF register buffers that change
// roles each step (no copies, so loads stay in flight across steps): bfloat16
// keeps the next two sub-blocks in flight, fp32 the next one. TAB: weights
// are read from the pre-scaled LDS tables tp / tq (bfloat16 only), whose
// values estimate the probabilities, so the target part is above the draft
// part where ep > eq; otherwise where a_p - a_q > dx. pre() runs once on
// every thread of the workgroup after each wave has issued the loads of its
// first sub-blocks and before any weight is read, so that work it does (the
// tables' scaling, and the barrier after it) hides under their latency.
//
// CHK (target row alone, bfloat16 table): also sets *chk when the row holds a
// code above the table window that is positive or NaN, i.e. when the row may
// not qualify for the table rule; other codes above the window (a < -63.25,
// -inf) read the zero slot as the rule says.
//
// RING > 0 keeps RING sub-blocks in flight per wave in a ring of register
// buffers (RING - 1 ahead of the one being reduced) instead of the default.
//
// FAST (TAB, not CHK): the tables hold kTabAlloc slots each (the
// running-product fill) and tq = tp + kTabAlloc. A vector pair whose codes
// all lie inside the window then takes its slots from tab_fast_off2, with
// the second table reached at byte 2^16; any other vector pair takes the
// general code below. Both read the same slots.
template <int DT, bool AL, bool TAB, bool RESID, bool PICK, int NW = kRWaves, class PRE, bool CHK = false,
          int RING = 0, bool FAST = false>
__device__ __forceinline__ void resolve_pass(const LinCfg& c, int64_t b, const char* prow, const char* qrow,
                                             int sb0, int sb1, const double* tp, const double* tq, const WRow& wp,
                                             const WRow& wq, float dx, ResRec* s_rec, PRE pre, int* chk = nullptr) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int VPL = kSB / (kWave * EPV);
  constexpr int NBUF = DT == kBF16 ? 3 : 2;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const double c64 = c.c64;
  struct Buf {
    uint4 p[VPL], q[VPL];
  };
  // Loads are issued unconditionally, so that the compiler can count the
  // ones in flight: a sub-block past this part's range re-reads the part's
  // last sub-block (never reduced), and vectors past the end of an aligned
  // row re-read its last vector and are replaced by -inf.
  auto load = [&](int s, Buf& x) {
    const int sc = min(s, sb1 - 1);
    const int64_t v0 = (int64_t)sc * (kSB / EPV) + lane;
    if constexpr (AL) {
      const uint4 ninf = make_uint4(E::kNegInfWord, E::kNegInfWord, E::kNegInfWord, E::kNegInfWord);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int64_t idx = v0 + (int64_t)v * kWave, ic = min(idx, (int64_t)c.nvec - 1);
        const uint4 lp = stream_load((const uint4*)prow + ic);
        x.p[v] = idx < c.nvec ? lp : ninf;
        if constexpr (RESID) {
          const uint4 lq = stream_load((const uint4*)qrow + ic);
          x.q[v] = idx < c.nvec ? lq : ninf;
        }
      }
    } else {
      load_raw<DT, AL, VPL, kWave>(prow, c.V, c.nvec, v0, x.p);
      if constexpr (RESID) load_raw<DT, AL, VPL, kWave>(qrow, c.V, c.nvec, v0, x.q);
    }
  };
  auto reduce = [&](int s, const Buf& x) {
    double sp = 0.0, sq = 0.0, a = 0.0, bq = 0.0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      bool general = TAB;
      if constexpr (TAB && FAST && !CHK) {
        uint32_t tw[2][4], out = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          tw[0][i] = tab_t2(word_of(x.p[v], i));
          tw[1][i] = RESID ? tab_t2(word_of(x.q[v], i)) : 0u;
          out |= tw[0][i] | tw[1][i];
        }
        general = __ballot((out & kTabOutside) != 0u) != 0ull;
        if (!general) {
          const char* const tb = (const char*)tp;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t op = tab_fast_off2(tw[0][i]);
            const uint32_t oq = RESID ? tab_fast_off2(tw[1][i]) : 0u;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const double ep = *(const double*)(tb + (hf ? op >> 16 : op & 0xffffu));
              sp += ep;
              if constexpr (RESID) {
                // the draft table starts at byte 2^16: bit 16 set on its offsets
                const uint32_t aq = hf ? __builtin_amdgcn_alignbit(1u, oq, 16u) : ((oq & 0xffffu) | 0x10000u);
                const double eq = *(const double*)(tb + aq);
                sq += eq;
                const double in = ep > eq ? 1.0 : 0.0;  // target part above draft part
                a = __builtin_fma(in, ep, a);
                bq = __builtin_fma(in, eq, bq);
              }
            }
          }
        }
      }
      if constexpr (TAB) {
        if (general) {
          // two bfloat16 codes per word; logits below the window read a zero
          // slot and get their exact weight in the rare call below
          uint32_t low = 0, high = 0;
          const char* const tpb = (const char*)tp;
          const char* const tqb = (const char*)tq;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t wpw = word_of(x.p[v], i), wqw = RESID ? word_of(x.q[v], i) : 0u;
            const uint32_t op = CHK ? tab_offsets2_chk(wpw, low, high) : tab_offsets2(wpw, low);
            const uint32_t oq = RESID ? tab_offsets2(wqw, low) : 0u;
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const double ep = *(const double*)(tpb + (hf ? op >> 16 : op & 0xffffu));
              sp += ep;
              if constexpr (RESID) {
                const double eq = *(const double*)(tqb + (hf ? oq >> 16 : oq & 0xffffu));
                sq += eq;
                const double in = ep > eq ? 1.0 : 0.0;  // target part above draft part
                a = __builtin_fma(in, ep, a);
                bq = __builtin_fma(in, eq, bq);
              }
            }
          }
          if constexpr (CHK) {
            if (__ballot((high & 0x80008000u) != 0u)) {
              // exact test of the flagged codes (codes below the window may set
              // the flag too)
              bool hit = false;
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                  const uint32_t h = (word_of(x.p[v], i) >> (16 * hf)) & 0xffffu;
                  const bool above = !tab_tiny(h) && tab_idx(h) == (uint32_t)kTabW;
                  hit |= above && (!(h & 0x8000u) || (h & 0x7fffu) > 0x7f80u);
                }
              if (hit) atomicOr(chk, 1);
            }
          }
          const bool tiny = (low & 0x80008000u) != 0u;
          if (__ballot(tiny)) {
            // a call, so that this rare work stays out of the common path
            const ResRec f = tiny_fixup(x.p[v], RESID ? x.q[v] : make_uint4(0, 0, 0, 0), RESID, c64, wp.scale,
                                        wq.scale, tp, tq);
            sp += f.sp;
            sq += f.sq;
            a += f.a;
            bq += f.bq;
          }
        }
      } else {
        float xp[EPV], xq[EPV];
        E::unpack(x.p[v], xp);
        if constexpr (RESID) E::unpack(x.q[v], xq);
#pragma unroll 2
        for (int e = 0; e < EPV; ++e) {
          const double ep = exp2_fast(__builtin_fma((double)xp[e], c64, -wp.mc));
          sp += ep;
          if constexpr (RESID) {
            const double eq = exp2_fast(__builtin_fma((double)xq[e], c64, -wq.mc));
            sq += eq;
            const double in = xp[e] - xq[e] > dx ? 1.0 : 0.0;
            a = __builtin_fma(in, ep, a);
            bq = __builtin_fma(in, eq, bq);
          }
        }
      }
    }
    ResRec* const rec = PICK ? s_rec + s : c.res + b * c.nsb + s;
    if constexpr (RESID) {
      // lanes 0, 16, 32, 48 hold the sums of sp, sq, a, bq
      const double tot = wave_sum4(sp, sq, a, bq);
      if ((lane & 15) == 0) reinterpret_cast<double*>(rec)[lane >> 4] = tot;  // ResRec is four doubles
    } else {
      const double tot = wave_sum_dpp(sp);
      if (lane == 0) *rec = ResRec{tot, 0.0, 0.0, 0.0};
    }
  };
  constexpr int W = NW;
  // waves from NW on take no part in the pass (they only run pre())
  const bool member = wave < W;
  if constexpr (RING > 0) {
    Buf x[RING];
    int s = sb0 + wave;
    if (member && s < sb1) {
#pragma unroll
      for (int k = 0; k < RING - 1; ++k) load(s + k * W, x[k]);
    }
    pre();
    if (!member || s >= sb1) return;
    for (; s < sb1; s += RING * W) {
#pragma unroll
      for (int k = 0; k < RING; ++k) {
        load(s + (k + RING - 1) * W, x[(k + RING - 1) % RING]);
        reduce(s + k * W, x[k]);
        if (s + (k + 1) * W >= sb1) return;
      }
    }
    return;
  }
  Buf x0, x1, x2;
  int s = sb0 + wave;
  if (member && s < sb1) {
    load(s, x0);
    if constexpr (NBUF == 3) load(s + W, x1);
  }
  pre();
  if (!member || s >= sb1) return;
  if constexpr (NBUF == 3) {
    for (; s < sb1; s += 3 * W) {
      load(s + 2 * W, x2);
      reduce(s, x0);
      if (s + W >= sb1) break;
      load(s + 3 * W, x0);
      reduce(s + W, x1);
      if (s + 2 * W >= sb1) break;
      load(s + 4 * W, x1);
      reduce(s + 2 * W, x2);
    }
  } else {
    for (; s < sb1; s += 2 * W) {
      load(s + W, x1);
      reduce(s, x0);
      if (s + W >= sb1) break;
      load(s + 2 * W, x0);
      reduce(s + W, x1);
    }
  }
}

// Weights of the 16 consecutive logits j0 .. j0+15 of one row (0 past V), for
// the rescan of the final pick: one or two 16-byte loads when aligned.
template <int DT, bool AL>
__device__ __forceinline__ void row16(const LinCfg& c, const char* row, int64_t j0, const WRow& w,
                                      const double* tab, double (&out)[16]) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  if (AL && j0 + 16 <= c.V) {
    const uint4* rp = (const uint4*)row + j0 / EPV;
#pragma unroll
    for (int v = 0; v < 16 / EPV; ++v) {
      float x[EPV];
      E::unpack(rp[v], x);
#pragma unroll
      for (int e = 0; e < EPV; ++e) out[v * EPV + e] = fweight<DT>(x[e], w, c.c64, tab);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) out[k] = j0 + k < c.V ? fweight<DT>(E::load1(row, j0 + k), w, c.c64, tab) : 0.0;
  }
}

// One resolve workgroup per (request, part): the decision of the request
// (every part computes it; part 0 publishes it), then per-sub-block fp64 sums
// over the one row pair the final draw needs (target row n and draft row n at
// a rejection, the bonus row K otherwise) for this part's sub-blocks. With
// PICK (one part per request) the workgroup also draws the final token from
// its sub-block sums kept in LDS; otherwise k_final does.
template <int DT, bool AL, bool PICK>
__global__ __launch_bounds__(kRT) void k_resolve(LinCfg c, int parts) {
  using E = Elem<DT>;
  extern __shared__ ResRec s_rec[];  // PICK: one record per sub-block
  const int64_t b = blockIdx.x / parts;
  const int part = (int)(blockIdx.x - b * parts);
  const int K = c.K, R = 2 * K + 1, t = threadIdx.x;
  const int wave = t / kWave, lane = t & (kWave - 1);
  __shared__ float s_m[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ int s_bad, s_n;
  // the 2^(a c) table, then the same multiplied by the scale of the final
  // target row (first half) and of the final draft row (second half)
  __shared__ double s_tab[2 * kTabAlloc];
  const bool tab = DT == kBF16 && c.tab;

  // ---- decision: row normalisers, accept tests, first rejection. Wave 0
  // gathers the drafted tokens' logits while waves 2.. reduce the statistics
  // records of the 2K+1 rows; the table fill overlaps both.
  if (t == 0) s_bad = 0;
  __syncthreads();
  int x = -1;
  float ap = 0.0f, aq = 0.0f;
  if (t < K) {
    x = c.draft[b * K + t];
    if (x < 0 || x >= c.V) {
      atomicOr(&s_bad, 1);
    } else {
      ap = E::load1(prow_of(c, b, t), x);
      aq = E::load1(qrow_of(c, b, t), x);
    }
  }
  const int r = t - 2 * kWave;
  if (r >= 0 && r < R) {
    float m;
    double S;
    // NaN, +inf, or an all -inf row
    const int bad = row_norm(c.st + (b * R + r) * (int64_t)c.nch32, c.nch32, c.c32, &m, &S) ? 0 : 1;
    s_m[r] = m;
    s_S[r] = S;
    if (bad) atomicOr(&s_bad, 1);
  }
  // the table by the running-product fill (one exp2 pair per 16 slots, by the
  // first kDT threads)
  if (tab && t < kDT) fill_tab_steps(s_tab, c.c64);
  __syncthreads();
  int acc = 1;
  double P = 0.0, Q = 0.0;
  if (t < K && x >= 0 && x < c.V) {
    P = ::exp(((double)ap - (double)s_m[t]) * c.invT - ::log(s_S[t]));
    Q = ::exp(((double)aq - (double)s_m[K + 1 + t]) * c.invT - ::log(s_S[K + 1 + t]));
    const double u = c.rng.u((uint32_t)b, (uint32_t)t, kDrawAccept);
    acc = u * Q < P;
  }
  if (t < kWave) {
    const unsigned long long rej = __ballot(t < K && !acc);
    if (t == 0) s_n = rej ? (__ffsll((long long)rej) - 1) : K;
  }
  __syncthreads();
  if (s_bad) {
    if (part == 0) {
      for (int i = t; i <= K; i += kRT) c.out_tokens[b * (K + 1) + i] = -1;
      if (c.out_probs)
        for (int i = t; i < 2 * K; i += kRT) c.out_probs[b * 2 * K + i] = 0.0f;
      if (c.fused)
        for (int i = t; i < K; i += kRT) c.draft[b * K + i] = -1;
      if (t == 0) {
        c.out_len[b] = -1;
        if (c.out_resid) c.out_resid[b] = 0.0;
        if (!PICK) {
          ReqState st = {};
          st.err = 1;
          c.rs[b] = st;
        }
      }
    }
    return;
  }
  const int n = s_n;
  const bool resid = n < K;
  if (part == 0 && t < K && c.out_probs) {
    c.out_probs[(b * K + t) * 2 + 0] = (float)P;
    c.out_probs[(b * K + t) * 2 + 1] = (float)Q;
  }
  const float mp = s_m[n], mq = resid ? s_m[K + 1 + n] : 0.0f;
  const double sph = s_S[n], sqh = resid ? s_S[K + 1 + n] : 1.0;
  const double c64 = c.c64;
  WRow wp, wq;
  wpair(tab, mp, mq, resid, c64, wp, wq);
  norm_pair(wp, wq, resid, sph, sqh);
  // target part above draft part (ep / sph > eq / sqh) <=> a_p - a_q > dx
  // (the rule of rows without the table)
  const float dx = wp.tab ? 0.0f : (float)((::log2(sph) - ::log2(sqh) + wp.mc - wq.mc) / c64);
  const double u_final = c.rng.u((uint32_t)b, (uint32_t)n, kDrawFinal);
  if (!PICK && part == 0 && t == 0) {
    ReqState st = {};
    st.n = n;
    st.err = 0;
    st.mp = mp;
    st.mq = mq;
    st.sp_hat = sph;
    st.sq_hat = sqh;
    st.u_final = u_final;
    c.rs[b] = st;
  }

  // ---- fp64 pass over this part's sub-blocks; the tables are scaled while
  // the first loads of the pass are in flight
  double* const tabp = s_tab;
  double* const tabq = s_tab + kTabAlloc;
  auto scale_tables = [&]() {
    if (DT == kBF16 && wp.tab) {
      for (int i = t; i < kTabAlloc; i += kRT) {
        const double e = s_tab[i];
        if (resid) tabq[i] = e * wq.scale;
        tabp[i] = e * wp.scale;
      }
    }
    __syncthreads();
  };
  const char* prow = prow_of(c, b, n);
  const char* qrow = resid ? qrow_of(c, b, n) : prow;
  const int nsb = c.nsb;
  const int sb0 = (int)((int64_t)part * nsb / parts), sb1 = (int)((int64_t)(part + 1) * nsb / parts);
  if (resid) {
    if (DT == kBF16 && wp.tab)
      resolve_pass<DT, AL, DT == kBF16, true, PICK, kRWaves, decltype(scale_tables), false, 0, true>(
          c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec, scale_tables);
    else
      resolve_pass<DT, AL, false, true, PICK>(c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec,
                                              scale_tables);
  } else {
    if (DT == kBF16 && wp.tab)
      resolve_pass<DT, AL, DT == kBF16, false, PICK, kRWaves, decltype(scale_tables), false, 0, true>(
          c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec, scale_tables);
    else
      resolve_pass<DT, AL, false, false, PICK>(c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec,
                                               scale_tables);
  }
  if constexpr (PICK) {
    __syncthreads();
    // ---- final draw (inverse CDF, fp64) from the sub-block sums in LDS, by wave 0
    if (wave != 0) return;
    const double* const tps = wp.tab ? tabp : nullptr;
    const double* const tqs = wq.tab ? tabq : nullptr;
    // Lane l owns a run of consecutive sub-blocks. The scaled sums estimate
    // probabilities, so the sub-block of the draw is known (except within
    // ~1e-7 of a sub-block edge) before the exact totals: its logits are
    // loaded while those are reduced, and loaded again in the rare case that
    // the exact selection differs.
    const int per = (nsb + kWave - 1) / kWave;
    const int s0 = min(nsb, lane * per), s1 = min(nsb, s0 + per);
    const double kpe = wp.tab ? 1.0 : 1.0 / sph, kqe = wq.tab ? 1.0 : 1.0 / sqh;
    auto west = [&](int i) {
      return resid ? fmax(0.0, s_rec[i].a * kpe - s_rec[i].bq * kqe) : s_rec[i].sp;
    };
    double me = 0.0, msp = 0.0, msq = 0.0;
    for (int i = s0; i < s1; ++i) {
      me += west(i);
      msp += s_rec[i].sp;
      msq += s_rec[i].sq;
    }
    double pref;
    const int sel_e = wave_select(nsb, u_final * wave_sum_dpp(me), west, pref);
    Raw16<DT> rp, rq;
    constexpr int EPL = kSB / kWave;
    if (sel_e >= 0) {
      const int64_t j0 = (int64_t)sel_e * kSB + (int64_t)lane * EPL;
      raw16<DT, AL>(c, prow, j0, rp);
      if (resid) raw16<DT, AL>(c, qrow, j0, rq);
    }
    // exact totals and masses
    const double Sp = wave_sum_dpp(msp), Sq = resid ? wave_sum_dpp(msq) : 1.0;
    const double iSp = 1.0 / Sp, iSq = 1.0 / Sq;
    double resid_mass = 0.0;
    if (resid) {
      double mine = 0.0;
      for (int i = s0; i < s1; ++i) mine += fmax(0.0, s_rec[i].a * iSp - s_rec[i].bq * iSq);
      resid_mass = wave_sum_dpp(mine);
    }
    // residual weights, or (bonus row, or a residual that vanished) the target row's
    const bool rmode = resid && resid_mass > 0.0;
    const double target = u_final * (rmode ? resid_mass : Sp);
    const int sel = rmode ? wave_select(nsb, target, [&](int i) { return fmax(0.0, s_rec[i].a * iSp - s_rec[i].bq * iSq); },
                                        pref)
                          : wave_select(nsb, target, [&](int i) { return s_rec[i].sp; }, pref);
    int y = -1;
    if (sel >= 0) {
      const int64_t j0 = (int64_t)sel * kSB + (int64_t)lane * EPL;
      if (sel != sel_e) {
        raw16<DT, AL>(c, prow, j0, rp);
        if (rmode) raw16<DT, AL>(c, qrow, j0, rq);
      }
      double w[EPL];
      weights16<DT>(c, rp, j0, wp, tps, w);
      if (rmode) {
        double wq16[EPL];
        weights16<DT>(c, rq, j0, wq, tqs, wq16);
#pragma unroll
        for (int k = 0; k < EPL; ++k) w[k] = fmax(0.0, w[k] * iSp - wq16[k] * iSq);
      }
      y = wave_rescan(sel, target - pref, w);
    }
    for (int i = lane; i <= K; i += kWave) {
      int v = -1;
      if (i < n) v = c.draft[b * K + i];
      else if (i == n) v = y;
      c.out_tokens[b * (K + 1) + i] = v;
    }
    if (lane == 0) {
      c.out_len[b] = n;
      if (c.out_resid) c.out_resid[b] = resid_mass;
    }
  }
}

// ----------------------------------------------------------- final step --
// Final draw when a request's sub-blocks were summed by several workgroups.
// Sub-blocks per lane whose records the one-wave picks keep in registers
// (V <= 64 * kPickPer * 1024); larger rows read them from memory.
constexpr int kPickPer = 4;

template <int DT, bool AL>
__global__ __launch_bounds__(kWave) void k_final(LinCfg c) {
  // one wave per request: the request's sub-block records from the resolve
  // parts (one round of loads into registers), the sub-block selection, and a
  // rescan of one sub-block
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x, K = c.K;
  const int nsb = c.nsb;
  const ResRec* rr = c.res + b * nsb;
  const bool inreg = nsb <= kWave * kPickPer;
  ResRec mr[kPickPer];
  if (inreg) {
#pragma unroll
    for (int k = 0; k < kPickPer; ++k) {
      const int sb = lane * kPickPer + k;
      mr[k] = sb < nsb ? rr[sb] : ResRec{0.0, 0.0, 0.0, 0.0};
    }
  }
  const ReqState st = c.rs[b];
  if (st.err) return;
  const int n = st.n;
  const bool bonus = n == K;
  const char* prow = prow_of(c, b, n);
  const char* qrow = bonus ? prow : qrow_of(c, b, n);
  // sum over this lane's records of f(record)
  auto lane_sum = [&](auto f) {
    double acc = 0.0;
    if (inreg) {
#pragma unroll
      for (int k = 0; k < kPickPer; ++k) acc += f(mr[k]);
    } else {
      for (int i = lane; i < nsb; i += kWave) acc += f(rr[i]);
    }
    return acc;
  };
  double Sp = 1.0, Sq = 1.0;
  if (!bonus) {
    Sp = wave_sum_dpp(lane_sum([](const ResRec& r) { return r.sp; }));
    Sq = wave_sum_dpp(lane_sum([](const ResRec& r) { return r.sq; }));
  }
  const double iSp = 1.0 / Sp, iSq = 1.0 / Sq;
  const double c64 = c.c64;
  WRow wp, wq;
  wpair(DT == kBF16 && c.tab, st.mp, st.mq, !bonus, c64, wp, wq);
  norm_pair(wp, wq, !bonus, st.sp_hat, st.sq_hat);
  auto wres = [&](const ResRec& r) { return fmax(0.0, r.a * iSp - r.bq * iSq); };
  const double resid = bonus ? 0.0 : wave_sum_dpp(lane_sum(wres));
  const bool rmode = !bonus && resid > 0.0;  // else the target row (bonus, or a vanished residual)
  const double W = rmode ? resid : wave_sum_dpp(lane_sum([](const ResRec& r) { return r.sp; }));
  const double target = st.u_final * W;
  double pref;
  int sel;
  if (inreg) {
    double v[kPickPer];
#pragma unroll
    for (int k = 0; k < kPickPer; ++k) v[k] = rmode ? wres(mr[k]) : mr[k].sp;
    sel = wave_select_reg(nsb, target, v, pref);
  } else {
    sel = rmode ? wave_select(nsb, target, [&](int i) { return wres(rr[i]); }, pref)
                : wave_select(nsb, target, [&](int i) { return rr[i].sp; }, pref);
  }
  int y = -1;
  if (sel >= 0) {
    const int64_t j0 = (int64_t)sel * kSB + (int64_t)lane * 16;
    Raw16<DT> rp, rq;
    raw16<DT, AL>(c, prow, j0, rp);
    if (rmode) raw16<DT, AL>(c, qrow, j0, rq);
    double w[16];
    weights16<DT>(c, rp, j0, wp, nullptr, w);
    if (rmode) {
      double wq16[16];
      weights16<DT>(c, rq, j0, wq, nullptr, wq16);
#pragma unroll
      for (int k = 0; k < 16; ++k) w[k] = fmax(0.0, w[k] * iSp - wq16[k] * iSq);
    }
    y = wave_rescan(sel, target - pref, w);
  }
  for (int i = lane; i <= K; i += kWave) {
    int v = -1;
    if (i < n) v = c.draft[b * K + i];
    else if (i == n) v = y;
    c.out_tokens[b * (K + 1) + i] = v;
  }
  if (lane == 0) {
    c.out_len[b] = n;
    if (c.out_resid) c.out_resid[b] = resid;
  }
}

// ----------------------------------------------------- draft sampling --
// One workgroup per draft row, after the statistics pass: the row maximum m
// and validity from the row's chunk records, then the fp64 weights of the
// row under the rule of the final draws (for a bfloat16 row that qualifies,
// an LDS table of 2^(a c) scaled by 2^(-m c)), summed per sub-block in LDS,
// then wave 0 draws x ~ q by inverse CDF over the sub-block sums and a rescan
// of the chosen sub-block ("Uno" research explainer, §3.3: the drafts of a
// block are drawn from the draft distributions). -1 for an invalid row.
template <int DT, bool AL>
__global__ __launch_bounds__(kDT) void k_draftrow(LinCfg c) {
  extern __shared__ ResRec s_rec[];  // one record per sub-block
  __shared__ double s_tab[kTabSize];
  __shared__ int s_bad;
  __shared__ float s_m;
  const int64_t qr = blockIdx.x;  // draft row in [0, B*K)
  const int K = c.K, t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1);
  const int64_t b = qr / K;
  const int i = (int)(qr - b * K);
  const char* row = qrow_of(c, b, i);
  // row maximum and validity from the statistics records (NaN, +inf, all -inf)
  if (wave == 0) {
    const StatRec* rec = c.st + (b * (c.rows.np + c.rows.nq) + c.rows.np + i) * (int64_t)c.nch32;
    float m = -INFINITY;
    int bad = 0;
    for (int ch = lane; ch < c.nch32; ch += kWave) {
      const StatRec rc = rec[ch];
      m = fmaxnan(m, rc.m);
      bad |= isnan(rc.s) ? 1 : 0;
    }
    m = wave_max(m);
    bad = wave_or(bad);
    if (lane == 0) {
      s_m = m;
      s_bad = bad || isnan(m) || isinf(m);
    }
  }
  const bool tab = DT == kBF16 && c.tab;
  if (tab) fill_tab<kDT>(s_tab, c.c64);
  __syncthreads();
  if (s_bad) {
    if (t == 0) c.draft[qr] = -1;
    return;
  }
  const WRow w = wrow(tab, s_m, c.c64);
  // the table is scaled while the first loads of the pass are in flight
  auto scale_table = [&]() {
    if (DT == kBF16 && w.tab)
      for (int j = t; j < kTabSize; j += kDT) s_tab[j] *= w.scale;
    __syncthreads();
  };
  if (DT == kBF16 && w.tab)
    resolve_pass<DT, AL, DT == kBF16, false, true, kDWaves>(c, b, row, row, 0, c.nsb, s_tab, s_tab, w, w, 0.0f,
                                                            s_rec, scale_table);
  else
    resolve_pass<DT, AL, false, false, true, kDWaves>(c, b, row, row, 0, c.nsb, s_tab, s_tab, w, w, 0.0f, s_rec,
                                                      scale_table);
  __syncthreads();
  if (wave != 0) return;
  const double* const tps = w.tab ? s_tab : nullptr;
  double mine = 0.0;
  for (int sb = lane; sb < c.nsb; sb += kWave) mine += s_rec[sb].sp;
  const double W = wave_sum_dpp(mine);
  const double u = c.rng.u((uint32_t)b, (uint32_t)i, kDrawDraft);
  const int x = wave_pick(
      c.nsb, c.V, u * W, [&](int sb) { return s_rec[sb].sp; },
      [&](int64_t j0, double(&wt)[16]) { row16<DT, AL>(c, row, j0, w, tps, wt); });
  if (lane == 0) c.draft[qr] = x;
}

// Statistics record of one (target row, chunk) by one wave, with no
// workgroup barrier: batches of 8 vectors per lane, a running maximum m of
// the wave, and the running sum of 2^((a - m) c) (binary32 exp2 of
// a c - round(m c), corrected by 2^(-(m c)_lo) in fp64 per batch; rescaled in
// fp64 when m rises). Same record as the statistics pass.
template <bool AL>
__device__ __forceinline__ void wave_stats_unit(const LinCfg& c, int64_t u) {
  using E = Elem<kBF16>;
  constexpr int EPV = E::kPerVec;
  constexpr int NVB = 8;
  constexpr int kVecs = kWG * kStatNV;  // 16-byte vectors per chunk
  const int lane = threadIdx.x & (kWave - 1);
  const int chunk = (int)(u % c.nch32);
  const int64_t pr = u / c.nch32;  // target row in [0, B * np)
  const int64_t b = pr / c.rows.np;
  const int64_t sr = b * (c.rows.np + c.rows.nq) + (pr - b * c.rows.np);
  const char* row = c.rows.row(sr);
  float m = -INFINITY;
  double s = 0.0;
  const float c32 = c.c32;
  for (int k0 = 0; k0 < kVecs / kWave; k0 += NVB) {
    float x[NVB][EPV];
    load_vecs<kBF16, AL, NVB, kWave>(row, c.V, c.nvec, (int64_t)chunk * kVecs + (int64_t)k0 * kWave + lane, x);
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < NVB; ++k)
#pragma unroll
      for (int e = 0; e < EPV; ++e) bm = fmaxnan(bm, x[k][e]);
    const float mn = fmaxnan(m, wave_max(bm));
    if (isnan(mn) || isinf(mn)) {  // NaN or +inf (the record is invalid), or all -inf so far
      m = mn;
      if (!is_neg_inf(mn)) break;
      continue;
    }
    if (mn > m && !is_neg_inf(m)) s *= exp2_fast(((double)m - (double)mn) * (double)c32);
    m = mn;
    const float mc_hi = m * c32;
    const float mc_lo = fmaf(m, c32, -mc_hi);
    double bs = 0.0;
#pragma unroll
    for (int k = 0; k < NVB; ++k) {
      float e[EPV];
#pragma unroll
      for (int j = 0; j < EPV; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(x[k][j], c32, -mc_hi));
      bs += (double)pairwise_sum(e);
    }
    s += bs * exp2_fast(-(double)mc_lo);
  }
  s = wave_sum_dpp(s);
  if (lane == 0) {
    StatRec r;
    r.m = m;
    r.pad = 0;
    r.s = (isnan(m) || (isinf(m) && m > 0.0f)) ? NAN : s;
    c.st[sr * c.nch32 + chunk] = r;
  }
}

// One pass over the bfloat16 draft row `row` (row i of request b), with no
// statistics pass before it (the table temperatures, c.tab): the fp64
// weights of the row are summed per sub-block into s_rec from the unscaled
// 2^(a c) table (the rule of fweight with scale 1), tracking whether the row
// holds a code that may break the table rule (positive or NaN above the
// window). The largest logit m_lo of the sub-block with the largest sum
// (read again, 2 KB) bounds the row maximum from below, so the row qualifies
// for the rule when (m_lo + 63.25) c >= 100 and nothing was flagged;
// otherwise it is read again: its exact maximum, then exp2 weights relative
// to it. Writes the row's chunk records for the verification that follows
// (reference m_lo, or the exact maximum) and returns the row's rule in w
// (with the LDS table, or exact exponentials) and its validity. Called by
// every thread of a kDT-thread workgroup.
// RING > 0: sub-blocks in flight per wave in the pass (more loads in flight
// for a workgroup that has its CU to itself). NP < kDWaves: only the first NP
// waves run the pass, and the others call during() meanwhile.
struct NoWork {
  __device__ void operator()() const {}
};
template <bool AL, int RING = 0, int NP = kDWaves, class DURING = NoWork>
__device__ bool qrow_pass(const LinCfg& c, int64_t b, int i, const char* row, ResRec* s_rec, double* s_tab,
                          float* shf, int* s_chk, double* s_smax, WRow& w, DURING during = DURING{}) {
  using E = Elem<kBF16>;
  const int t = threadIdx.x, wave = t / kWave, lane = t & (kWave - 1);
  const int nsb = c.nsb;
  const double c64 = c.c64;
  const WRow w1 = {0.0, 1.0, true};
  // the table is filled while the first loads of the pass are in flight
  auto fill = [&]() {
    fill_tab_steps(s_tab, c64);
    if (t == 0) *s_chk = 0;
    __syncthreads();
  };
  resolve_pass<kBF16, AL, true, false, true, NP, decltype(fill), true, RING>(c, b, row, row, 0, nsb, s_tab, s_tab,
                                                                            w1, w1, 0.0f, s_rec, fill, s_chk);
  if constexpr (NP < kDWaves) {
    if (wave >= NP) during();  // waves outside the pass do other work meanwhile
  }
  __syncthreads();
  if (wave == 0) {
    // the sub-block with the largest sum (lowest index on ties), then its largest logit
    double mx = 0.0;
    int at = 0;
    for (int sb = lane; sb < nsb; sb += kWave) {
      const double v = s_rec[sb].sp;
      if (v > mx) {
        mx = v;
        at = sb;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const double ov = __shfl_xor(mx, o);
      const int oa = __shfl_xor(at, o);
      if (ov > mx || (ov == mx && oa < at)) {
        mx = ov;
        at = oa;
      }
    }
    float xm = -INFINITY;
    if (mx > 0.0) {
      float x[2][E::kPerVec];
      load_vecs<kBF16, AL, 2, 1>(row, c.V, c.nvec, ((int64_t)at * kSB + (int64_t)lane * 16) / E::kPerVec, x);
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < E::kPerVec; ++e) xm = fmaxnan(xm, x[k][e]);
      xm = wave_max(xm);
    }
    if (lane == 0) {
      *s_smax = mx;
      shf[0] = xm;
    }
  }
  __syncthreads();
  const double smax = *s_smax;
  const float m_lo = shf[0];
  __syncthreads();  // shf is reused below
  const bool fast = !*s_chk && smax > 0.0 && !isnan(m_lo) && ((double)m_lo + kTabMaxAbs) * c64 >= 100.0;
  float m;
  w = w1;
  if (fast) {
    m = m_lo;
  } else {
    // exact maximum and validity, then the weights relative to it
    constexpr int EPV = E::kPerVec;
    float mx = -INFINITY;
    for (int64_t v0 = t; v0 < c.nvec || (!AL && v0 * EPV < c.V); v0 += kDT * 4) {
      float x[4][EPV];
      load_vecs<kBF16, AL, 4, kDT>(row, c.V, c.nvec, v0, x);
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < EPV; ++e) mx = fmaxnan(mx, x[k][e]);
    }
    m = block_max<kDT>(mx, shf);
    if (!isnan(m) && !isinf(m)) {
      w = wrow(false, m, c64);
      resolve_pass<kBF16, AL, false, false, true, kDWaves>(c, b, row, row, 0, nsb, s_tab, s_tab, w, w, 0.0f, s_rec,
                                                           [] {});
    }
    __syncthreads();
  }
  const bool bad = isnan(m) || isinf(m);  // NaN, +inf, or an all -inf row
  // chunk records of this row: sums of 2^((a - m) c) over each chunk's sub-blocks
  constexpr int kSbPerChunk = kWG * kStatNV * E::kPerVec / kSB;
  StatRec* rec = c.st + (b * (c.rows.np + c.rows.nq) + c.rows.np + i) * (int64_t)c.nch32;
  const double scale = fast ? exp2_fast(-(double)m * c64) : 1.0;
  for (int ch = t; ch < c.nch32; ch += kDT) {
    double sc = 0.0;
    for (int sb = ch * kSbPerChunk; sb < min(nsb, (ch + 1) * kSbPerChunk); ++sb) sc += s_rec[sb].sp;
    StatRec r;
    r.m = m;
    r.pad = 0;
    r.s = bad && !is_neg_inf(m) ? NAN : sc * scale;
    rec[ch] = r;
  }
  return !bad;
}

// One inverse-CDF draw from the sub-block sums of qrow_pass (uniform u) by
// one whole wave, the chosen sub-block rescanned under the row's rule.
template <bool AL>
__device__ __forceinline__ int qrow_draw(const LinCfg& c, const char* row, const ResRec* s_rec,
                                         const double* s_tab, const WRow& w, double u) {
  const int lane = threadIdx.x & (kWave - 1);
  const double* const tps = w.tab ? s_tab : nullptr;
  double mine = 0.0;
  for (int sb = lane; sb < c.nsb; sb += kWave) mine += s_rec[sb].sp;
  const double W = wave_sum_dpp(mine);
  return wave_pick(c.nsb, c.V, u * W, [&](int sb) { return s_rec[sb].sp; },
                   [&](int64_t j0, double(&wt)[16]) { row16<kBF16, AL>(c, row, j0, w, tps, wt); });
}

// The target-row chunk records of a launch: wave `slot` of workgroup g takes
// the units g * kDWaves + slot + k * (kDWaves * grid), `nunits` in all.
template <bool AL>
__device__ __forceinline__ void stats_units(const LinCfg& c, int64_t nunits, int slot) {
  for (int64_t un = (int64_t)blockIdx.x * kDWaves + slot; un < nunits; un += (int64_t)gridDim.x * kDWaves)
    wave_stats_unit<AL>(c, un);
}

// Waves of a fused draft-row workgroup that stream target rows while the
// others run the pass over its draft row, and the statistics units each of
// them takes meanwhile.
constexpr int kQrowEarlyWaves = 2;
constexpr int kQrowEarlyUnits = 1;

// One workgroup per draft row of linear verification: qrow_pass, then wave 0
// draws x ~ q with U(seed, step, b, i, 0x40000000) ("Uno" research explainer,
// §3.3: the drafts of a block are drawn from the draft distributions; -1 for
// an invalid row). The target rows' chunk records (wave_stats_unit, `nunits`
// of them over the whole grid) come in two parts. SPLIT: the last
// kQrowEarlyWaves waves compute kQrowEarlyUnits each while the others run
// the pass over the draft row (the table-bound pass and the streaming of
// target rows share the CU); then every wave takes the rest slot-major, wave 0
// (busy drawing) taking the last slot, which the grid reaches last. Held to
// 128 registers (four waves per SIMD), so that two workgroups share a CU.
template <bool AL, bool SPLIT>
__global__ __launch_bounds__(kDT) __attribute__((amdgpu_waves_per_eu(4))) void k_qrow(LinCfg c, int64_t nunits) {
  extern __shared__ ResRec s_rec[];  // one record per sub-block (.sp)
  __shared__ double s_tab[kTabAlloc];  // the running-product fill
  __shared__ float shf[kDWaves];
  __shared__ int s_chk;
  __shared__ double s_smax;
  const int64_t qr = blockIdx.x;  // draft row in [0, B*K)
  const int K = c.K, wave = threadIdx.x / kWave;
  const int64_t b = qr / K;
  const int i = (int)(qr - b * K);
  const char* row = qrow_of(c, b, i);
  const int64_t g = blockIdx.x, G = gridDim.x;
  constexpr int NP = SPLIT ? kDWaves - kQrowEarlyWaves : kDWaves;
  const int64_t early = SPLIT ? (int64_t)kQrowEarlyWaves * kQrowEarlyUnits * G : 0;
  auto during = [&]() {
    for (int r = 0; r < kQrowEarlyUnits; ++r) {
      const int64_t un = ((int64_t)r * kQrowEarlyWaves + (wave - NP)) * G + g;
      if (un < nunits) wave_stats_unit<AL>(c, un);
    }
  };
  WRow w;
  const bool ok = qrow_pass<AL, 0, NP>(c, b, i, row, s_rec, s_tab, shf, &s_chk, &s_smax, w, during);
  if (wave == 0) {
    const int x = ok ? qrow_draw<AL>(c, row, s_rec, s_tab, w, c.rng.u((uint32_t)b, (uint32_t)i, kDrawDraft)) : -1;
    if ((threadIdx.x & (kWave - 1)) == 0) c.draft[qr] = x;
  }
  const int slot = wave == 0 ? kDWaves - 1 : wave - 1;
  for (int64_t un = early + slot * G + g; un < nunits; un += G * kDWaves) wave_stats_unit<AL>(c, un);
}

// Tree node drafts: workgroups [0, nextra) compute target-row chunk records
// only; workgroup nextra + (b (N + 1) + r) runs qrow_pass on draft row r of
// request b and draws each child of row r, the j-th (ascending node id) with
// U(seed, step, b, r, 0x40000000 + j) ("Uno" research explainer, §3.4: the
// candidates of a row are drawn i.i.d. from its draft distribution), one wave
// per child; -1 for an invalid row (the walk then marks every node of the
// request).
constexpr int64_t kTreeQrowFill = 256;  // workgroups of a tree draft-row launch, at least

template <bool AL>
__global__ __launch_bounds__(kDT) void k_tqrow(LinCfg c, TreeTopo tp, TreeCfg tc, int64_t nunits, int nextra) {
  extern __shared__ ResRec s_rec[];
  __shared__ double s_tab[kTabAlloc];  // the running-product fill
  __shared__ float shf[kDWaves];
  __shared__ int s_chk;
  __shared__ double s_smax;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  if ((int)blockIdx.x < nextra) {
    stats_units<AL>(c, nunits, wave);
    return;
  }
  const int R = tc.N + 1;
  const int64_t qr = blockIdx.x - nextra;  // draft row in [0, B (N + 1))
  const int64_t b = qr / R;
  const int r = (int)(qr - b * R);
  const char* row = c.rows.q + (qr * (int64_t)c.V) * c.rows.esz;
  WRow w;
  const bool ok = qrow_pass<AL>(c, b, r, row, s_rec, s_tab, shf, &s_chk, &s_smax, w);
  const int k0 = tp.off[r], nk = tp.off[r + 1] - k0;
  for (int j = wave; j < nk; j += kDWaves) {
    const int x = ok ? qrow_draw<AL>(c, row, s_rec, s_tab, w,
                                     c.rng.u((uint32_t)b, (uint32_t)r, kDrawDraft + (uint32_t)j))
                     : -1;
    if (lane == 0) tc.tokens[b * tc.N + tp.kids[k0 + j]] = x;
  }
  stats_units<AL>(c, nunits, wave);
}

// Draft sampling alone: a request with an invalid draft row gets -1 for all
// its drafts.
__global__ __launch_bounds__(kWave) void k_draft_fix(LinCfg c) {
  const int64_t b = blockIdx.x;
  const int K = c.K, lane = threadIdx.x;
  int bad = 0;
  for (int i = lane; i < K; i += kWave) bad |= c.draft[b * K + i] < 0 ? 1 : 0;
  bad = wave_or(bad);
  if (bad)
    for (int i = lane; i < K; i += kWave) c.draft[b * K + i] = -1;
}

// fp64 sub-block sums (with per-sub-block maxima) of draft rows, for the node
// drafts of tree verification.
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_draftpass(LinCfg c) {
  constexpr int EPV = Elem<DT>::kPerVec;
  constexpr int VPL = kSB / (kWave * EPV);
  const int64_t qr = blockIdx.y;  // draft row in [0, B*K)
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int sb = blockIdx.x * kWaves + wave;
  if (sb >= c.nsb) return;
  const char* row = c.rows.q + (qr * (int64_t)c.V) * c.rows.esz;
  float x[VPL][EPV];
  load_vecs<DT, AL, VPL, kWave>(row, c.V, c.nvec, (int64_t)sb * (kSB / EPV) + lane, x);
  float m = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxnan(m, x[v][e]);
  m = wave_max(m);
  double s = 0.0;
  if (!is_neg_inf(m)) {
    const double md = m;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int e = 0; e < EPV; ++e) s += exp2_fast(((double)x[v][e] - md) * c.c64);
    s = wave_sum_dpp(s);
  }
  if (lane == 0) {
    DraftRec r;
    r.m = m;
    r.pad = 0;
    r.s = s;
    c.dr[qr * c.nsb + sb] = r;
  }
}

// ------------------------------------------------------------- greedy --
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_argmax(LinCfg c) {
  constexpr int EPV = Elem<DT>::kPerVec;
  const int64_t item = blockIdx.x;
  const int chunk = (int)(item % c.nch32);
  const int64_t sr = item / c.nch32;
  const char* row = c.rows.row(sr);
  float x[kStatNV][EPV];
  const int64_t vfirst = (int64_t)chunk * kWG * kStatNV + threadIdx.x;
  load_vecs<DT, AL, kStatNV, kWG>(row, c.V, c.nvec, vfirst, x);
  float best = -INFINITY;
  int idx = 0x7fffffff, bad = 0;
#pragma unroll
  for (int k = 0; k < kStatNV; ++k)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const float v = x[k][e];
      const int j = (int)((vfirst + (int64_t)k * kWG) * EPV + e);
      bad |= isnan(v) || (isinf(v) && v > 0.0f);
      if (v > best) {
        best = v;
        idx = j;
      }
    }
  // workgroup reduction: larger value first, then lower index
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ov = __shfl_xor(best, o);
    const int oi = __shfl_xor(idx, o);
    if (ov > best || (ov == best && oi < idx)) {
      best = ov;
      idx = oi;
    }
  }
  bad = wave_or(bad);
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves], sb_[kWaves];
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    sv[w] = best;
    si[w] = idx;
    sb_[w] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgRec r;
    r.v = sv[0];
    r.idx = si[0];
    r.bad = sb_[0];
    for (int k = 1; k < kWaves; ++k) {
      if (sv[k] > r.v || (sv[k] == r.v && si[k] < r.idx)) {
        r.v = sv[k];
        r.idx = si[k];
      }
      r.bad |= sb_[k];
    }
    r.pad = 0;
    c.ar[item] = r;
  }
}

__global__ __launch_bounds__(kWG) void k_greedy_decide(LinCfg c) {
  const int64_t b = blockIdx.x;
  const int K = c.K, R = 2 * K + 1, t = threadIdx.x;
  __shared__ int s_g[2 * kMaxK + 1];
  __shared__ int s_bad, s_n;
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < R; i += kWG) {
    int bad;
    s_g[i] = row_argmax(c.ar + (b * R + i) * (int64_t)c.nch32, c.nch32, &bad);
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  int acc = 1, x = 0;
  if (t < K) {
    x = c.fused ? s_g[K + 1 + t] : c.draft[b * K + t];
    if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
    acc = x == s_g[t];
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
    if (c.fused) c.draft[b * K + t] = x;
    if (c.out_probs) {
      c.out_probs[(b * K + t) * 2 + 0] = x == s_g[t] ? 1.0f : 0.0f;
      c.out_probs[(b * K + t) * 2 + 1] = x == s_g[K + 1 + t] ? 1.0f : 0.0f;
    }
  }
  __syncthreads();
  for (int i = t; i <= K; i += kWG) {
    int v = -1;
    if (i < n) v = c.fused ? s_g[K + 1 + i] : c.draft[b * K + i];
    else if (i == n) v = s_g[n];
    c.out_tokens[b * (K + 1) + i] = v;
  }
  if (t == 0) {
    c.out_len[b] = n;
    if (c.out_resid) c.out_resid[b] = 0.0;
  }
}

__global__ __launch_bounds__(kWG) void k_greedy_draft(LinCfg c) {
  const int64_t b = blockIdx.x;
  const int K = c.K, t = threadIdx.x;
  __shared__ int s_bad;
  __shared__ int s_g[kMaxK];
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < K; i += kWG) {
    int bad;
    s_g[i] = row_argmax(c.ar + (b * K + i) * (int64_t)c.nch32, c.nch32, &bad);
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  for (int i = t; i < K; i += kWG) c.draft[b * K + i] = s_bad ? -1 : s_g[i];
}

// ------------------------------------------------------------ launchers --
template <int DT, bool AL>
static hipError_t linear_sampled_t(const LinCfg& c, hipStream_t s) {
  const int64_t rows = c.B * (2 * c.K + 1);
  if (c.fused && DT == kBF16 && c.tab) {
    // drafts drawn in one pass over their rows, whose workgroups also write
    // those rows' chunk records and, wave by wave, the target rows' ones
    PSI_LAUNCH_LDS(s, (k_qrow<AL, true>), dim3((unsigned)(c.B * c.K)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec),
                   c, c.B * c.rows.np * (int64_t)c.nch32);
  } else {
    const hipError_t e = launch_stats32(c, rows, DT, s);
    if (e != hipSuccess) return e;
    // drafts drawn inside the call, from the statistics of their rows
    if (c.fused)
      PSI_LAUNCH_LDS(s, (k_draftrow<DT, AL>), dim3((unsigned)(c.B * c.K)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec),
                     c);
  }
  // One resolve workgroup per request when there are enough requests to fill
  // the chip (and its sub-block records fit in LDS); otherwise several per
  // request and a separate final step.
  const size_t lds = (size_t)c.nsb * sizeof(ResRec);
  if (c.B >= kResolveOneWgMinB && lds <= kResolveMaxLds) {
    PSI_LAUNCH_LDS(s, (k_resolve<DT, AL, true>), dim3((unsigned)c.B), dim3(kRT), lds, c, 1);
  } else {
    const int parts = (int)std::min<int64_t>(std::max<int64_t>(1, (kResolveTargetWgs + c.B - 1) / c.B),
                                             std::max(1, c.nsb / kRWaves));
    PSI_LAUNCH(s, (k_resolve<DT, AL, false>), dim3((unsigned)(c.B * parts)), dim3(kRT), c, parts);
    PSI_LAUNCH(s, (k_final<DT, AL>), dim3((unsigned)c.B), dim3(kWave), c);
  }
  return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t linear_greedy_t(const LinCfg& c, hipStream_t s) {
  const int64_t rows = c.B * (2 * c.K + 1);
  PSI_LAUNCH(s, (k_argmax<DT, AL>), dim3((unsigned)(rows * c.nch32)), dim3(kWG), c);
  PSI_LAUNCH(s, k_greedy_decide, dim3((unsigned)c.B), dim3(kWG), c);
  return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t draft_sampled_t(const LinCfg& c, hipStream_t s) {
  if (DT == kBF16 && c.tab) {
    PSI_LAUNCH_LDS(s, (k_qrow<AL, false>), dim3((unsigned)(c.B * c.K)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec),
                   c, (int64_t)0);
  } else {
    const hipError_t e = launch_stats32(c, c.B * c.K, DT, s);
    if (e != hipSuccess) return e;
    PSI_LAUNCH_LDS(s, (k_draftrow<DT, AL>), dim3((unsigned)(c.B * c.K)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec),
                   c);
  }
  PSI_LAUNCH(s, k_draft_fix, dim3((unsigned)c.B), dim3(kWave), c);
  return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t draft_greedy_t(const LinCfg& c, hipStream_t s) {
  const int64_t rows = c.B * c.K;
  PSI_LAUNCH(s, (k_argmax<DT, AL>), dim3((unsigned)(rows * c.nch32)), dim3(kWG), c);
  PSI_LAUNCH(s, k_greedy_draft, dim3((unsigned)c.B), dim3(kWG), c);
  return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t draftpass_t(const LinCfg& c, int64_t rows, hipStream_t s) {
  PSI_LAUNCH(s, (k_draftpass<DT, AL>), dim3((c.nsb + kWaves - 1) / kWaves, (unsigned)rows), dim3(kWG), c);
  return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t argmax_t(const LinCfg& c, int64_t rows, hipStream_t s) {
  PSI_LAUNCH(s, (k_argmax<DT, AL>), dim3((unsigned)(rows * c.nch32)), dim3(kWG), c);
  return hipGetLastError();
}

hipError_t launch_linear_sampled(const LinCfg& c, int dtype, hipStream_t s) {
  return PSI_DISPATCH(linear_sampled_t, dtype, c.aligned, c, s);
}
hipError_t launch_linear_greedy(const LinCfg& c, int dtype, hipStream_t s) {
  return PSI_DISPATCH(linear_greedy_t, dtype, c.aligned, c, s);
}
hipError_t launch_draft_sampled(const LinCfg& c, int dtype, hipStream_t s) {
  return PSI_DISPATCH(draft_sampled_t, dtype, c.aligned, c, s);
}
hipError_t launch_draft_greedy(const LinCfg& c, int dtype, hipStream_t s) {
  return PSI_DISPATCH(draft_greedy_t, dtype, c.aligned, c, s);
}
template <bool AL>
static hipError_t tree_qrows_t(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, hipStream_t s) {
  const int64_t nq = c.B * (int64_t)(tc.N + 1);
  const int64_t nunits = c.B * c.rows.np * (int64_t)c.nch32;
  // statistics-only workgroups on the CUs the draft rows leave idle, at most
  // one per kDWaves target chunks
  const int64_t spare = std::max<int64_t>(0, kTreeQrowFill - nq);
  const int nextra = (int)std::min<int64_t>(spare, (nunits + kDWaves - 1) / kDWaves);
  PSI_LAUNCH_LDS(s, (k_tqrow<AL>), dim3((unsigned)(nextra + nq)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec), c, tp,
                 tc, nunits, nextra);
  return hipGetLastError();
}

hipError_t launch_tree_qrows(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, hipStream_t s) {
  return c.aligned ? tree_qrows_t<true>(c, tp, tc, s) : tree_qrows_t<false>(c, tp, tc, s);
}

hipError_t launch_draftpass(const LinCfg& c, int64_t rows, int dtype, hipStream_t s) {
  return PSI_DISPATCH(draftpass_t, dtype, c.aligned, c, rows, s);
}
hipError_t launch_argmax(const LinCfg& c, int64_t rows, int dtype, hipStream_t s) {
  return PSI_DISPATCH(argmax_t, dtype, c.aligned, c, rows, s);
}

}  // namespace psi
