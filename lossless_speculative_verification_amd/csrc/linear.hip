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
constexpr size_t kResolveMaxLds = 64 * 1024;

// ------------------------------------------------------------ resolve --
// Threads of a resolve workgroup: 16 waves, so that one workgroup per request
// keeps every SIMD of a CU busy through the fp64 final-row pass.
constexpr int kRT = 1024;
constexpr int kRWaves = kRT / kWave;

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

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
// every NW-th, NW the workgroup's waves). Software-pipelined over NBUF register buffers that change
// roles each step (no copies, so loads stay in flight across steps): bfloat16
// keeps the next two sub-blocks in flight, fp32 the next one. TAB: weights
// are read from the pre-scaled LDS tables tp / tq (bfloat16 only), whose
// values estimate the probabilities, so the target part is above the draft
// part where ep > eq; otherwise where a_p - a_q > dx.
template <int DT, bool AL, bool TAB, bool RESID, bool PICK, int NW = kRWaves>
__device__ __forceinline__ void resolve_pass(const LinCfg& c, int64_t b, const char* prow, const char* qrow,
                                             int sb0, int sb1, const double* tp, const double* tq, const WRow& wp,
                                             const WRow& wq, float dx, ResRec* s_rec) {
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
      if constexpr (TAB) {
        // two bfloat16 codes per word; logits below the window read a zero
        // slot and get their exact weight in the rare call below
        uint32_t low = 0;
        const char* const tpb = (const char*)tp;
        const char* const tqb = (const char*)tq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t wpw = word_of(x.p[v], i), wqw = RESID ? word_of(x.q[v], i) : 0u;
          const uint32_t op = tab_offsets2(wpw, low);
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
      const double tot = wave_sum(sp);
      if (lane == 0) *rec = ResRec{tot, 0.0, 0.0, 0.0};
    }
  };
  constexpr int W = NW;
  Buf x0, x1, x2;
  int s = sb0 + wave;
  if (s >= sb1) return;
  load(s, x0);
  if constexpr (NBUF == 3) {
    load(s + W, x1);
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
                                      const double* tab_scaled, double (&out)[16]) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  if (AL && j0 + 16 <= c.V) {
    const uint4* rp = (const uint4*)row + j0 / EPV;
#pragma unroll
    for (int v = 0; v < 16 / EPV; ++v) {
      float x[EPV];
      E::unpack(rp[v], x);
#pragma unroll
      for (int e = 0; e < EPV; ++e) out[v * EPV + e] = fweight<DT>(x[e], w, c.c64, tab_scaled);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) out[k] = j0 + k < c.V ? fweight<DT>(E::load1(row, j0 + k), w, c.c64, tab_scaled) : 0.0;
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
  // the 2^(a c) table, then the same multiplied by 2^(-m_p c) (first half)
  // and by 2^(-m_q c) (second half) once the final rows are known
  __shared__ double s_tab[2 * kTabSize];
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
    const StatRec* rec = c.st + (b * R + r) * (int64_t)c.nch32;
    float m = -INFINITY;
    for (int ch = 0; ch < c.nch32; ++ch) m = fmaxnan(m, rec[ch].m);
    double S = 0.0;
    int bad = isnan(m) || isinf(m);  // NaN, +inf, or an all -inf row
    if (!bad)
      for (int ch = 0; ch < c.nch32; ++ch) {
        const StatRec rc = rec[ch];
        if (isnan(rc.s)) bad = 1;
        else if (!is_neg_inf(rc.m)) S += rc.s * ::exp2(((double)rc.m - (double)m) * (double)c.c32);
      }
    if (!(S > 0.0)) bad = 1;
    s_m[r] = m;
    s_S[r] = S;
    if (bad) atomicOr(&s_bad, 1);
  }
  if (tab) fill_tab<kRT>(s_tab, c.c64);
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
  const float dx = (float)((::log2(sph) - ::log2(sqh) + wp.mc - wq.mc) / c64);
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
  double* const tabp = s_tab;
  double* const tabq = s_tab + kTabSize;
  if (DT == kBF16 && wp.tab) {
    for (int i = t; i < kTabSize; i += kRT) {
      const double e = s_tab[i];
      if (resid) tabq[i] = e * wq.scale;
      tabp[i] = e * wp.scale;
    }
    __syncthreads();
  }

  // ---- fp64 pass over this part's sub-blocks
  const char* prow = prow_of(c, b, n);
  const char* qrow = resid ? qrow_of(c, b, n) : prow;
  const int nsb = c.nsb;
  const int sb0 = (int)((int64_t)part * nsb / parts), sb1 = (int)((int64_t)(part + 1) * nsb / parts);
  if (resid) {
    if (DT == kBF16 && wp.tab)
      resolve_pass<DT, AL, DT == kBF16, true, PICK>(c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec);
    else resolve_pass<DT, AL, false, true, PICK>(c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec);
  } else {
    if (DT == kBF16 && wp.tab)
      resolve_pass<DT, AL, DT == kBF16, false, PICK>(c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec);
    else resolve_pass<DT, AL, false, false, PICK>(c, b, prow, qrow, sb0, sb1, tabp, tabq, wp, wq, dx, s_rec);
  }
  if constexpr (PICK) {
    __syncthreads();
    // ---- final draw (inverse CDF, fp64) from the sub-block sums in LDS, by wave 0
    if (wave != 0) return;
    const double* const tps = wp.tab ? tabp : nullptr;
    const double* const tqs = wq.tab ? tabq : nullptr;
    double resid_mass = 0.0;
    int y;
    if (resid) {
      double sa = 0.0, sb_ = 0.0;
      for (int i = lane; i < nsb; i += kWave) {
        sa += s_rec[i].sp;
        sb_ += s_rec[i].sq;
      }
      const double iSp = 1.0 / wave_sum(sa), iSq = 1.0 / wave_sum(sb_);
      double mine = 0.0;
      for (int i = lane; i < nsb; i += kWave) mine += fmax(0.0, s_rec[i].a * iSp - s_rec[i].bq * iSq);
      resid_mass = wave_sum(mine);
      if (resid_mass > 0.0) {
        y = wave_pick(
            nsb, c.V, u_final * resid_mass, [&](int i) { return fmax(0.0, s_rec[i].a * iSp - s_rec[i].bq * iSq); },
            [&](int64_t j0, double(&w)[16]) {
              double wq16[16];
              row16<DT, AL>(c, prow, j0, wp, tps, w);
              row16<DT, AL>(c, qrow, j0, wq, tqs, wq16);
#pragma unroll
              for (int k = 0; k < 16; ++k) w[k] = fmax(0.0, w[k] * iSp - wq16[k] * iSq);
            });
      }
    }
    if (!resid || !(resid_mass > 0.0)) {  // bonus row, or a residual that vanished: the target row
      double mine = 0.0;
      for (int i = lane; i < nsb; i += kWave) mine += s_rec[i].sp;
      const double W = wave_sum(mine);
      y = wave_pick(
          nsb, c.V, u_final * W, [&](int i) { return s_rec[i].sp; },
          [&](int64_t j0, double(&w)[16]) { row16<DT, AL>(c, prow, j0, wp, tps, w); });
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
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_final(LinCfg c) {
  using E = Elem<DT>;
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, K = c.K;
  const ReqState st = c.rs[b];
  if (st.err) return;
  const int n = st.n;
  const bool bonus = n == K;
  const int nsb = c.nsb;
  const ResRec* rr = c.res + b * nsb;
  __shared__ double sh[kWaves];
  double Sp = 1.0, Sq = 1.0;
  if (!bonus) {
    double a = 0.0, q = 0.0;
    for (int i = t; i < nsb; i += kWG) {
      a += rr[i].sp;
      q += rr[i].sq;
    }
    Sp = block_sum(a, sh);
    Sq = block_sum(q, sh);
  }
  const char* prow = prow_of(c, b, n);
  const char* qrow = bonus ? prow : qrow_of(c, b, n);
  const double c64 = c.c64;
  WRow wp, wq;
  wpair(DT == kBF16 && c.tab, st.mp, st.mq, !bonus, c64, wp, wq);
  norm_pair(wp, wq, !bonus, st.sp_hat, st.sq_hat);
  double resid = 0.0;
  int mode = 0;  // 0: target weights of the final row; 1: residual; 2: residual vanished -> target
  if (!bonus) {
    double mine = 0.0;
    for (int i = t; i < nsb; i += kWG) mine += fmax(0.0, rr[i].a * (1.0 / Sp) - rr[i].bq * (1.0 / Sq));
    resid = block_sum(mine, sh);
    mode = resid > 0.0 ? 1 : 2;
  }
  int y;
  if (mode == 1) {
    y = pick_index(
        nsb, c.V, st.u_final * resid, [&](int i) { return fmax(0.0, rr[i].a * (1.0 / Sp) - rr[i].bq * (1.0 / Sq)); },
        [&](int64_t j) {
          const double ep = fweight<DT>(E::load1(prow, j), wp, c64, nullptr);
          const double eq = fweight<DT>(E::load1(qrow, j), wq, c64, nullptr);
          return fmax(0.0, ep * (1.0 / Sp) - eq * (1.0 / Sq));
        },
        sh);
  } else {
    double mine = 0.0;
    for (int i = t; i < nsb; i += kWG) mine += rr[i].sp;
    const double W = block_sum(mine, sh);
    y = pick_index(
        nsb, c.V, st.u_final * W, [&](int i) { return rr[i].sp; },
        [&](int64_t j) { return fweight<DT>(E::load1(prow, j), wp, c64, nullptr); }, sh);
  }
  for (int i = t; i <= K; i += kWG) {
    int v = -1;
    if (i < n) v = c.draft[b * K + i];
    else if (i == n) v = y;
    c.out_tokens[b * (K + 1) + i] = v;
  }
  if (t == 0) {
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
constexpr int kDT = 512;
constexpr int kDWaves = kDT / kWave;

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
  if (DT == kBF16 && w.tab) {
    for (int j = t; j < kTabSize; j += kDT) s_tab[j] *= w.scale;
    __syncthreads();
    resolve_pass<DT, AL, DT == kBF16, false, true, kDWaves>(c, b, row, row, 0, c.nsb, s_tab, s_tab, w, w, 0.0f,
                                                            s_rec);
  } else {
    resolve_pass<DT, AL, false, false, true, kDWaves>(c, b, row, row, 0, c.nsb, s_tab, s_tab, w, w, 0.0f, s_rec);
  }
  __syncthreads();
  if (wave != 0) return;
  const double* const tps = w.tab ? s_tab : nullptr;
  double mine = 0.0;
  for (int sb = lane; sb < c.nsb; sb += kWave) mine += s_rec[sb].sp;
  const double W = wave_sum(mine);
  const double u = c.rng.u((uint32_t)b, (uint32_t)i, kDrawDraft);
  const int x = wave_pick(
      c.nsb, c.V, u * W, [&](int sb) { return s_rec[sb].sp; },
      [&](int64_t j0, double(&wt)[16]) { row16<DT, AL>(c, row, j0, w, tps, wt); });
  if (lane == 0) c.draft[qr] = x;
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
    s = wave_sum(s);
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
  const hipError_t e = launch_stats32(c, rows, DT, s);
  if (e != hipSuccess) return e;
  // drafts drawn inside the call, from the statistics of their rows
  if (c.fused)
    PSI_LAUNCH_LDS(s, (k_draftrow<DT, AL>), dim3((unsigned)(c.B * c.K)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec), c);
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
    PSI_LAUNCH(s, (k_final<DT, AL>), dim3((unsigned)c.B), dim3(kWG), c);
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
  const hipError_t e = launch_stats32(c, c.B * c.K, DT, s);
  if (e != hipSuccess) return e;
  PSI_LAUNCH_LDS(s, (k_draftrow<DT, AL>), dim3((unsigned)(c.B * c.K)), dim3(kDT), (size_t)c.nsb * sizeof(ResRec), c);
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
hipError_t launch_draftpass(const LinCfg& c, int64_t rows, int dtype, hipStream_t s) {
  return PSI_DISPATCH(draftpass_t, dtype, c.aligned, c, rows, s);
}
hipError_t launch_argmax(const LinCfg& c, int64_t rows, int dtype, hipStream_t s) {
  return PSI_DISPATCH(argmax_t, dtype, c.aligned, c, rows, s);
}

}  // namespace psi
