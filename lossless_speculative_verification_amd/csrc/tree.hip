// Tree verification of Psi-Spec on gfx950 ("Uno" research explainer, §3.4
// Tree Sampler: several candidate continuations are checked in one verify
// pass).
//
// Rule at a row with children c_0 < c_1 < ... (each drawn i.i.d. from the
// row's draft distribution Q): the running target starts at P; child j is
// accepted iff u * Q(tok_j) < r(tok_j); after a rejection r <- norm((r - Q)+)
// (kept when that vanishes); the walk descends into the first accepted child;
// at a leaf, or once every child is rejected, the final token is drawn from r.
//
// The running target after j rejections has the closed form
//   r_j = (P - c_j Q)+ / G(c_j),  G(c) = sum_t max(0, P(t) - c Q(t)),
//   c_0 = 0, c_{j+1} = c_j + G(c_j),
// (induction: (r_j - Q)+ = (P - (c_j + G(c_j)) Q)+ / G(c_j)), so each
// rejection costs one fp64 pass over the row pair for a scalar G, and every
// test needs only P(tok), Q(tok) and (c_j, G(c_j)).
//
// Pipeline on the caller's stream:
//   k_tqrow            (linear.hip; fused bfloat16 node drafts) one pass per
//                      draft row, which draws the row's children and writes its
//                      chunk records, and the target rows' chunk records; or
//                      k_draftpass + k_tree_draft (node drafts) and k_stats32.
//   k_tree_wp          (sub-block group, request), launched rounds + 1 times:
//                      every workgroup of a request takes the walk step (row
//                      statistics and checks first; then G(c) from the previous
//                      round's sums, and the accept tests until the next
//                      rejection), then sums its sub-blocks of the row pair
//                      the new state needs (the next G(c), or the final row).
//   k_tree_pick        one workgroup per request: inverse-CDF draw of the final
//                      token from r at the stopping row, outputs.
// The LM-head path (lmhead.hip) draws its final token with k_tree_pass and
// k_tree_pick (launch_tree_final).
// Greedy (temperature 0): k_argmax then k_tree_greedy. Filtered sampling:
// k_filter_row (filter.hip) then k_tree_filt, which runs the recursive update
// directly on the at most 2 * top_k entry union of the two kept sets.
#include "rowops.hpp"

namespace psi {

namespace {

__device__ __forceinline__ const char* tree_prow(const LinCfg& c, int64_t b, int r) {
  return c.rows.p + ((b * c.rows.np + r) * (int64_t)c.V) * c.rows.esz;
}
__device__ __forceinline__ const char* tree_qrow(const LinCfg& c, int64_t b, int r) {
  return c.rows.q + ((b * c.rows.nq + r) * (int64_t)c.V) * c.rows.esz;
}

// Fills the outputs of one request with -1 (tokens and path) ahead of the walk.
__device__ __forceinline__ void tree_clear_outputs(const LinCfg& c, const TreeCfg& tc, int64_t b) {
  const int D = tc.D;
  for (int i = threadIdx.x; i <= D; i += blockDim.x) c.out_tokens[b * (D + 1) + i] = -1;
  for (int i = threadIdx.x; i < D; i += blockDim.x) tc.out_path[b * D + i] = -1;
}

__device__ __forceinline__ void load_row_stats(TreeState& s, const RowStat* rs, int N, int row) {
  s.mp = rs[row].m;
  s.sp_hat = rs[row].s;
  s.mq = rs[N + 1 + row].m;
  s.sq_hat = rs[N + 1 + row].s;
  s.has_exact = 0;
  s.Sp = 0.0;
  s.Sq = 0.0;
  s.cj = 0.0;
  s.Gj = 1.0;
  s.j = 0;
}

}  // namespace

// ----------------------------------------------------------- node drafts --
// Node n, the j-th child of row r, drawn from row r of q with draw id
// kDrawDraft + j; -1 for every node when any draft row of the request is invalid.
template <int DT>
__global__ __launch_bounds__(kWG) void k_tree_draft(LinCfg c, TreeTopo tp, TreeCfg tc) {
  const int N = tc.N, R = N + 1, nsb = c.nsb, t = threadIdx.x;
  const int64_t b = blockIdx.x / N;
  const int n = (int)(blockIdx.x - b * N);
  __shared__ int s_bad;
  __shared__ int s_alive[kMaxNodes + 1];
  __shared__ float shf[kWaves];
  __shared__ double sh[kWG + kWaves];
  for (int r = t; r < R; r += kWG) s_alive[r] = 0;
  if (t == 0) s_bad = 0;
  __syncthreads();
  const DraftRec* req = c.dr + b * R * (int64_t)nsb;
  for (int idx = t; idx < R * nsb; idx += kWG) {
    const DraftRec r = req[idx];
    if (isnan(r.m) || (isinf(r.m) && r.m > 0.0f) || isnan(r.s)) atomicOr(&s_bad, 1);
    if (!is_neg_inf(r.m)) atomicOr(&s_alive[idx / nsb], 1);
  }
  __syncthreads();
  int bad = s_bad;
  for (int r = 0; r < R; ++r) bad |= !s_alive[r];
  if (bad) {
    if (t == 0) tc.tokens[b * N + n] = -1;
    return;
  }
  const int row = tp.prow[n];
  const int64_t qr = b * R + row;
  const double u = c.rng.u((uint32_t)b, (uint32_t)row, kDrawDraft + (uint32_t)tp.sib[n]);
  const int y = draft_pick<DT>(c, c.rows.q + (qr * (int64_t)c.V) * c.rows.esz, c.dr + qr * nsb, u, shf, sh);
  if (t == 0) tc.tokens[b * N + n] = y;
}

// ------------------------------------------------------------------ walk --
// Thread 0's accept tests down the tree from state s until the next
// rejection (phase kTreeWaitG: a G(c_new) is needed) or the final row (phase
// kTreeFinal). rs holds the request's row statistics; the accepted path is
// written to the outputs when `write` is set.
// Per node of a request, gathered by the workgroup before the walk: its
// token, the logits of that token in its parent's target and draft rows, and
// the uniform of its accept test.
struct NodeIn {
  int32_t tok;
  float ap, aq;
  double u;
};

template <int DT>
__device__ __forceinline__ void gather_nodes(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int64_t b,
                                             NodeIn* nodes) {
  using E = Elem<DT>;
  // threads from wave 1 on first, so that wave 0 is free for other work when N
  // is below the workgroup size less a wave
  const int first = (int)((threadIdx.x + blockDim.x - kWave) % blockDim.x);
  for (int n = first; n < tc.N; n += blockDim.x) {
    const int r = tp.prow[n];
    NodeIn o;
    o.tok = tc.tokens[b * tc.N + n];
    const bool ok = o.tok >= 0 && o.tok < c.V;
    o.ap = ok ? E::load1(tree_prow(c, b, r), o.tok) : 0.0f;
    o.aq = ok ? E::load1(tree_qrow(c, b, r), o.tok) : 0.0f;
    o.u = c.rng.u((uint32_t)b, (uint32_t)r, (uint32_t)(kDrawAccept + tp.sib[n]));
    nodes[n] = o;
  }
}

template <int DT>
__device__ void tree_walk_steps(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int64_t b, TreeState& s,
                                const RowStat* rs, const NodeIn* nodes, bool write) {
  const int N = tc.N, D = tc.D;
  for (;;) {
    const int row = s.row;
    const int k0 = tp.off[row], nk = tp.off[row + 1] - k0;
    if (nk == 0) {  // leaf: draw from P
      s.phase = kTreeFinal;
      s.c_new = 0.0;
      s.c_old = 0.0;
      return;
    }
    const int child = tp.kids[k0 + s.j];
    const NodeIn nd = nodes[child];
    const int tok = nd.tok;
    double P, Q;
    if (s.has_exact) {
      WRow wp, wq;  // exact sums come from a residual-type pass over this row pair
      wpair(DT == kBF16 && c.tab, s.mp, s.mq, true, c.c64, wp, wq);
      P = fweight<DT>(nd.ap, wp, c.c64, nullptr) / s.Sp;
      Q = fweight<DT>(nd.aq, wq, c.c64, nullptr) / s.Sq;
    } else {
      P = ::exp(((double)nd.ap - (double)s.mp) * c.invT - ::log(s.sp_hat));
      Q = ::exp(((double)nd.aq - (double)s.mq) * c.invT - ::log(s.sq_hat));
    }
    const double r = s.cj == 0.0 ? P : fmax(0.0, P - s.cj * Q) / s.Gj;
    const double u = nd.u;  // U(seed, step, b, row, 1 + j) of the j-th child of this row
    if (u * Q < r) {
      if (write) {
        tc.out_path[b * D + s.len] = child;
        c.out_tokens[b * (D + 1) + s.len] = tok;
      }
      ++s.len;
      s.row = child + 1;
      load_row_stats(s, rs, N, s.row);
      continue;
    }
    ++s.j;
    s.c_old = s.cj;
    s.c_new = s.cj + s.Gj;
    s.phase = s.j < nk ? kTreeWaitG : kTreeFinal;
    return;
  }
}

// One round of the walk with the row pass it asks for, grid (sub-block
// group, request), launched rounds + 1 times. Every workgroup of a request
// takes the same walk step: in round 0 it reduces the row statistics and
// checks the request, in later rounds it turns the previous round's sums into
// the fp64-grade normalisers of the row pair and G(c_new); then the accept
// tests until the next rejection or the final row. Workgroup 0 writes the
// state and the outputs; every workgroup then sums its sub-blocks of the row
// pair the new state needs. States and sums alternate between two buffers,
// so that a round reads only what the previous round wrote.
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_tree_wp(LinCfg c, TreeTopo tp, TreeCfg tc, int round) {
  const int64_t b = blockIdx.y;
  const bool lead = blockIdx.x == 0;
  const int t = threadIdx.x, N = tc.N, R2 = 2 * (N + 1);
  TreeState* const ts_out = (round & 1) ? tc.ts2 : tc.ts;
  const TreeState* const ts_in = (round & 1) ? tc.ts : tc.ts2;
  TreeRes* const tres_out = (round & 1) ? tc.tres2 : tc.tres;
  const TreeRes* const tres_in = (round & 1) ? tc.tres : tc.tres2;
  __shared__ int s_bad, s_badq;
  __shared__ RowStat s_rs[2 * (kMaxNodes + 1)];
  __shared__ NodeIn s_nodes[kMaxNodes];
  __shared__ TreeState s_st;
  const RowStat* rs = tc.rst + b * R2;
  TreeState s = {};
  if (round == 0) {
    if (t == 0) {
      s_bad = 0;
      s_badq = 0;
    }
    __syncthreads();
    for (int i = t; i < R2; i += kWG) {
      // same reduction as the linear decide step, so that a chain-shaped tree
      // reproduces the linear result bit for bit
      float m;
      double S;
      const int bad = row_norm(c.st + (b * R2 + i) * (int64_t)c.nch32, c.nch32, c.c32, &m, &S) ? 0 : 1;
      RowStat o;
      o.m = m;
      o.bad = bad;
      o.s = S;
      s_rs[i] = o;
      if (lead) tc.rst[b * R2 + i] = o;
      if (bad) atomicOr(&s_bad, 1);
      if (bad && i > N) atomicOr(&s_badq, 1);
    }
    __syncthreads();
    for (int n = t; n < N; n += kWG) {
      int x = tc.tokens[b * N + n];
      if (c.fused && s_badq) {  // drafts drawn in the call: every node of the request is -1
        x = -1;
        if (lead) tc.tokens[b * N + n] = -1;
      }
      if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
    }
    if (lead) tree_clear_outputs(c, tc, b);
    __syncthreads();
    if (s_bad) {
      if (lead && t == 0) {
        c.out_len[b] = -1;
        TreeState d = {};
        d.phase = kTreeDone;
        ts_out[b] = d;
      }
      return;
    }
    rs = s_rs;
    if (t == 0) {
      s.row = 0;
      s.len = 0;
      s.phase = kTreeTest;
      load_row_stats(s, rs, N, 0);
    }
  } else {
    s = ts_in[b];
    if (s.phase != kTreeWaitG) {  // final or done: carried over
      if (lead && t == 0) ts_out[b] = s;
      return;
    }
    // fp64-grade normalisers of the row pair and G(c_new) from the previous
    // pass, by wave 0 (thread 0 takes the walk), while the other waves gather
    // the node inputs
    if (t < kWave) {
      const TreeRes* rr = tres_in + b * c.nsb;
      double sp = 0.0, sq = 0.0;
      for (int sb = t; sb < c.nsb; sb += kWave) {
        sp += rr[sb].sp;
        sq += rr[sb].sq;
      }
      const double Sp = wave_sum_dpp(sp);
      const double Sq = wave_sum_dpp(sq);
      double g = 0.0;
      for (int sb = t; sb < c.nsb; sb += kWave) g += fmax(0.0, rr[sb].a / Sp - s.c_new * rr[sb].bq / Sq);
      const double G = wave_sum_dpp(g);
      s.Sp = Sp;
      s.Sq = Sq;
      s.has_exact = 1;
      if (G > 0.0) {
        s.cj = s.c_new;
        s.Gj = G;
      }
      s.phase = kTreeTest;
    }
  }
  gather_nodes<DT>(c, tp, tc, b, s_nodes);
  __syncthreads();
  if (t == 0) {
    tree_walk_steps<DT>(c, tp, tc, b, s, rs, s_nodes, lead);
    s.buf = round & 1;
    s_st = s;
    if (lead) ts_out[b] = s;
  }
  __syncthreads();
  const int sb = blockIdx.x * kWaves + t / kWave;
  if (sb < c.nsb) tree_pass_sb<DT, AL>(c, s_st, b, sb, tres_out);
}

// -------------------------------------------------------------- row pass --
// fp64 sums of sub-block sb of the row pair of state s (request b), one wave:
// the target row alone at a leaf, else the residual parts for c_new and c_old.
template <int DT, bool AL>
__device__ __forceinline__ void tree_pass_sb(const LinCfg& c, const TreeState& s, int64_t b, int sb, TreeRes* dst) {
  constexpr int EPV = Elem<DT>::kPerVec;
  constexpr int VPL = kSB / (kWave * EPV);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t vfirst = (int64_t)sb * (kSB / EPV) + lane;
  TreeRes out = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  const double c64 = c.c64;
  const bool leaf = s.c_new == 0.0 && s.c_old == 0.0;
  WRow wp, wq;
  wpair(DT == kBF16 && c.tab, s.mp, s.mq, !leaf, c64, wp, wq);
  if (leaf) {  // draw from P: target row only
    float x[VPL][EPV];
    load_vecs<DT, AL, VPL, kWave>(tree_prow(c, b, s.row), c.V, c.nvec, vfirst, x);
    double sp = 0.0;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int e = 0; e < EPV; ++e) sp += fweight<DT>(x[v][e], wp, c64, nullptr);
    out.sp = wave_sum_dpp(sp);
    out.a = out.sp;
    out.a0 = out.sp;
  } else {
    float xp[VPL][EPV], xq[VPL][EPV];
    load_vecs<DT, AL, VPL, kWave>(tree_prow(c, b, s.row), c.V, c.nvec, vfirst, xp);
    load_vecs<DT, AL, VPL, kWave>(tree_qrow(c, b, s.row), c.V, c.nvec, vfirst, xq);
    // P > c Q <=> ep / sph > c eq / sqh <=> a_p - a_q > dx(c), with the best
    // normalisers at hand; entries near the boundary carry almost no weight
    const double sph = s.has_exact ? s.Sp : s.sp_hat, sqh = s.has_exact ? s.Sq : s.sq_hat;
    const double c1 = s.c_new, c0 = s.c_old;
    const float dx1 = (float)((::log2(sph) - ::log2(sqh) + ::log2(c1) + wp.mc - wq.mc) / c64);
    const float dx0 = (float)((::log2(sph) - ::log2(sqh) + ::log2(c0) + wp.mc - wq.mc) / c64);
    double sp = 0.0, sq = 0.0, a = 0.0, bq = 0.0, a0 = 0.0, bq0 = 0.0;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const double ep = fweight<DT>(xp[v][e], wp, c64, nullptr);
        const double eq = fweight<DT>(xq[v][e], wq, c64, nullptr);
        sp += ep;
        sq += eq;
        const double in1 = xp[v][e] - xq[v][e] > dx1 ? 1.0 : 0.0;
        a = __builtin_fma(in1, ep, a);
        bq = __builtin_fma(in1, eq, bq);
        const double in0 = xp[v][e] - xq[v][e] > dx0 ? 1.0 : 0.0;
        a0 = __builtin_fma(in0, ep, a0);
        bq0 = __builtin_fma(in0, eq, bq0);
      }
    out.sp = wave_sum_dpp(sp);
    out.sq = wave_sum_dpp(sq);
    out.a = wave_sum_dpp(a);
    out.bq = wave_sum_dpp(bq);
    out.a0 = wave_sum_dpp(a0);
    out.bq0 = wave_sum_dpp(bq0);
  }
  if (lane == 0) dst[b * c.nsb + sb] = out;
}

template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_tree_pass(LinCfg c, TreeCfg tc, int final_pass) {
  const int64_t b = blockIdx.y;
  const int sb = blockIdx.x * kWaves + threadIdx.x / kWave;
  if (sb >= c.nsb) return;
  const TreeState s = tc.ts[b];
  if (s.phase != (final_pass ? kTreeFinal : kTreeWaitG)) return;
  tree_pass_sb<DT, AL>(c, s, b, sb, tc.tres);
}

// ------------------------------------------------------------ final pick --
// One wave per request: the final token from the running target at the
// stopping row, with the state's sub-block sums loaded once into registers
// (V <= 64 * kTreePickPer * 1024; larger rows read them from memory), the
// sub-block selection, and a rescan of one sub-block with 16-byte loads.
constexpr int kTreePickPer = 4;

template <int DT, bool AL>
__global__ __launch_bounds__(kWave) void k_tree_pick(LinCfg c, TreeCfg tc) {
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x;
  const TreeState s = tc.ts[b];
  if (s.phase != kTreeFinal) return;
  const int nsb = c.nsb, D = tc.D;
  const TreeRes* rr = (s.buf ? tc.tres2 : tc.tres) + b * nsb;
  const bool inreg = nsb <= kWave * kTreePickPer;
  TreeRes mr[kTreePickPer];
  if (inreg) {
#pragma unroll
    for (int k = 0; k < kTreePickPer; ++k) {
      const int sb = lane * kTreePickPer + k;
      mr[k] = sb < nsb ? rr[sb] : TreeRes{0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    }
  }
  auto lane_sum = [&](auto f) {
    double acc = 0.0;
    if (inreg) {
#pragma unroll
      for (int k = 0; k < kTreePickPer; ++k) acc += f(mr[k]);
    } else {
      for (int i = lane; i < nsb; i += kWave) acc += f(rr[i]);
    }
    return acc;
  };
  const char* prow = tree_prow(c, b, s.row);
  const char* qrow = tree_qrow(c, b, s.row);
  const double c64 = c.c64;
  WRow rwp, rwq;
  wpair(DT == kBF16 && c.tab, s.mp, s.mq, s.c_new != 0.0, c64, rwp, rwq);
  const double u = c.rng.u((uint32_t)b, (uint32_t)(s.urow1 > 0 ? s.urow1 - 1 : s.row), kDrawFinal);
  // 0: target weights (a leaf, or a residual (P - Q)+ that vanished); 1: (P - c_new Q)+;
  // 2: (r - Q)+ vanished, so r stays (P - c_old Q)+
  int mode = 0;
  double Sp = 1.0, Sq = 1.0, cm = 0.0, W = 0.0;
  if (s.c_new != 0.0) {
    Sp = wave_sum_dpp(lane_sum([](const TreeRes& r) { return r.sp; }));
    Sq = wave_sum_dpp(lane_sum([](const TreeRes& r) { return r.sq; }));
    const double c1 = s.c_new;
    W = wave_sum_dpp(lane_sum([&](const TreeRes& r) { return fmax(0.0, r.a / Sp - c1 * r.bq / Sq); }));
    if (W > 0.0) {
      mode = 1;
      cm = c1;
    } else if (s.c_old > 0.0) {
      const double c0 = s.c_old;
      W = wave_sum_dpp(lane_sum([&](const TreeRes& r) { return fmax(0.0, r.a0 / Sp - c0 * r.bq0 / Sq); }));
      mode = 2;
      cm = c0;
    }
  }
  auto wsb = [&](const TreeRes& r) {
    return mode == 1 ? fmax(0.0, r.a / Sp - cm * r.bq / Sq) : (mode == 2 ? fmax(0.0, r.a0 / Sp - cm * r.bq0 / Sq) : r.sp);
  };
  if (mode == 0) W = wave_sum_dpp(lane_sum([](const TreeRes& r) { return r.sp; }));
  const double target = u * W;
  double pref;
  int sel;
  if (inreg) {
    double v[kTreePickPer];
#pragma unroll
    for (int k = 0; k < kTreePickPer; ++k) v[k] = wsb(mr[k]);
    sel = wave_select_reg(nsb, target, v, pref);
  } else {
    sel = wave_select(nsb, target, [&](int i) { return wsb(rr[i]); }, pref);
  }
  int y = -1;
  if (sel >= 0) {
    const int64_t j0 = (int64_t)sel * kSB + (int64_t)lane * 16;
    Raw16<DT> rp, rq;
    raw16<DT, AL>(c, prow, j0, rp);
    if (mode != 0) raw16<DT, AL>(c, qrow, j0, rq);
    double w[16];
    weights16<DT>(c, rp, j0, rwp, nullptr, w);
    if (mode != 0) {
      double wq16[16];
      weights16<DT>(c, rq, j0, rwq, nullptr, wq16);
#pragma unroll
      for (int k = 0; k < 16; ++k) w[k] = fmax(0.0, w[k] / Sp - cm * wq16[k] / Sq);
    }
    y = wave_rescan(sel, target - pref, w);
  }
  if (lane == 0) {
    c.out_tokens[b * (D + 1) + s.len] = y;
    c.out_len[b] = s.len;
    TreeState d = s;
    d.phase = kTreeDone;
    tc.ts[b] = d;
  }
}

// ---------------------------------------------------------------- greedy --
__global__ __launch_bounds__(kWG) void k_tree_greedy(LinCfg c, TreeTopo tp, TreeCfg tc) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, N = tc.N, D = tc.D, R2 = 2 * (N + 1);
  __shared__ int s_bad, s_badq;
  __shared__ int s_g[2 * (kMaxNodes + 1)];
  __shared__ int s_tok[kMaxNodes];
  if (t == 0) {
    s_bad = 0;
    s_badq = 0;
  }
  __syncthreads();
  for (int i = t; i < R2; i += kWG) {
    int bad;
    s_g[i] = row_argmax(c.ar + (b * R2 + i) * (int64_t)c.nch32, c.nch32, &bad);
    if (bad) {
      atomicOr(&s_bad, 1);
      if (i > N) atomicOr(&s_badq, 1);
    }
  }
  __syncthreads();
  for (int n = t; n < N; n += kWG) {
    int x;
    if (c.fused) {
      x = s_badq ? -1 : s_g[N + 1 + tp.prow[n]];  // argmax of the parent row's draft logits
      tc.tokens[b * N + n] = x;
    } else {
      x = tc.tokens[b * N + n];
    }
    s_tok[n] = x;
    if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
  }
  tree_clear_outputs(c, tc, b);
  __syncthreads();
  if (t != 0) return;
  if (s_bad) {
    c.out_len[b] = -1;
    return;
  }
  int row = 0, len = 0;
  for (;;) {
    const int g = s_g[row];
    int acc = -1;
    for (int k = tp.off[row]; k < tp.off[row + 1]; ++k)
      if (s_tok[tp.kids[k]] == g) {
        acc = tp.kids[k];
        break;
      }
    if (acc < 0) {
      c.out_tokens[b * (D + 1) + len] = g;
      break;
    }
    tc.out_path[b * D + len] = acc;
    c.out_tokens[b * (D + 1) + len] = g;
    ++len;
    row = acc + 1;
  }
  c.out_len[b] = len;
}

// -------------------------------------------------------------- filtered --
// Union of the kept sets of a target row and a draft row, in token-id order.
constexpr int kUnion = 2 * kMaxTopK;

__global__ __launch_bounds__(kWG) void k_tree_filt(LinCfg c, FiltCfg f, TreeTopo tp, TreeCfg tc) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, N = tc.N, D = tc.D, R2 = 2 * (N + 1);
  const FiltRow* H = f.hdr + b * R2;
  const FiltEnt* Ent = f.ent + b * R2 * (int64_t)f.stride;
  __shared__ int s_bad, s_badq;
  __shared__ int s_id[kUnion];
  __shared__ int s_tok[kMaxNodes];
  __shared__ double s_r[kUnion], s_q[kUnion], s_pe[kMaxTopK], s_qe[kMaxTopK];
  if (t == 0) {
    s_bad = 0;
    s_badq = 0;
  }
  __syncthreads();
  for (int i = t; i < R2; i += kWG)
    if (H[i].bad || H[i].cnt <= 0) {
      atomicOr(&s_bad, 1);
      if (i > N) atomicOr(&s_badq, 1);
    }
  __syncthreads();
  for (int n = t; n < N; n += kWG) {
    int x;
    if (c.fused) {
      x = -1;
      if (!s_badq) {
        const int r = tp.prow[n];
        const FiltRow hq = H[N + 1 + r];
        const FiltEnt* eq = Ent + (N + 1 + r) * (int64_t)f.stride;
        const double u = c.rng.u((uint32_t)b, (uint32_t)r, kDrawDraft + (uint32_t)tp.sib[n]);
        x = draw_list(hq.cnt, u, [&](int k) { return ::exp(eq[k].z - hq.m); }, eq);
      }
      tc.tokens[b * N + n] = x;
    } else {
      x = tc.tokens[b * N + n];
    }
    s_tok[n] = x;
    if (x < 0 || x >= c.V) atomicOr(&s_bad, 1);
  }
  tree_clear_outputs(c, tc, b);
  __syncthreads();
  if (s_bad) {
    if (t == 0) c.out_len[b] = -1;
    return;
  }
  int row = 0, len = 0;  // uniform across the workgroup
  for (;;) {
    const FiltRow hp = H[row], hq = H[N + 1 + row];
    const FiltEnt* ep = Ent + row * (int64_t)f.stride;
    const FiltEnt* eq = Ent + (N + 1 + row) * (int64_t)f.stride;
    const int k0 = tp.off[row], nk = tp.off[row + 1] - k0;
    // normalised probabilities of the two kept sets
    for (int k = t; k < hp.cnt; k += kWG) s_pe[k] = ::exp(ep[k].z - hp.L);
    for (int k = t; k < hq.cnt; k += kWG) s_qe[k] = ::exp(eq[k].z - hq.L);
    __syncthreads();
    __shared__ int s_next, s_y;
    if (t == 0) {
      int y = -1, next = -1;
      if (nk == 0) {
        const double u = c.rng.u((uint32_t)b, (uint32_t)row, kDrawFinal);
        y = draw_list(hp.cnt, u, [&](int k) { return s_pe[k]; }, ep);
      } else {
        // merge the two id-ordered lists
        int nu = 0, i = 0, k = 0;
        while (i < hp.cnt || k < hq.cnt) {
          const int ip = i < hp.cnt ? ep[i].i : 0x7fffffff;
          const int iq = k < hq.cnt ? eq[k].i : 0x7fffffff;
          const int id = min(ip, iq);
          s_id[nu] = id;
          s_r[nu] = id == ip ? s_pe[i++] : 0.0;
          s_q[nu] = id == iq ? s_qe[k++] : 0.0;
          ++nu;
        }
        auto find = [&](int x) {
          int lo = 0, hi = nu - 1;
          while (lo <= hi) {
            const int mid = (lo + hi) >> 1;
            if (s_id[mid] == x) return mid;
            if (s_id[mid] < x) lo = mid + 1;
            else hi = mid - 1;
          }
          return -1;
        };
        for (int j = 0; j < nk; ++j) {
          const int child = tp.kids[k0 + j];
          const int tok = s_tok[child];
          const int at = find(tok);
          const double Qt = at >= 0 ? s_q[at] : 0.0, rt = at >= 0 ? s_r[at] : 0.0;
          const double u = c.rng.u((uint32_t)b, (uint32_t)row, (uint32_t)(kDrawAccept + j));
          if (u * Qt < rt) {
            next = child;
            break;
          }
          double S = 0.0;
          for (int e = 0; e < nu; ++e) S += fmax(0.0, s_r[e] - s_q[e]);
          if (S > 0.0)
            for (int e = 0; e < nu; ++e) s_r[e] = fmax(0.0, s_r[e] - s_q[e]) / S;
        }
        if (next < 0) {
          const double u = c.rng.u((uint32_t)b, (uint32_t)row, kDrawFinal);
          double W = 0.0;
          for (int e = 0; e < nu; ++e) W += s_r[e];
          const double target = u * W;
          double acc = 0.0;
          int last = -1;
          for (int e = 0; e < nu; ++e) {
            acc += s_r[e];
            if (s_r[e] > 0.0) last = e;
            if (acc > target) {
              y = s_id[e];
              break;
            }
          }
          if (y < 0 && last >= 0) y = s_id[last];
        }
      }
      s_next = next;
      s_y = y;
    }
    __syncthreads();
    const int next = s_next;
    if (next < 0) {
      if (t == 0) {
        c.out_tokens[b * (D + 1) + len] = s_y;
        c.out_len[b] = len;
      }
      return;
    }
    if (t == 0) {
      tc.out_path[b * D + len] = next;
      c.out_tokens[b * (D + 1) + len] = s_tok[next];
    }
    ++len;
    row = next + 1;
    __syncthreads();
  }
}

// ------------------------------------------------------------- launchers --
template <int DT, bool AL>
static hipError_t tree_sampled_t(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int rounds, hipStream_t s) {
  const dim3 grid((c.nsb + kWaves - 1) / kWaves, (unsigned)c.B);
  for (int r = 0; r <= rounds; ++r) PSI_LAUNCH(s, (k_tree_wp<DT, AL>), grid, dim3(kWG), c, tp, tc, r);
  TreeCfg tf = tc;  // the last round's states
  tf.ts = (rounds & 1) ? tc.ts2 : tc.ts;
  PSI_LAUNCH(s, (k_tree_pick<DT, AL>), dim3((unsigned)c.B), dim3(kWave), c, tf);
  return hipGetLastError();
}

hipError_t launch_tree_sampled(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int rounds, int dtype,
                               hipStream_t s) {
  hipError_t e = hipSuccess;
  if (c.fused && dtype == kBF16 && c.tab) {
    // node drafts in one pass per draft row (which writes that row's chunk
    // records); the target rows' records by waves of the same launch
    e = launch_tree_qrows(c, tp, tc, s);
    if (e != hipSuccess) return e;
    return c.aligned ? tree_sampled_t<kBF16, true>(c, tp, tc, rounds, s)
                     : tree_sampled_t<kBF16, false>(c, tp, tc, rounds, s);
  }
  if (c.fused) {
    // node drafts: fp64 sub-block records of every draft row, then one pick per node
    e = launch_draftpass(c, c.B * (int64_t)(tc.N + 1), dtype, s);
    if (e != hipSuccess) return e;
    if (dtype == kBF16) PSI_LAUNCH(s, (k_tree_draft<kBF16>), dim3((unsigned)(c.B * tc.N)), dim3(kWG), c, tp, tc);
    else PSI_LAUNCH(s, (k_tree_draft<kF32>), dim3((unsigned)(c.B * tc.N)), dim3(kWG), c, tp, tc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  e = launch_stats32(c, c.B * (int64_t)(2 * (tc.N + 1)), dtype, s);
  if (e != hipSuccess) return e;
  if (dtype == kBF16)
    return c.aligned ? tree_sampled_t<kBF16, true>(c, tp, tc, rounds, s)
                     : tree_sampled_t<kBF16, false>(c, tp, tc, rounds, s);
  return c.aligned ? tree_sampled_t<kF32, true>(c, tp, tc, rounds, s) : tree_sampled_t<kF32, false>(c, tp, tc, rounds, s);
}

template <int DT, bool AL>
static hipError_t tree_final_t(const LinCfg& c, const TreeCfg& tc, hipStream_t s) {
  PSI_LAUNCH(s, (k_tree_pass<DT, AL>), dim3((unsigned)((c.nsb + kWaves - 1) / kWaves), (unsigned)c.B), dim3(kWG), c,
             tc, 1);
  PSI_LAUNCH(s, (k_tree_pick<DT, AL>), dim3((unsigned)c.B), dim3(kWave), c, tc);
  return hipGetLastError();
}

hipError_t launch_tree_final(const LinCfg& c, const TreeCfg& tc, int dtype, hipStream_t s) {
  return PSI_DISPATCH(tree_final_t, dtype, c.aligned, c, tc, s);
}

hipError_t launch_tree_greedy(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int dtype, hipStream_t s) {
  hipError_t e = launch_argmax(c, c.B * (int64_t)(2 * (tc.N + 1)), dtype, s);
  if (e != hipSuccess) return e;
  PSI_LAUNCH(s, k_tree_greedy, dim3((unsigned)c.B), dim3(kWG), c, tp, tc);
  return hipGetLastError();
}

hipError_t launch_tree_filtered(const LinCfg& c, const FiltCfg& f, const TreeTopo& tp, const TreeCfg& tc, int dtype,
                                hipStream_t s) {
  hipError_t e = launch_filter_rows(c, f, c.B * (int64_t)(2 * (tc.N + 1)), dtype, s);
  if (e != hipSuccess) return e;
  PSI_LAUNCH(s, k_tree_filt, dim3((unsigned)c.B), dim3(kWG), c, f, tp, tc);
  return hipGetLastError();
}

}  // namespace psi
