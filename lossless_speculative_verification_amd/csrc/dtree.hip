// Tree Sampler on gfx950 ("Uno" research explainer, §3.4 Tree Sampler: every
// draft position keeps its top-K tokens, only the most probable prefixes over
// them are kept, and the resulting tree is verified in one pass; §6.3 uses
// block 16, K = 32 and 32 kept prefixes).
//
// Candidates, per request:
//   q_i = softmax(d_i / T), C_i = the `cands` most probable tokens of
//   position i (ties: lower id), score of a prefix = sum of log q_i(t_i);
//   keep the `nodes` best prefixes under (score desc, length asc, position of
//   the parent prefix asc, rank of the last token asc).
// Pipeline: the filter kernels with top_k = cands, whose chunk pass also
// stores each chunk's maximum and sum of 2^((a - m) c) (for log q) and whose
// merge stores each kept set in rank order, then
// k_cand_tree: one workgroup per request turns the kept sets into log q
// values in LDS and one wave enumerates the prefixes best first (every kept
// prefix offers its best child not yet kept; the best offer is kept).
//
// Verification of deterministic candidates (a point-mass proposal at tok is
// accepted with probability r(tok)), per request with its own tree:
//   at a row r = P, E = 0; children in ascending node id, child j accepted iff
//   U(b, row, 1 + j) * (1 - E) < P(tok) (0 if tok was already removed), a
//   rejection removes tok (E += P(tok)); the walk descends into the first
//   accepted child; at a leaf or once every child is rejected the final token
//   is drawn from P without the removed tokens with U(b, row, 0).
// Pipeline: k_stats32 over the N + 1 target rows; k_dtree_walk (one workgroup
// per request: row normalisers, every node's P(tok), sibling order and
// uniforms in parallel, then the walk by one thread over LDS); k_dtree_pass
// (sub-block sums of the final row with and without the removed tokens);
// k_dtree_pick (inverse-CDF draw). Greedy: k_argmax then k_dtree_greedy.
#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kSlots = kMaxNodes + 1;                       // the empty prefix, then one per node
constexpr int kSlotsPerLane = (kSlots + kWave - 1) / kWave;  // slot s lives on lane s % 64

// Unsigned key increasing with the double x; its upper 32 bits order the
// values up to ties within 2^-20 relative.
__device__ __forceinline__ uint32_t order_hi(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint64_t k = (b >> 63) ? ~b : (b | 0x8000000000000000ull);
  return (uint32_t)(k >> 32);
}

__device__ __forceinline__ double rd_lane(double v, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), l);
  return __hiloint2double(hi, lo);
}


}  // namespace

// ------------------------------------------------------------ candidates --
// Best-first enumeration by one whole wave. Slot s (0 = the empty prefix,
// n + 1 = node n) lives on lane s % 64, register j = s / 64 (SPL registers per
// lane): its log score, length, the rank of its best child not yet kept, and
// that child's offer (-inf when none). Per step: each lane's best offer under
// (score desc, length asc, slot asc), the wave maximum of the upper 32 bits of
// the scores' order keys (DPP), a ballot, and a full compare only when upper
// words tie; the kept slot then offers its next child and the new slot its
// first, from two broadcast LDS reads. Writes s_par[n] and s_ent[n] (position
// * C + rank) for n < NN, -1 past the last prefix of positive probability.
template <int SPL>
__device__ void cand_enumerate(const double* s_lq, int K, int C, int NN, int* s_par, int* s_ent) {
  const int lane = threadIdx.x & (kWave - 1);
  double ls[SPL], off[SPL];
  int dep[SPL], nxt[SPL];
#pragma unroll
  for (int j = 0; j < SPL; ++j) {
    ls[j] = 0.0;
    off[j] = -INFINITY;
    dep[j] = 0;
    nxt[j] = 0;
  }
  if (lane == 0) off[0] = s_lq[0];  // the empty prefix offers the best position-0 candidate
  int n = 0;
  for (; n < NN; ++n) {
    double bo = off[0], bl = ls[0];
    int bk = dep[0] * 512 + lane, bn = nxt[0];
#pragma unroll
    for (int j = 1; j < SPL; ++j) {
      const int key = dep[j] * 512 + lane + kWave * j;
      const bool better = off[j] > bo || (off[j] == bo && key < bk);
      bo = better ? off[j] : bo;
      bl = better ? ls[j] : bl;
      bk = better ? key : bk;
      bn = better ? nxt[j] : bn;
    }
    const uint32_t hi = bo > -INFINITY ? order_hi(bo) : 0u;
    const uint32_t M = wave_max_u32(hi);
    if (M == 0u) break;  // no prefix of positive probability is left
    unsigned long long cand = __ballot(hi == M);
    int w = __ffsll((long long)cand) - 1;
    if (__popcll(cand) > 1) {  // upper words tie: compare in full
      double wo = rd_lane(bo, w);
      int wk = __builtin_amdgcn_readlane(bk, w);
      cand &= cand - 1;
      while (cand) {
        const int l = __ffsll((long long)cand) - 1;
        cand &= cand - 1;
        const double o = rd_lane(bo, l);
        const int k = __builtin_amdgcn_readlane(bk, l);
        if (o > wo || (o == wo && k < wk)) {
          w = l;
          wo = o;
          wk = k;
        }
      }
    }
    const double wo = rd_lane(bo, w);
    const double wl = rd_lane(bl, w);
    const int wk = __builtin_amdgcn_readlane(bk, w);
    const int wn = __builtin_amdgcn_readlane(bn, w);
    const int ws = wk & 511, wd = wk >> 9;
    if (lane == 0) {
      s_par[n] = ws - 1;
      s_ent[n] = wd * C + wn;
    }
    const double x1 = wn + 1 < C ? s_lq[wd * C + wn + 1] : -INFINITY;  // the kept slot's next child
    const double x0 = wd + 1 < K ? s_lq[(wd + 1) * C] : -INFINITY;     // the new slot's first child
    const int sn = n + 1;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      const bool kept = j == (ws >> 6) && lane == (ws & (kWave - 1));
      const bool born = j == (sn >> 6) && lane == (sn & (kWave - 1));
      nxt[j] = kept ? wn + 1 : (born ? 0 : nxt[j]);
      off[j] = kept ? wl + x1 : (born ? wo + x0 : off[j]);
      ls[j] = born ? wo : ls[j];
      dep[j] = born ? wd + 1 : dep[j];
    }
  }
  if (lane == 0)
    for (int m = n; m < NN; ++m) {
      s_par[m] = -1;
      s_ent[m] = -1;
    }
}

__global__ __launch_bounds__(kWG) void k_cand_tree(LinCfg c, FiltCfg f, CandCfg cc) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int K = c.K, C = cc.cands, NN = cc.nodes;
  __shared__ double s_lq[kMaxCandEntries];  // [K][C] log q of rank r at position i, -inf past the kept set
  __shared__ double s_L[kMaxK];
  __shared__ int s_cnt[kMaxK];
  __shared__ int s_ent[kMaxNodes];
  __shared__ int s_par[kMaxNodes];
  __shared__ int s_bad;
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int i = t; i < K; i += kWG) {
    const int64_t sr = b * K + i;
    const FiltRow h = f.hdr[sr];
    float m;
    double S;
    const bool ok = row_norm(f.cst + sr * f.nchf, f.nchf, c.c32, &m, &S);
    if (!ok || h.bad || h.cnt <= 0) atomicOr(&s_bad, 1);
    // log of the full-row normaliser of z = a / T
    s_L[i] = (double)m / f.T + ::log(S);
    s_cnt[i] = h.cnt;
  }
  __syncthreads();
  if (s_bad) {
    for (int n = t; n < NN; n += kWG) {
      cc.out_parent[b * NN + n] = -1;
      cc.out_tokens[b * NN + n] = -1;
    }
    return;
  }
  const FiltEnt* ent = f.ent + b * K * (int64_t)f.stride;
  for (int e = t; e < K * C; e += kWG) {
    const int i = e / C, r = e - i * C;
    s_lq[e] = r < s_cnt[i] ? ent[i * (int64_t)f.stride + r].z - s_L[i] : -INFINITY;
  }
  __syncthreads();
  if (t >= kWave) return;
  switch ((NN + kWave) / kWave) {  // slots per lane: ceil((NN + 1) / 64)
    case 1: cand_enumerate<1>(s_lq, K, C, NN, s_par, s_ent); break;
    case 2: cand_enumerate<2>(s_lq, K, C, NN, s_par, s_ent); break;
    case 3: cand_enumerate<3>(s_lq, K, C, NN, s_par, s_ent); break;
    case 4: cand_enumerate<4>(s_lq, K, C, NN, s_par, s_ent); break;
    default: cand_enumerate<5>(s_lq, K, C, NN, s_par, s_ent); break;
  }
  wave_sync();
  for (int m = lane; m < NN; m += kWave) {
    const int e = s_ent[m];
    int tok = -1;
    if (e >= 0) {
      const int i = e / C, r = e - i * C;
      tok = ent[i * (int64_t)f.stride + r].i;
    }
    cc.out_parent[b * NN + m] = s_par[m];
    cc.out_tokens[b * NN + m] = tok;
  }
}

// ---------------------------------------------------------- verification --
// Walk outcome of one request, for the final pick.
struct DTreeState {
  int32_t row;   // final row
  int32_t len;   // accepted path length; -1 = request error (outputs written)
  int32_t nrem;  // removed tokens (the final row's children when it has any)
  int32_t pad;
  float m;       // exact maximum of the final row
  float pad2;
};
static_assert(sizeof(DTreeState) <= sizeof(TreeState), "DTreeState lives in the tree-state section");

namespace {

__device__ __forceinline__ const char* det_row(const LinCfg& c, int64_t b, int r) {
  return c.rows.p + ((b * c.rows.np + r) * (int64_t)c.V) * c.rows.esz;
}

// Bit k of the result: element j0 + k (k < 32) is one of the removed tokens.
__device__ __forceinline__ uint32_t removed_mask(const int32_t* rem, int nrem, int64_t j0) {
  uint32_t gone = 0;
  for (int k = 0; k < nrem; ++k) {
    const int64_t rel = (int64_t)rem[k] - j0;
    if (rel >= 0 && rel < 32) gone |= 1u << rel;
  }
  return gone;
}

}  // namespace

// Validates the request and, for node n: sibling index j (ascending node id
// among the children of its parent row), whether an earlier sibling carries
// the same token, and the child lists in node order (s_par / s_tok filled and
// *s_bad set by the caller before). The writer workgroup clears the outputs
// and reports a malformed request. Returns false for one.
template <int NT>
__device__ bool det_topology(const LinCfg& c, const DTreeCfg& d, int64_t b, bool writer, const int* s_par,
                             const int* s_tok, int* s_sib, int* s_dup, int* s_off, int* s_kid, int* s_bad) {
  const int t = threadIdx.x, N = d.N;
  if (writer) {
    for (int i = t; i <= N; i += NT) d.out_tokens[b * (N + 1) + i] = -1;
    for (int i = t; i < N; i += NT) d.out_path[b * N + i] = -1;
  }
  __syncthreads();
  if (*s_bad) {
    if (writer && t == 0) c.out_len[b] = -1;
    return false;
  }
  // off[r] = nodes whose parent row is below r; sibling index and duplicates
  for (int r = t; r <= N; r += NT) {
    int k = 0;
    for (int m = 0; m < N; ++m) k += s_par[m] + 1 < r ? 1 : 0;
    s_off[r] = k;
  }
  for (int n = t; n < N; n += NT) {
    const int p = s_par[n], x = s_tok[n];
    int j = 0, dup = 0;
    for (int m = 0; m < n; ++m)
      if (s_par[m] == p) {
        ++j;
        dup |= s_tok[m] == x;
      }
    s_sib[n] = j;
    s_dup[n] = dup;
  }
  __syncthreads();
  for (int n = t; n < N; n += NT) s_kid[s_off[s_par[n] + 1] + s_sib[n]] = n;
  __syncthreads();
  return true;
}

// Grid (sub-block groups, request). Every workgroup of a request repeats the
// walk (row normalisers from the statistics records, every node's P(tok) and
// uniform, the walk by thread 0 over LDS); workgroup 0 writes the path and the
// walk outcome. Then each wave sums one sub-block of the final row under the
// final-draw weight rule: res.sp without the removed tokens, res.sq over all.
template <int DT, bool AL>
__global__ __launch_bounds__(kWG) void k_dtree_walkpass(LinCfg c, DTreeCfg d) {
  using E = Elem<DT>;
  constexpr int EPV = E::kPerVec;
  constexpr int VPL = kSB / (kWave * EPV);
  const int64_t b = blockIdx.y;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int N = d.N, R = N + 1;
  const bool writer = blockIdx.x == 0;
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_sib[kMaxNodes], s_dup[kMaxNodes], s_kid[kMaxNodes];
  __shared__ int s_off[kMaxNodes + 1];
  __shared__ double s_P[kMaxNodes], s_u[kMaxNodes];
  __shared__ float s_m[kMaxNodes + 1];
  __shared__ double s_S[kMaxNodes + 1];
  __shared__ int s_rem[kMaxNodes];
  __shared__ int s_bad, s_row, s_nrem;
  if (t == 0) s_bad = 0;
  __syncthreads();
  // node data, and the logit of each node's token at its parent row
  float a_node[(kMaxNodes + kWG - 1) / kWG];
#pragma unroll
  for (int k = 0; k < (kMaxNodes + kWG - 1) / kWG; ++k) {
    const int n = t + k * kWG;
    a_node[k] = 0.0f;
    if (n < N) {
      const int p = d.parent[b * N + n], x = d.tokens[b * N + n];
      const bool ok = p >= -1 && p < n && x >= 0 && x < c.V;
      if (!ok) atomicOr(&s_bad, 1);
      s_par[n] = p;
      s_tok[n] = x;
      if (ok) a_node[k] = E::load1(det_row(c, b, p + 1), x);
    }
  }
  for (int r = t; r < R; r += kWG) {
    float m;
    double S;
    if (!row_norm(c.st + (b * R + r) * (int64_t)c.nch32, c.nch32, c.c32, &m, &S)) atomicOr(&s_bad, 1);
    s_m[r] = m;
    s_S[r] = S;
  }
  if (!det_topology<kWG>(c, d, b, writer, s_par, s_tok, s_sib, s_dup, s_off, s_kid, &s_bad)) {
    if (writer && t == 0) ((DTreeState*)d.state)[b] = DTreeState{0, -1, 0, 0, 0.0f, 0.0f};
    return;
  }
#pragma unroll
  for (int k = 0; k < (kMaxNodes + kWG - 1) / kWG; ++k) {
    const int n = t + k * kWG;
    if (n < N) {
      const int row = s_par[n] + 1;
      s_P[n] = ::exp(((double)a_node[k] - (double)s_m[row]) * c.invT - ::log(s_S[row]));
      s_u[n] = c.rng.u((uint32_t)b, (uint32_t)row, kDrawAccept + (uint32_t)s_sib[n]);
    }
  }
  __syncthreads();
  if (t == 0) {
    int row = 0, len = 0, k0 = 0, nk = 0;
    for (;;) {
      k0 = s_off[row];
      nk = (row < N ? s_off[row + 1] : N) - k0;
      double E = 0.0;  // probability removed at this row
      int acc = -1;
      for (int k = 0; k < nk; ++k) {
        const int n = s_kid[k0 + k];
        const double pt = s_dup[n] ? 0.0 : s_P[n];
        if (s_u[n] * (1.0 - E) < pt) {
          acc = n;
          break;
        }
        E += pt;
      }
      if (acc < 0) break;
      if (writer) {
        d.out_path[b * N + len] = acc;
        d.out_tokens[b * (N + 1) + len] = s_tok[acc];
      }
      ++len;
      row = acc + 1;
    }
    for (int k = 0; k < nk; ++k) s_rem[k] = s_tok[s_kid[k0 + k]];
    s_row = row;
    s_nrem = nk;
    if (writer) ((DTreeState*)d.state)[b] = DTreeState{row, len, nk, 0, s_m[row], 0.0f};
  }
  __syncthreads();
  const int row = s_row, nrem = s_nrem;
  if (writer)
    for (int k = t; k < nrem; k += kWG) d.rem[b * N + k] = s_rem[k];
  const int sb = blockIdx.x * kWaves + wave;
  if (sb >= c.nsb) return;
  const int64_t vfirst = (int64_t)sb * (kSB / EPV) + lane;
  float x[VPL][EPV];
  load_vecs<DT, AL, VPL, kWave>(det_row(c, b, row), c.V, c.nvec, vfirst, x);
  // removed tokens held by this lane: element (vfirst + v * 64) * EPV + e is bit v * EPV + e
  uint32_t gone = 0;
#pragma unroll
  for (int v = 0; v < VPL; ++v)
    gone |= (removed_mask(s_rem, nrem, (vfirst + (int64_t)v * kWave) * EPV) & ((1u << EPV) - 1u)) << (v * EPV);
  const WRow wr = wrow(DT == kBF16 && c.tab, s_m[row], c.c64);
  double all = 0.0, kept = 0.0;
#pragma unroll
  for (int v = 0; v < VPL; ++v)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const double w = fweight<DT>(x[v][e], wr, c.c64, nullptr);
      all += w;
      kept += (gone >> (v * EPV + e)) & 1u ? 0.0 : w;
    }
  all = wave_sum_dpp(all);
  kept = wave_sum_dpp(kept);
  if (lane == 0) c.res[b * c.nsb + sb] = ResRec{kept, all, 0.0, 0.0};
}

// One wave per request: inverse-CDF draw from the final row's weights without
// the removed tokens (from all of them if nothing is left), then the outputs.
template <int DT>
__global__ __launch_bounds__(kWave) void k_dtree_pick(LinCfg c, DTreeCfg d) {
  using E = Elem<DT>;
  constexpr int EPL = kSB / kWave;
  const int64_t b = blockIdx.x;
  const int lane = threadIdx.x, nsb = c.nsb, N = d.N;
  __shared__ int32_t s_rem[kMaxNodes];
  for (int k = lane; k < N; k += kWave) s_rem[k] = d.rem[b * N + k];  // entries past nrem are not read
  const DTreeState s = ((const DTreeState*)d.state)[b];
  if (s.len < 0) return;
  wave_sync();
  const int32_t* rem = s_rem;
  const ResRec* rr = c.res + b * nsb;
  double W = 0.0, W0 = 0.0;
  for (int sb = lane; sb < nsb; sb += kWave) {
    const ResRec r = rr[sb];
    W += r.sp;
    W0 += r.sq;
  }
  W = wave_sum_dpp(W);
  W0 = wave_sum_dpp(W0);
  const char* row = det_row(c, b, s.row);
  const WRow wr = wrow(DT == kBF16 && c.tab, s.m, c.c64);
  const double u = c.rng.u((uint32_t)b, (uint32_t)s.row, kDrawFinal);
  const bool none_left = !(W > 0.0);  // every token of positive probability was removed: draw from P
  const int y = wave_pick(
      nsb, c.V, u * (none_left ? W0 : W), [&](int sb) { return none_left ? rr[sb].sq : rr[sb].sp; },
      [&](int64_t j0, double (&w)[EPL]) {
        const uint32_t gone = none_left ? 0u : removed_mask(rem, s.nrem, j0);
#pragma unroll
        for (int k = 0; k < EPL; ++k) {
          const int64_t j = j0 + k;
          const double e = j < c.V ? fweight<DT>(E::load1(row, j), wr, c.c64, nullptr) : 0.0;
          w[k] = (gone >> k) & 1u ? 0.0 : e;
        }
      });
  if (lane == 0) {
    d.out_tokens[b * (N + 1) + s.len] = y;
    c.out_len[b] = s.len;
  }
}

// Temperature 0: a child is accepted iff its token is its row's argmax.
__global__ __launch_bounds__(kWG) void k_dtree_greedy(LinCfg c, DTreeCfg d) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, N = d.N, R = N + 1;
  __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_sib[kMaxNodes], s_dup[kMaxNodes], s_kid[kMaxNodes];
  __shared__ int s_off[kMaxNodes + 1];
  __shared__ int s_g[kMaxNodes + 1];
  __shared__ int s_bad;
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int r = t; r < R; r += kWG) {
    int bad;
    s_g[r] = row_argmax(c.ar + (b * R + r) * (int64_t)c.nch32, c.nch32, &bad);
    if (bad) atomicOr(&s_bad, 1);
  }
  for (int n = t; n < N; n += kWG) {
    const int p = d.parent[b * N + n], x = d.tokens[b * N + n];
    if (p < -1 || p >= n || x < 0 || x >= c.V) atomicOr(&s_bad, 1);
    s_par[n] = p;
    s_tok[n] = x;
  }
  if (!det_topology<kWG>(c, d, b, true, s_par, s_tok, s_sib, s_dup, s_off, s_kid, &s_bad)) return;
  if (t != 0) return;
  int row = 0, len = 0;
  for (;;) {
    const int g = s_g[row];
    const int k0 = s_off[row], nk = (row < N ? s_off[row + 1] : N) - k0;
    int acc = -1;
    for (int k = 0; k < nk && acc < 0; ++k)
      if (s_tok[s_kid[k0 + k]] == g) acc = s_kid[k0 + k];
    if (acc < 0) {
      d.out_tokens[b * (N + 1) + len] = g;
      break;
    }
    d.out_path[b * N + len] = acc;
    d.out_tokens[b * (N + 1) + len] = g;
    ++len;
    row = acc + 1;
  }
  c.out_len[b] = len;
}

// ------------------------------------------------------------- launchers --
template <int DT, bool AL>
static hipError_t cand_t(const LinCfg& c, const FiltCfg& f, const CandCfg& cc, hipStream_t s) {
  hipError_t e = launch_filter_rows(c, f, c.B * c.K, DT, s);  // with the chunk statistics (f.cst)
  if (e != hipSuccess) return e;
  PSI_LAUNCH(s, k_cand_tree, dim3((unsigned)c.B), dim3(kWG), c, f, cc);
  return hipGetLastError();
}

hipError_t launch_tree_candidates(const LinCfg& c, const FiltCfg& f, const CandCfg& cc, int dtype, hipStream_t s) {
  return PSI_DISPATCH(cand_t, dtype, c.aligned, c, f, cc, s);
}

template <int DT, bool AL>
static hipError_t dtree_t(const LinCfg& c, const DTreeCfg& d, hipStream_t s) {
  const int64_t rows = c.B * (d.N + 1);
  if (c.c64 == 0.0) {
    hipError_t e = launch_argmax(c, rows, DT, s);
    if (e != hipSuccess) return e;
    PSI_LAUNCH(s, k_dtree_greedy, dim3((unsigned)c.B), dim3(kWG), c, d);
    return hipGetLastError();
  }
  hipError_t e = launch_stats32(c, rows, DT, s);
  if (e != hipSuccess) return e;
  PSI_LAUNCH(s, (k_dtree_walkpass<DT, AL>), dim3((unsigned)((c.nsb + kWaves - 1) / kWaves), (unsigned)c.B),
             dim3(kWG), c, d);
  PSI_LAUNCH(s, k_dtree_pick<DT>, dim3((unsigned)c.B), dim3(kWave), c, d);
  return hipGetLastError();
}

hipError_t launch_verify_tree_det(const LinCfg& c, const DTreeCfg& d, int dtype, hipStream_t s) {
  return PSI_DISPATCH(dtree_t, dtype, c.aligned, c, d, s);
}

}  // namespace psi
