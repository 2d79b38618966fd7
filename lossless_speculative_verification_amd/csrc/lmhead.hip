// Linear verification fused with the LM head on gfx950: the target and draft
// logits are products of hidden states with the vocabulary matrix
// ("Uno" research explainer, §3.1: the AR path and the diffusion path share
// the base model and its output head; §3.3: the verifier needs p and q of the
// drafted tokens, then one residual or bonus row), computed tile by tile with
// bf16 matrix cores and reduced in the tile's epilogue, so that the logits of
// the K + 1 target and K draft rows never reach HBM.
//
// Pipeline on the caller's stream:
//   k_lmh_gemm<kLmhStats>   every target and draft row against every 256-token
//                           vocabulary tile: per (row, tile) the maximum and a
//                           binary32-grade sum of 2^((z - m) c), and the logit
//                           of the row's drafted token;
//   k_lmh_decide            per request: row normalisers, accept tests
//                           u * Q(x) < P(x), first rejection n; the draw state;
//   k_lmh_gemm<kLmhLogits>  the final rows only (target row n and draft row n,
//                           or the bonus row): fp32 logits;
//   k_tree_pass, k_tree_pick (tree.hip) the fp64 residual / bonus draw over them.
//
// GEMM: C[M, V] = A[M, H] * W[V, H]^T, A rows from the target and draft hidden
// states. A workgroup computes a 128-row x 256-token tile with four waves (2 x
// 2, 64 x 128 each, as 2 x 4 blocks of v_mfma_f32_32x32x16_bf16), stepping over
// H by 32 with both operand tiles double-buffered in LDS (rows padded by 16
// bytes so that the 16-byte fragment reads of a wave do not collide in banks),
// the global loads issued two steps ahead and two workgroups per CU.
// Block operand layout of the instruction (checked on the device): lane l
// holds A[l % 32][8 (l / 32) .. +7] and W[col l % 32][8 (l / 32) .. +7]; result
// element i of lane l is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
// Tiles are ordered so that the row tiles of one vocabulary tile run one after
// another on the same XCD and share its L2 copy of the W tile.
#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kLmhBM = kLmhTileM, kLmhBN = kLmhTileN, kLmhBK = 32;
static_assert(kLmhBM == 128 && kLmhBN == 256, "four 64 x 128 wave tiles");
static_assert(kLmhStepK % kLmhBK == 0, "the hidden size is a multiple of the step");
constexpr int kLmhPad = 8;                      // bf16 elements of padding per LDS row
constexpr int kLmhLd = kLmhBK + kLmhPad;        // LDS row stride (elements)
constexpr int kXcds = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ const uint16_t* lmh_arow(const LmhCfg& g, int64_t r) {
  return r < g.Mp ? g.hp + r * (int64_t)g.H : g.hq + (r - g.Mp) * (int64_t)g.H;
}

// Drafted token of combined row r (target rows b (K + 1) + i, then draft rows
// b K + i); -1 for a bonus row.
__device__ __forceinline__ int lmh_token(const LmhCfg& g, int64_t r) {
  if (r < g.Mp) {
    const int64_t b = r / (g.K + 1);
    const int i = (int)(r - b * (g.K + 1));
    return i < g.K ? g.draft[b * g.K + i] : -1;
  }
  return g.draft[r - g.Mp];
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(2))) void k_lmh_gemm(LmhCfg g) {
  __shared__ __attribute__((aligned(16))) uint16_t s_a[2][kLmhBM * kLmhLd];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][kLmhBN * kLmhLd];
  __shared__ int64_t s_row[kLmhBM];  // combined row index of each tile row (-1 past the end)
  __shared__ int s_tok[kLmhBM];
  __shared__ float s_wm[2][kLmhBM];
  __shared__ float s_ws[2][kLmhBM];
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  // tile order: row tiles of one vocabulary tile consecutive on one XCD
  // (workgroup g runs on XCD g % 8; the grid is a multiple of 8)
  const int64_t per = (int64_t)gridDim.x / kXcds;
  const int64_t lt = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (lt >= (int64_t)g.ntm * g.ntn) return;  // the whole workgroup
  const int64_t tn = lt / g.ntm, tm = lt - tn * g.ntm;
  const int64_t m0 = tm * kLmhBM, n0 = tn * kLmhBN;
  if (t < kLmhBM) {
    const int64_t i = m0 + t;
    int64_t r = -1;
    if (i < g.M) r = g.rows ? (int64_t)g.rows[i] : i;
    s_row[t] = r;
    s_tok[t] = (MODE == kLmhStats && r >= 0) ? lmh_token(g, r) : -1;
  }
  __syncthreads();

  // global -> register staging: thread t always loads the 16-byte column
  // t % VPR of tile rows t / VPR + RPP j (VPR vectors per row of the step,
  // RPP rows per pass of the workgroup), addresses formed once here; rows
  // past the end read a valid row and are zeroed (no branches)
  constexpr int VPR = kLmhBK / 8, RPP = kWG / VPR;
  constexpr int NA = kLmhBM / RPP, NB = kLmhBN / RPP;
  const int kv = t % VPR, r0 = t / VPR;
  const uint16_t* pa[NA];
  const uint16_t* pb[NB];
  uint32_t live = 0;  // bit j: A row j valid; bit NA + j: W row j valid
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int64_t r = s_row[r0 + RPP * j];
    live |= r >= 0 ? 1u << j : 0u;
    pa[j] = lmh_arow(g, r >= 0 ? r : 0) + kv * 8;
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int64_t n = n0 + r0 + RPP * j;
    live |= n < g.V ? 1u << (NA + j) : 0u;
    pb[j] = g.w + (n < g.V ? n : 0) * (int64_t)g.H + kv * 8;
  }
  // two register sets: the loads of step s + 2 are issued while step s is
  // multiplied, and step s + 1 (loaded during step s - 1) is stored to LDS
  uint4 ra0[NA], rb0[NB], ra1[NA], rb1[NB];
  auto load_step = [&](int k0, uint4 (&ra)[NA], uint4 (&rb)[NB]) {
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const uint4 x = *(const uint4*)(pa[j] + k0);
      ra[j] = (live >> j) & 1u ? x : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint4 x = *(const uint4*)(pb[j] + k0);
      rb[j] = (live >> (NA + j)) & 1u ? x : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_step = [&](int buf, const uint4 (&ra)[NA], const uint4 (&rb)[NB]) {
#pragma unroll
    for (int j = 0; j < NA; ++j) *(uint4*)&s_a[buf][(r0 + RPP * j) * kLmhLd + kv * 8] = ra[j];
#pragma unroll
    for (int j = 0; j < NB; ++j) *(uint4*)&s_b[buf][(r0 + RPP * j) * kLmhLd + kv * 8] = rb[j];
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.0f;

  const int steps = g.H / kLmhBK;
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  // operand fragments of one 16-deep slice, read one slice ahead of the MFMAs
  bf16x8_t fa[2][2], fb[2][4];
  auto read_frag = [&](int buf, int kk, int slot) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
      fa[slot][bi] = *(const bf16x8_t*)&s_a[buf][(wm * 64 + bi * 32 + fr) * kLmhLd + kk + fk];
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
      fb[slot][bj] = *(const bf16x8_t*)&s_b[buf][(wn * 128 + bj * 32 + fr) * kLmhLd + kk + fk];
  };
  auto step = [&](int s, uint4 (&la)[NA], uint4 (&lb)[NB], const uint4 (&sa)[NA], const uint4 (&sb)[NB]) {
    const int buf = s & 1;
    if (s + 2 < steps) load_step((s + 2) * kLmhBK, la, lb);
#pragma unroll
    for (int q = 0; q < kLmhBK / 16; ++q) {
      if (q + 1 < kLmhBK / 16) read_frag(buf, (q + 1) * 16, (q + 1) & 1);
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 4; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q & 1][bi], fb[q & 1][bj], acc[bi][bj], 0, 0, 0);
    }
    if (s + 1 < steps) store_step(buf ^ 1, sa, sb);
    __syncthreads();
    if (s + 1 < steps) read_frag(buf ^ 1, 0, 0);
  };
  load_step(0, ra0, rb0);
  store_step(0, ra0, rb0);
  if (steps > 1) load_step(kLmhBK, ra1, rb1);
  __syncthreads();
  read_frag(0, 0, 0);
  for (int s = 0; s < steps; s += 2) {
    step(s, ra0, rb0, ra1, rb1);  // loads step s + 2 into set 0, stores step s + 1 from set 1
    if (s + 1 < steps) step(s + 1, ra1, rb1, ra0, rb0);
  }

  // ---- epilogue. Element e of block (bi, bj) on this lane: tile row
  // wm 64 + bi 32 + 8 (e / 4) + 4 (lane / 32) + e % 4, tile column
  // wn 128 + bj 32 + lane % 32.
  const int half = lane >> 5;
  if constexpr (MODE == kLmhLogits) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * 64 + bi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        const int64_t i = m0 + row;
        if (i >= g.M) continue;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int64_t n = n0 + wn * 128 + bj * 32 + fr;
          if (n < g.V) g.out[i * (int64_t)g.V + n] = acc[bi][bj][e];
        }
      }
  } else {
    const float c32 = g.c32;
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * 64 + bi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        float m = -INFINITY;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int64_t n = n0 + wn * 128 + bj * 32 + fr;
          if (n < g.V) m = fmaxnan(m, acc[bi][bj][e]);
        }
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) m = fmaxnan(m, __shfl_xor(m, o));  // within the 32-lane half
        float sl = 0.0f;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int64_t n = n0 + wn * 128 + bj * 32 + fr;
          if (n < g.V) sl += __builtin_amdgcn_exp2f((acc[bi][bj][e] - m) * c32);
        }
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) sl += __shfl_xor(sl, o);
        if (fr == 0) {
          s_wm[wn][row] = m;
          s_ws[wn][row] = sl;
        }
        // the drafted token's logit, from the lane that holds its column
        const int x = s_tok[row];
        const int64_t rel = (int64_t)x - (n0 + wn * 128);
        if (x >= 0 && rel >= 0 && rel < 128 && (int)(rel & 31) == fr) {
          const int bj = (int)(rel >> 5);
          const float z = bj == 0 ? acc[bi][0][e] : bj == 1 ? acc[bi][1][e] : bj == 2 ? acc[bi][2][e] : acc[bi][3][e];
          g.glog[s_row[row]] = z;
        }
      }
    __syncthreads();
    if (t < kLmhBM) {
      const int64_t r = s_row[t];
      if (r >= 0) {
        const float ma = s_wm[0][t], mb = s_wm[1][t];
        const float m = fmaxnan(ma, mb);
        double s = 0.0;
        if (!is_neg_inf(m)) {
          if (!is_neg_inf(ma)) s += (double)s_ws[0][t] * ::exp2(((double)ma - (double)m) * (double)c32);
          if (!is_neg_inf(mb)) s += (double)s_ws[1][t] * ::exp2(((double)mb - (double)m) * (double)c32);
        }
        if (isnan(m) || isinf(m)) s = NAN;
        g.st[r * (int64_t)g.ntn + tn] = StatRec{m, 0u, s};
      }
    }
  }
}

// Per request (one workgroup): the row normalisers of the K + 1 target and K
// draft rows from the tile records (a wave per row), the accept tests, the
// first rejection n, the accepted tokens, and the state of the final draw.
__global__ __launch_bounds__(kWG) void k_lmh_decide(LmhCfg g, LinCfg c, TreeCfg tc) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int K = g.K;
  __shared__ float s_m[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ int s_bad, s_n;
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int j = wave; j < 2 * K + 1; j += kWaves) {
    const int64_t r = j <= K ? b * (K + 1) + j : g.Mp + b * K + (j - K - 1);
    const StatRec* rec = g.st + r * (int64_t)g.ntn;
    float m = -INFINITY;
    int bad = 0;
    for (int i = lane; i < g.ntn; i += kWave) {
      const StatRec x = rec[i];
      m = fmaxnan(m, x.m);
      bad |= isnan(x.s) ? 1 : 0;
    }
    m = wave_max(m);
    double S = 0.0;
    if (!isnan(m) && !isinf(m))
      for (int i = lane; i < g.ntn; i += kWave) {
        const StatRec x = rec[i];
        if (!is_neg_inf(x.m)) S += x.s * ::exp2(((double)x.m - (double)m) * (double)g.c32);
      }
    S = wave_sum(S);
    bad = wave_or(bad);
    if (lane == 0) {
      s_m[j] = m;
      s_S[j] = S;
      if (bad || isnan(m) || isinf(m) || !(S > 0.0)) atomicOr(&s_bad, 1);
    }
  }
  for (int i = t; i < K; i += kWG) {
    const int x = g.draft[b * K + i];
    if (x < 0 || x >= g.V) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (t != 0) return;
  int n = K;
  if (!s_bad) {
    for (int i = 0; i < K; ++i) {
      const double P = ::exp(((double)g.glog[b * (K + 1) + i] - (double)s_m[i]) * c.invT - ::log(s_S[i]));
      const double Q = ::exp(((double)g.glog[g.Mp + b * K + i] - (double)s_m[K + 1 + i]) * c.invT -
                             ::log(s_S[K + 1 + i]));
      const double u = c.rng.u((uint32_t)b, (uint32_t)i, kDrawAccept);
      if (!(u * Q < P)) {
        n = i;
        break;
      }
    }
  }
  for (int i = 0; i <= K; ++i) c.out_tokens[b * (K + 1) + i] = (!s_bad && i < n) ? g.draft[b * K + i] : -1;
  TreeState st = {};
  if (s_bad) {
    c.out_len[b] = -1;
    st.phase = kTreeDone;
  } else {
    st.phase = kTreeFinal;
    st.row = 0;  // the final rows are row b of the target and draft final-row buffers
    st.urow1 = n + 1;  // the final draw's uniform is that of position n
    st.len = n;
    st.mp = s_m[n];
    st.sp_hat = s_S[n];
    st.mq = n < K ? s_m[K + 1 + n] : 0.0f;
    st.sq_hat = n < K ? s_S[K + 1 + n] : 1.0;
    st.cj = 0.0;
    st.Gj = 1.0;
    st.c_new = n < K ? 1.0 : 0.0;  // residual max(0, P - Q), or the bonus row P
    st.c_old = 0.0;
  }
  tc.ts[b] = st;
  // final rows: target row n, then draft row n (the target row again for a bonus)
  g.fin[b] = (int32_t)(b * (K + 1) + n);
  g.fin[g.B + b] = (int32_t)(n < K ? g.Mp + b * K + n : b * (K + 1) + n);
}

namespace {
// Workgroups of a product: the tile count rounded up to a multiple of the XCD
// count, so that the XCD-major tile order covers every tile once.
inline unsigned lmh_grid(const LmhCfg& g) {
  const int64_t G = (int64_t)g.ntm * g.ntn;
  return (unsigned)((G + kXcds - 1) / kXcds * kXcds);
}
}  // namespace

hipError_t launch_lmh_stats(const LmhCfg& g, hipStream_t s) {
  PSI_LAUNCH(s, k_lmh_gemm<kLmhStats>, dim3(lmh_grid(g)), dim3(kWG), g);
  return hipGetLastError();
}
hipError_t launch_lmh_decide(const LmhCfg& g, const LinCfg& c, const TreeCfg& tc, hipStream_t s) {
  PSI_LAUNCH(s, k_lmh_decide, dim3((unsigned)g.B), dim3(kWG), g, c, tc);
  return hipGetLastError();
}
hipError_t launch_lmh_logits(const LmhCfg& g, hipStream_t s) {
  PSI_LAUNCH(s, k_lmh_gemm<kLmhLogits>, dim3(lmh_grid(g)), dim3(kWG), g);
  return hipGetLastError();
}

}  // namespace psi
