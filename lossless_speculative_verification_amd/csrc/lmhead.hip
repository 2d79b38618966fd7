// Linear verification fused with the LM head on gfx950: the target and draft
// logits are products of hidden states with the vocabulary matrix
// ("Uno" research explainer, §3.1: the AR path and the diffusion path share
// the base model and its output head; §3.3: the verifier needs p and q of the
// drafted tokens, then one residual or bonus row), computed tile by tile with
// bf16 matrix cores and reduced in the tile's epilogue, so that the logits of
// the K + 1 target and K draft rows never reach HBM.
//
// Pipeline on the caller's stream:
//   k_lmh_gemm<kLmhStats>   every target and draft row against every 512-token
//                           vocabulary tile: per (row, tile) the maximum and a
//                           binary32-grade sum of 2^((z - m) c);
//   k_lmh_decide            per request: row normalisers, the drafted tokens'
//                           logits (dot products), accept tests
//                           u * Q(x) < P(x), first rejection n; the draw state;
//   k_lmh_gemm<kLmhLogits>  the final rows only (target row n and draft row n,
//                           or the bonus row): fp32 logits;
//   k_tree_pass, k_tree_pick (tree.hip) the fp64 residual / bonus draw over them.
//
// GEMM: C[M, V] = A[M, H] * W[V, H]^T, A rows from the target and draft hidden
// states. A workgroup computes a 128-row x 512-token tile with four waves, each
// owning 128 tokens of the tile (all 128 rows): 4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, 256 accumulator registers, one wave per SIMD.
// Operand tiles of 32 hidden elements per step go from global memory straight
// into LDS (16-byte direct loads, no register staging) through a four-stage
// ring: the loads of step s + 3 are issued during step s, one between each
// pair of its products, into the slot step s - 1 has left. A tile row is 64 bytes in
// LDS: its four 16-byte slots are permuted by an XOR of row bits 2..3, so that
// the 16-byte fragment reads of a wave do not conflict in the LDS banks. The
// tile epilogue reduces each row over the wave's 128 columns with a butterfly
// across the half-wave (every stage halves the rows a lane carries), then
// over the four waves through LDS.
// Block operand layout of the instruction (checked on the device): lane l
// holds A[l % 32][8 (l / 32) .. +7] and W[col l % 32][8 (l / 32) .. +7]; result
// element i of lane l is C[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
// Tiles are ordered so that the row tiles of one vocabulary tile run one after
// another on the same XCD and share its L2 copy of the W tile.
#include <type_traits>

#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kLmhBM = kLmhTileM, kLmhBN = kLmhTileN, kLmhBK = 32;
static_assert(kLmhBM == 128 && kLmhBN == 512, "four 128 x 128 wave tiles side by side");
static_assert(kLmhStepK % kLmhBK == 0, "the hidden size is a multiple of the step");
constexpr int kStages = 4;                        // ring depth (160 KB): loads of step s + 3 spread over step s
constexpr int kRowB = kLmhBK * 2;                 // bytes of a tile row per step
constexpr int kAStage = kLmhBM * kRowB;           // 8 KB
constexpr int kBStage = kLmhBN * kRowB;           // 32 KB
constexpr int kStage = kAStage + kBStage;
constexpr int kLoadB = kWave * 16;                // bytes of one wave-wide direct load
constexpr int kRowsPerLoad = kLoadB / kRowB;      // 16 rows of 4 slots
constexpr int kIA = kAStage / kLoadB / kWaves;    // direct loads per wave per step: A
constexpr int kIB = kBStage / kLoadB / kWaves;    //                               W
constexpr int kLoads = kIA + kIB;
static_assert(kIA * kLoadB * kWaves == kAStage && kIB * kLoadB * kWaves == kBStage, "whole loads");
static_assert(kRowsPerLoad == 16 && kLoads == 10, "a load covers 16 rows of 4 slots; 5 loads per half step");
constexpr int kHalfLoads = kLoads / 2;
constexpr int kXcds = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Slot permutation of tile row r (its 4 16-byte slots, by bits 2..3 of r: a
// function of r % 16, the same for every load of a lane). With it the 16-byte
// fragment reads of a wave, 32 rows at one logical slot, are free of LDS bank
// conflicts (measured).
__device__ __forceinline__ int lmh_swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ const uint16_t* lmh_arow(const LmhCfg& g, int64_t r) {
  return r < g.Mp ? g.hp + r * (int64_t)g.H : g.hq + (r - g.Mp) * (int64_t)g.H;
}

// One wave-wide direct load: 16 bytes per lane from gptr into LDS at
// lds + 16 * lane. Written as an asm statement so that the compiler does not
// add a full vmcnt wait before every LDS read of the ring (it cannot tell the
// stages apart); the ring's waits are explicit (wait_vm) and the statement
// has no register output. The LDS base goes through M0, which the compiler
// does not otherwise use in these kernels (M0 is a reserved register and
// cannot be listed as clobbered).
__device__ __forceinline__ void lmh_dma16(const uint16_t* gptr, const unsigned char* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_void_t*)lds;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(la)
               : "memory");
}
// Waits until at most N direct loads of this wave are outstanding (vmcnt; the
// other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt field (bits 3:0 and 15:14)");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Workgroup barrier with no memory fence: the direct loads are waited for
// explicitly; the asm statements keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void lmh_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int MODE>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(1))) void k_lmh_gemm(LmhCfg g) {
  // ring of operand tiles; after the main loop its start holds the
  // epilogue's per-wave row maxima and sums
  __shared__ __attribute__((aligned(1024))) unsigned char s_mem[kStages * kStage];
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  // tile order: row tiles of one vocabulary tile consecutive on one XCD
  // (workgroup g runs on XCD g % 8; the grid is a multiple of 8)
  const int64_t per = (int64_t)gridDim.x / kXcds;
  const int64_t lt = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (lt >= (int64_t)g.ntm * g.ntn) return;  // the whole workgroup
  const int64_t tn = lt / g.ntm, tm = lt - tn * g.ntm;
  const int64_t m0 = tm * kLmhBM, n0 = tn * kLmhBN;
  auto combined_row = [&](int row) -> int64_t {  // combined row index of tile row `row` (-1 past the end)
    const int64_t i = m0 + row;
    if (i >= g.M) return -1;
    return g.rows ? (int64_t)g.rows[i] : i;
  };

  // direct loads: load j of this wave fills 16 tile rows; lane l writes LDS
  // slot l % 4 of row l / 4 of them, i.e. logical slot (l % 4) ^ swz(row),
  // swz(row) = swz(l / 4). Rows past the end read a valid row (their results
  // are never used).
  const int lr = lane >> 2;
  const int kvo = ((lane & 3) ^ lmh_swz(lr)) * 8;  // element offset of this lane's slot
  const uint16_t* src[kLoads];                     // loads 0 .. kIA - 1: A rows; then W rows
#pragma unroll
  for (int j = 0; j < kIA; ++j) {
    const int64_t r = combined_row((wave * kIA + j) * kRowsPerLoad + lr);
    src[j] = lmh_arow(g, r >= 0 ? r : 0) + kvo;
  }
#pragma unroll
  for (int j = 0; j < kIB; ++j) {
    const int64_t n = n0 + (int64_t)(wave * kIB + j) * kRowsPerLoad + lr;
    src[kIA + j] = g.w + (n < g.V ? n : (int64_t)g.V - 1) * g.H + kvo;
  }
  auto dst = [&](unsigned char* st, int j) {
    return j < kIA ? st + (wave * kIA + j) * kLoadB : st + kAStage + (wave * kIB + (j - kIA)) * kLoadB;
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int bj = 0; bj < 4; ++bj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.0f;

  // fragment reads: lane l reads row (block + l % 32), logical slot
  // 2 q + l / 32 of slice q; swz(row) = swz(l % 16)
  const int fr = lane & 31, half = lane >> 5;
  const int frow = fr * kRowB;
  const int fsw = lmh_swz(fr);
  const int bw = kAStage + wave * 128 * kRowB;  // this wave's W rows in a stage
  bf16x8_t fa[2][4], fb[2][4];
  auto read_frag = [&](const unsigned char* st, int q, int slot) {
    const int fo = frow + (((2 * q + half) ^ fsw) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[slot][i] = *(const bf16x8_t*)(st + i * 32 * kRowB + fo);
#pragma unroll
    for (int i = 0; i < 4; ++i) fb[slot][i] = *(const bf16x8_t*)(st + bw + i * 32 * kRowB + fo);
  };
  // row blocks of 32 that hold rows of the product (a last row tile may be
  // partial: its empty blocks are not multiplied)
  const int mblocks = (int)((g.M - m0 + 31) / 32 < 4 ? (g.M - m0 + 31) / 32 : 4);
  auto mfma1 = [&](int slot, int i) {
    if ((i >> 2) < mblocks)
      acc[i >> 2][i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i >> 2], fb[slot][i & 3],
                                                                   acc[i >> 2][i & 3], 0, 0, 0);
  };

  const int steps = g.H / kLmhBK;
  auto ring = [&](int i) { return s_mem + i * kStage; };
  // Waits until at most n direct loads of this wave are outstanding.
  auto wait_loads = [&](int n) {
    if (n >= 3 * kHalfLoads) wait_vm<3 * kHalfLoads>();
    else if (n >= 2 * kHalfLoads) wait_vm<2 * kHalfLoads>();
    else if (n >= kHalfLoads) wait_vm<kHalfLoads>();
    else wait_vm<0>();
  };
  // prologue: steps 0 .. kStages - 2 in flight, wait for step 0
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < steps)
#pragma unroll
      for (int j = 0; j < kLoads; ++j) lmh_dma16(src[j] + p * kLmhBK, dst(ring(p), j));
  wait_loads(((steps > 1) + (steps > 2)) * kLoads);
  lmh_barrier();
  read_frag(ring(0), 0, 0);
  int cur = 0;  // ring slot of step s
  // One step; REFILL: the loads of step s + 3 are issued (every step but the
  // last three, which run a copy of the body without them).
  auto step = [&](int s, auto refill_tag) {
    constexpr bool kRefill = decltype(refill_tag)::value;
    unsigned char* st = ring(cur);
    const int nxt = cur == kStages - 1 ? 0 : cur + 1;
    // The loads of step s + 3 go to the slot of step s - 1, free since the
    // middle of step s - 1; they are spread over the products of step s, one
    // between each pair (the load unit takes them as fast as they come).
    unsigned char* fill = ring(cur == 0 ? kStages - 1 : cur - 1);
    const int k0 = (s + 3) * kLmhBK;
    // slice 0 of step s is in fa[0] / fb[0]; slice 1 is read after the first
    // product (so that the wait for slice 0 does not include its reads)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mfma1(0, i);
      if (i == 0) {
        __builtin_amdgcn_sched_barrier(0);
        read_frag(st, 1, 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kRefill && (i & 1) && i / 2 < kHalfLoads) lmh_dma16(src[i / 2] + k0, dst(fill, i / 2));
    }
    // step s + 1 is in; the loads of step s + 2 and the first half of step
    // s + 3 may stay in flight
    if (kRefill) wait_vm<kLoads + kHalfLoads>();
    else wait_loads(s + 2 < steps ? kLoads : 0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of this stage are done
    lmh_barrier();
    if (s + 1 < steps) read_frag(ring(nxt), 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mfma1(1, i);
      if (kRefill && (i & 1) && i / 2 < kHalfLoads)
        lmh_dma16(src[kHalfLoads + i / 2] + k0, dst(fill, kHalfLoads + i / 2));
    }
    cur = nxt;
  };
  int s = 0;
  for (; s + 3 < steps; ++s) step(s, std::true_type{});
  for (; s < steps; ++s) step(s, std::false_type{});

  // epilogue tables at the start of the ring (no longer read: every wave
  // passed the last step's barrier after its last read)
  float(*s_wm)[kLmhBM] = (float(*)[kLmhBM])s_mem;
  float(*s_ws)[kLmhBM] = (float(*)[kLmhBM])(s_mem + kWaves * kLmhBM * sizeof(float));

  // ---- epilogue. Element e of block (bi, bj) on this lane: tile row
  // bi 32 + 8 (e / 4) + 4 (lane / 32) + e % 4, tile column
  // wave 128 + bj 32 + lane % 32.
  if constexpr (MODE == kLmhLogits) {
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = bi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
        const int64_t i = m0 + row;
        if (i >= g.M) continue;
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
          const int64_t n = n0 + wave * 128 + bj * 32 + fr;
          if (n < g.V) g.out[i * (int64_t)g.V + n] = acc[bi][bj][e];
        }
      }
  } else {
    const float c32 = g.c32;
    // Per row of the tile (item it = 16 bi + e of this lane: row
    // 32 bi + 8 (e / 4) + 4 (lane / 32) + e % 4): the maximum and the sum of
    // 2^((z - m) c) over this lane's 4 columns, then over the 32 lanes of the
    // half-wave by a butterfly that halves the items at every stage (at offset
    // o a lane keeps the items whose index bit matches its lane bit and sends
    // the others), so that lane l ends with items 2 (l % 32) and 2 (l % 32) + 1.
    bool vcol[4];  // this lane's column of block bj is inside the vocabulary
#pragma unroll
    for (int bj = 0; bj < 4; ++bj) vcol[bj] = n0 + wave * 128 + bj * 32 + fr < g.V;
    float im[64], is[64];
#pragma unroll
    for (int it = 0; it < 64; ++it) {
      const int bi = it >> 4, e = it & 15;
      float m = -INFINITY;
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) m = vcol[bj] ? fmaxnan(m, acc[bi][bj][e]) : m;
      const float mo = is_neg_inf(m) ? 0.0f : m;  // an empty part sums to 0
      float sl = 0.0f;
#pragma unroll
      for (int bj = 0; bj < 4; ++bj) sl += vcol[bj] ? __builtin_amdgcn_exp2f((acc[bi][bj][e] - mo) * c32) : 0.0f;
      im[it] = m;
      is[it] = sl;
    }
    auto part = [&](float mx, float sx, float m) {  // sx 2^((mx - m) c), 0 for an empty part
      return is_neg_inf(mx) ? 0.0f : sx * __builtin_amdgcn_exp2f((mx - m) * c32);
    };
#pragma unroll
    for (int stg = 0; stg < 5; ++stg) {
      const int off = 16 >> stg, n = 32 >> stg;
      const bool up = (fr & off) != 0;
#pragma unroll
      for (int i = 0; i < n; ++i) {
        const float mk = up ? im[i + n] : im[i], sk = up ? is[i + n] : is[i];
        const float mo = up ? im[i] : im[i + n], so = up ? is[i] : is[i + n];
        const float mr = __shfl_xor(mo, off), sr = __shfl_xor(so, off);
        const float m = fmaxnan(mk, mr);
        im[i] = m;
        is[i] = is_neg_inf(m) ? 0.0f : part(mk, sk, m) + part(mr, sr, m);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = 2 * fr + i, bi = it >> 4, e = it & 15;
      const int row = bi * 32 + 8 * (e >> 2) + 4 * half + (e & 3);
      s_wm[wave][row] = im[i];
      s_ws[wave][row] = is[i];
    }
    __syncthreads();
    if (t < kLmhBM) {
      const int64_t r = combined_row(t);
      if (r >= 0) {
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) m = fmaxnan(m, s_wm[w][t]);
        double s = 0.0;
        if (!is_neg_inf(m)) {
#pragma unroll
          for (int w = 0; w < kWaves; ++w) {
            const float mw = s_wm[w][t];
            if (!is_neg_inf(mw)) s += (double)s_ws[w][t] * ::exp2(((double)mw - (double)m) * (double)c32);
          }
        }
        if (isnan(m) || isinf(m)) s = NAN;
        g.st[r * (int64_t)g.ntn + tn] = StatRec{m, 0u, s};
      }
    }
  }
}

// Per request (one workgroup): the row normalisers of the K + 1 target and K
// draft rows from the tile records (a wave per row), the logits of the drafted
// tokens as dot products of the hidden states with the tokens' rows of W (fp32
// products, summed per lane in order and across lanes in fp64), the accept
// tests, the first rejection n, the accepted tokens, and the state of the
// final draw.
constexpr int kDecideWG = 1024;  // 16 waves: about one row of the request per wave
__global__ __launch_bounds__(kDecideWG) void k_lmh_decide(LmhCfg g, LinCfg c, TreeCfg tc) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int K = g.K;
  __shared__ float s_m[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ float s_z[2 * kMaxK + 1];  // logit of the row's drafted token
  __shared__ int s_bad;
  if (t == 0) s_bad = 0;
  __syncthreads();
  for (int j = wave; j < 2 * K + 1; j += kDecideWG / kWave) {
    const int64_t r = j <= K ? b * (K + 1) + j : g.Mp + b * K + (j - K - 1);
    if (j != K) {  // row K is the bonus row: no drafted token
      const int x = g.draft[b * K + (j < K ? j : j - K - 1)];
      float z = NAN;
      if (x >= 0 && x < g.V) {
        const uint4* hv = (const uint4*)lmh_arow(g, r);
        const uint4* wv = (const uint4*)(g.w + (int64_t)x * g.H);
        float a = 0.0f;
        for (int v = lane; v < g.H / 8; v += kWave) {
          float h8[8], w8[8];
          Elem<kBF16>::unpack(hv[v], h8);
          Elem<kBF16>::unpack(wv[v], w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) a = __builtin_fmaf(h8[e], w8[e], a);
        }
        z = (float)wave_sum((double)a);
      }
      if (lane == 0) s_z[j] = z;
    }
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
  for (int i = t; i < K; i += kDecideWG) {
    const int x = g.draft[b * K + i];
    if (x < 0 || x >= g.V) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (t != 0) return;
  int n = K;
  if (!s_bad) {
    for (int i = 0; i < K; ++i) {
      const double P = ::exp(((double)s_z[i] - (double)s_m[i]) * c.invT - ::log(s_S[i]));
      const double Q = ::exp(((double)s_z[K + 1 + i] - (double)s_m[K + 1 + i]) * c.invT -
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
  PSI_LAUNCH(s, k_lmh_decide, dim3((unsigned)g.B), dim3(kDecideWG), g, c, tc);
  return hipGetLastError();
}
hipError_t launch_lmh_logits(const LmhCfg& g, hipStream_t s) {
  PSI_LAUNCH(s, k_lmh_gemm<kLmhLogits>, dim3(lmh_grid(g)), dim3(kWG), g);
  return hipGetLastError();
}

}  // namespace psi
