// Linear verification fused with the LM head on gfx950: the target and draft
// logits are products of hidden states with the vocabulary matrix
// ("Uno" research explainer, §3.1: the AR path and the diffusion path share
// the base model and its output head; §3.3: the verifier needs p and q of the
// drafted tokens, then one residual or bonus row), computed tile by tile with
// bf16 matrix cores and reduced in the tile's epilogue. The product is made
// once: its epilogue also stores the fp32 logits, of which the final draw
// reads only target row n and draft row n of each request.
//
// Pipeline on the caller's stream:
//   k_lmh_gemm              every target and draft row against every 256-token
//                           vocabulary tile: per row and 128-token chunk the
//                           maximum and a binary32-grade sum of 2^((z - m) c),
//                           and the logits;
//   k_lmh_decide            per request: row normalisers, the drafted tokens'
//                           logits (dot products), accept tests
//                           u * Q(x) < P(x), first rejection n; the draw state;
//   k_tree_pass, k_tree_pick (tree.hip) the fp64 residual / bonus draw over the
//                           kept logits of the final rows.
//
// GEMM: C[M, V] = A[M, H] * W[V, H]^T, A rows from the target and draft hidden
// states, in 256-row x 256-token tiles. The grid is persistent, one workgroup
// per compute unit: workgroup b runs on XCD b % 8 and walks its share of the
// tiles, which are ordered so that the row tiles of one vocabulary tile run at
// the same time on one XCD and share its L2 copy of the W tile. Four waves,
// one per SIMD, each own a 128 x 128 quarter of the tile as 8 x 8 blocks of
// v_mfma_f32_16x16x32_bf16 (256 accumulator registers); on gfx950 this block
// shape issues at a higher rate than 32 x 32 x 16 (measured: 2.4 against 2.1
// PFLOP/s from registers); a last row tile with fewer rows is split evenly
// between the two wave rows, whose empty blocks are skipped. Operand tiles of
// 32 hidden elements per step go from global memory straight into LDS
// (16-byte direct loads, no register staging) through a four-stage ring that
// runs on across tile boundaries: the loads of the next tile's first steps
// are in flight while a tile's epilogue runs. The loads of step s + 3 are issued during step s, one after each
// group of 8 products, into the slot step s - 1 has left; the fragments of
// step s + 1 are read from LDS during the second half of step s (double
// buffered by step parity). A tile row is 64 bytes in LDS: its four 16-byte
// slots are permuted by an XOR of row bits 2..3, so that the fragment reads
// of each 16-lane group fall in distinct banks. The tile epilogue stores the
// logits and reduces each row over the wave's 128 columns with a butterfly
// across the 16 lanes of a column group (DPP moves within the row of 16
// lanes; every stage halves the rows a lane carries): a record per row and
// wave, so the epilogue has no barrier and the waves of a tile do not wait
// for one another.
// Block operand layout of the instruction (checked on the device against the
// 32 x 32 x 16 form): lane l holds A[l % 16][8 (l / 16) .. +7] and
// W[col l % 16][8 (l / 16) .. +7]; result element i of lane l is
// C[4 (l / 16) + i][l % 16].
#include <type_traits>

#include "rowops.hpp"

namespace psi {

namespace {

constexpr int kLmhBM = kLmhTileM, kLmhBN = kLmhTileN, kLmhBK = 32;
static_assert(kLmhBM == 256 && kLmhBN == 256, "2 x 2 wave quarters of 128 x 128");
static_assert(kLmhChunk * 2 == kLmhBN, "a statistics record per wave column");
static_assert(kLmhStepK == 4 * kLmhBK, "at least 4 steps, an even number (fragment buffers alternate)");
constexpr int kWN = 2;                            // waves side by side along the vocabulary
constexpr int kStages = 4;                        // ring depth (128 KB): loads of step s + 3 spread over step s
constexpr int kRowB = kLmhBK * 2;                 // bytes of a tile row per step
constexpr int kAStage = kLmhBM * kRowB;           // 16 KB
constexpr int kBStage = kLmhBN * kRowB;           // 16 KB
constexpr int kStage = kAStage + kBStage;
constexpr int kLoadB = kWave * 16;                // bytes of one wave-wide direct load
constexpr int kRowsPerLoad = kLoadB / kRowB;      // 16 rows of 4 slots
constexpr int kIA = kAStage / kLoadB / kWaves;    // direct loads per wave per step: A
constexpr int kIB = kBStage / kLoadB / kWaves;    //                               W
constexpr int kLoads = kIA + kIB;
static_assert(kIA * kLoadB * kWaves == kAStage && kIB * kLoadB * kWaves == kBStage, "whole loads");
static_assert(kRowsPerLoad == 16 && kLoads == 8, "a load covers 16 rows of 4 slots; 4 loads per half step");
constexpr int kHalfLoads = kLoads / 2;
constexpr int kXcds = 8;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
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
// The lane index, computed where it is used: an asm statement is neither
// merged with another nor moved, so the value is not kept live (or spilled)
// across the main loop.
__device__ __forceinline__ int lane_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}
__device__ __forceinline__ void lmh_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// A value from another lane of the same row of 16 lanes, by DPP: lane
// l ^ 15 (row mirror), l ^ 7 (half-row mirror), l ^ 3 and l ^ 1 (quad
// permutations 3 2 1 0 and 1 0 3 2).
constexpr int kDppRowMirror = 0x140, kDppHalfMirror = 0x141, kDppXor3 = 0x1B, kDppXor1 = 0xB1;
template <int kCtrl>
__device__ __forceinline__ float dpp_row(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

}  // namespace

__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(1))) void k_lmh_gemm(LmhCfg g) {
  __shared__ __attribute__((aligned(1024))) unsigned char s_mem[kStages * kStage];  // operand ring
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int wm = wave / kWN, wn = wave % kWN;
  // tiles of this workgroup: XCD x (workgroups x, x + 8, ...) takes the
  // consecutive tiles [x per, (x + 1) per); its workgroup j the tiles
  // x per + j + i slots (the grid is a multiple of 8)
  const int G = g.ntm * g.ntn;
  const int per = (G + kXcds - 1) / kXcds;
  const int slots = (int)(gridDim.x / kXcds);
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int lt_lo = xcd * per, lt_hi = (xcd + 1) * per < G ? (xcd + 1) * per : G;
  const int mine = lt_lo + slot < lt_hi ? (lt_hi - lt_lo - slot + slots - 1) / slots : 0;
  if (mine == 0) return;  // the whole workgroup
  const int steps = g.H / kLmhBK;
  // Tile coordinates (row tile tm, vocabulary tile tn = lt / ntm) of this
  // workgroup's tiles, stepped by `slots` tiles without a division.
  struct TilePos {
    int tm, tn;
  };
  const int ntm = g.ntm;
  const int dn = __builtin_amdgcn_readfirstlane(slots / ntm), dm = slots - dn * ntm;
  auto next_tile = [&](TilePos p) {
    p.tm += dm;
    p.tn += dn;
    if (p.tm >= ntm) {
      p.tm -= ntm;
      ++p.tn;
    }
    p.tm = __builtin_amdgcn_readfirstlane(p.tm);
    p.tn = __builtin_amdgcn_readfirstlane(p.tn);
    return p;
  };
  TilePos first;
  first.tn = __builtin_amdgcn_readfirstlane((lt_lo + slot) / ntm);
  first.tm = __builtin_amdgcn_readfirstlane(lt_lo + slot - first.tn * ntm);

  // direct loads: load j of this wave fills 16 tile rows; lane l writes LDS
  // slot l % 4 of row l / 4 of them, i.e. logical slot (l % 4) ^ swz(row),
  // swz(row) = swz(l / 4). Rows past the end read a valid row (their results
  // are never used). src[j]: the next load of j, advanced by a step per load.
  const uint16_t* src[kLoads];  // loads 0 .. kIA - 1: A rows; then W rows
  auto set_src = [&](TilePos p) {
    // the lane terms are taken again here (once per tile), not kept live
    const int lid = lane_here();
    const int lr = lid >> 2;
    const int kvo = ((lid & 3) ^ lmh_swz(lr)) * 8;  // element offset of this lane's slot
    const int64_t m0 = (int64_t)p.tm * kLmhBM, n0 = (int64_t)p.tn * kLmhBN;
#pragma unroll
    for (int j = 0; j < kIA; ++j) {
      const int64_t r = m0 + (wave * kIA + j) * kRowsPerLoad + lr;
      src[j] = lmh_arow(g, r < g.M ? r : 0) + kvo;
    }
#pragma unroll
    for (int j = 0; j < kIB; ++j) {
      const int64_t n = n0 + (int64_t)(wave * kIB + j) * kRowsPerLoad + lr;
      src[kIA + j] = g.w + (n < g.V ? n : (int64_t)g.V - 1) * g.H + kvo;
    }
  };
  auto dst = [&](unsigned char* st, int j) {
    return j < kIA ? st + (wave * kIA + j) * kLoadB : st + kAStage + (wave * kIB + (j - kIA)) * kLoadB;
  };
  auto ring = [&](int i) { return s_mem + i * kStage; };
  // load cursor: step ls of tile lk (at lpos) is loaded next
  int lk = 0, ls = 0;
  TilePos lpos = first;
  auto issue = [&](unsigned char* st, int j) {
    lmh_dma16(src[j], dst(st, j));
    src[j] += kLmhBK;
  };
  auto advance = [&]() {
    if (++ls == steps) {
      ls = 0;
      ++lk;
      if (lk < mine) {
        lpos = next_tile(lpos);
        set_src(lpos);
      }
    }
  };

  // fragment reads: lane l reads row 16 i + l % 16, logical slot l / 16;
  // swz(row) = swz(l % 16)
  const int r16 = lane & 15, q4 = lane >> 4;
  const int fo = r16 * kRowB + ((q4 ^ lmh_swz(r16)) * 16);
  const int ba = wm * 128 * kRowB + fo, bw = kAStage + wn * 128 * kRowB + fo;
  bf16x8_t fa[2][8], fb[2][8];  // by step parity

  // prologue: the first kStages - 1 steps in flight, wait for the first
  set_src(lpos);
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) issue(ring(p), j);
    advance();
  }
  wait_vm<(kStages - 2) * kLoads>();  // steps 1 and 2 may stay in flight
  lmh_barrier();
  int cur = 0;  // ring slot of the current step
  TilePos pos = first;
  for (int k = 0; k < mine; ++k, pos = next_tile(pos)) {
    const int tn = pos.tn;
    const int64_t m0 = (int64_t)pos.tm * kLmhBM, n0 = (int64_t)tn * kLmhBN;
    // Rows of the tile per wave row: 128, or in a last row tile with fewer
    // than 256 rows of the product an even split of its 16-row blocks
    // between the two wave rows (wave row wm takes tile rows [wm rpw,
    // (wm + 1) rpw)); mb of the wave's row blocks hold rows of the product,
    // the others are not multiplied, stored or recorded.
    const int64_t rrem = g.M - m0;
    const int rpw = rrem >= kLmhBM ? 128 : 16 * (int)((rrem + 31) / 32);
    const int64_t mrem = rrem - wm * rpw;
    const int mb = __builtin_amdgcn_readfirstlane(
        mrem <= 0 ? 0 : (int)((mrem + 15) / 16 < rpw / 16 ? (mrem + 15) / 16 : rpw / 16));
    const int64_t mw = m0 + wm * rpw;      // first row of the wave's share
    const int bat = ba - wm * (128 - rpw) * kRowB;  // its fragment reads
    f32x4_t acc[8][8];
#pragma unroll
    for (int bi = 0; bi < 8; ++bi)
#pragma unroll
      for (int bj = 0; bj < 8; ++bj)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[bi][bj][e] = 0.0f;
    {
      const unsigned char* st = ring(cur);
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[0][i] = *(const bf16x8_t*)(st + bat + i * 16 * kRowB);
#pragma unroll
      for (int i = 0; i < 8; ++i) fb[0][i] = *(const bf16x8_t*)(st + bw + i * 16 * kRowB);
    }
    // One step of the tile with its fragments in buffer P. REFILL: the loads
    // of stream step q + 3 are issued; otherwise (the last three steps of the
    // stream) LEFT steps beyond q + 1 are still loading.
    auto step = [&](auto refill_tag, auto par_tag, auto left_tag) {
      constexpr bool kRefill = decltype(refill_tag)::value;
      constexpr int P = decltype(par_tag)::value;
      constexpr int kLeft = decltype(left_tag)::value;
      const int nxt = cur == kStages - 1 ? 0 : cur + 1;
      unsigned char* fill = ring(cur == 0 ? kStages - 1 : cur - 1);
      // first half: row blocks 0..3, a load after each group of 8 products
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        if (bi < mb) {
#pragma unroll
          for (int bj = 0; bj < 8; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[P][bi], fb[P][bj], acc[bi][bj], 0, 0, 0);
        }
        if (kRefill) issue(fill, bi);
      }
      // step q + 1 is in (and visible after the barrier); the later steps'
      // loads may stay in flight: steps q + 2 and half of q + 3 while
      // refilling, else what the stream has left
      if (kRefill) wait_vm<kLoads + kHalfLoads>();
      else wait_vm<kLeft * kLoads>();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of this slot are done
      lmh_barrier();
      // second half: row blocks 4..7, the next step's fragments read into
      // buffer 1 - P (after a tile's last step they are read and not used)
      const unsigned char* sn = ring(nxt);
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        fa[1 - P][2 * gq] = *(const bf16x8_t*)(sn + bat + (2 * gq) * 16 * kRowB);
        fa[1 - P][2 * gq + 1] = *(const bf16x8_t*)(sn + bat + (2 * gq + 1) * 16 * kRowB);
        fb[1 - P][2 * gq] = *(const bf16x8_t*)(sn + bw + (2 * gq) * 16 * kRowB);
        fb[1 - P][2 * gq + 1] = *(const bf16x8_t*)(sn + bw + (2 * gq + 1) * 16 * kRowB);
        const int bi = 4 + gq;
        if (bi < mb) {
#pragma unroll
          for (int bj = 0; bj < 8; ++bj)
            acc[bi][bj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[P][bi], fb[P][bj], acc[bi][bj], 0, 0, 0);
        }
        if (kRefill) issue(fill, kHalfLoads + gq);
      }
      if (kRefill) advance();
      cur = nxt;
    };
    using R = std::true_type;
    using N = std::false_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using L0 = std::integral_constant<int, 0>;
    using L1 = std::integral_constant<int, 1>;
    if (k + 1 < mine) {
      // the stream goes on into the next tile: every step loads (steps >= 4)
      for (int s = 0; s < steps; s += 2) {
        step(R{}, P0{}, L0{});
        step(R{}, P1{}, L0{});
      }
    } else {
      // the stream's last tile: its last three steps load nothing
      int s = 0;
      for (; s + 4 < steps; s += 2) {
        step(R{}, P0{}, L0{});
        step(R{}, P1{}, L0{});
      }
      step(R{}, P0{}, L0{});
      step(N{}, P1{}, L1{});
      step(N{}, P0{}, L0{});
      step(N{}, P1{}, L0{});
    }

    // ---- epilogue of the tile (the next tile's first steps are loading).
    // Element e of block (bi, bj) on this lane: tile row wm rpw + bi 16 +
    // 4 (lane / 16) + e, tile column wn 128 + bj 16 + lane % 16. The lane
    // index is taken again here so that the epilogue's address arithmetic is
    // not kept live across the main loop. No barrier: each wave writes the
    // records of its own 128 columns.
    const int lid = lane_here();
    const int er = lid & 15, eq = lid >> 4;
    const int64_t c0 = n0 + wn * 128;  // first column of the wave's chunk
    const bool fullc = c0 + 128 <= g.V;
    const float c32 = g.c32;
    // Row block by row block: the block's logits are stored (kept for the
    // final draw; a block whose 16 rows and 128 columns are all in the product
    // without per-element tests, the columns of block bj at immediate
    // offsets), then, from the same values, per row of the wave's chunk (item
    // it = 4 bi + e of this lane: row 16 bi + 4 (lane / 16) + e of the wave's
    // share) the maximum and the sum of 2^((z - m) c) over this lane's 8
    // columns; columns past the vocabulary (a last tile) are left out. Then
    // the items are reduced over the 16 lanes of the column group by a
    // butterfly that halves them at every stage (with the partner lane ^ 15,
    // ^ 7, ^ 3, ^ 1, moved by DPP within the row of 16 lanes: a lane keeps the
    // items whose index bit 3, 2, 1, 0 matches that bit of its lane and sends
    // the others), so that lane l ends with items 2 (l % 16) and
    // 2 (l % 16) + 1.
    float im[32], is[32];
#pragma unroll
    for (int bi = 0; bi < 8; ++bi) {
      const int64_t rb = mw + bi * 16;
      if (bi >= mb) {  // not the wave's rows of the product: an empty part
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          im[4 * bi + e] = -INFINITY;
          is[4 * bi + e] = 0.0f;
        }
        continue;
      }
      if (g.all) {
        if (fullc && rb + 16 <= g.M) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* const p = g.all + (rb + 4 * eq + e) * (int64_t)g.V + c0 + er;
#pragma unroll
            for (int bj = 0; bj < 8; ++bj) p[bj * 16] = acc[bi][bj][e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t i = rb + 4 * eq + e;
            if (i >= g.M) continue;
#pragma unroll
            for (int bj = 0; bj < 8; ++bj) {
              const int64_t n = c0 + bj * 16 + er;
              if (n < g.V) g.all[i * (int64_t)g.V + n] = acc[bi][bj][e];
            }
          }
        }
      }
      auto item = [&](auto full_tag, int e) {
        constexpr bool kFull = decltype(full_tag)::value;
        float x[8];
#pragma unroll
        for (int bj = 0; bj < 8; ++bj)
          x[bj] = kFull || c0 + bj * 16 + er < g.V ? acc[bi][bj][e] : -INFINITY;
        float m = x[0];
#pragma unroll
        for (int bj = 1; bj < 8; ++bj) m = fmaxnan(m, x[bj]);
        const float mo = is_neg_inf(m) ? 0.0f : m;  // an empty part sums to 0
        float sl = 0.0f;
#pragma unroll
        for (int bj = 0; bj < 8; ++bj) sl += __builtin_amdgcn_exp2f((x[bj] - mo) * c32);
        im[4 * bi + e] = m;
        is[4 * bi + e] = sl;
      };
      if (fullc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) item(std::true_type{}, e);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) item(std::false_type{}, e);
      }
    }
    // two parts (ma, sa), (mb, sb) as one: the part with the smaller maximum
    // is scaled by 2^((min - max) c), the other is exact
    auto merge = [&](float ma, float sa, float mb, float sb, float& m, float& sm) {
      m = fmaxnan(ma, mb);
      const bool ab = ma >= mb;
      const float big = ab ? sa : sb, small = ab ? sb : sa;
      const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(ma - mb) * c32);
      sm = is_neg_inf(m) ? 0.0f : big + small * e;
    };
    auto stage = [&](auto ctrl_tag, int bit, int n) {
      constexpr int kCtrl = decltype(ctrl_tag)::value;
      const bool up = (er & bit) != 0;
#pragma unroll
      for (int i = 0; i < n; ++i) {
        const float mk = up ? im[i + n] : im[i], sk = up ? is[i + n] : is[i];
        const float mo = up ? im[i] : im[i + n], so = up ? is[i] : is[i + n];
        merge(mk, sk, dpp_row<kCtrl>(mo), dpp_row<kCtrl>(so), im[i], is[i]);
      }
    };
    stage(std::integral_constant<int, kDppRowMirror>{}, 8, 16);
    stage(std::integral_constant<int, kDppHalfMirror>{}, 4, 8);
    stage(std::integral_constant<int, kDppXor3>{}, 2, 4);
    stage(std::integral_constant<int, kDppXor1>{}, 1, 2);
    // the records of the wave's chunk: an overflowed or NaN maximum marks the
    // record invalid; an empty chunk (past the vocabulary) has maximum -inf
    // and sum 0
    const int nch = g.ntn * (kLmhBN / kLmhChunk);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int it = 2 * er + i, bi = it >> 2, e = it & 3;
      const int64_t r = mw + bi * 16 + 4 * eq + e;
      if (bi < mb && r < g.M) {
        const float m = im[i];
        const double s = (isnan(m) || m == INFINITY) ? (double)NAN : (double)is[i];
        g.st[r * nch + 2 * tn + wn] = StatRec{m, 0u, s};
      }
    }
  }
}

// Per request (one workgroup): the row normalisers of the K + 1 target and K
// draft rows from the chunk records (a half-wave per row: 2K + 1 <= 32 rows
// for K <= 15, else a second pass), the logits of the drafted tokens as dot
// products of the hidden states with the tokens' rows of W (fp32 products,
// summed per lane in order and across lanes in fp64), the accept tests (a lane
// per position, the first rejection n by a ballot), the accepted tokens, and
// the state of the final draw.
constexpr int kDecideWG = 1024;
__global__ __launch_bounds__(kDecideWG) void k_lmh_decide(LmhCfg g, LinCfg c, TreeCfg tc) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x, lane = t & (kWave - 1);
  const int hl = t & 31, hw = t >> 5;  // lane in the half-wave, half-wave
  const int K = g.K;
  const int nch = g.ntn * (kLmhTileN / kLmhChunk);  // records per row
  __shared__ float s_m[2 * kMaxK + 1];
  __shared__ double s_S[2 * kMaxK + 1];
  __shared__ float s_z[2 * kMaxK + 1];  // logit of the row's drafted token
  __shared__ int s_bad;
  if (t == 0) s_bad = 0;
  __syncthreads();
  // half-wave sums and maxima (xor distances below 32 stay in the half-wave)
  auto hsum = [](double v) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
  };
  auto hmax = [](float v) {
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v = fmaxnan(v, __shfl_xor(v, o));
    return v;
  };
  for (int j = hw; j < 2 * K + 1; j += kDecideWG / 32) {
    const int64_t r = j <= K ? b * (K + 1) + j : g.Mp + b * K + (j - K - 1);
    const StatRec* rec = g.st + r * (int64_t)nch;
    // loads are issued in batches before their values are used, so that a
    // row costs a few memory latencies rather than one per iteration
    constexpr int kDecB = 8;
    float z = NAN;
    if (j != K) {  // row K is the bonus row: no drafted token
      const int x = g.draft[b * K + (j < K ? j : j - K - 1)];
      if (x >= 0 && x < g.V) {
        const uint4* hv = (const uint4*)lmh_arow(g, r);
        const uint4* wv = (const uint4*)(g.w + (int64_t)x * g.H);
        float a = 0.0f;
        const int nv = g.H / 8;
        for (int v0 = hl; v0 < nv; v0 += 32 * kDecB) {
          uint4 hh[kDecB], ww[kDecB];
#pragma unroll
          for (int u = 0; u < kDecB; ++u) {
            const int v = v0 + 32 * u;
            hh[u] = v < nv ? hv[v] : make_uint4(0, 0, 0, 0);
            ww[u] = v < nv ? wv[v] : make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < kDecB; ++u) {
            if (v0 + 32 * u >= nv) break;
            float h8[8], w8[8];
            Elem<kBF16>::unpack(hh[u], h8);
            Elem<kBF16>::unpack(ww[u], w8);
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_fmaf(h8[e], w8[e], a);
          }
        }
        z = (float)hsum((double)a);
      }
    }
    // one pass over the row's records: a running maximum ml per lane and the
    // sum Sl of 2^((z - ml) c), rescaled in fp64 when ml rises
    constexpr int kRecB = 16;
    const double c32 = (double)g.c32;
    float ml = -INFINITY;
    double Sl = 0.0;
    int bad = 0;
    for (int i0 = hl; i0 < nch; i0 += 32 * kRecB) {
      float mm[kRecB];
      double ss[kRecB];
#pragma unroll
      for (int u = 0; u < kRecB; ++u) {
        const int i = i0 + 32 * u;
        mm[u] = i < nch ? rec[i].m : -INFINITY;
        ss[u] = i < nch ? rec[i].s : 0.0;
      }
#pragma unroll
      for (int u = 0; u < kRecB; ++u) {
        bad |= (isnan(ss[u]) || isnan(mm[u])) ? 1 : 0;
        if (is_neg_inf(mm[u]) || isnan(mm[u])) continue;
        if (is_neg_inf(ml)) {
          ml = mm[u];
          Sl = ss[u];
        } else if (mm[u] > ml) {
          Sl = Sl * exp2_fast(((double)ml - (double)mm[u]) * c32) + ss[u];
          ml = mm[u];
        } else {
          Sl += ss[u] * exp2_fast(((double)mm[u] - (double)ml) * c32);
        }
      }
    }
    const float m = hmax(ml);
    double S = 0.0;
    if (!isnan(m) && !isinf(m) && !is_neg_inf(ml)) S = Sl * exp2_fast(((double)ml - (double)m) * c32);
    S = hsum(S);
    bad = (int)hsum((double)bad);
    if (hl == 0) {
      s_m[j] = m;
      s_S[j] = S;
      s_z[j] = z;
      if (bad || isnan(m) || isinf(m) || !(S > 0.0)) atomicOr(&s_bad, 1);
    }
  }
  for (int i = t; i < K; i += kDecideWG) {
    const int x = g.draft[b * K + i];
    if (x < 0 || x >= g.V) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (t >= kWave) return;
  // accept tests u Q(x) < P(x), a lane per position (positions K .. are
  // never rejected); n = the first rejection
  const int nbad = s_bad;
  int n = K;
  if (!nbad) {
    for (int i0 = 0; i0 < K; i0 += kWave) {
      const int i = i0 + lane;
      bool rej = false;
      if (i < K) {
        const double P = ::exp(((double)s_z[i] - (double)s_m[i]) * c.invT - ::log(s_S[i]));
        const double Q = ::exp(((double)s_z[K + 1 + i] - (double)s_m[K + 1 + i]) * c.invT -
                               ::log(s_S[K + 1 + i]));
        const double u = c.rng.u((uint32_t)b, (uint32_t)i, kDrawAccept);
        rej = !(u * Q < P);
      }
      const unsigned long long mask = __ballot(rej);
      if (mask) {
        n = i0 + __builtin_ctzll(mask);
        break;
      }
    }
  }
  for (int i = lane; i <= K; i += kWave)
    c.out_tokens[b * (K + 1) + i] = (!nbad && i < n) ? g.draft[b * K + i] : -1;
  if (lane != 0) return;
  TreeState st = {};
  if (nbad) {
    c.out_len[b] = -1;
    st.phase = kTreeDone;
  } else {
    st.phase = kTreeFinal;
    st.row = n;  // target row n and draft row n of the request, in the kept logits
    st.urow1 = 0;  // the final draw's uniform is that of position n
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
}

namespace {
// Workgroups of the persistent product: one per compute unit, a multiple of
// the XCD count (the device's compute units, read once per device).
hipError_t lmh_grid(unsigned* grid) {
  static int cus[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (cus[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus[dev] = n / kXcds * kXcds > 0 ? n / kXcds * kXcds : kXcds;
  }
  *grid = (unsigned)cus[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_lmh_stats(const LmhCfg& g, hipStream_t s) {
  unsigned grid = 0;
  if (hipError_t e = lmh_grid(&grid)) return e;
  PSI_LAUNCH(s, k_lmh_gemm, dim3(grid), dim3(kWG), g);
  return hipGetLastError();
}
hipError_t launch_lmh_decide(const LmhCfg& g, const LinCfg& c, const TreeCfg& tc, hipStream_t s) {
  PSI_LAUNCH(s, k_lmh_decide, dim3((unsigned)g.B), dim3(kDecideWG), g, c, tc);
  return hipGetLastError();
}

}  // namespace psi
