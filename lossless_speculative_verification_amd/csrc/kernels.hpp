// Internal interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "psispec.h"

namespace psi {

// Benchmark timing hook (psispec_set_timing_events, capi.hip): timing_begin
// starts an entry point's sequence; while armed, timing_pair hands out the
// next two events, which the launch of the next kernel records as that
// kernel's start and end (its dispatch's own timestamps).
void timing_begin(hipStream_t s);
bool timing_pair(hipEvent_t* start, hipEvent_t* stop);

// Every kernel launch of the library goes through PSI_LAUNCH (or
// PSI_LAUNCH_LDS with dynamic LDS bytes).
#define PSI_LAUNCH_LDS(s, kernel, grid, block, lds, ...)                                  \
  do {                                                                                     \
    hipEvent_t psi_ev0_, psi_ev1_;                                                         \
    if (::psi::timing_pair(&psi_ev0_, &psi_ev1_))                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, lds, s, psi_ev0_, psi_ev1_, 0u, __VA_ARGS__); \
    else                                                                                   \
      hipLaunchKernelGGL(kernel, grid, block, lds, s, __VA_ARGS__);                        \
  } while (0)
#define PSI_LAUNCH(s, kernel, grid, block, ...) PSI_LAUNCH_LDS(s, kernel, grid, block, 0, __VA_ARGS__)
// Calls the instance fn<dtype, aligned> of a launcher template.
#define PSI_DISPATCH(fn, dtype, aligned, ...)                                                    \
  ((dtype) == kBF16 ? ((aligned) ? fn<kBF16, true>(__VA_ARGS__) : fn<kBF16, false>(__VA_ARGS__)) \
                    : ((aligned) ? fn<kF32, true>(__VA_ARGS__) : fn<kF32, false>(__VA_ARGS__)))

constexpr int kMaxK = 64;
constexpr int kMaxTopK = 256;  // largest top_k of the filtered path
constexpr int kStatNV = 16;  // 16-byte vectors per thread in the fp32-grade statistics pass
// Window of the per-call 2^(a c) table for bfloat16 logits: magnitude codes
// [kTabLo, kTabLo + kTabW) = |a| in [2^-26, 63.25], both signs. Positive codes
// take slots [0, kTabW), negative ones [kTabNeg, kTabNeg + kTabW); slot kTabW
// of each half is a zero slot. 8 * kTabSize < 2^16, so the byte offset of a
// slot fits a 16-bit lane (the sign is its bit 15).
constexpr uint32_t kTabLo = 101u << 7;
constexpr int kTabW = 4094;
constexpr int kTabNeg = 4096;
constexpr int kTabSize = kTabNeg + kTabW + 1;
// Slots of a table filled by the running-product fill: both halves whole
// (4096 slots each, slots kTabW .. kTabNeg - 1 of a half zero), 64 KB, so
// that a code whose magnitude lies in [kTabLo, kTabLo + kTabNeg) finds its
// slot without the clamp to the zero slot, and a second such table placed
// right after the first starts at byte 2^16.
constexpr int kTabAlloc = 2 * kTabNeg;
constexpr double kTabMaxAbs = 63.25;  // the largest magnitude in the window

// Per (row, chunk) record of the fp32-grade statistics pass: chunk maximum of
// the raw logits and sum of 2^((a - m) * c) with c = log2(e) / T (binary32),
// accumulated in fp64. s is NaN when the chunk holds a NaN or +inf.
struct StatRec {
  float m;
  uint32_t pad;
  double s;
};

// Per (row, chunk) record of the greedy pass: maximum, lowest index holding
// it, and a flag for NaN / +inf.
struct ArgRec {
  float v;
  int32_t idx;
  int32_t bad;
  int32_t pad;
};

// Per (row, sub-block) record of the fp64-grade draft pass: sub-block maximum
// and sum of exp((a - m_sb) / T).
struct DraftRec {
  float m;
  uint32_t pad;
  double s;
};

// Per (request, sub-block) record of the fp64-grade final-row pass.
// Residual: sp = sum P-part, sq = sum Q-part, a / bq = the same sums over the
// entries where the target part exceeds the draft part. Bonus: sp only.
struct ResRec {
  double sp, sq, a, bq;
};

// Per-request decision state written by the decide step.
struct ReqState {
  int32_t n;    // accepted prefix length (K = all accepted, bonus row)
  int32_t err;  // 1 = request error (outputs already written)
  float mp;     // exact maximum of the final target row
  float mq;     // exact maximum of the final draft row (residual only)
  double sp_hat, sq_hat;  // fp32-grade normalisers of those rows
  double u_final;         // uniform of the final draw
  double pad[3];
};

// Filtered row: header and entries of the kept set (token-id order, or rank
// order with FiltCfg::by_rank).
struct FiltRow {
  int32_t cnt;  // kept tokens (0 for an invalid row)
  int32_t bad;  // NaN / +inf / all -inf
  double m;     // max z over the kept set
  double L;     // log-normaliser over the kept set
};
struct FiltEnt {
  int32_t i;
  int32_t pad;
  double z;  // a / T
};
// Top-k candidates of one row chunk (kFiltChunk logits, 64 per thread): tau
// is a lower bound of the chunk's kk-th largest logit, and the chunk's
// candidates are all its finite logits >= tau (cnt of them; more than
// kFiltChunkCap are not stored and the chunk is read again).
constexpr int kFiltVals = 64;
constexpr int kFiltChunk = 256 * kFiltVals;
constexpr int kFiltChunkCap = 128;
struct FiltChunk {
  float tau;
  int32_t cnt;
  int32_t flags;  // bit 0: NaN or +inf seen; bit 1: a finite logit seen
  int32_t pad;
};
struct FiltCand {
  float v;
  int32_t i;
};
struct FiltCfg {
  FiltRow* hdr;     // [rows]
  FiltEnt* ent;     // [rows][stride]
  FiltChunk* chk;   // [rows][nchf]
  FiltCand* fc;     // [rows][nchf][kFiltChunkCap]
  int32_t* nfall;   // rows left to the workgroup merge, then their indices
  int32_t* fall;    // [rows]
  StatRec* cst;     // [rows][nchf] chunk statistics, stored by the chunk pass when not null
  int stride;       // entries per row: min(V, kMaxTopK) >= any admissible top_k
  int nchf;         // chunks per row
  int kk;           // top_k in effect
  int by_rank;      // 1: kept set stored by (logit desc, id asc) instead of token-id order
  double T;         // temperature (binary32 value)
  double top_p;     // binary32 value
};

// Filters with no small bound on the kept set (top-p alone, or top_k above
// kMaxTopK), wide.hip. The kept set of a row is a prefix of the order (logit
// descending, id ascending), described by its last token: token j is kept iff
// key(a_j) > key, or key(a_j) == key and j <= id, with key the order key of
// the binary32 logit (-0 as +0).
struct CutRec {
  float m;       // maximum logit of the row
  uint32_t key;  // order key of the last kept token
  int32_t id;    // its token id
  int32_t bad;   // NaN / +inf / all -inf
  double S;      // sum over the kept set of 2^((a - m) c), c = log2(e) / T
  double cnt;    // kept tokens sharing the last key (diagnostic)
};
struct WideCfg {
  CutRec* cut;   // [rows]
  int top_k;     // 0: no top-k stage
  double top_p;  // binary32 value; 1: no top-p stage
};

// Candidate tree topology, passed by value in the kernel arguments. Row 0 is
// the root context and row n+1 the context after node n; the children of row
// r are the nodes kids[off[r] .. off[r+1]) in ascending node id.
constexpr int kMaxNodes = 256;
struct TreeTopo {
  int16_t off[kMaxNodes + 2];
  int16_t kids[kMaxNodes];
  int16_t prow[kMaxNodes];  // row of node n's parent (parent[n] + 1)
  uint8_t sib[kMaxNodes];   // index of node n among the children of that row
  int32_t N, D;
};

// Per-row normaliser of the tree path: exact maximum and fp32-grade sum of
// 2^((a - m) * c) (from the statistics pass).
struct RowStat {
  float m;
  int32_t bad;
  double s;
};

// Walk state of one request. After j rejections at a row the running target
// is (P - cj * Q)+ / Gj with c_0 = 0, G_0 = 1 and c_{j+1} = c_j + G(c_j),
// G(c) = sum_t max(0, P(t) - c Q(t)).
enum TreePhase : int32_t { kTreeTest = 0, kTreeWaitG = 1, kTreeFinal = 2, kTreeDone = 3 };
struct TreeState {
  int32_t row, j, len, phase, has_exact;
  int32_t urow1;          // row of the final draw's uniform + 1 when it differs from row (0: row)
  int32_t buf;            // which of the two TreeRes buffers holds the sums of this state's pass
  float mp, mq;      // exact row maxima of the current row pair
  double sp_hat, sq_hat;  // fp32-grade normalisers of the current row pair
  double Sp, Sq;          // fp64-grade normalisers (valid when has_exact)
  double cj, Gj;          // current coefficient and normaliser
  double c_new, c_old;    // coefficient asked of the next row pass, and the one to fall back to
};

// Per (request, sub-block) sums of a tree row pass: sp, sq = sums of the
// unnormalised P and Q parts; (a, bq) = the same over the entries where
// P > c_new Q; (a0, bq0) = over the entries where P > c_old Q.
struct TreeRes {
  double sp, sq, a, bq, a0, bq0;
};

struct TreeCfg {
  int32_t* tokens;        // [B, N] node tokens (written first when drafts are fused)
  int32_t* out_path;      // [B, D]
  RowStat* rst;           // [B, 2 (N + 1)]
  TreeState* ts;          // [B]
  TreeRes* tres;          // [B, nsb]
  TreeState* ts2;         // [B] second state buffer of the fused walk rounds (k_tree_wp)
  TreeRes* tres2;         // [B, nsb] second sum buffer of the fused walk rounds
  int N, D;
};

// Tree Sampler: candidate prefixes from the draft rows, and the verification
// of deterministic candidates with a tree per request.
constexpr int kMaxCandEntries = 4096;  // draft positions x candidates per position
struct CandCfg {
  int cands, nodes;
  int32_t* out_parent;  // [B, nodes]
  int32_t* out_tokens;  // [B, nodes]
};
struct DTreeCfg {
  int N;
  const int32_t* parent;  // [B, N]
  const int32_t* tokens;  // [B, N]
  int32_t* out_tokens;    // [B, N + 1]
  int32_t* out_path;      // [B, N]
  void* state;            // [B] walk outcome (tree-state workspace section)
  int32_t* rem;           // [B, N] removed tokens of the final row
};

// Rows of one request: np target rows then nq draft rows.
struct RowMap {
  const char* p;
  const char* q;
  int np, nq;
  int64_t V;
  int esz;
  __device__ __forceinline__ const char* row(int64_t sr) const {
    const int64_t per = np + nq;
    const int64_t b = sr / per;
    const int i = (int)(sr - b * per);
    return i < np ? p + ((b * np + i) * V) * esz : q + ((b * nq + (i - np)) * V) * esz;
  }
};

struct LinCfg {
  RowMap rows;  // np = K + 1, nq = K (linear) or np = 0, nq = K (draft only)
  int64_t B;
  int K;
  int V;
  int aligned;  // rows are 16-byte aligned and V is a multiple of the vector width
  int nvec;     // 16-byte vectors per row (aligned path)
  int nch32;    // chunks per row in the statistics pass
  int nsb;      // sub-blocks per row in the fp64-grade passes
  float c32;    // log2(e) / T rounded to binary32
  double invT;  // 1 / T
  double c64;   // log2(e) / T in fp64
  int tab;      // bf16 weights may use the 2^(a c) table (window below); 0 for small T
  Rng rng;
  int fused;
  int32_t* draft;
  int32_t* out_tokens;
  int32_t* out_len;
  float* out_probs;
  double* out_resid;
  StatRec* st;
  ArgRec* ar;
  ReqState* rs;
  ResRec* res;
  DraftRec* dr;
};

// Launchers (linear.hip). Each returns hipSuccess or the launch error.
hipError_t launch_linear_sampled(const LinCfg& c, int dtype, hipStream_t s);
hipError_t launch_linear_greedy(const LinCfg& c, int dtype, hipStream_t s);
hipError_t launch_draft_sampled(const LinCfg& c, int dtype, hipStream_t s);
hipError_t launch_draft_greedy(const LinCfg& c, int dtype, hipStream_t s);
hipError_t launch_filtered(const LinCfg& c, const FiltCfg& f, int dtype, bool draft_only, hipStream_t s);
hipError_t launch_wide(const LinCfg& c, const WideCfg& wc, int dtype, bool draft_only, hipStream_t s);
// Draft sampling alone: -1 for all drafts of a request with an invalid row.
__global__ void k_draft_fix(LinCfg c);
// Tree verification (tree.hip); c.rows holds N + 1 target and N + 1 draft rows
// per request; `rounds` bounds the rejections that need a new G(c) before the
// final one along any walk.
// With c.fused the node tokens are drawn first: the j-th child of row r from
// row r of q with draw id kDrawDraft + j (argmax when greedy).
hipError_t launch_tree_sampled(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int rounds, int dtype,
                               hipStream_t s);
hipError_t launch_tree_greedy(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, int dtype, hipStream_t s);
hipError_t launch_tree_wide(const LinCfg& c, const WideCfg& wc, const TreeTopo& tp, const TreeCfg& tc, int dtype,
                            hipStream_t s);
hipError_t launch_tree_filtered(const LinCfg& c, const FiltCfg& f, const TreeTopo& tp, const TreeCfg& tc, int dtype,
                                hipStream_t s);
// Row passes over the first `rows` rows of c.rows, reused by the tree:
// filtering (filter.hip), statistics and argmax (linear.hip).
hipError_t launch_filter_rows(const LinCfg& c, const FiltCfg& f, int64_t rows, int dtype, hipStream_t s);
// Tree Sampler (dtree.hip): candidates (c.rows: the K draft rows of each
// request) and the verification of deterministic candidates (c.rows: the N + 1
// target rows of each request).
hipError_t launch_tree_candidates(const LinCfg& c, const FiltCfg& f, const CandCfg& cc, int dtype, hipStream_t s);
hipError_t launch_verify_tree_det(const LinCfg& c, const DTreeCfg& d, int dtype, hipStream_t s);
hipError_t launch_stats32(const LinCfg& c, int64_t rows, int dtype, hipStream_t s);
// Total-variation distillation loss (tv.hip): c.rows holds one teacher (p) and
// one student (q) row per loss row (c.B rows); rn: [c.B, 2] row maxima and
// normalisers (written by the call); sgn: ceil(V / per-vector) 16-bit sign
// words per row (written by the first pass when a gradient is asked for).
hipError_t launch_tv_loss(const LinCfg& c, RowStat* rn, uint16_t* sgn, const float* w_row, double* loss, void* grad,
                          double T, int dtype, hipStream_t s);
hipError_t launch_argmax(const LinCfg& c, int64_t rows, int dtype, hipStream_t s);
// Multi-round generation on the toy model (driver.hip).
struct GenState {
  int32_t* t12;     // [B, 2] last two committed tokens
  int32_t* x0;      // [B] the block's first token
  int32_t* drafts;  // [B, K]
  int32_t* vtok;    // [B, K + 1]
  int32_t* vlen;    // [B]
  int32_t* ctx;     // [B (K + 1), 2]
  int32_t* pos;     // [B K]
};
struct GenLayout {
  size_t first, q, p, inner, inner_bytes, st, total;
};
GenLayout gen_layout(int64_t B, int K, int V, int esz, size_t inner_bytes);
GenState gen_state(void* ws, const GenLayout& L, int64_t B, int K);
hipError_t launch_gen_init(int64_t B, const int32_t* prompt, const GenState& g, int32_t* len, int32_t* seq,
                           int max_len, hipStream_t s);
hipError_t launch_round_ctx(int64_t B, int K, int kind, const GenState& g, hipStream_t s);
hipError_t launch_commit(int64_t B, int K, int r, int rounds, int max_len, const GenState& g, int32_t* seq,
                         int32_t* len, int32_t* round_tokens, hipStream_t s);
hipError_t launch_toy_logits(int64_t rows, int V, const int32_t* ctx, const int32_t* pos, int kind,
                             const psispec_toy_model& m, int dtype, void* out, hipStream_t s);
// Linear verification fused with the LM head (lmhead.hip).
constexpr int kLmhTileM = 256;  // rows of a product tile
constexpr int kLmhTileN = 256;  // vocabulary entries of a product tile
constexpr int kLmhChunk = 128;  // vocabulary entries of a statistics record (a wave's share of a tile)
constexpr int kLmhStepK = 128;  // the hidden size must be a multiple of this
struct LmhCfg {
  const uint16_t* hp;     // [Mp, H] target hidden states (bf16 bits)
  const uint16_t* hq;     // [Mq, H] draft hidden states
  const uint16_t* w;      // [V, H] vocabulary matrix
  int64_t Mp, Mq;         // B (K + 1) target rows, B K draft rows
  int64_t M;              // rows of this product
  int64_t B;
  int K, H, V;
  int ntm, ntn;           // row tiles, vocabulary tiles
  const int32_t* draft;   // [B, K]
  float c32;
  StatRec* st;            // [Mp + Mq][ntn V-tiles x 2 chunks] per (row, 128-token chunk)
  float* all;             // [Mp + Mq][V] fp32 logits of every row, kept for the final draw
                          // (nullptr: not kept)
};
hipError_t launch_lmh_stats(const LmhCfg& g, hipStream_t s);
hipError_t launch_lmh_decide(const LmhCfg& g, const LinCfg& c, const TreeCfg& tc, hipStream_t s);
// The final draw of a tree-state row pair (tree.hip): the fp64 pass over the
// rows in c.rows and the pick, for every request whose state is kTreeFinal.
hipError_t launch_tree_final(const LinCfg& c, const TreeCfg& tc, int dtype, hipStream_t s);
// Fused bfloat16 node drafts of tree verification at a table temperature
// (linear.hip): one pass per draft row, which draws the row's children and
// writes its chunk records, and the target rows' chunk records.
hipError_t launch_tree_qrows(const LinCfg& c, const TreeTopo& tp, const TreeCfg& tc, hipStream_t s);
// fp64 draft-row sub-block records of the first `rows` rows of c.rows.q (linear.hip).
hipError_t launch_draftpass(const LinCfg& c, int64_t rows, int dtype, hipStream_t s);


}  // namespace psi
