// C ABI of libpsispec: argument validation, workspace carving and launches on
// the caller's stream. See include/psispec.h for the contract of each call.
#include <math.h>
#include <string.h>

#include <mutex>

#include "psispec.h"
#include "kernels.hpp"

// Scratch of psispec_verify_linear_noalloc: the workspace of that call lives
// in this file-scope array instead of a caller buffer. Each GPU the library
// runs on holds its own copy until the process ends. In host code the name is
// only a stand-in for the device array: its device address comes from
// hipGetSymbolAddress (scratch_of below), and only that address is used.
static __device__ __align__(256) unsigned char scratch[PSISPEC_NOALLOC_SCRATCH_BYTES];

namespace psi {

// Benchmark timing hook: caller-owned events, two per kernel launch in order.
static hipEvent_t* g_timing_events = nullptr;
static int g_timing_n = 0;
static int g_timing_next = 0;

void timing_begin(hipStream_t) { g_timing_next = 0; }

bool timing_pair(hipEvent_t* start, hipEvent_t* stop) {
  if (!g_timing_events || g_timing_next + 1 >= g_timing_n) return false;
  *start = g_timing_events[g_timing_next];
  *stop = g_timing_events[g_timing_next + 1];
  g_timing_next += 2;
  return true;
}

namespace {

constexpr int kVersion = 100;  // 0.1.0

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int elem_bytes(int dtype) { return dtype == PSISPEC_DTYPE_BF16 ? 2 : 4; }
inline int per_vec(int dtype) { return dtype == PSISPEC_DTYPE_BF16 ? 8 : 4; }

inline int nch32_of(int V, int dtype) {
  const int64_t chunk = (int64_t)kWG * kStatNV * per_vec(dtype);
  return (int)((V + chunk - 1) / chunk);
}
inline int nsb_of(int V) { return (V + kSB - 1) / kSB; }

// Kept-set entries stored per filtered row (top_k < V and top_k <= kMaxTopK).
inline int filt_stride(int32_t V) { return V < kMaxTopK ? V : kMaxTopK; }

// Workspace sections, each 256-byte aligned.
struct Layout {
  size_t st, rs, res, dr, fh, fe, fk, fc, ff, wc, rst, ts, tres, total;
};

inline int nchf_of(int32_t V) { return (V + kFiltChunk - 1) / kFiltChunk; }

inline Layout layout(int64_t B, int32_t rows_per_req, int32_t V, int dtype) {
  Layout L;
  size_t off = 0;
  const size_t nch = (size_t)nch32_of(V, dtype), nsb = (size_t)nsb_of(V);
  L.st = off;
  off = align_up(off + (size_t)B * rows_per_req * nch * sizeof(StatRec), 256);
  L.rs = off;
  off = align_up(off + (size_t)B * sizeof(ReqState), 256);
  L.res = off;
  off = align_up(off + (size_t)B * nsb * sizeof(ResRec), 256);
  L.dr = off;
  off = align_up(off + (size_t)B * rows_per_req * nsb * sizeof(DraftRec), 256);
  L.fh = off;
  off = align_up(off + (size_t)B * rows_per_req * sizeof(FiltRow), 256);
  L.fe = off;
  off = align_up(off + (size_t)B * rows_per_req * filt_stride(V) * sizeof(FiltEnt), 256);
  L.fk = off;
  off = align_up(off + (size_t)B * rows_per_req * nchf_of(V) * sizeof(FiltChunk), 256);
  L.fc = off;
  off = align_up(off + (size_t)B * rows_per_req * nchf_of(V) * kFiltChunkCap * sizeof(FiltCand), 256);
  L.ff = off;
  off = align_up(off + ((size_t)B * rows_per_req + 1) * sizeof(int32_t), 256);
  L.wc = off;
  off = align_up(off + (size_t)B * rows_per_req * sizeof(CutRec), 256);
  L.rst = off;
  off = align_up(off + (size_t)B * rows_per_req * sizeof(RowStat), 256);
  L.ts = off;  // two state buffers (the fused walk rounds alternate between them)
  off = align_up(off + 2 * (size_t)B * sizeof(TreeState), 256);
  L.tres = off;  // two sum buffers
  off = align_up(off + 2 * (size_t)B * nsb * sizeof(TreeRes), 256);
  L.total = off;
  return L;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Common checks of the sampling parameters.
inline int check_params(const psispec_params* prm, int32_t V) {
  if (!prm) return PSISPEC_EINVAL;
  if (!(prm->temperature >= 0.0f) || !isfinite(prm->temperature)) return PSISPEC_EINVAL;
  if (!(prm->top_p > 0.0f && prm->top_p <= 1.0f)) return PSISPEC_EINVAL;
  if (prm->top_k < 0) return PSISPEC_EINVAL;
  (void)V;
  return PSISPEC_OK;
}

inline bool filtered(const psispec_params* prm, int32_t V) {
  return prm->temperature > 0.0f && ((prm->top_k > 0 && prm->top_k < V) || prm->top_p < 1.0f);
}

// Filtered sampling whose kept set is not bounded by a top_k in
// [1, kMaxTopK]: top-p alone (top_k 0 or >= V), or a larger top_k. Such rows
// go to the cut search of wide.hip instead of the kept-set lists of filter.hip.
inline bool wide_filter(const psispec_params* prm, int32_t V) {
  return filtered(prm, V) && (prm->top_k <= 0 || prm->top_k >= V || prm->top_k > kMaxTopK);
}

inline WideCfg wide_cfg(const psispec_params* prm, void* ws, int64_t B, int32_t rows_per_req, int32_t V, int dtype) {
  WideCfg w;
  w.cut = (CutRec*)((char*)ws + layout(B, rows_per_req, V, dtype).wc);
  w.top_k = (prm->top_k > 0 && prm->top_k < V) ? prm->top_k : 0;
  w.top_p = (double)prm->top_p;
  return w;
}

inline FiltCfg filt_cfg(const psispec_params* prm, void* ws, int64_t B, int32_t rows_per_req, int32_t V, int dtype) {
  const Layout L = layout(B, rows_per_req, V, dtype);
  FiltCfg f;
  f.hdr = (FiltRow*)((char*)ws + L.fh);
  f.ent = (FiltEnt*)((char*)ws + L.fe);
  f.chk = (FiltChunk*)((char*)ws + L.fk);
  f.fc = (FiltCand*)((char*)ws + L.fc);
  f.nfall = (int32_t*)((char*)ws + L.ff);
  f.fall = f.nfall + 1;
  f.stride = filt_stride(V);
  f.nchf = nchf_of(V);
  f.kk = prm->top_k;
  f.by_rank = 0;
  f.cst = nullptr;
  f.T = (double)prm->temperature;
  f.top_p = (double)prm->top_p;
  return f;
}

inline void fill_common(LinCfg& c, const void* p, const void* q, int dtype, int64_t B, int32_t K, int32_t V,
                        const psispec_params* prm, void* ws, int np) {
  memset(&c, 0, sizeof(c));
  c.rows.p = (const char*)p;
  c.rows.q = (const char*)q;
  c.rows.np = np;
  c.rows.nq = K;
  c.rows.V = V;
  c.rows.esz = elem_bytes(dtype);
  c.B = B;
  c.K = K;
  c.V = V;
  const int pv = per_vec(dtype);
  c.aligned = (V % pv == 0) && aligned16(q) && (p == nullptr || aligned16(p));
  c.nvec = V / pv;
  c.nch32 = nch32_of(V, dtype);
  c.nsb = nsb_of(V);
  const double T = (double)prm->temperature;
  c.invT = T > 0.0 ? 1.0 / T : 0.0;
  c.c32 = T > 0.0 ? (float)(1.4426950408889634074 / T) : 0.0f;
  c.c64 = T > 0.0 ? 1.4426950408889634074 / T : 0.0;
  // the 2^(a c) table covers |a| < 64: keep every entry inside the fp64 range
  c.tab = (dtype == PSISPEC_DTYPE_BF16 && c.c64 * kTabMaxAbs <= 1000.0) ? 1 : 0;
  c.rng.k0 = (uint32_t)(prm->seed & 0xffffffffu);
  c.rng.k1 = (uint32_t)(prm->seed >> 32);
  c.rng.step = prm->step;
  c.fused = (prm->flags & PSISPEC_FUSED_DRAFT) ? 1 : 0;
  const Layout L = layout(B, np + K, V, dtype);
  char* w = (char*)ws;
  c.st = (StatRec*)(w + L.st);
  c.ar = (ArgRec*)(w + L.st);
  c.rs = (ReqState*)(w + L.rs);
  c.res = (ResRec*)(w + L.res);
  c.dr = (DraftRec*)(w + L.dr);
}

// Children lists of every row from a validated parent array, and the largest
// number of rejections along one walk that need a new G(c) before the final
// one: at a row with C children at most C - 1 of them, summed down a path.
inline int build_topo(const int32_t* parent, int32_t N, int32_t D, TreeTopo& tp) {
  memset(&tp, 0, sizeof(tp));
  tp.N = N;
  tp.D = D;
  int cnt[kMaxNodes + 1] = {0};
  for (int n = 0; n < N; ++n) ++cnt[parent[n] + 1];
  tp.off[0] = 0;
  for (int r = 0; r <= N; ++r) tp.off[r + 1] = (int16_t)(tp.off[r] + cnt[r]);
  int fill[kMaxNodes + 1] = {0};
  for (int n = 0; n < N; ++n) {
    const int r = parent[n] + 1;
    tp.prow[n] = (int16_t)r;
    tp.sib[n] = (uint8_t)fill[r];
    tp.kids[tp.off[r] + fill[r]++] = (int16_t)n;
  }
  int cost[kMaxNodes + 1];
  int rounds = 0;
  for (int r = 0; r <= N; ++r) {
    const int own = cnt[r] > 1 ? cnt[r] - 1 : 0;
    cost[r] = own + (r == 0 ? 0 : cost[parent[r - 1] + 1]);
    if (cost[r] > rounds) rounds = cost[r];
  }
  return rounds;
}

// Device address of the scratch array on device `dev`, looked up once per
// device with that device current. Returns the lookup's status.
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

hipError_t scratch_of(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace
}  // namespace psi

using namespace psi;

extern "C" {

size_t psispec_workspace_bytes(int64_t B, int32_t rows_per_req, int32_t V, int dtype) {
  if (B <= 0 || rows_per_req <= 0 || V <= 0) return 0;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return 0;
  return layout(B, rows_per_req, V, dtype).total;
}

int psispec_draft_sample(const void* q_logits, int dtype, int64_t B, int32_t K, int32_t V,
                         const psispec_params* params, int32_t* draft_tokens, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  if (!q_logits || !draft_tokens || !workspace) return PSISPEC_EINVAL;
  if (B <= 0 || K <= 0 || V <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (K > PSISPEC_MAX_K) return PSISPEC_EUNSUPPORTED;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  if (ws_bytes < psispec_workspace_bytes(B, K, V, dtype)) return PSISPEC_EWORKSPACE;
  LinCfg c;
  fill_common(c, nullptr, q_logits, dtype, B, K, V, params, workspace, 0);
  c.draft = draft_tokens;
  timing_begin(stream);
  hipError_t e;
  if (params->temperature == 0.0f) e = launch_draft_greedy(c, dtype, stream);
  else if (wide_filter(params, V)) e = launch_wide(c, wide_cfg(params, workspace, B, K, V, dtype), dtype, true, stream);
  else if (filtered(params, V)) e = launch_filtered(c, filt_cfg(params, workspace, B, K, V, dtype), dtype, true, stream);
  else e = launch_draft_sampled(c, dtype, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

int psispec_verify_linear(const void* p_logits, const void* q_logits, int dtype, int64_t B, int32_t K, int32_t V,
                          int32_t* draft_tokens, const psispec_params* params, int32_t* out_tokens,
                          int32_t* out_len, float* out_probs, double* out_resid_mass, void* workspace,
                          size_t ws_bytes, hipStream_t stream) {
  if (!p_logits || !q_logits || !draft_tokens || !out_tokens || !out_len || !workspace) return PSISPEC_EINVAL;
  if (B <= 0 || K <= 0 || V <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (K > PSISPEC_MAX_K) return PSISPEC_EUNSUPPORTED;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  if (ws_bytes < psispec_workspace_bytes(B, 2 * K + 1, V, dtype)) return PSISPEC_EWORKSPACE;
  LinCfg c;
  fill_common(c, p_logits, q_logits, dtype, B, K, V, params, workspace, K + 1);
  c.draft = draft_tokens;
  c.out_tokens = out_tokens;
  c.out_len = out_len;
  c.out_probs = out_probs;
  c.out_resid = out_resid_mass;
  timing_begin(stream);
  hipError_t e;
  if (params->temperature == 0.0f) {
    e = launch_linear_greedy(c, dtype, stream);
  } else if (wide_filter(params, V)) {
    e = launch_wide(c, wide_cfg(params, workspace, B, 2 * K + 1, V, dtype), dtype, false, stream);
  } else if (filtered(params, V)) {
    e = launch_filtered(c, filt_cfg(params, workspace, B, 2 * K + 1, V, dtype), dtype, false, stream);
  } else {
    e = launch_linear_sampled(c, dtype, stream);  // draws the drafts itself when fused
  }
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

int psispec_verify_linear_noalloc(const void* p_logits, const void* q_logits, int dtype, int64_t B, int32_t K,
                                  int32_t V, int32_t* draft_tokens, const psispec_params* params,
                                  int32_t* out_tokens, int32_t* out_len, float* out_probs, double* out_resid_mass,
                                  hipStream_t stream) {
  if (!p_logits || !q_logits || !draft_tokens || !out_tokens || !out_len) return PSISPEC_EINVAL;
  if (B <= 0 || K <= 0 || V <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (K > PSISPEC_MAX_K) return PSISPEC_EUNSUPPORTED;
  // Sections of the workspace layout this call uses: statistics, request and
  // sub-block records, then the kept sets when filtering (the tree sections
  // after them are never touched by linear verification).
  const Layout L = layout(B, 2 * K + 1, V, dtype);
  const size_t need = (params->temperature > 0.0f && filtered(params, V)) ? L.rst : L.fh;
  if (need > (size_t)PSISPEC_NOALLOC_SCRATCH_BYTES) return PSISPEC_ESCRATCH;
  int dev = -1;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return PSISPEC_EHIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return PSISPEC_EHIP;
  }
  void* ws = nullptr;
  if (scratch_of(dev, &ws) != hipSuccess || !ws) return PSISPEC_EHIP;
  return psispec_verify_linear(p_logits, q_logits, dtype, B, K, V, draft_tokens, params, out_tokens, out_len,
                               out_probs, out_resid_mass, ws, L.total, stream);
}

int32_t psispec_tree_depth(const int32_t* parent, int32_t N) {
  if (!parent || N <= 0) return PSISPEC_EINVAL;
  if (N > PSISPEC_MAX_TREE_NODES) return PSISPEC_EUNSUPPORTED;
  int32_t depth[PSISPEC_MAX_TREE_NODES];
  int32_t D = 0;
  for (int32_t n = 0; n < N; ++n) {
    if (parent[n] < -1 || parent[n] >= n) return PSISPEC_EINVAL;
    depth[n] = parent[n] < 0 ? 1 : depth[parent[n]] + 1;
    if (depth[n] > D) D = depth[n];
  }
  if (D > PSISPEC_MAX_K) return PSISPEC_EUNSUPPORTED;
  return D;
}

int psispec_verify_tree(const void* p_logits, const void* q_logits, int dtype, int64_t B, int32_t N, int32_t V,
                        const int32_t* parent, int32_t* node_tokens, const psispec_params* params,
                        int32_t* out_tokens, int32_t* out_path, int32_t* out_len, void* workspace, size_t ws_bytes,
                        hipStream_t stream) {
  if (!p_logits || !q_logits || !parent || !node_tokens || !out_tokens || !out_path || !out_len || !workspace)
    return PSISPEC_EINVAL;
  if (B <= 0 || N <= 0 || V <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  const int32_t D = psispec_tree_depth(parent, N);
  if (D < 0) return D;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  const int32_t rows = 2 * (N + 1);
  if (ws_bytes < psispec_workspace_bytes(B, rows, V, dtype)) return PSISPEC_EWORKSPACE;
  TreeTopo tp;
  const int rounds = build_topo(parent, N, D, tp);
  LinCfg c;
  fill_common(c, p_logits, q_logits, dtype, B, N + 1, V, params, workspace, N + 1);
  c.out_tokens = out_tokens;
  c.out_len = out_len;
  const Layout L = layout(B, rows, V, dtype);
  char* w = (char*)workspace;
  TreeCfg tc;
  tc.tokens = node_tokens;
  tc.out_path = out_path;
  tc.rst = (RowStat*)(w + L.rst);
  tc.ts = (TreeState*)(w + L.ts);
  tc.tres = (TreeRes*)(w + L.tres);
  tc.ts2 = tc.ts + B;
  tc.tres2 = tc.tres + B * (int64_t)nsb_of(V);
  tc.N = N;
  tc.D = D;
  timing_begin(stream);
  hipError_t e;
  if (params->temperature == 0.0f) e = launch_tree_greedy(c, tp, tc, dtype, stream);
  else if (wide_filter(params, V)) e = launch_tree_wide(c, wide_cfg(params, workspace, B, rows, V, dtype), tp, tc, dtype, stream);
  else if (filtered(params, V)) e = launch_tree_filtered(c, filt_cfg(params, workspace, B, rows, V, dtype), tp, tc, dtype, stream);
  else e = launch_tree_sampled(c, tp, tc, rounds, dtype, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

static_assert(PSISPEC_MAX_CAND_ENTRIES == kMaxCandEntries && PSISPEC_MAX_TOPK == kMaxTopK &&
                  PSISPEC_MAX_TREE_NODES == kMaxNodes,
              "public limits match the kernels");

int psispec_tree_candidates(const void* q_logits, int dtype, int64_t B, int32_t K, int32_t V,
                            const psispec_params* params, int32_t cands, int32_t nodes, int32_t* out_parent,
                            int32_t* out_tokens, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (!q_logits || !out_parent || !out_tokens || !workspace) return PSISPEC_EINVAL;
  if (B <= 0 || K <= 0 || V <= 0 || cands <= 0 || nodes <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (!(params->temperature > 0.0f)) return PSISPEC_EINVAL;
  if (params->top_k != 0 || params->top_p != 1.0f) return PSISPEC_EUNSUPPORTED;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (K > PSISPEC_MAX_K || cands > V || cands > kMaxTopK || (int64_t)K * cands > kMaxCandEntries ||
      nodes > kMaxNodes)
    return PSISPEC_EUNSUPPORTED;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  if (ws_bytes < psispec_workspace_bytes(B, K, V, dtype)) return PSISPEC_EWORKSPACE;
  LinCfg c;
  fill_common(c, nullptr, q_logits, dtype, B, K, V, params, workspace, 0);
  psispec_params fp = *params;
  fp.top_k = cands;
  FiltCfg f = filt_cfg(&fp, workspace, B, K, V, dtype);
  f.by_rank = 1;
  f.cst = (StatRec*)((char*)workspace + layout(B, K, V, dtype).dr);  // nchf <= nsb records per row
  static_assert(sizeof(StatRec) == sizeof(DraftRec) && kFiltChunk >= kSB, "chunk statistics fit the draft section");
  CandCfg cc;
  cc.cands = cands;
  cc.nodes = nodes;
  cc.out_parent = out_parent;
  cc.out_tokens = out_tokens;
  timing_begin(stream);
  const hipError_t e = launch_tree_candidates(c, f, cc, dtype, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

int psispec_verify_tree_det(const void* p_logits, int dtype, int64_t B, int32_t N, int32_t V,
                            const int32_t* parent, const int32_t* node_tokens, const psispec_params* params,
                            int32_t* out_tokens, int32_t* out_path, int32_t* out_len, void* workspace,
                            size_t ws_bytes, hipStream_t stream) {
  if (!p_logits || !parent || !node_tokens || !out_tokens || !out_path || !out_len || !workspace)
    return PSISPEC_EINVAL;
  if (B <= 0 || N <= 0 || V <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (params->top_k != 0 || params->top_p != 1.0f) return PSISPEC_EUNSUPPORTED;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (N > PSISPEC_MAX_TREE_NODES) return PSISPEC_EUNSUPPORTED;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  const int32_t rows = N + 1;
  if (ws_bytes < psispec_workspace_bytes(B, rows, V, dtype)) return PSISPEC_EWORKSPACE;
  LinCfg c;
  fill_common(c, p_logits, nullptr, dtype, B, 0, V, params, workspace, rows);
  c.out_len = out_len;
  const Layout L = layout(B, rows, V, dtype);
  char* w = (char*)workspace;
  DTreeCfg d;
  d.N = N;
  d.parent = parent;
  d.tokens = node_tokens;
  d.out_tokens = out_tokens;
  d.out_path = out_path;
  d.state = w + L.ts;
  d.rem = (int32_t*)(w + L.rst);
  timing_begin(stream);
  const hipError_t e = launch_verify_tree_det(c, d, dtype, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

size_t psispec_tv_workspace_bytes(int64_t R, int32_t V, int dtype) {
  if (R <= 0 || V <= 0 || (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16)) return 0;
  const int64_t nv = ((int64_t)V + per_vec(dtype) - 1) / per_vec(dtype);
  return layout(R, 2, V, dtype).total + align_up((size_t)(R * nv) * sizeof(uint16_t), 256);
}

int psispec_tv_loss(const void* p_logits, const void* q_logits, int dtype, int64_t R, int32_t V, float temperature,
                    const float* row_weights, double* out_loss, void* out_grad, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  if (!p_logits || !q_logits || !out_loss || !workspace) return PSISPEC_EINVAL;
  if (R <= 0 || V <= 0 || !(temperature > 0.0f) || !isfinite(temperature)) return PSISPEC_EINVAL;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  if (ws_bytes < psispec_tv_workspace_bytes(R, V, dtype)) return PSISPEC_EWORKSPACE;
  psispec_params prm = {};
  prm.temperature = temperature;
  prm.top_p = 1.0f;
  LinCfg c;
  fill_common(c, p_logits, q_logits, dtype, R, 1, V, &prm, workspace, 1);
  c.aligned = c.aligned && (out_grad == nullptr || aligned16(out_grad));
  const Layout L = layout(R, 2, V, dtype);
  uint16_t* sgn = (uint16_t*)((char*)workspace + L.total);
  RowStat* rn = (RowStat*)((char*)workspace + L.rst);  // [R, 2] teacher and student row normalisers
  timing_begin(stream);
  const hipError_t e =
      launch_tv_loss(c, rn, sgn, row_weights, out_loss, out_grad, (double)temperature, dtype, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

int psispec_toy_logits(int64_t rows, int32_t V, const int32_t* ctx, const int32_t* pos, int kind,
                       const psispec_toy_model* model, int dtype, void* out, hipStream_t stream) {
  if (!ctx || !model || !out || rows <= 0 || V <= 0 || (kind != 0 && kind != 1) || (kind == 1 && !pos))
    return PSISPEC_EINVAL;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  const hipError_t e = launch_toy_logits(rows, V, ctx, pos, kind, *model, dtype, out, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

size_t psispec_generate_workspace_bytes(int64_t B, int32_t block, int32_t V, int dtype) {
  if (B <= 0 || block < 2 || block - 1 > PSISPEC_MAX_K || V <= 0) return 0;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return 0;
  const int K = block - 1;
  return gen_layout(B, K, V, elem_bytes(dtype), psispec_workspace_bytes(B, 2 * K + 1, V, dtype)).total;
}

int psispec_generate_toy(int64_t B, int32_t block, int32_t V, int dtype, const psispec_toy_model* model,
                         const psispec_params* params, const int32_t* prompt, int32_t rounds, int32_t* out_seq,
                         int32_t* out_len, int32_t* out_round_tokens, void* workspace, size_t ws_bytes,
                         hipStream_t stream) {
  if (!model || !prompt || !out_seq || !out_len || !out_round_tokens || !workspace) return PSISPEC_EINVAL;
  if (B <= 0 || V <= 0 || rounds <= 0 || block < 2) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (params->top_k != 0 || params->top_p != 1.0f) return PSISPEC_EUNSUPPORTED;
  if (dtype != PSISPEC_DTYPE_F32 && dtype != PSISPEC_DTYPE_BF16) return PSISPEC_EUNSUPPORTED;
  if (block - 1 > PSISPEC_MAX_K) return PSISPEC_EUNSUPPORTED;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  if (ws_bytes < psispec_generate_workspace_bytes(B, block, V, dtype)) return PSISPEC_EWORKSPACE;
  const int K = block - 1;
  const int max_len = rounds * (block + 1);
  const GenLayout L = gen_layout(B, K, V, elem_bytes(dtype), psispec_workspace_bytes(B, 2 * K + 1, V, dtype));
  char* w = (char*)workspace;
  const GenState g = gen_state(workspace, L, B, K);
  void* first = w + L.first;
  void* q = w + L.q;
  void* p = w + L.p;
  void* inner = w + L.inner;
  psispec_params prm = *params;
  prm.flags = 0;
  hipError_t e = launch_gen_init(B, prompt, g, out_len, out_seq, max_len, stream);
  for (int r = 0; r < rounds && e == hipSuccess; ++r) {
    int rc = PSISPEC_OK;
    prm.step = params->step + 2u * (uint32_t)r;
    if ((e = launch_round_ctx(B, K, 0, g, stream)) != hipSuccess) break;
    if ((e = launch_toy_logits(B, V, g.ctx, nullptr, 0, *model, dtype, first, stream)) != hipSuccess) break;
    if ((rc = psispec_draft_sample(first, dtype, B, 1, V, &prm, g.x0, inner, L.inner_bytes, stream))) return rc;
    prm.step = params->step + 2u * (uint32_t)r + 1u;
    if ((e = launch_round_ctx(B, K, 1, g, stream)) != hipSuccess) break;
    if ((e = launch_toy_logits(B * K, V, g.ctx, g.pos, 1, *model, dtype, q, stream)) != hipSuccess) break;
    if ((rc = psispec_draft_sample(q, dtype, B, K, V, &prm, g.drafts, inner, L.inner_bytes, stream))) return rc;
    if ((e = launch_round_ctx(B, K, 2, g, stream)) != hipSuccess) break;
    if ((e = launch_toy_logits(B * (K + 1), V, g.ctx, nullptr, 0, *model, dtype, p, stream)) != hipSuccess) break;
    if ((rc = psispec_verify_linear(p, q, dtype, B, K, V, g.drafts, &prm, g.vtok, g.vlen, nullptr, nullptr, inner,
                                    L.inner_bytes, stream)))
      return rc;
    e = launch_commit(B, K, r, rounds, max_len, g, out_seq, out_len, out_round_tokens, stream);
  }
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

namespace psi {
namespace {
struct LmhLayout {
  size_t st, ts, tres, out, total;
};
inline LmhLayout lmh_layout(int64_t B, int32_t K, int32_t V) {
  LmhLayout L;
  const int64_t rows = B * (2 * (int64_t)K + 1);
  const int64_t ntn = (V + kLmhTileN - 1) / kLmhTileN;
  size_t off = 0;
  L.st = off;
  off = align_up(off + (size_t)(rows * ntn * (kLmhTileN / kLmhChunk)) * sizeof(StatRec), 256);
  L.ts = off;
  off = align_up(off + (size_t)B * sizeof(TreeState), 256);
  L.tres = off;
  off = align_up(off + (size_t)B * nsb_of(V) * sizeof(TreeRes), 256);
  L.out = off;  // the logits of every row, kept by the product for the final draw
  off = align_up(off + (size_t)rows * V * sizeof(float), 256);
  L.total = off;
  return L;
}
}  // namespace
}  // namespace psi

size_t psispec_lmhead_workspace_bytes(int64_t B, int32_t K, int32_t V) {
  if (B <= 0 || K <= 0 || K > PSISPEC_MAX_K || V <= 0) return 0;
  return lmh_layout(B, K, V).total;
}

int psispec_verify_lmhead(const void* h_target, const void* h_draft, const void* w_vocab, int64_t B, int32_t K,
                          int32_t H, int32_t V, const int32_t* draft_tokens, const psispec_params* params,
                          int32_t* out_tokens, int32_t* out_len, void* workspace, size_t ws_bytes,
                          hipStream_t stream) {
  if (!h_target || !h_draft || !w_vocab || !draft_tokens || !out_tokens || !out_len || !workspace)
    return PSISPEC_EINVAL;
  if (B <= 0 || K <= 0 || H <= 0 || V <= 0) return PSISPEC_EINVAL;
  if (int rc = check_params(params, V)) return rc;
  if (!(params->temperature > 0.0f) || params->top_k != 0 || params->top_p != 1.0f) return PSISPEC_EUNSUPPORTED;
  if (K > PSISPEC_MAX_K || H % kLmhStepK != 0) return PSISPEC_EUNSUPPORTED;
  if (!aligned16(h_target) || !aligned16(h_draft) || !aligned16(w_vocab)) return PSISPEC_EINVAL;
  if (((uintptr_t)workspace & 255u) != 0) return PSISPEC_EINVAL;
  if (ws_bytes < psispec_lmhead_workspace_bytes(B, K, V)) return PSISPEC_EWORKSPACE;
  const LmhLayout L = lmh_layout(B, K, V);
  char* w = (char*)workspace;
  LmhCfg g;
  memset(&g, 0, sizeof(g));
  g.hp = (const uint16_t*)h_target;
  g.hq = (const uint16_t*)h_draft;
  g.w = (const uint16_t*)w_vocab;
  g.Mp = B * (K + 1);
  g.Mq = B * K;
  g.B = B;
  g.K = K;
  g.H = H;
  g.V = V;
  g.ntn = (V + kLmhTileN - 1) / kLmhTileN;
  g.draft = draft_tokens;
  g.c32 = (float)(1.4426950408889634074 / (double)params->temperature);
  g.st = (StatRec*)(w + L.st);
  g.all = (float*)(w + L.out);
  // the draw over the final rows, read from the kept logits: target rows [B, K + 1, V], then
  // draft rows [B, K, V] (fp32)
  psispec_params prm = *params;
  prm.flags = 0;
  LinCfg c;
  fill_common(c, g.all, g.all + (size_t)g.Mp * V, PSISPEC_DTYPE_F32, B, K, V, &prm, workspace, K + 1);
  c.st = nullptr;  // the draw uses only the tree-state sections below
  c.ar = nullptr;
  c.rs = nullptr;
  c.res = nullptr;
  c.dr = nullptr;
  c.K = K;
  c.out_tokens = out_tokens;
  c.out_len = out_len;
  TreeCfg tc;
  memset(&tc, 0, sizeof(tc));
  tc.ts = (TreeState*)(w + L.ts);
  tc.tres = (TreeRes*)(w + L.tres);
  tc.ts2 = nullptr;  // one walk state per request: no fused walk rounds here
  tc.tres2 = nullptr;
  tc.N = K;
  tc.D = K;
  timing_begin(stream);
  LmhCfg gs = g;
  gs.M = g.Mp + g.Mq;
  gs.ntm = (int)((gs.M + kLmhTileM - 1) / kLmhTileM);
  hipError_t e = launch_lmh_stats(gs, stream);
  if (e == hipSuccess) e = launch_lmh_decide(gs, c, tc, stream);
  if (e == hipSuccess) e = launch_tree_final(c, tc, PSISPEC_DTYPE_F32, stream);
  return e == hipSuccess ? PSISPEC_OK : PSISPEC_EHIP;
}

const char* psispec_strerror(int status) {
  switch (status) {
    case PSISPEC_OK:
      return "success";
    case PSISPEC_EINVAL:
      return "invalid argument";
    case PSISPEC_EUNSUPPORTED:
      return "unsupported dtype, size or mode";
    case PSISPEC_EWORKSPACE:
      return "workspace too small";
    case PSISPEC_EHIP:
      return "HIP launch failed";
    case PSISPEC_ESCRATCH:
      return "the call needs more than the no-alloc entry point's fixed scratch";
    default:
      return "unknown status";
  }
}

int psispec_version(void) { return kVersion; }

int psispec_set_timing_events(hipEvent_t* events, int n) {
  if (events == nullptr || n <= 0) {
    g_timing_events = nullptr;
    g_timing_n = 0;
    return PSISPEC_OK;
  }
  g_timing_events = events;
  g_timing_n = n;
  return PSISPEC_OK;
}

int psispec_timing_count(void) { return g_timing_next; }

}  // extern "C"
