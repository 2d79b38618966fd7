/*
 * psispec.h — C ABI of libpsispec, the lossless block-verification step of the
 * Psi-Spec sampler on AMD MI355X (gfx950).
 *
 * What the library computes (sources are the web pages on Uno, a
 * diffusion-augmented LLM):
 *   - "Uno" research explainer, §3.3 (Psi-Spec): a diffusion pass proposes a
 *     block of draft tokens x_i drawn from per-position draft distributions q_i;
 *     the AR pass gives target distributions p_i; draft i is kept with
 *     probability a_i = min(1, p_i(x_i) / q_i(x_i)); the longest run of kept
 *     drafts from the start of the block survives; at the first rejected
 *     position one token is drawn from norm(max(0, p - q)); when the whole block
 *     survives one extra token is drawn from the last target row.
 *   - same page, §3.3 TPF bound: one verify call emits between 1 and K+1 tokens.
 *   - same page, §3.4 (Linear vs Tree sampler) and §7 (what "lossless" means:
 *     the output law equals the AR law; bitwise equality with plain AR decoding
 *     is not promised).
 *   - Uno repository README (inference section): the user-facing sampling
 *     controls temperature / top-p / top-k.
 * Randomness: counter-based Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC'11), see PSISPEC RNG below.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership   Every tensor pointer is a caller-owned DEVICE buffer unless the
 *             argument says "host". The library never allocates, frees or
 *             synchronises; work is enqueued on `stream` (NULL = the default
 *             stream) and the call returns right after the enqueue. Calls are
 *             re-entrant when they use distinct workspaces; two calls that
 *             share a workspace must be ordered on one stream.
 * Layout      Logit tensors are contiguous row-major: a row is V consecutive
 *             values of `dtype`. Rows that are 16-byte aligned take the
 *             vectorised path, others a slower element-wise one; the workspace
 *             must be 256-byte aligned.
 * dtype       PSISPEC_DTYPE_F32 (IEEE binary32) or PSISPEC_DTYPE_BF16
 *             (bfloat16, upper half of a binary32).
 * Errors      Argument errors are returned synchronously (negative codes
 *             below) and nothing is enqueued. Errors that can only be seen in
 *             the data (a token outside [0, V), a NaN or +inf logit, a row that
 *             is entirely -inf) are reported per request: out_len[b] = -1 and
 *             that request's output tokens are all -1; other requests are
 *             unaffected.
 * Determinism The same inputs, parameters, seed and step give bitwise
 *             identical outputs on every run; there are no floating-point
 *             atomics anywhere in the library.
 */
#ifndef PSISPEC_H
#define PSISPEC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PSISPEC_OK            0
#define PSISPEC_EINVAL       -1 /* null pointer, size <= 0, temperature < 0 or not finite,
                                   top_p outside (0, 1], top_k < 0, workspace not 256-byte
                                   aligned, malformed tree topology */
#define PSISPEC_EUNSUPPORTED -2 /* dtype other than F32/BF16, K or tree depth > 64,
                                   tree with more than 256 nodes; the Tree Sampler
                                   calls' own limits (see there) */
#define PSISPEC_EWORKSPACE   -3 /* ws_bytes smaller than psispec_workspace_bytes(...) */
#define PSISPEC_EHIP         -4 /* a HIP launch failed */
#define PSISPEC_ESCRATCH     -5 /* psispec_verify_linear_noalloc: the call needs more than
                                   PSISPEC_NOALLOC_SCRATCH_BYTES of scratch */

/* ---- dtypes --------------------------------------------------------------- */
#define PSISPEC_DTYPE_F32  0
#define PSISPEC_DTYPE_BF16 1

/* ---- flags ------------------------------------------------------------------ */
/* psispec_verify_linear draws the drafts itself from q (exactly as
   psispec_draft_sample with the same params would) and writes them to
   draft_tokens, instead of reading them from there. psispec_verify_tree
   likewise draws the node tokens (see there) and writes them to node_tokens. */
#define PSISPEC_FUSED_DRAFT 1u

/* ---- limits ----------------------------------------------------------------- */
#define PSISPEC_MAX_K         64   /* draft positions per request (one wave64 ballot) */
#define PSISPEC_MAX_TREE_NODES 256 /* tree nodes per request */
#define PSISPEC_MAX_TOPK      256  /* largest top_k of the kept-set-list filter path, and
                                      of the Tree Sampler's candidates per position */
#define PSISPEC_NOALLOC_SCRATCH_BYTES (32u << 20) /* device scratch of psispec_verify_linear_noalloc */

/*
 * Sampling parameters (Uno README, inference controls: temperature, top-p,
 * top-k).
 *   temperature  > 0: logits z = a / temperature; == 0: greedy mode (argmax,
 *                lowest index on ties; draft accepted iff it equals the target
 *                argmax; no random numbers are drawn; top_k/top_p ignored).
 *   top_k        0 or >= V disables; otherwise keep the top_k largest z per
 *                row (ties: the lower token id wins). Every top_k is accepted:
 *                up to PSISPEC_MAX_TOPK the kept set is gathered as a list in
 *                one pass over the row; above it, and for top-p without a
 *                top-k, a cut search reads each row several times (slower).
 *   top_p        1 disables; otherwise, among the tokens kept by top-k, keep the
 *                shortest prefix of the probability-sorted list (ties: lower id
 *                first) whose cumulative probability reaches top_p (at least
 *                one token). Filtering is applied in the order temperature ->
 *                top-k -> top-p -> renormalise, identically and independently
 *                to every target row and every draft row; losslessness then
 *                holds with respect to the filtered target distribution.
 *   seed, step   Philox key and the step word of the counter (see RNG).
 *   flags        bitwise OR of PSISPEC_* flags.
 */
typedef struct psispec_params {
  float temperature;
  int32_t top_k;
  float top_p;
  uint32_t flags;
  uint64_t seed;
  uint32_t step;
  uint32_t reserved; /* must be 0 */
} psispec_params;

/*
 * PSISPEC RNG. Every uniform is U(seed, step, b, r, d) = word0 * 2^-32 (a
 * double in [0, 1)) where word0 is the first output word of Philox4x32-10 with
 *   key     = (lo32(seed), hi32(seed))
 *   counter = (d, r, b, step)
 * b is the request, r the logit row within the request, and d the draw id:
 *   d = 0               final sample (residual, bonus or tree stop) at row r
 *   d = 1 + j           accept test of the j-th candidate child at row r
 *                       (the linear sampler uses j = 0 at every position)
 *   d = 0x40000000 + j  j-th draft drawn from draft row r
 * Because the tree sampler uses the same layout, a chain-shaped tree gives
 * bit-for-bit the result of psispec_verify_linear.
 */

/*
 * Bytes of workspace sufficient for any call of this library on B requests,
 * each reading at most `rows_per_req` logit rows of length V:
 *   psispec_draft_sample   rows_per_req = K
 *   psispec_verify_linear  rows_per_req = 2*K + 1
 *   psispec_verify_tree    rows_per_req = 2*(N + 1)
 *   psispec_tree_candidates rows_per_req = K
 *   psispec_verify_tree_det rows_per_req = N + 1
 * (psispec_tv_loss has its own: psispec_tv_workspace_bytes.)
 * Returns 0 for arguments out of range. Pure host function.
 */
size_t psispec_workspace_bytes(int64_t B, int32_t rows_per_req, int32_t V, int dtype);

/*
 * Draft sampling (Uno explainer §3.3: the diffusion pass proposes every block
 * position in parallel, each token drawn independently from its own draft
 * distribution q_i).
 *   q_logits      [B, K, V] draft logits.
 *   draft_tokens  [B, K] int32 out: x_{b,i} drawn from softmax(filter(q_{b,i} / T))
 *                 by inverse CDF in token-id order with U(seed, step, b, i,
 *                 0x40000000); greedy mode (T == 0): argmax of q_{b,i}.
 *                 A request with an invalid q row gets -1 in every slot.
 */
int psispec_draft_sample(const void* q_logits, int dtype, int64_t B, int32_t K, int32_t V,
                         const psispec_params* params, int32_t* draft_tokens, void* workspace,
                         size_t ws_bytes, hipStream_t stream);

/*
 * Linear verification (Uno explainer §3.3 and §3.4 "Linear Sampler").
 *   p_logits      [B, K+1, V] target logits; row i scores draft position i and
 *                 row K is the bonus row used when every draft is accepted.
 *   q_logits      [B, K, V] draft logits.
 *   draft_tokens  [B, K] int32; input, or output with PSISPEC_FUSED_DRAFT.
 *   out_tokens    [B, K+1] int32 out: the n accepted drafts, then the final
 *                 token y, then -1 padding. Emitted tokens per request = n + 1.
 *   out_len       [B] int32 out: n in [0, K] (or -1 for a request error).
 *   out_probs     nullable [B, K, 2] float out: (p_i(x_i), q_i(x_i)) for every
 *                 position i, after temperature and filtering; greedy mode
 *                 writes the one-hot limits (x_i == argmax p_i, x_i == argmax q_i).
 *   out_resid_mass nullable [B] double out: sum_j max(0, p_n(j) - q_n(j)) when
 *                 n < K (= 1 - alpha_n, alpha = sum_j min(p, q)), 0 when n == K
 *                 or in greedy mode.
 * Decision rules (U as in PSISPEC RNG):
 *   accept_i  <=>  U(seed, step, b, i, 1) * q_i(x_i) < p_i(x_i)
 *   n         =    first i with !accept_i, else K
 *   y         =    inverse-CDF draw, in token-id order, with U(seed, step, b, n, 0)
 *                  from max(0, p_n - q_n) if n < K (from p_n if that is all zero),
 *                  or from p_K if n == K.
 */
int psispec_verify_linear(const void* p_logits, const void* q_logits, int dtype, int64_t B, int32_t K,
                          int32_t V, int32_t* draft_tokens, const psispec_params* params,
                          int32_t* out_tokens, int32_t* out_len, float* out_probs, double* out_resid_mass,
                          void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Linear verification that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Arguments, outputs,
 * rules and errors are those of psispec_verify_linear (same kernels, same
 * bits). The workspace is a fixed device array of
 * PSISPEC_NOALLOC_SCRATCH_BYTES (32 MiB) inside the library. Each GPU the
 * library runs on holds its own copy from the first call on that GPU (the GPU
 * of `stream`, or the current one for NULL) until the process ends.
 *   Limit   the call needs, of psispec_workspace_bytes' layout for
 *           rows_per_req = 2K + 1, the statistics and request records (about
 *           16 B per logit chunk of 32768 (bf16) or 16384 (fp32) logits per
 *           row, plus 32 B per 1024 logits of each request and 16 B per 1024
 *           logits of each row); filtered sampling also needs the kept-set
 *           sections. B = 256, K = 8, V = 151936 bf16 takes about 12 MB;
 *           beyond 32 MiB the call returns PSISPEC_ESCRATCH and enqueues
 *           nothing.
 *   Races   every call on one GPU shares that GPU's array: calls that may
 *           overlap on one GPU (different streams, or different threads'
 *           streams) race and give undefined outputs; order them on one
 *           stream. The kernels initialise everything they read from the
 *           array, so it needs no clearing between calls.
 */
int psispec_verify_linear_noalloc(const void* p_logits, const void* q_logits, int dtype, int64_t B, int32_t K,
                                  int32_t V, int32_t* draft_tokens, const psispec_params* params,
                                  int32_t* out_tokens, int32_t* out_len, float* out_probs, double* out_resid_mass,
                                  hipStream_t stream);

/*
 * Depth of a candidate tree given its HOST parent array (parent[n] in
 * [-1, n-1]; -1 = child of the root). Returns the depth D >= 1, or a negative
 * status for a malformed topology. Pure host function.
 */
int32_t psispec_tree_depth(const int32_t* parent, int32_t N);

/*
 * Tree verification (Uno explainer §3.4 "Tree Sampler": several candidate
 * continuations checked in one verify pass). Verification rule: at a node
 * with children c_0 < c_1 < ... (ascending node id), each child drawn i.i.d.
 * from that node's draft distribution Q, start with r = P; child j is accepted
 * iff U(seed, step, b, row, 1+j) * Q(tok_j) < r(tok_j); after a rejection
 * r <- norm(max(0, r - Q)) (kept unchanged when that is all zero); the walk
 * descends into the first accepted child; at a leaf, or when every child is
 * rejected, the final token is drawn from r with U(seed, step, b, row, 0).
 *   p_logits, q_logits  [B, N+1, V]; row 0 is the root context, row n+1 the
 *                 context after node n.
 *   parent        HOST [N] int32, parent[n] < n, -1 for children of the root;
 *                 shared by every request.
 *   node_tokens   [B, N] int32 candidate token of each node; input, or output
 *                 with PSISPEC_FUSED_DRAFT: node n, the j-th child (ascending
 *                 id) of row r, is then drawn from softmax(filter(q_r / T)) by
 *                 inverse CDF with U(seed, step, b, r, 0x40000000 + j) (argmax
 *                 of q_r in greedy mode), -1 for every node of a request with
 *                 an invalid row. The rule is lossless only for children drawn
 *                 i.i.d. from their row's draft distribution, as these are.
 *   out_tokens    [B, D+1] int32 out (D = psispec_tree_depth): path tokens, the
 *                 final token, then -1 padding.
 *   out_path      [B, D] int32 out: node ids of the accepted path, -1 padding.
 *   out_len       [B] int32 out: accepted path length (or -1 on error).
 */
int psispec_verify_tree(const void* p_logits, const void* q_logits, int dtype, int64_t B, int32_t N,
                        int32_t V, const int32_t* parent, int32_t* node_tokens,
                        const psispec_params* params, int32_t* out_tokens, int32_t* out_path,
                        int32_t* out_len, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Tree Sampler candidates (Uno explainer §3.4 "Tree Sampler": every draft
 * position keeps its top-K tokens and only the most probable prefixes over
 * them are verified in one pass; §6.3 uses block 16, K = 32 and 32 kept
 * prefixes). The pages give no formula; this call computes, per request:
 *   q_i = softmax(q_logits_i / T) over the full row, for position i < K;
 *   C_i = the `cands` tokens of largest q_i (ties: lower id first), rank 0 first;
 *   score(t_0 .. t_{l-1}) = sum_i log q_i(t_i), t_i in C_i, l <= K;
 *   the kept prefixes: the first `nodes` in the order score descending, then
 *   length ascending, then the position of the parent prefix in this same
 *   order (the empty prefix first), then the rank of the last token in C.
 * A parent's score is at least its child's, so the kept set is closed under
 * taking prefixes. Prefixes of probability zero are never kept.
 *   q_logits     [B, K, V] draft logits (K draft positions, K <= 64).
 *   params       temperature > 0 (no greedy mode); top_k / top_p must be
 *                disabled (0 and 1); seed, step and flags are not used.
 *   cands        tokens per position, 1 <= cands <= min(V, PSISPEC_MAX_TOPK),
 *                K * cands <= PSISPEC_MAX_CAND_ENTRIES.
 *   nodes        kept prefixes, 1 <= nodes <= PSISPEC_MAX_TREE_NODES.
 *   out_parent   [B, nodes] int32 out: node n is the n-th kept prefix; its
 *                parent is the node of its prefix one shorter (-1 at length 1),
 *                so out_parent[b, n] < n.
 *   out_tokens   [B, nodes] int32 out: the last token of prefix n.
 * Nodes past the last prefix of positive probability, and every node of a
 * request with an invalid draft row, get -1 in both outputs.
 * Workspace: psispec_workspace_bytes(B, K, V, dtype).
 */
#define PSISPEC_MAX_CAND_ENTRIES 4096 /* K * cands */
int psispec_tree_candidates(const void* q_logits, int dtype, int64_t B, int32_t K, int32_t V,
                            const psispec_params* params, int32_t cands, int32_t nodes, int32_t* out_parent,
                            int32_t* out_tokens, void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * Verification of deterministic candidates, one tree per request (Uno
 * explainer §3.4 "Tree Sampler": the candidates are chosen, not drawn, so the
 * draft-ratio test of psispec_verify_tree does not apply; the pages state no
 * rule for them and this is the plain lossless one for point-mass proposals).
 * At a row with children c_0 < c_1 < ... (ascending node id), r = P =
 * softmax(p_row / T) and E = 0; child j with token tok is accepted iff
 *   U(seed, step, b, row, 1 + j) * (1 - E) < P(tok),
 * with P(tok) counted as 0 when tok was already rejected at this row; after a
 * rejection tok is removed from r (E += P(tok)). The walk descends into the
 * first accepted child; at a leaf, or once every child is rejected, the final
 * token is an inverse-CDF draw in token-id order with U(seed, step, b, row, 0)
 * from P without the removed tokens (from P itself if nothing remains).
 * Greedy mode (T == 0): a child is accepted iff its token is the argmax of the
 * row (lowest id on ties), and the final token is that argmax.
 *   p_logits     [B, N+1, V] target logits; row 0 is the root context, row
 *                n+1 the context after node n.
 *   parent       [B, N] int32, per request: parent[b, n] in [-1, n-1].
 *   node_tokens  [B, N] int32 candidate token of each node.
 *   params       top_k / top_p must be disabled (0 and 1).
 *   out_tokens   [B, N+1] int32 out: path tokens, the final token, -1 padding.
 *   out_path     [B, N] int32 out: node ids of the accepted path, -1 padding.
 *   out_len      [B] int32 out: accepted path length, or -1 for a request
 *                error (a parent outside [-1, n-1], a token outside [0, V),
 *                an invalid target row).
 * Workspace: psispec_workspace_bytes(B, N + 1, V, dtype). N <= 256.
 */
int psispec_verify_tree_det(const void* p_logits, int dtype, int64_t B, int32_t N, int32_t V,
                            const int32_t* parent, const int32_t* node_tokens, const psispec_params* params,
                            int32_t* out_tokens, int32_t* out_path, int32_t* out_len, void* workspace,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Total-variation distillation loss (Uno explainer §3.2, Diffusion
 * Distillation: one forward gives the frozen AR teacher's logits and the
 * diffusion student's; the TV term minimises the total-variation distance of
 * the two token distributions of every position, which governs the verifier's
 * acceptance since sum_v min(p_v, q_v) = 1 - TV).
 *   p_logits     [R, V] teacher logits; q_logits [R, V] student logits.
 *   temperature  > 0: p = softmax(p_logits / T), q = softmax(q_logits / T).
 *   row_weights  nullable [R] float: upstream gradient of each row's loss
 *                (e.g. 1/R for a mean); NULL means 1.
 *   out_loss     [R] double out: 1/2 sum_v |p_v - q_v|.
 *   out_grad     nullable [R, V] out, in the logits' dtype (bf16: rounded to
 *                nearest even): the gradient of w_r * loss_r with respect to
 *                the student logits, w_r q_j (g_j - sum_v g_v q_v) / T with
 *                g_v = sign(q_v - p_v) / 2 (0 where q_v == p_v). The teacher is
 *                frozen and gets no gradient. NULL computes the loss only.
 * p and q are evaluated in binary32 from binary32-grade normalisers (about
 * 1e-7 relative); the loss is accumulated in fp64. A row with a NaN or +inf
 * logit, or entirely -inf, gets a NaN loss and a NaN gradient row.
 * Workspace: psispec_tv_workspace_bytes(R, V, dtype): the statistics and
 * partial sums of the passes, and two bits per logit for the sign of q - p
 * (written by the second pass, read by the gradient pass instead of p).
 */
size_t psispec_tv_workspace_bytes(int64_t R, int32_t V, int dtype);
int psispec_tv_loss(const void* p_logits, const void* q_logits, int dtype, int64_t R, int32_t V, float temperature,
                    const float* row_weights, double* out_loss, void* out_grad, void* workspace, size_t ws_bytes,
                    hipStream_t stream);

/*
 * Linear verification fused with the LM head (Uno explainer §3.1: the AR path
 * and the diffusion path share the base model's output head; §3.3: the
 * verification rule of psispec_verify_linear). The logits are products of
 * hidden states with the vocabulary matrix, p_logits = h_target W^T and
 * q_logits = h_draft W^T, computed on bf16 matrix cores (fp32 accumulation)
 * tile by tile and reduced as they are produced (per row and 128-token chunk,
 * the maximum and the sum of exponentials); the same pass stores the fp32
 * logits in the workspace, from which the final draw reads the residual or
 * bonus rows, so the product is made once.
 *   h_target      [B, K+1, H] bf16 target hidden states (row K: the bonus row).
 *   h_draft       [B, K, H] bf16 draft hidden states.
 *   w_vocab       [V, H] bf16 vocabulary matrix (row v gives token v's logit).
 *   draft_tokens  [B, K] int32 drafts (input).
 *   params        temperature > 0; top_k / top_p disabled; seed, step as for
 *                 psispec_verify_linear, whose decision rules apply unchanged
 *                 to these logits.
 *   out_tokens    [B, K+1], out_len [B]: as psispec_verify_linear.
 * H must be a multiple of 128 and the three inputs 16-byte aligned. The logits
 * carry the fp32 accumulation error of an H-term dot product.
 * Workspace: psispec_lmhead_workspace_bytes(B, K, V), about 4 B (2K + 1) V
 * bytes (the logits of every row), 256-byte aligned.
 */
size_t psispec_lmhead_workspace_bytes(int64_t B, int32_t K, int32_t V);
int psispec_verify_lmhead(const void* h_target, const void* h_draft, const void* w_vocab, int64_t B, int32_t K,
                          int32_t H, int32_t V, const int32_t* draft_tokens, const psispec_params* params,
                          int32_t* out_tokens, int32_t* out_len, void* workspace, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Synthetic order-2 toy language model: a stand-in for the AR target and the
 * diffusion drafter in tests and benchmarks of multi-round generation (it is
 * not part of the method). Logits depend on the last two tokens (t1, t2):
 *   ctx  = (uint32 t1 << 32) | uint32 t2
 *   bits(s, stream, i) = mix(mix(s ^ mix(stream * 0x632BE59BD9B4E019 + 0x2545F4914F6CDD1D))
 *                            ^ (i * 0xD1B54A32D192ED03)),  mix = SplitMix64 (Steele, Lea,
 *                        Flood, OOPSLA 2014)
 *   z(r) = ((sum of the four 16-bit fields of r) / 65536 - 2) * sqrt(3)
 *   target a(v) = float(sd * z(bits(seed, ctx, v)) + (top 10 bits of mix(r) < n_heavy ? boost : 0))
 *   drafter at block position i:
 *          d(v) = float(rho * a(v) + noise * z(bits(seed ^ 0xA5A5A5A55A5A5A5A, ctx * 64 + i, v)))
 * every double operation rounded on its own, then bfloat16 (round to nearest
 * even) or float32.
 */
typedef struct psispec_toy_model {
  uint64_t seed;
  float sd;
  int32_t n_heavy; /* out of 1024 tokens, on average, get the boost */
  float boost;
  float rho;
  float noise;
  uint32_t reserved; /* must be 0 */
} psispec_toy_model;

/*
 * Toy-model logits of `rows` rows into out [rows, V] (dtype): ctx [rows, 2]
 * int32 (t1, t2) and, for kind 1 (drafter), pos [rows] int32 block positions;
 * kind 0 is the target. Device pointers; enqueued on `stream`.
 */
int psispec_toy_logits(int64_t rows, int32_t V, const int32_t* ctx, const int32_t* pos, int kind,
                       const psispec_toy_model* model, int dtype, void* out, hipStream_t stream);

/*
 * Multi-round Psi-Spec generation (Uno explainer §3.3: each round is one draft
 * pass and one verify pass; the block's first position comes from the AR
 * weights and is always kept; the other block - 1 positions are proposed in
 * parallel; the verifier keeps the longest accepted prefix and adds the
 * residual or bonus token, and the rejected drafts are dropped; tokens per
 * forward pass lie in [1, (block + 1) / 2]) on the toy model, all requests in
 * parallel, every step on the device. Round r:
 *   x0    = psispec_draft_sample of the target row at (t1, t2), step + 2r;
 *   d     = psispec_draft_sample of the drafter rows at (t2, x0), positions
 *           1 .. block - 1, step + 2r + 1;
 *   p     = target rows at (h_i, h_{i+1}), h = (t2, x0, d_0 .. d_{block-2});
 *   verify = psispec_verify_linear(p, drafter rows, d), step + 2r + 1;
 *   commit x0, the accepted drafts and the final token; (t1, t2) advance.
 *   params       temperature (0 = greedy), seed and step (top_k / top_p must
 *                be disabled).
 *   prompt       [B, 2] int32 (t1, t2) of each request.
 *   block        2 .. 65 (so block - 1 <= PSISPEC_MAX_K drafts).
 *   out_seq      [B, rounds * (block + 1)] int32 out: the committed tokens, -1 padded.
 *   out_len      [B] int32 out: committed tokens (-1 after a verification error).
 *   out_round_tokens [B, rounds] int32 out: tokens committed by each round.
 * Workspace: psispec_generate_workspace_bytes(B, block, V, dtype).
 */
size_t psispec_generate_workspace_bytes(int64_t B, int32_t block, int32_t V, int dtype);
int psispec_generate_toy(int64_t B, int32_t block, int32_t V, int dtype, const psispec_toy_model* model,
                         const psispec_params* params, const int32_t* prompt, int32_t rounds, int32_t* out_seq,
                         int32_t* out_len, int32_t* out_round_tokens, void* workspace, size_t ws_bytes,
                         hipStream_t stream);

/*
 * Benchmark timing hook (not part of the method; for measuring each kernel of
 * a call live on the caller's stream). While armed with n > 0 caller-created
 * HIP events (timing enabled), every compute entry point launches its i-th
 * kernel (0-based, while 2i + 1 < n) with events[2i] and events[2i + 1] as
 * its start and stop events (hipExtLaunchKernelGGL: the timestamps of the
 * kernel's own dispatch), so hipEventElapsedTime(events[2i], events[2i + 1])
 * is kernel i's execution time, without the gaps between kernels. The events
 * stay owned by the caller and must outlive every armed call. The setting is
 * process-wide and not thread-safe; events == NULL or n <= 0 disarms it.
 */
int psispec_set_timing_events(hipEvent_t* events, int n);

/* Number of events the most recent compute call used while armed (two per
   kernel launch). */
int psispec_timing_count(void);

/* Static message for a status code. */
const char* psispec_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int psispec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PSISPEC_H */
