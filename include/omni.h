/*
 * omni.h - C ABI of libomni.so, the MI355X (gfx950) routed-branch forward of
 * OmniMoE ("OmniMoE: An Efficient MoE by Orchestrating Atomic Experts at
 * Scale", arXiv 2602.05711).
 *
 * The routed branch runs in three calls on one HIP stream:
 *   omni_router          Cartesian Product Router: ids, scores, gates
 *   omni_schedule        expert-centric schedule: sorted tasks, group offsets
 *   omni_expert_forward  Dynamic Expert Assembly: y
 * or in two, with the schedule and the assembly in the form the device picks
 * for the routing: omni_router, then omni_expert_forward_auto.
 * with a dense variant of the assembly for routing in which many tokens share
 * experts, omni_expert_forward_blocked, and one comparison baseline,
 * omni_expert_forward_token_centric.
 * The backward of the branch runs in two more calls:
 *   omni_expert_backward  dx (expert part), d gate, dW and dV of used experts
 *                         (omni_expert_backward_blocked: its blocked form)
 *   omni_router_backward  dW_r, dW_c, and the router part added into dx
 * and the layer's other branch in one:
 *   omni_shared_mlp       the shared dense MLP, added into (or written to) y
 * The router the pages' ablation substitutes is also provided, as a baseline:
 *   omni_dense_router     fully connected router over all N experts
 *
 * Conventions shared by every call
 *   - Every array pointer is DEVICE memory owned by the caller, row-major and
 *     contiguous, with a 16-byte-aligned base.  The library never allocates,
 *     frees or synchronises; scratch memory comes in through (ws, ws_bytes),
 *     sized by omni_workspace_bytes, device memory, 256-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *     enqueued on it; results are ready when the stream reaches that point.
 *   - x, W_r, W_c, W and V share one dtype (omni_dtype).  Arithmetic is fp32
 *     (bf16 values are widened exactly; products accumulate in fp32).
 *   - Arguments are validated on the host before anything is launched; on an
 *     error nothing is enqueued and no output is touched.  omni_last_error()
 *     returns a message for the calling thread's last failed call.
 *     OMNI_ERR_HIP reports a launch error; faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Expert ids in idx must lie in [0, N) (a precondition, not checked on
 *     the device).
 *   - Calls are reentrant; two calls that share output or workspace buffers
 *     must be ordered by the caller (same stream, or events).
 */
#ifndef OMNI_H
#define OMNI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OMNI_ABI_VERSION 10

#if defined(__GNUC__) || defined(__clang__)
#define OMNI_API __attribute__((visibility("default")))
#else
#define OMNI_API
#endif

typedef enum {
  OMNI_OK = 0,
  OMNI_ERR_INVALID_ARG = 1, /* null pointer, non-positive or inconsistent size */
  OMNI_ERR_UNSUPPORTED = 2, /* valid request beyond the compiled limits below */
  OMNI_ERR_WORKSPACE = 3,   /* ws_bytes below omni_workspace_bytes() */
  OMNI_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} omni_status;

typedef enum { OMNI_F32 = 0, OMNI_BF16 = 1 } omni_dtype;

typedef enum {
  OMNI_OP_ROUTER = 0,
  OMNI_OP_SCHEDULE = 1,
  OMNI_OP_EXPERT_FORWARD = 2,
  OMNI_OP_EXPERT_BACKWARD = 3,
  OMNI_OP_ROUTER_BACKWARD = 4,
  OMNI_OP_SHARED_MLP = 5, /* omni_workspace_bytes takes d_ff in its N argument */
  OMNI_OP_DENSE_ROUTER = 6,
  OMNI_OP_EXPERT_FORWARD_BLOCKED = 7,
  OMNI_OP_EXPERT_BACKWARD_BLOCKED = 8,
  OMNI_OP_EXPERT_FORWARD_AUTO = 9,
  OMNI_OP_EXPERT_BACKWARD_AUTO = 10
} omni_op;

/* Compiled limits (OMNI_ERR_UNSUPPORTED beyond them). */
#define OMNI_MAX_GRID_SIDE 4096 /* N_r, N_c */
#define OMNI_MAX_K 512
#define OMNI_MAX_D_BF16 4096 /* d for bf16 inputs */
#define OMNI_MAX_D_F32 2048  /* d for fp32 inputs */

/*
 * omni_router - Cartesian Product Router.
 * Source: OmniMoE digest (paper.rainbus.top), method paragraph, step 2;
 * gist.science resume section 2.2 ("Cartesian product router").
 *
 * For each token t (row of x):
 *   s_r = x_t W_r,  s_c = x_t W_c                       (row / column logits)
 *   p_r = LogSoftmax(s_r),  p_c = LogSoftmax(s_c)
 *   S_ij = p_r[i] + p_c[j] over the implicit N_r x N_c grid (never built)
 *   the K best grid cells under (S descending, n ascending), n = i*N_c + j
 *   gate = softmax of the K selected S
 *
 *   x      [L, d]     dtype dt
 *   Wr     [N_r, d]   dtype dt   row i is grid row i's projection vector
 *   Wc     [N_c, d]   dtype dt   row j is grid column j's projection vector
 *   idx    [L, K]     int32  out  expert ids, each row ordered by (S desc, n asc)
 *   score  [L, K]     fp32   out  S of each selected id
 *   gate   [L, K]     fp32   out  softmax over the row's K scores
 * Requires 1 <= K <= N_r*N_c, K <= OMNI_MAX_K, N_r, N_c <= OMNI_MAX_GRID_SIDE,
 * d % 8 == 0, d <= OMNI_MAX_D_BF16 (bf16) or OMNI_MAX_D_F32 (fp32),
 * L*K < 2^31, N_r*N_c < 2^31.
 * Workspace: fp32 logits [L, N_r + N_c].
 */
OMNI_API omni_status omni_router(const void* x, const void* Wr, const void* Wc,
                        int64_t L, int64_t d, int64_t Nr, int64_t Nc,
                        int64_t K, omni_dtype dt,
                        int32_t* idx, float* score, float* gate,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * omni_schedule - expert-centric scheduling.
 * Source: OmniMoE digest, method paragraph, step 3 (task collection, sort by
 * expert id into contiguous groups of size B, group id primary and token id
 * secondary key); gist.science resume section 2.2 (groups are contiguous
 * ranges of expert ids, tasks sorted by token id inside each group).
 *
 * Task m = t*K + k is (token t, expert idx[m]); its group is idx[m] / B.
 *   perm       [L*K]    int32 out  task ids sorted by (group, token, m)
 *   group_off  [G+1]    int32 out  G = ceil(N/B); group_off[q] = number of
 *                                  tasks whose group is < q, so group q's
 *                                  tasks are perm[group_off[q] .. group_off[q+1])
 *                                  (empty for an inactive group)
 *                                  perm and group_off are both given or both
 *                                  NULL (then only token_order is computed,
 *                                  which is all omni_expert_forward_blocked
 *                                  reads)
 *   token_order [L]     int32 out, optional (NULL: not computed)
 *                                  the tokens stably sorted by the group of
 *                                  their first expert, idx[t*K] / B (ties by
 *                                  token id).  Not part of the pages' method:
 *                                  an execution order for omni_expert_forward's
 *                                  output pass that puts tokens sharing their
 *                                  leading experts side by side; it never
 *                                  changes y.
 * Bit-exact and deterministic.  Requires N >= 1, 1 <= B < 2^31 (every
 * B >= N gives the single group 0), L*K < 2^31, N < 2^31 (and
 * L <= 2^31-8 with token_order); B >= 2^31 is OMNI_ERR_UNSUPPORTED.
 * Workspace: sort buffers, O(L*K) int32.
 */
OMNI_API omni_status omni_schedule(const int32_t* idx, int64_t L, int64_t K,
                          int64_t N, int64_t B,
                          int32_t* perm, int32_t* group_off, int32_t* token_order,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * omni_schedule_noalloc - omni_schedule for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, outputs, checks and results as omni_schedule (bit for
 * bit), without ws / ws_bytes: the sort buffers live in a fixed array of
 * OMNI_SCHEDULE_NOALLOC_MAX_WS bytes inside the library's code object, one
 * copy per GPU, held until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine).  Sizes whose workspace
 * (omni_workspace_bytes(OMNI_OP_SCHEDULE, ...)) exceeds that maximum are
 * refused with OMNI_ERR_UNSUPPORTED before anything is launched: the
 * 80 MiB cover up to about 4.9 million tasks (L*K), e.g. 16384 tokens x
 * K = 256.
 * Every call on one GPU uses that GPU's single array, which keeps whatever
 * the last call left there (every word the kernels read is written earlier
 * in the same call, so nothing needs clearing): two calls that may overlap
 * on one GPU (different streams without an ordering event, or different
 * host threads) race on it and give undefined results.  The first call on a
 * device looks the array's device address up once (hipGetSymbolAddress).
 */
#define OMNI_SCHEDULE_NOALLOC_MAX_WS (80u << 20) /* bytes of scratch per GPU */
OMNI_API omni_status omni_schedule_noalloc(const int32_t* idx, int64_t L, int64_t K,
                                           int64_t N, int64_t B, int32_t* perm,
                                           int32_t* group_off, int32_t* token_order,
                                           void* stream);

/*
 * omni_expert_forward - Dynamic Expert Assembly over the schedule.
 * Source: OmniMoE digest, method paragraph, step 1 (global matrices
 * W = [w_in^0 .. w_in^{N-1}]^T and V likewise; y = (g . sigma(x w_x^T)) v_x)
 * and step 3 (per active group O_q = (G_q . sigma(X_q W_q^T)) V_q);
 * gist.science resume section 2.1.
 *
 *   x     [L, d]  dtype dt
 *   W, V  [N, d]  dtype dt    row e holds atomic expert e's input / output vector
 *   idx   [L, K]  int32       expert ids (from omni_router)
 *   gate  [L, K]  fp32        gates      (from omni_router)
 *   perm  [L*K]   int32       schedule   (from omni_schedule, same B)
 *   group_off [G+1] int32     group offsets (from omni_schedule, same B),
 *                             G = ceil(N/B)
 *   token_order [L] int32     optional (NULL: tokens by id); the order in which
 *                             the output pass visits tokens, each of the 8
 *                             XCDs taking a contiguous eighth (from
 *                             omni_schedule's token_order).  Must be a
 *                             permutation of [0, L): entries outside [0, L)
 *                             are skipped and a token that never appears keeps
 *                             its old y row.  y itself does not depend on it.
 *   B                         group size the schedule was built with
 *                             (1 <= B < 2^31; every B >= N is one group)
 *   y     [L, d]  fp32 out    y_t = sum_k gate[t,k] * SiLU(x_t . W[idx[t,k]]) * V[idx[t,k]]
 *                             fully overwritten (no accumulation into old y)
 * SiLU(h) = h / (1 + exp(-h)).  The activation pass walks the scheduled tasks
 * group by group: the sorted tasks are cut into chunks along the group
 * boundaries that group_off gives (a group larger than a chunk is split), so
 * a group's tasks of one token class run in one wave, one after another, and
 * a W row that several of them use is fetched once; each task's gated
 * activation g * SiLU(x_t . W[e]) is the (G_q . sigma(X_q W_q^T)) factor.
 * The output pass then sums each token's K terms a V[e] in k order without
 * atomics, so y is deterministic.  perm and group_off must be the schedule of
 * this idx with this B (they are read, not checked: other values give other
 * sums, never an out-of-bounds access as long as perm is a permutation of
 * [0, L*K) and group_off is non-decreasing from 0 to L*K).
 * Requires d % 8 == 0, d <= OMNI_MAX_D_BF16 (bf16) or OMNI_MAX_D_F32 (fp32),
 * K <= OMNI_MAX_K, L*K < 2^31, N < 2^31.  Workspace: fp32 activations [L*K]
 * and the chunk starts (omni_workspace_bytes(OMNI_OP_EXPERT_FORWARD, ...,
 * B, ...)).
 */
OMNI_API omni_status omni_expert_forward(const void* x, const void* W, const void* V,
                                const int32_t* idx, const float* gate,
                                const int32_t* perm, const int32_t* group_off,
                                const int32_t* token_order, int64_t L, int64_t d, int64_t N,
                                int64_t K, int64_t B, omni_dtype dt, float* y,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * omni_expert_forward_blocked - the same y as omni_expert_forward, as dense
 * MFMA products over blocks of tokens, for routing in which many tokens share
 * their experts.
 * Source: the assembly O_q = (G_q . sigma(X_q W_q^T)) V_q of the OmniMoE
 * digest, method paragraph, step 3 (gist.science resume section 2.1), with
 * the group formed the other way round: the tokens are cut into blocks of
 * 64 consecutive entries of token_order, and block b's group is the union
 * U_b of its tokens' experts.  Each block computes
 *   A_b = G_b . SiLU(X_b W[U_b]^T)  (G_b: the gates, zero off the tasks)
 *   y_b = A_b V[U_b]
 * so each weight row of the union is read once per block and serves all of
 * the block's tokens.  The W-side product is exact in bf16 x bf16 with fp32
 * accumulation; A enters the V-side product as two bf16 terms (hi + lo,
 * about 16 significant bits); sums are fp32, in an order that differs from
 * omni_expert_forward's, so y agrees with it to fp32 rounding, not bitwise
 * (deterministic run to run).
 *
 *   x, W, V, idx, gate, y   as for omni_expert_forward
 *   token_order [L] int32   a permutation of [0, L) (omni_schedule's
 *                           token_order groups tokens that share experts;
 *                           any permutation gives the same y, at a cost that
 *                           grows with the blocks' union sizes)
 * Requires bf16, d % 256 == 0, K <= OMNI_MAX_K, the K ids of each token
 * distinct (as omni_router returns them), L*K < 2^31, N < 2^31.  Entries of
 * token_order outside [0, L) are skipped (their y rows are not written).
 * Workspace (omni_workspace_bytes(OMNI_OP_EXPERT_FORWARD_BLOCKED)): the
 * unions, the gate and activation tiles at the largest union each block can
 * have (64 * min(64 K, N) entries per block); roughly 8 B * 64 * L * K.
 */
OMNI_API omni_status omni_expert_forward_blocked(const void* x, const void* W, const void* V,
                                                 const int32_t* idx, const float* gate,
                                                 const int32_t* token_order, int64_t L, int64_t d,
                                                 int64_t N, int64_t K, omni_dtype dt, float* y,
                                                 void* ws, size_t ws_bytes, void* stream);

/*
 * omni_expert_forward_auto - the expert-centric schedule and assembly, in the
 * form that suits the step's routing, chosen on the device per call (the
 * host never waits).
 * Source: the schedule and assembly of omni_schedule and omni_expert_forward
 * (OmniMoE digest, method paragraph, steps 1 and 3); the choice answers the
 * digest's weaknesses paragraph, which names grouping efficiency under
 * changing active-expert sets as the open problem of expert-centric
 * scheduling.
 *
 * A first kernel counts the distinct experts among a fixed sample of the
 * tasks (all L*K tasks when there are at most 65536, else tasks
 * i * 2654435761 mod L*K for i < 65536).  When the sample repeats its
 * experts twice or more on average, the blocked form runs: the token order
 * (as omni_schedule's token_order), then omni_expert_forward_blocked over it.
 * Otherwise the pages' schedule runs (perm and group_off with group size B,
 * as omni_schedule, kept in the workspace) and then the per-task passes of
 * omni_expert_forward.  The launches of the form not chosen return at once.
 * y is the same up to the rounding of the form taken (see
 * omni_expert_forward_blocked).  The blocked form is only considered for
 * bf16 inputs with d % 256 == 0.
 *
 *   x, W, V, idx, gate, B, y   as for omni_expert_forward
 *   chosen  [1] int32 out, optional (NULL: not written): 1 when the blocked
 *           form ran, 0 for the schedule and the per-task passes
 * Requires what omni_schedule and omni_expert_forward require, and the K ids
 * of each token distinct (as omni_router returns them).  Workspace
 * (omni_workspace_bytes(OMNI_OP_EXPERT_FORWARD_AUTO, ..., B, ...)): the
 * choice, a bitmap of N bits, and the larger of the two forms' buffers.
 */
OMNI_API omni_status omni_expert_forward_auto(const void* x, const void* W, const void* V,
                                              const int32_t* idx, const float* gate, int64_t L,
                                              int64_t d, int64_t N, int64_t K, int64_t B,
                                              omni_dtype dt, float* y, int32_t* chosen,
                                              void* ws, size_t ws_bytes, void* stream);

/*
 * omni_expert_forward_token_centric - the same y as omni_expert_forward,
 * computed in token-centric order: each token fetches the W and V rows of
 * its own K experts, with no schedule.  This is the execution order that the
 * expert-centric scheduling replaces (makerbund article, section 5: the
 * ablation that reverts to token-centric execution keeps the quality and
 * costs latency); it is provided as the measured baseline for that
 * comparison.  Arguments as for omni_expert_forward, without perm and
 * without workspace.  y is fully overwritten.
 */
OMNI_API omni_status omni_expert_forward_token_centric(const void* x, const void* W,
                                                       const void* V, const int32_t* idx,
                                                       const float* gate, int64_t L, int64_t d,
                                                       int64_t N, int64_t K, omni_dtype dt,
                                                       float* y, void* stream);

/*
 * omni_expert_backward - gradients of the expert assembly for an upstream
 * gradient dy = dLoss/dy.
 * Source: the chain rule of omni_expert_forward's definition (OmniMoE digest,
 * method paragraph, steps 1 and 3: y_t = sum_k g_k sigma(x_t . w_k) v_k,
 * sigma = SiLU).  Per task (t, k, e = idx[t,k]), h = x_t . W[e],
 * u = V[e] . dy_t:
 *   dgate[t,k] = SiLU(h) u
 *   dh         = gate[t,k] u SiLU'(h),  SiLU'(h) = sig(h) (1 + h (1 - sig(h)))
 *   dx_t       = sum_k dh W[e]                    (expert part only)
 *   dW[e]      = sum over e's tasks of dh x_t
 *   dV[e]      = sum over e's tasks of gate SiLU(h) dy_t
 *
 *   x, W, V, idx, gate   as for omni_expert_forward (the forward's routing)
 *   dy      [L, d]  fp32      upstream gradient
 *   dx      [L, d]  fp32 out  expert part of dLoss/dx, fully overwritten
 *   dgate   [L, K]  fp32 out  dLoss/dgate, fully overwritten
 *   uniq    [U_cap] int32 out the experts that have tasks, ascending
 *   n_uniq  [1]     int32 out U, the number of entries of uniq
 *   grad_dt          dtype of the two gradient-row arrays (OMNI_F32, or
 *                    OMNI_BF16: the fp32 sums rounded to nearest even)
 *   dW_rows [U_cap, d] grad_dt out  row r = dLoss/dW[uniq[r]] for r < U
 *   dV_rows [U_cap, d] grad_dt out  row r = dLoss/dV[uniq[r]] for r < U
 * with U_cap = min(N, L*K); rows and entries at or past U are left as they
 * were.  Experts without tasks have zero gradient and no row (a sparse row
 * gradient: dense fp32 dW and dV would be 2*N*d*4 bytes).  Each row is summed
 * by one workgroup over the expert's tasks in (token, k) order, so the
 * result is deterministic.  Writing the rows is most of this call's memory
 * traffic; bf16 rows halve it.  Same size limits as omni_expert_forward,
 * and L <= 2^31-9 (OMNI_ERR_UNSUPPORTED above).
 * Workspace: per-task terms, the tasks sorted by expert id, the per-expert
 * segment table and the order in which the rows are summed
 * (omni_workspace_bytes(OMNI_OP_EXPERT_BACKWARD)).
 */
OMNI_API omni_status omni_expert_backward(const void* x, const void* W, const void* V,
                                          const int32_t* idx, const float* gate, const float* dy,
                                          int64_t L, int64_t d, int64_t N, int64_t K,
                                          omni_dtype dt, float* dx, float* dgate, int32_t* uniq,
                                          int32_t* n_uniq, omni_dtype grad_dt, void* dW_rows,
                                          void* dV_rows, void* ws, size_t ws_bytes,
                                          void* stream);

/*
 * omni_expert_backward_blocked - the same gradients as omni_expert_backward,
 * with the per-token part (dgate, the per-task terms and dx) computed over
 * the blocked assembly's token blocks: for block b (64 consecutive entries
 * of token_order) and the union U_b of its experts,
 *   H = X_b W[U_b]^T,  D = dy_b V[U_b]^T      (dense MFMA products)
 *   at each task: dgate = D SiLU(h), dh = g D SiLU'(h), g SiLU(h)
 *   dx_b = dH W[U_b]                          (dH: dh at the tasks, else 0)
 * dy enters the MFMA products as two bf16 terms (hi + lo, about 16
 * significant bits), dH likewise; sums are fp32.  For routing in which many
 * tokens share experts; on spread-out routing omni_expert_backward is faster.
 *   token_order [L] int32  a permutation of [0, L), as for
 *                          omni_expert_forward_blocked; every token must
 *                          appear once (a token that does not gets no dx row
 *                          or dgate entries, and the dW, dV rows of its
 *                          experts are undefined; entries outside [0, L) are
 *                          skipped, nothing is accessed out of bounds)
 * The dW and dV rows are summed over sets of 64 used experts (ordered by the
 * first position of their tokens in token_order) as dense products with the
 * union of the set's tokens: dW rows = DhT X[T_s], dV rows = GaT dy[T_s],
 * each row written once (deterministic; the summation order differs from
 * omni_expert_backward's, so the rows agree to fp32 rounding).
 * Other arguments, outputs and limits as omni_expert_backward, plus those of
 * omni_expert_forward_blocked (bf16, d % 256 == 0, distinct ids per token)
 * and L <= 524288.
 * Workspace: omni_workspace_bytes(OMNI_OP_EXPERT_BACKWARD_BLOCKED).
 */
OMNI_API omni_status omni_expert_backward_blocked(const void* x, const void* W, const void* V,
                                                  const int32_t* idx, const float* gate,
                                                  const float* dy, const int32_t* token_order,
                                                  int64_t L, int64_t d, int64_t N, int64_t K,
                                                  omni_dtype dt, float* dx, float* dgate,
                                                  int32_t* uniq, int32_t* n_uniq,
                                                  omni_dtype grad_dt, void* dW_rows,
                                                  void* dV_rows, void* ws, size_t ws_bytes,
                                                  void* stream);

/*
 * omni_expert_backward_auto - the gradients of omni_expert_backward, in the
 * form that suits the routing, chosen on the device per call by the rule of
 * omni_expert_forward_auto (the same sample of the tasks, so on the same idx
 * and up to 524288 tokens both passes of a step take the same form; the host
 * never waits).
 * Source: as omni_expert_backward; the choice answers the digest's
 * weaknesses paragraph as omni_expert_forward_auto does.
 *
 * When the sampled tasks repeat their experts twice or more on average, the
 * blocked form runs (omni_expert_backward_blocked) over the tokens stably
 * sorted by their first expert id; otherwise the per-task form
 * (omni_expert_backward).  The launches of the form not chosen return at
 * once.  Both forms share the sort of the tasks by expert.  The outputs are
 * those of omni_expert_backward (the same layout in both forms), equal up to
 * the rounding of the form taken.  The blocked form is only considered for
 * bf16 inputs with d % 256 == 0 and L <= 524288.
 *
 *   arguments as for omni_expert_backward, plus
 *   chosen  [1] int32 out, optional (NULL: not written): 1 when the blocked
 *           form ran, 0 for the per-task form
 * Requires what omni_expert_backward requires, and the K ids of each token
 * distinct (as omni_router returns them).  Workspace
 * (omni_workspace_bytes(OMNI_OP_EXPERT_BACKWARD_AUTO)): the choice, a bitmap
 * of N bits, the token order and its sort, and the blocked form's buffers
 * (which hold the per-task form's).
 */
OMNI_API omni_status omni_expert_backward_auto(const void* x, const void* W, const void* V,
                                               const int32_t* idx, const float* gate,
                                               const float* dy, int64_t L, int64_t d, int64_t N,
                                               int64_t K, omni_dtype dt, float* dx, float* dgate,
                                               int32_t* uniq, int32_t* n_uniq, omni_dtype grad_dt,
                                               void* dW_rows, void* dV_rows, int32_t* chosen,
                                               void* ws, size_t ws_bytes, void* stream);

/*
 * omni_router_backward - gradients of the Cartesian Product Router.
 * Source: the chain rule of omni_router's definition (OmniMoE digest,
 * method paragraph, step 2: s = x W^T, p = LogSoftmax(s), S_ij = p_r[i] +
 * p_c[j], gate = softmax over the K selected S).  The top-K selection is
 * piecewise constant and passes no gradient.  Per token:
 *   dS_k    = gate_k (dgate_k - sum_j gate_j dgate_j)
 *   ds_r[i] = sum of dS_k over the selected ids in grid row i (n = i*N_c + j),
 *   ds_c[j] likewise over grid column j; the LogSoftmax Jacobian's other term,
 *   -softmax(s) * sum_k dS_k, is zero because sum_k dS_k = 0
 *   dW_r = ds_r^T x,  dW_c = ds_c^T x,  dx += ds_r W_r + ds_c W_c
 *
 *   x, Wr, Wc, idx, gate   as for omni_router (idx, gate: its outputs)
 *   dgate   [L, K]  fp32      dLoss/dgate (e.g. from omni_expert_backward)
 *   dx      [L, d]  fp32 in/out  the router part is ADDED to it
 *   dWr     [N_r, d], dWc [N_c, d]  fp32 out, fully overwritten
 * bf16 inputs: ds is split into two bf16 terms (high part and remainder,
 * about 16 significant bits) for the MFMA products, accumulated in fp32.
 * Same size limits as omni_router.  Workspace: the logit gradients and
 * transposed operands (omni_workspace_bytes(OMNI_OP_ROUTER_BACKWARD)).
 */
OMNI_API omni_status omni_router_backward(const void* x, const void* Wr, const void* Wc,
                                          const int32_t* idx, const float* gate,
                                          const float* dgate, int64_t L, int64_t d, int64_t Nr,
                                          int64_t Nc, int64_t K, omni_dtype dt, float* dx,
                                          float* dWr, float* dWc, void* ws, size_t ws_bytes,
                                          void* stream);

/*
 * omni_shared_mlp - the shared dense MLP branch of the layer.
 * Source: OmniMoE digest, method paragraph, step 1 (y = (g . sigma(x w^T)) v
 * + MLP(x)); gist.science resume section 2.1 (a standard dense MLP branch,
 * active for every input).  The pages give no shape; it is read as a SwiGLU
 * block (the digest's SwiGLU remark has no gate vector to act on in an
 * atomic expert):
 *   MLP(x) = (SiLU(x Wg^T) * (x Wu^T)) Wd^T
 *
 *   x       [L, d]      dtype dt
 *   Wg, Wu  [d_ff, d]   dtype dt   gate and up projections
 *   Wd      [d, d_ff]   dtype dt   down projection
 *   y       [L, d] fp32 out: y = MLP(x) when accumulate == 0, y += MLP(x)
 *                       otherwise (after omni_expert_forward this gives the
 *                       whole layer, routed branch + MLP)
 * bf16: products on MFMA with fp32 accumulation; the intermediate
 * SiLU(g) * u is rounded to bf16 before the down projection.  fp32: fp32
 * throughout.  Requires d_ff >= 1; bf16 also needs d % 64 == 0 and
 * d_ff % 64 == 0.  Workspace: the intermediate [L, d_ff]
 * (omni_workspace_bytes(OMNI_OP_SHARED_MLP, ..., N = d_ff, ...)).
 */
OMNI_API omni_status omni_shared_mlp(const void* x, const void* Wg, const void* Wu, const void* Wd,
                                     int64_t L, int64_t d, int64_t d_ff, omni_dtype dt, float* y,
                                     int accumulate, void* ws, size_t ws_bytes, void* stream);

/*
 * omni_dense_router - the fully connected router of the pages' ablation.
 * Source: makerbund article, section 5 (replacing the Cartesian Product
 * Router by a conventional fully connected router raises latency and memory
 * sharply); the router conventions of omni_router otherwise:
 *   s = x Wn^T over all N experts, p = LogSoftmax(s) over the N experts,
 *   top-K under (p desc, n asc), gate = softmax over the K selected p.
 *
 *   x      [L, d]   dtype dt
 *   Wn     [N, d]   dtype dt   one routing vector per expert
 *   idx    [L, K]   int32 out  ids, rows ordered by (score desc, id asc)
 *   score  [L, K]   fp32 out   p at the selected ids
 *   gate   [L, K]   fp32 out   softmax over the K selected scores
 * It costs O(N d) per token against O(sqrt(N) d) for omni_router.  The
 * logits are formed 65536 experts at a time (a [L, 65536] fp32 buffer in the
 * workspace), never for all N at once.  Requires 1 <= K <= min(N,
 * OMNI_MAX_K), N < 2^31; bf16 also needs d % 64 == 0.
 */
OMNI_API omni_status omni_dense_router(const void* x, const void* Wn, int64_t L, int64_t d,
                                       int64_t N, int64_t K, omni_dtype dt, int32_t* idx,
                                       float* score, float* gate, void* ws, size_t ws_bytes,
                                       void* stream);

/*
 * omni_gather_probe - measurement aid, not part of the method: reads the
 * listed rows of a row-major matrix A [n_rows_A, row_bytes] in random order
 * (one wave per row, eight rows in flight, non-temporal loads), as the
 * expert assembly reads the rows of W and V, and writes a checksum per
 * thread to sink.  Timed on the
 * rows a step uses, it gives the gather rate the memory system delivers for
 * that pattern, beside the nominal HBM peak.
 *   rows  [n] int32   row ids; ids outside [0, n_rows_A) are skipped
 *   sink  [sink_floats] fp32 out, at least 256 * min(8192, ceil(n / 32))
 * Requires row_bytes a multiple of 16 in [16, 65536].
 */
OMNI_API omni_status omni_gather_probe(const void* A, int64_t n_rows_A, int64_t row_bytes,
                                       const int32_t* rows, int64_t n, float* sink,
                                       size_t sink_floats, void* stream);

/*
 * omni_workspace_bytes - workspace size needed by one call of `op` with
 * these sizes (arguments an op does not use are ignored).  Writes *out.
 * Returns the same validation status the call itself would return for the
 * sizes (pointers are not checked).
 */
OMNI_API omni_status omni_workspace_bytes(omni_op op, int64_t L, int64_t d, int64_t Nr,
                                 int64_t Nc, int64_t K, int64_t N, int64_t B,
                                 omni_dtype dt, size_t* out);

/* Static description of a status code. */
OMNI_API const char* omni_status_string(omni_status s);

/* Detail message of the calling thread's last failed call ("" if none). */
OMNI_API const char* omni_last_error(void);

/* OMNI_ABI_VERSION of the built library. */
OMNI_API int omni_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* OMNI_H */
