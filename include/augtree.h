/*
 * augtree.h -- C ABI of exact shared-prefix attention on MI355X (gfx950).
 *
 * One attention layer over a replay tree: one prompt of P tokens shared by G response
 * branches ("Splitting Prompt Prefill from Response Replay for Context-Parallel
 * Long-Context LLM Post-Training", Bao et al., §2.1 replay tree; §3.2 Eq. 1 dependency).
 * A prompt token attends causally to the prompt; a token of branch i attends to the whole
 * prompt and causally to branch i, never to a sibling. The prompt is evaluated once
 * (prefill, §3.2); the branches are evaluated against the stationary prompt K/V plus
 * their own K/V (replay, §3.3 MoveQ), and the two partial softmax states are merged
 * exactly (§3.3, Fig. 8). Backward sums every branch's prompt K/V gradient into one
 * prompt gradient (§3.2, equation after Eq. 1) and then adds the prompt queries' own
 * contribution, as the accumulated prompt gradient flows back through the prefill graph.
 *
 * Call order for one layer (§3.2): augtree_prefill_fwd -> augtree_replay_fwd ->
 * augtree_replay_bwd -> augtree_prefill_bwd.
 *
 * Data layout (all device buffers, row-major, contiguous, no strides):
 *   prompt   q_p, o_p, do_p, dq_p          [P][Hq][D]     (dtype)
 *            k_p, v_p, dk_p, dv_p          [P][Hkv][D]    (dtype)
 *   response q_r, o_r, do_r, dq_r          [T_R][Hq][D]   (dtype), branches packed back to back
 *            k_r, v_r, dk_r, dv_r          [T_R][Hkv][D]  (dtype)
 *   lse_p [Hq][P], lse_r [Hq][T_R]         float32, natural log of sum_j exp(scale*q.k_j)
 *   dk_p_acc, dv_p_acc [P][Hkv][D]         float32, branches' summed prompt K/V gradient
 * where T_R = branch_offsets[G] and query head h reads key/value head h / (Hq/Hkv).
 * dtype is float32 or bfloat16; accumulation is always float32 and each bf16 output is
 * rounded once, to nearest even. Every device pointer must be 16-byte aligned.
 *
 * Ownership: the caller allocates every buffer, the workspace included (size from
 * augtree_workspace_bytes). The library allocates no device memory (only the host-side
 * planner call augtree_assign_units uses host scratch of its own), frees and synchronises
 * nothing, keeps
 * no pointer after a call returns, and enqueues all work on `stream` (a hipStream_t; NULL
 * is the null stream). Buffers must stay alive until that work completes.
 *
 * Errors: arguments are validated on the host before anything is enqueued. On an error
 * the call returns a non-zero status and enqueues nothing, except AUGTREE_ERR_HIP, which
 * may follow a partial enqueue. augtree_last_error() then describes the failure (per
 * thread). No C++ exception crosses this interface. The library may be called from several
 * host threads; its only mutable global state is the per-device address table of the static
 * scratch of augtree_replay_fwd_noalloc (filled once per device, under a lock).
 *
 * Results are bitwise reproducible for identical inputs and dims: no floating-point
 * atomics are used anywhere; every reduction runs in a fixed order.
 *
 * Workspaces: every entry point that takes one writes transposed copies of some of its
 * operands there (sequence-contiguous, each branch padded to 64 positions, stored tile by
 * tile: one 32- or 64-position tile of all head_dim rows is one contiguous block), plus the
 * partial results named at the entry point. augtree_workspace_bytes gives the size; the
 * pointer must be 256-byte aligned. The workspace holds nothing between calls.
 */
#ifndef AUGTREE_H
#define AUGTREE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AUGTREE_ABI_VERSION 4
#define AUGTREE_MAX_BRANCHES 128

typedef enum { AUGTREE_F32 = 0, AUGTREE_BF16 = 1 } augtree_dtype;

typedef enum {
  AUGTREE_OK = 0,
  AUGTREE_ERR_INVALID_ARGUMENT = 1, /* bad size, offsets, pointer or alignment */
  AUGTREE_ERR_UNSUPPORTED = 2,      /* valid but not built: head_dim other than 64/128
                                       (64 for float32), Hq*head_dim*element size >= 2^24
                                       bytes per row, or a tensor beyond 2^31 elements */
  AUGTREE_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than required */
  AUGTREE_ERR_HIP = 4               /* a HIP launch or runtime call failed */
} augtree_status;

/* Operation codes for augtree_workspace_bytes: one per entry point that takes a workspace. */
enum { AUGTREE_OP_PREFILL_FWD = 0, AUGTREE_OP_REPLAY_FWD = 1, AUGTREE_OP_REPLAY_BWD = 2,
       AUGTREE_OP_PREFILL_BWD = 3, AUGTREE_OP_REPLAY_PROMPT_BWD = 4,
       AUGTREE_OP_REPLAY_PROMPT_FWD = 5, AUGTREE_OP_REPLAY_LOCAL_FWD = 6,
       AUGTREE_OP_REPLAY_LOCAL_BWD = 7, AUGTREE_OP_REPLAY_DQ = 8, AUGTREE_OP_PREFILL_KV_BWD = 9,
       AUGTREE_OP_PREFILL_DQ = 10, AUGTREE_OP_REPLAY_PROMPT_DQ = 11,
       AUGTREE_OP_REPLAY_LOCAL_DQ = 12 };

/* Most partial states augtree_merge_partials accepts in one call. */
#define AUGTREE_MAX_PARTS 8

/* Sizes of one replay tree. Only branch_offsets is a HOST pointer. */
typedef struct {
  int32_t prompt_len;             /* P >= 1 */
  int32_t num_branches;           /* 1 <= G <= AUGTREE_MAX_BRANCHES */
  const int32_t *branch_offsets;  /* host, G+1 entries: [0] = 0, strictly increasing (every
                                     branch has >= 1 token), [G] = T_R; branch i is packed
                                     rows [offsets[i], offsets[i+1]) */
  int32_t num_q_heads;            /* Hq >= 1 */
  int32_t num_kv_heads;           /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;               /* D: 64 or 128 */
  float softmax_scale;            /* > 0 and finite; attention uses softmax(scale*QK^T) */
  int32_t dtype;                  /* augtree_dtype of Q, K, V, O, dO and every gradient */
} augtree_dims;

/* Causal attention of the prompt over itself, computed once for all branches (§3.2,
 * shared prompt prefill; attention definition §2.2).
 * in:  q_p [P][Hq][D], k_p/v_p [P][Hkv][D]   out: o_p [P][Hq][D], lse_p [Hq][P].
 * Workspace: augtree_workspace_bytes(dims, AUGTREE_OP_PREFILL_FWD) (a transposed V). */
augtree_status augtree_prefill_fwd(const augtree_dims *dims, const void *q_p, const void *k_p,
                                   const void *v_p, void *o_p, float *lse_p, void *ws,
                                   size_t ws_bytes, void *stream);

/* Response replay against the stationary prompt K/V (§3.3 MoveQ; §3.2 response replay
 * with the cached prompt state): every branch row attends to all P prompt keys (one dense
 * partial state per row), then causally to its own branch (a second partial state); the
 * two states are merged by the log-sum-exp rule of §3.3 (Fig. 8).
 * in:  k_p/v_p [P][Hkv][D], q_r [T_R][Hq][D], k_r/v_r [T_R][Hkv][D]
 * out: o_r [T_R][Hq][D], lse_r [Hq][T_R].
 * Workspace: the two partial states (2 * T_R*Hq*(D+1) floats) and transposed V copies. */
augtree_status augtree_replay_fwd(const augtree_dims *dims, const void *k_p, const void *v_p,
                                  const void *q_r, const void *k_r, const void *v_r, void *o_r,
                                  float *lse_r, void *ws, size_t ws_bytes, void *stream);

/* Backward of augtree_replay_fwd for the loss sum(o_r * do_r) (§3.3: gradients return to
 * the query and K/V owners; §3.2: prompt K/V gradient summed over branches).
 * in:  k_p, v_p, q_r, k_r, v_r, o_r, lse_r (as produced by augtree_replay_fwd), do_r
 * out: dq_r [T_R][Hq][D], dk_r/dv_r [T_R][Hkv][D] (own-branch contributions; complete),
 *      dk_p_acc/dv_p_acc [P][Hkv][D] float32: the sum over all branches and all query
 *      heads of each group of the prompt K/V gradient (overwritten, not accumulated into).
 * Workspace: row statistics, transposed Q/dO/K copies and, when the prompt has few key
 * tiles, split partial sums. */
augtree_status augtree_replay_bwd(const augtree_dims *dims, const void *k_p, const void *v_p,
                                  const void *q_r, const void *k_r, const void *v_r,
                                  const void *o_r, const float *lse_r, const void *do_r,
                                  void *dq_r, void *dk_r, void *dv_r, float *dk_p_acc,
                                  float *dv_p_acc, void *ws, size_t ws_bytes, void *stream);

/* Backward of augtree_prefill_fwd for the loss sum(o_p * do_p), with the branches'
 * prompt K/V gradient added in (§3.2: accumulated prompt gradients flow back through the
 * prefill graph).
 * in:  q_p, k_p, v_p, o_p, lse_p (as produced by augtree_prefill_fwd), do_p,
 *      dk_p_acc/dv_p_acc from augtree_replay_bwd, or both NULL (no branches: plain causal
 *      attention backward)
 * out: dq_p [P][Hq][D], dk_p/dv_p [P][Hkv][D] = prompt queries' contribution + acc,
 *      rounded once to dtype.
 * Workspace: row statistics, transposed Q/dO/K copies and, when the prompt dK/dV walk is
 * cut into row chunks (prompts with few key tiles, or long prompts), the chunks' float32
 * partial sums (2 * chunks * P*Hkv*D floats, at most 16 chunks). */
augtree_status augtree_prefill_bwd(const augtree_dims *dims, const void *q_p, const void *k_p,
                                   const void *v_p, const void *o_p, const float *lse_p,
                                   const void *do_p, const float *dk_p_acc,
                                   const float *dv_p_acc, void *dq_p, void *dk_p, void *dv_p,
                                   void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same computation, kernels and results as
 * augtree_replay_fwd (bitwise), but the workspace is a static array of the library's code
 * object, AUGTREE_NOALLOC_SCRATCH_BYTES per GPU, reserved on each GPU the library runs on
 * until the process ends. The caller still passes inputs and outputs (device pointers, as
 * for augtree_replay_fwd); the call allocates and frees nothing. The current device
 * (hipGetDevice) must be the device of the buffers and of `stream`; its scratch address is
 * looked up on the first call on that device.
 * Every call on one GPU shares that GPU's scratch, and the scratch keeps the last call's
 * contents (nothing in it needs to start at zero: every byte read is first written by the
 * same call). Calls that overlap in time on one GPU (several streams, or several host
 * threads) race on the scratch and give undefined results: serialise them.
 * Errors: as augtree_replay_fwd; AUGTREE_ERR_WORKSPACE (before anything is enqueued) when
 * the tree needs more scratch than AUGTREE_NOALLOC_SCRATCH_BYTES, i.e. when
 * augtree_workspace_bytes(dims, AUGTREE_OP_REPLAY_FWD) exceeds it (about 2*T_R*Hq*(D+1)*4
 * bytes plus two transposed V copies: T_R*Hq up to about 2.5e5 at D = 128). */
#define AUGTREE_NOALLOC_SCRATCH_BYTES (256u << 20)
augtree_status augtree_replay_fwd_noalloc(const augtree_dims *dims, const void *k_p,
                                          const void *v_p, const void *q_r, const void *k_r,
                                          const void *v_r, void *o_r, float *lse_r,
                                          void *stream);

/* ---------------------------------------------------------------------------------------
 * Single steps. The four calls above are compositions of these (each launches one kernel,
 * augtree_replay_prompt_bwd one or two):
 *   replay_fwd  = replay_prompt_fwd(0, P) + replay_local_fwd + merge_partials(2 parts)
 *   replay_bwd  = row_dot(T_R rows) + replay_prompt_bwd(0, P) + replay_local_bwd + replay_dq
 *   prefill_bwd = row_dot(P rows) + prefill_kv_bwd + prefill_dq
 * and, in the prompt-K/V shard layout, replay_dq = sum_parts(replay_prompt_dq per shard range
 * + replay_local_dq) up to float32 rounding.
 * A prompt key range [key_begin, key_end) lets one call act as one stationary prompt-K/V
 * shard of §3.3 MoveQ: the shard's partial states are later merged per query row.
 * Each step with a workspace takes the size of its own AUGTREE_OP_* code.
 * Partial states are (normalised output, LSE) pairs: o_part [T_R][Hq][D] float32 and
 * lse_part [Hq][T_R]; a row with no visible key in the range has lse = -inf and o = 0.
 * rowdot [Hq][rows] float32 is sum_d dO[r][h][d] * O[r][h][d] of the saved outputs.
 * --------------------------------------------------------------------------------------- */

/* Partial state of every branch row over prompt keys [key_begin, key_end), no mask
 * (§3.3 MoveQ: a stationary prompt K/V shard evaluates all branch queries).
 * 0 <= key_begin < key_end <= P. Workspace: augtree_range_workspace_bytes(dims,
 * AUGTREE_OP_REPLAY_PROMPT_FWD, key_begin, key_end) (a transposed copy of the range's V). */
augtree_status augtree_replay_prompt_fwd(const augtree_dims *dims, const void *k_p,
                                         const void *v_p, const void *q_r, int32_t key_begin,
                                         int32_t key_end, float *o_part, float *lse_part,
                                         void *ws, size_t ws_bytes, void *stream);

/* Partial state of every branch row over its own branch, causally (§3.2, Eq. 1: a branch
 * token sees its own earlier tokens and itself, never a sibling).
 * Workspace: AUGTREE_OP_REPLAY_LOCAL_FWD. */
augtree_status augtree_replay_local_fwd(const augtree_dims *dims, const void *q_r,
                                        const void *k_r, const void *v_r, float *o_part,
                                        float *lse_part, void *ws, size_t ws_bytes,
                                        void *stream);

/* Exact merge of num_parts (1..AUGTREE_MAX_PARTS) partial states per branch row (§3.3,
 * Fig. 8: states along a query row are combined by the log-sum-exp rule, not by
 * averaging normalised outputs). o_parts/lse_parts are HOST arrays of device pointers.
 * out: o_r [T_R][Hq][D] (dtype), lse_r [Hq][T_R]. Parts are combined in index order. */
augtree_status augtree_merge_partials(const augtree_dims *dims, int32_t num_parts,
                                      const float *const *o_parts,
                                      const float *const *lse_parts, void *o_r, float *lse_r,
                                      void *stream);

/* rowdot[h][r] = sum_d d_o[r][h][d] * o[r][h][d] for rows = P (prompt) or T_R (branches);
 * the row statistic of the softmax backward. */
augtree_status augtree_row_dot(const augtree_dims *dims, int32_t rows, const void *o,
                               const void *d_o, float *rowdot, void *stream);

/* Prompt K/V gradient from every branch row, for prompt keys [key_begin, key_end): writes
 * rows [key_begin, key_end) of dk_p_acc/dv_p_acc [P][Hkv][D] float32 with the sum over all
 * branches and over the query heads of each group (§3.2, equation after Eq. 1), in a fixed
 * order. Workspace: augtree_range_workspace_bytes(dims, AUGTREE_OP_REPLAY_PROMPT_BWD,
 * key_begin, key_end): transposed Q/dO copies, row statistics and, when the range has few key
 * tiles, split partial sums (their count depends on dims and range only). */
augtree_status augtree_replay_prompt_bwd(const augtree_dims *dims, const void *k_p,
                                         const void *v_p, const void *q_r, const float *lse_r,
                                         const float *rowdot_r, const void *do_r,
                                         int32_t key_begin, int32_t key_end, float *dk_p_acc,
                                         float *dv_p_acc, void *ws, size_t ws_bytes,
                                         void *stream);

/* dK/dV of the branch keys (own-branch rows only, causal): dk_r/dv_r [T_R][Hkv][D].
 * Workspace: AUGTREE_OP_REPLAY_LOCAL_BWD. */
augtree_status augtree_replay_local_bwd(const augtree_dims *dims, const void *q_r,
                                        const void *k_r, const void *v_r, const float *lse_r,
                                        const float *rowdot_r, const void *do_r, void *dk_r,
                                        void *dv_r, void *ws, size_t ws_bytes, void *stream);

/* dQ of every branch row over the whole prompt and its own branch: dq_r [T_R][Hq][D].
 * Workspace: AUGTREE_OP_REPLAY_DQ. */
augtree_status augtree_replay_dq(const augtree_dims *dims, const void *k_p, const void *v_p,
                                 const void *q_r, const void *k_r, const void *v_r,
                                 const float *lse_r, const float *rowdot_r, const void *do_r,
                                 void *dq_r, void *ws, size_t ws_bytes, void *stream);

/* dQ of every branch row over prompt keys [key_begin, key_end) only, as float32 partial sums
 * dq_part [T_R][Hq][D] (§3.3 MoveQ: a stationary prompt-K/V shard returns each query's gradient
 * share to the query's owner through the reverse communication of its custom autograd
 * operator). lse_r and rowdot_r are the rows' full statistics (over all their keys), so the
 * shards' partials plus the own-branch partial add up to dQ; augtree_sum_parts adds them in
 * a fixed order. 0 <= key_begin < key_end <= P. Workspace: augtree_range_workspace_bytes(dims,
 * AUGTREE_OP_REPLAY_PROMPT_DQ, key_begin, key_end) (a transposed copy of the range's K). */
augtree_status augtree_replay_prompt_dq(const augtree_dims *dims, const void *k_p, const void *v_p,
                                        const void *q_r, const float *lse_r, const float *rowdot_r,
                                        const void *do_r, int32_t key_begin, int32_t key_end,
                                        float *dq_part, void *ws, size_t ws_bytes, void *stream);

/* dQ of every branch row over its own branch keys only (causal, §3.2 Eq. 1), as float32
 * partial sums dq_part [T_R][Hq][D]. Workspace: AUGTREE_OP_REPLAY_LOCAL_DQ (a transposed K_R). */
augtree_status augtree_replay_local_dq(const augtree_dims *dims, const void *q_r, const void *k_r,
                                       const void *v_r, const float *lse_r, const float *rowdot_r,
                                       const void *do_r, float *dq_part, void *ws, size_t ws_bytes,
                                       void *stream);

/* out [rows][Hq][D] (dtype) = sum of num_parts (1..AUGTREE_MAX_PARTS) float32 partials of the
 * same layout, added in index order and rounded once; rows = P or T_R. parts is a HOST array of
 * device pointers. Used for the dQ partials of several prompt-K/V shards plus the own-branch
 * partial. */
augtree_status augtree_sum_parts(const augtree_dims *dims, int32_t rows, int32_t num_parts,
                                 const float *const *parts, void *out, void *stream);

/* Prompt dK/dV: the prompt queries' causal contribution plus dk_p_acc/dv_p_acc (or
 * nothing when both are NULL), rounded once: dk_p/dv_p [P][Hkv][D] (dtype).
 * Workspace: AUGTREE_OP_PREFILL_KV_BWD. */
augtree_status augtree_prefill_kv_bwd(const augtree_dims *dims, const void *q_p,
                                      const void *k_p, const void *v_p, const float *lse_p,
                                      const float *rowdot_p, const void *do_p,
                                      const float *dk_p_acc, const float *dv_p_acc, void *dk_p,
                                      void *dv_p, void *ws, size_t ws_bytes, void *stream);

/* dQ of the prompt rows (causal over the prompt): dq_p [P][Hq][D].
 * Workspace: AUGTREE_OP_PREFILL_DQ. */
augtree_status augtree_prefill_dq(const augtree_dims *dims, const void *q_p, const void *k_p,
                                  const void *v_p, const float *lse_p, const float *rowdot_p,
                                  const void *do_p, void *dq_p, void *ws, size_t ws_bytes,
                                  void *stream);

/* ---------------------------------------------------------------------------------------
 * Replay-unit assignment of the online planner (§3.4, "Replay units and grid assignment"):
 * place num_units replay units (one complete response path each) with work estimates w on a
 * grid of `rounds` response-replay rounds x `lanes` replay lanes per round, every cell holding
 * at least one unit, minimising  sum over rounds of (largest lane load in the round).
 * Exact (dynamic programming over subsets of units) when num_units <= exact_max, otherwise
 * largest-first greedy: units by decreasing weight (equal weights: lower index first), each to
 * the cell whose use raises the objective least, empty cells first while any remain (equal
 * rises: the less loaded cell, then the lower cell index).
 * in:  w HOST [num_units], finite and >= 0; rounds, lanes >= 1; rounds * lanes <= num_units;
 *      0 <= exact_max <= AUGTREE_ASSIGN_EXACT_MAX (the exact path takes about
 *      (rounds + lanes) * 3^num_units / 2 steps and 12 * lanes * 2^num_units bytes of host
 *      memory).
 * out: cell HOST [num_units]: round * lanes + lane of each unit; *cost: the objective.
 * Errors: AUGTREE_ERR_INVALID_ARGUMENT for a NULL pointer, a size out of range, fewer units
 * than cells, a negative or non-finite weight, or host memory running out on the exact path;
 * nothing is written then.
 * Host only: touches no device memory or stream. Deterministic for identical inputs. */
#define AUGTREE_ASSIGN_EXACT_MAX 16
augtree_status augtree_assign_units(const double *w, int32_t num_units, int32_t rounds,
                                    int32_t lanes, int32_t exact_max, int32_t *cell,
                                    double *cost);

/* Bytes of workspace operation `op` (AUGTREE_OP_*) needs for `dims`; 0 for invalid dims.
 * For the ops that take a prompt key range this covers every range. */
size_t augtree_workspace_bytes(const augtree_dims *dims, int op);

/* Bytes of workspace one call of `op` over prompt keys [key_begin, key_end) needs: a
 * stationary prompt-K/V shard of §3.3 (MoveQ) sizes its own workspace with this. Never more
 * than augtree_workspace_bytes(dims, op). For ops without a key range it equals
 * augtree_workspace_bytes. 0 for invalid dims or an empty or out-of-range key range.
 * Host only. */
size_t augtree_range_workspace_bytes(const augtree_dims *dims, int op, int32_t key_begin,
                                     int32_t key_end);

/* Static text of a status code. */
const char *augtree_status_string(augtree_status status);

/* Detail of the last failed call on the calling thread ("" if none). */
const char *augtree_last_error(void);

/* AUGTREE_ABI_VERSION of the built library. */
int augtree_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AUGTREE_H */
