/*
 * harts.h -- C ABI of the MI355X (gfx950) tree-packed chunkwise gated-delta
 * path: rollout trajectories -> compact tokens -> minimum-call packed rounds
 * -> per-round chunkwise gated-delta forward / backward with state handoffs
 * -> per-position log-probabilities.
 *
 * Sources (HARTS, arXiv 2608.28158; cited by page and section):
 *   [blog]   close-reading blog (inkeast.github.io), sections 3.2, 4.2, 4.3, 4.4
 *   [plsum]  paperlayer.ai summary of v1, sections 3 and 4
 *   [tla]    thelatestinai.com page: Figures 1, 2, C.1
 *
 * Conventions for every entry point
 *   - Return value: HARTS_OK (0) or a negative HARTS_E* code; nothing is
 *     thrown across the ABI.  harts_last_error() returns a thread-local
 *     message describing the last failure of the calling thread.
 *   - Host calls (tree, plan) are synchronous and thread-safe per handle.
 *   - Device calls only enqueue work on the caller's HIP stream (hipStream_t
 *     passed as void*, NULL = the null stream); they never synchronise.
 *   - Device buffers are allocated by the caller and passed as raw device
 *     pointers with their sizes; the library never frees them.  Opaque handles
 *     are owned by the library and released by the matching *_free call.
 *   - Dense tensors are row-major, token-major: q, k, g [N, H, dk]; v, o
 *     [N, H, dv]; beta [N, H]; states [n, H, dk, dv] (float32).  N is the
 *     number of compact rows C for tree plans, the total token count for
 *     varlen plans.  q and k are used as given (no normalisation, no scale).
 *   - NaN / Inf in inputs are not checked; they propagate.
 */
#ifndef HARTS_H
#define HARTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HARTS_OK 0
#define HARTS_EINVAL (-1)  /* bad shape, dtype, size or argument */
#define HARTS_ERANGE (-2)  /* an index or offset outside its range */
#define HARTS_ENOMEM (-3)  /* host or device allocation failed */
#define HARTS_EHIP (-4)    /* a HIP runtime call failed */
#define HARTS_ESTATE (-5)  /* handle in the wrong state for this call */

#define HARTS_DTYPE_BF16 0
#define HARTS_DTYPE_FP32 1

typedef struct harts_tree harts_tree;
typedef struct harts_plan harts_plan;
typedef struct harts_dev_plan harts_dev_plan;

/* ---------------------------------------------------------------- trajectories -> compact tokens
 * [blog 3.2] semantic positions s = (x, i) and compact tokens C with the map
 * m: S -> C; [plsum 3] trajectories are sorted lexicographically (stable) and
 * merged into a compressed trie whose unique nodes are the compact tokens.
 *
 * tokens: host int32 [traj_offsets[n_traj]], trajectories concatenated.
 * traj_offsets: host int64 [n_traj + 1], non-decreasing, traj_offsets[0] = 0.
 * Trajectories may repeat, be prefixes of one another and come in any order;
 * the semantic order S is the caller's order.  An empty trajectory, n_traj < 1
 * or decreasing offsets give HARTS_EINVAL.
 */
int harts_tree_build(const int32_t *tokens, const int64_t *traj_offsets, int64_t n_traj, harts_tree **out);

/* S (semantic positions), C (compact tokens), fork-free segments and forks. */
int harts_tree_stats(const harts_tree *tree, int64_t *S, int64_t *C, int64_t *n_segments, int64_t *n_forks);

void harts_tree_free(harts_tree *tree);

/* ---------------------------------------------------------------- minimum-call round plan
 * [blog 4.2] segment tree (segment = maximal fork-free token path); packed
 * chunkwise calls with at most one direct continuation per fork; T_pre/T_in
 * bottom-up recursion (leaves = 1, minimum calls = T_pre(root)), top-down
 * recovery; a side branch restarts at a(p) = B*floor(p/B) and replays [a(p), p).
 * [blog 4.3] compact layout: round-major, sequences contiguous, replay rows
 * and requested boundary states addressable.  [tla Figure 2] three boundary
 * cases.
 *
 * chunk_B must be 16, 32 or 64 (HARTS_EINVAL otherwise).
 */
int harts_plan_create(const harts_tree *tree, int32_t chunk_B, harts_plan **out);

/*
 * A plan for independent packed sequences (no tree, no replay): one round.
 * cu_seqlens: host int64 [n_seq + 1] (lengths >= 1).  has_init: host uint8
 * [n_seq] or NULL; sequence i starts from init_states[i] when has_init[i] != 0,
 * from zero otherwise.  emit_boundaries != 0 requests the state after every
 * multiple of chunk_B inside each sequence (in (0, L_i], sequence-major,
 * chunk order); harts_plan_boundary_offsets() gives where each sequence's
 * states start.
 */
int harts_plan_create_varlen(const int64_t *cu_seqlens, int64_t n_seq, int32_t chunk_B, const uint8_t *has_init,
                             int32_t emit_boundaries, harts_plan **out);

typedef struct {
  int64_t S, C;           /* semantic positions, compact rows (= N) */
  int32_t chunk_B;
  int32_t n_rounds;       /* packed calls per layer pass = minimum calls for trees */
  int32_t min_calls;      /* T_pre(root) (trees); 1 for varlen plans */
  int32_t n_sequences;    /* = number of leaves for trees */
  int32_t n_slots;        /* handed-off boundary states (trees) */
  int32_t n_boundaries;   /* emitted boundary states (varlen plans) */
  int64_t replay_total;   /* sum of replay lengths (= forced replay R) */
  int64_t n_chunks;       /* chunks over all rounds */
  int64_t n_vrows;        /* virtual rows (own + replay) over all rounds */
} harts_plan_info_t;

int harts_plan_info(const harts_plan *plan, harts_plan_info_t *out);

/*
 * Host copies of the maps [blog 3.2, 4.4]: m int64 [S] (semantic position ->
 * compact row), q int32 [C] (multiplicity, sum = S), node_to_row int64 [C]
 * (trie node in DFS preorder, children by token id -> compact row).  Any
 * pointer may be NULL.  Varlen plans: m and node_to_row are the identity.
 */
int harts_plan_maps(const harts_plan *plan, int64_t *m, int32_t *q, int64_t *node_to_row);

/* One packed sequence of the plan (host view). */
typedef struct {
  int32_t round;       /* 1-based round (packed call) */
  int32_t init_slot;   /* slot of the initial state, -1 = zero state (varlen: index into init states) */
  int64_t start;       /* absolute position of the virtual stream's first token = a(s_head) */
  int64_t row_begin;   /* own compact rows [row_begin, row_end) */
  int64_t row_end;
  int64_t replay_off;  /* replay rows [replay_off, replay_off + n_replay) of harts_plan_replay_rows() */
  int32_t n_replay;    /* < chunk_B */
  int32_t n_emits;     /* emitted states [emit_off, emit_off + n_emits) of harts_plan_emits() */
  int64_t emit_off;
} harts_seq_view;

/* seqs: host [n_sequences], ordered by round, then head segment DFS preorder. */
int harts_plan_sequences(const harts_plan *plan, harts_seq_view *seqs);
/* rows: host int64 [replay_total]: compact rows replayed, per sequence in path order. */
int harts_plan_replay_rows(const harts_plan *plan, int64_t *rows);
/* Emitted states: boundary index (local chunk boundary, >= 1) and target
 * (slot id for trees, boundary-state index for varlen plans); host int32 [total emits]. */
int harts_plan_emits(const harts_plan *plan, int32_t *boundary, int32_t *target);
/* Varlen plans with emit_boundaries: host int64 [n_seq + 1]. */
int harts_plan_boundary_offsets(const harts_plan *plan, int64_t *offsets);

/*
 * Host view of one round (one packed call) [blog 4.2, 4.3]: its sequences in launch order, with
 * their own compact rows, the absolute position their virtual stream starts at, the rows they
 * replay, their initial state and the states they emit.  r is 0-based (< n_rounds, else
 * HARTS_EINVAL).  The arrays belong to the plan and stay valid until harts_plan_free; the call
 * is thread-safe.
 */
typedef struct {
  int32_t n_seq;
  const int64_t *row_start, *row_end; /* own compact rows [row_start[i], row_end[i]) */
  const int64_t *abs_start;           /* absolute position of the first (replayed or own) token */
  const int64_t *replay_off;          /* [n_seq + 1]: sequence i replays replay_rows[replay_off[i] ..) */
  const int64_t *replay_rows;         /* compact rows replayed, per sequence in path order */
  const int32_t *init_slot;           /* slot (trees) or init-state index (varlen) of the initial state, -1 = zero */
  const int64_t *emit_off;            /* [n_seq + 1] into emit_chunk and emit_slot */
  const int32_t *emit_chunk;          /* local chunk boundary (>= 1) after which a state is emitted */
  const int32_t *emit_slot;           /* its target: slot id (trees) or boundary-state index (varlen) */
} harts_round_view;

int harts_plan_round(const harts_plan *plan, int32_t r, harts_round_view *out);

void harts_plan_free(harts_plan *plan);

/* ---------------------------------------------------------------- device plan
 * Uploads the per-round descriptors (virtual-row gather lists, chunk and
 * sequence tables, emit targets) for heads H and key / value width dk, dv on
 * the given stream, and records the workspace size the device calls need.
 * dk, dv in {16, 32, 64, 128}; dtype HARTS_DTYPE_BF16 (dk = dv = 128 or 64 with
 * chunk_B = 64; dk = dv = 64 or 32 with chunk_B = 32) or HARTS_DTYPE_FP32
 * (dk = dv = 16 with chunk_B = 16, dk = dv = 32 with chunk_B = 32).  The descriptor memory belongs to the
 * handle (hipMalloc here, hipFree in harts_dev_plan_free).
 */
int harts_plan_upload(const harts_plan *plan, int32_t H, int32_t dk, int32_t dv, int32_t dtype, void *stream,
                      harts_dev_plan **out);

/* Bytes of caller-provided device workspace for harts_kda_fwd (backward = 0),
 * harts_kda_bwd (backward = 1), or a forward/backward pair with keep = 1
 * (backward = 2; the same size as 1).  Other values: HARTS_EINVAL. */
int harts_kda_workspace_size(const harts_dev_plan *dplan, int32_t backward, size_t *bytes);

void harts_dev_plan_free(harts_dev_plan *dplan);

/* ---------------------------------------------------------------- gated-delta forward
 * [blog 1.2, 4.3] one packed varlen chunkwise call per round: the root starts
 * from the zero state, other sequences from boundary states returned by
 * earlier rounds; replay (< B ancestor tokens) updates only the state and
 * writes no outputs; requested boundary states {S[c]} are materialised
 * (equation 16, cited not printed).  Per token (equation 1, cited not printed;
 * KDA-style gated delta rule, per head):
 *     S'_t = diag(exp(g_t)) S_{t-1};  S_t = S'_t - beta_t k_t (k_t^T S'_t - v_t^T);  o_t = S_t^T q_t
 *
 * q, k, g, v, beta, o: device, dtype of the device plan (beta [N, H]).
 * states: device float32 [n_slots, H, dk, dv] for tree plans (written for
 *   every produced slot, read for every consumed one); for varlen plans the
 *   emitted boundary states [n_boundaries, H, dk, dv] (NULL if not requested).
 * init_states: varlen plans only, device float32 [n_seq, H, dk, dv] read for
 *   sequences with has_init != 0 (NULL when none).
 * final_states: varlen plans only, device float32 [n_seq, H, dk, dv] or NULL.
 * workspace: device, >= harts_kda_workspace_size(dplan, keep ? 2 : 0, ...) bytes.
 * keep (0 or 1): 1 makes the forward also write, into the workspace, every
 *   round's per-chunk backward operands and every chunk-start state, so that a
 *   following harts_kda_bwd with keep = 1 on the same inputs, states and
 *   workspace (untouched in between) skips the per-round preparation and state
 *   recompute.  Results are the same either way.  Honoured for the bf16
 *   configurations; elsewhere both calls recompute as with keep = 0.  The
 *   device plan records the workspace of its last forward with keep = 1 (a
 *   forward without keep on that workspace clears the record); harts_kda_bwd
 *   with keep = 1 on any other workspace returns HARTS_EINVAL.  That the inputs
 *   are the same is the caller's contract.
 */
typedef struct {
  const void *q, *k, *v, *g, *beta;
  void *o;
  float *states;
  const float *init_states;
  float *final_states;
  void *workspace;
  size_t workspace_bytes;
  int32_t keep;
} harts_kda_io;

int harts_kda_fwd(const harts_dev_plan *dplan, const harts_kda_io *io, void *stream);

/*
 * The flat packed call in one function [blog 1.2, 4.3]: independent sequences (no tree, no
 * replay) given by host cu_seqlens [n_seq + 1] (lengths >= 1, else HARTS_EINVAL before any device
 * work, as for harts_plan_create_varlen), one round, from the zero state or from
 * init_states[i] where init_mask[i] != 0 (init_mask host uint8 [n_seq], or NULL: every sequence
 * with init_states != NULL starts from it), writing o and, when boundary_states != NULL, the state
 * after every multiple of chunk_B inside each sequence (sum_i floor(L_i / chunk_B) states,
 * sequence-major, chunk order; boundary_offsets, host int64 [n_seq + 1] or NULL, receives where
 * each sequence's states start) and, when final_states != NULL, every final state.  Device
 * tensors as for harts_kda_fwd (N = cu_seqlens[n_seq]).  For one-off calls: it builds and uploads
 * its plan, allocates its workspace with hipMalloc, enqueues the forward on stream, waits for the
 * stream and frees both; repeated calls on the same lengths should create the plan once
 * (harts_plan_create_varlen, harts_plan_upload) and call harts_kda_fwd.
 */
typedef struct {
  const void *q, *k, *v, *g, *beta;
  const int64_t *cu_seqlens;
  int64_t n_seq;
  const float *init_states;
  const uint8_t *init_mask;
  void *o;
  float *boundary_states;
  int64_t *boundary_offsets;
  float *final_states;
  int32_t H, dk, dv, chunk_B, dtype;
} harts_varlen_args;

int harts_kda_fwd_varlen(const harts_varlen_args *args, void *stream);

/* ---------------------------------------------------------------- gated-delta backward
 * [blog 4.3] differentiable handoff: initial-state gradients accumulate back
 * into the call that produced the boundary; [plsum 4] recomputation under the
 * fixed plan (same layout, rounds, replay and state links; activations are
 * recomputed per round unless the forward kept them, see keep above).  Rounds
 * run in reverse order.
 *
 * Loss L = sum_rows <dO, o>.  Outputs (device, plan dtype unless noted):
 *   dq, dk, dg [N, H, dk]; dv [N, H, dv]; dbeta [N, H]: gradients of the compact
 *   rows, summed over every use (own row and every replay of it);
 *   dstates (float32 [n_slots, H, dk, dv], tree plans, may be NULL): for every
 *   slot, the sum over its consumer sequences of dL/d(initial state);
 *   dinit (float32 [n_seq, H, dk, dv], varlen plans, may be NULL): dL/d(init state).
 * io->states must hold the slots written by harts_kda_fwd on the same inputs
 * (tree plans), io->init_states the same initial states (varlen plans).
 * workspace: >= harts_kda_workspace_size(dplan, 1, ...) bytes.
 */
typedef struct {
  const void *dO;
  void *dq, *dk, *dv, *dg, *dbeta;
  float *dstates;
  float *dinit;
} harts_kda_grad;

int harts_kda_bwd(const harts_dev_plan *dplan, const harts_kda_io *io, const harts_kda_grad *grad, void *stream);

/* ---------------------------------------------------------------- compact -> semantic log-probs
 * [blog 4.4; plsum 3] max and sum-exp computed once per compact logit row,
 * then each semantic position reads its target logit in the original order:
 *     logp[s] = logits[m[s], labels[s]] - logsumexp(logits[m[s], :])
 * and the multiplicity q[c] = #{s : m[s] = c}.
 *
 * logits: device [C, V] (dtype bf16 or fp32), rows contiguous.
 * m: device int64 [S] in [0, C); labels: device int32 [S] in [0, V).
 * logp_out: device float32 [S]; q_out: device int32 [C] (may be NULL);
 * lse_out: device float32 [C] (may be NULL).
 * workspace: device, >= harts_logprob_workspace_size(C) bytes.
 * A position whose m is outside [0, C) or whose label is outside [0, V) reads
 * no logit, gets NaN and is not counted in q (harts_logprob_check_map checks
 * host copies of m and labels beforehand).
 */
size_t harts_logprob_workspace_size(int64_t C);
/* The same size for C compact rows and S semantic positions (the gather's workspace depends on C
 * alone). */
size_t harts_logprob_workspace(int64_t C, int64_t S);
int harts_logprob_gather(const void *logits, int64_t C, int64_t V, int32_t dtype, const int64_t *m,
                         const int32_t *labels, int64_t S, float *logp_out, int32_t *q_out, float *lse_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/* No-allocation variant of harts_logprob_gather, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same logp_out and q_out as
 * harts_logprob_gather (lse is not returned); the per-row log-sum-exp lives in
 * a device array of HARTS_LOGPROB_NOALLOC_MAX_ROWS floats (4 MiB) that the
 * library's code object holds on each GPU it runs on until the process ends.
 * No hipMalloc, hipFree or allocating routine is called.  C above the maximum:
 * HARTS_EINVAL, before any device work.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller; the array needs no clearing (every
 * call writes the rows it reads). */
#define HARTS_LOGPROB_NOALLOC_MAX_ROWS (1 << 20)
int harts_logprob_gather_noalloc(const void *logits, int64_t C, int64_t V, int32_t dtype, const int64_t *m,
                                 const int32_t *labels, int64_t S, float *logp_out, int32_t *q_out, void *stream);

/* ---------------------------------------------------------------- log-prob gradient
 * [blog 4.4, equation 19] For L = sum_s dlogp[s] * logp[s], every semantic
 * position forms its own gradient and the positions that read one compact row
 * are summed into it (never a reuse count times one term):
 *     dlogits[c, v] = sum_{s : m[s] = c, labels[s] = v} dlogp[s]
 *                     - (sum_{s : m[s] = c} dlogp[s]) * softmax(logits[c, :])[v]
 * each row's positions summed in increasing s (results do not depend on the
 * schedule); the S x V expansion is never formed.  One streaming read of the
 * logits and one write of the gradient.
 *
 * logits: device [C, V] (dtype bf16 or fp32), as given to harts_logprob_gather.
 * lse: device float32 [C], that call's lse_out on the same logits.
 * row_off: device int64 [C + 1]; row_pos: device int64 [S]: the semantic
 *   positions of row c are row_pos[row_off[c] .. row_off[c + 1]) in increasing
 *   order (harts_logprob_rows builds both from m on the host).
 * labels: device int32 [S] in [0, V); dlogp: device float32 [S].
 * dlogits_out: device [C, V], the logits' dtype, every element written; must
 *   not overlap logits.
 * Offsets and positions are not checked on the device (caller contract); a
 * label outside [0, V) adds nothing to its row.
 */
int harts_logprob_backward(const void *logits, int64_t C, int64_t V, int32_t dtype, const float *lse,
                           const int64_t *row_off, const int64_t *row_pos, const int32_t *labels,
                           const float *dlogp, int64_t S, void *dlogits_out, void *stream);

/* Host: checks host copies of m (int64 [S]) and labels (int32 [S], may be NULL)
 * against C rows and V labels.  HARTS_OK, or HARTS_ERANGE naming the first
 * position out of range. */
int harts_logprob_check_map(const int64_t *m, const int32_t *labels, int64_t S, int64_t C, int64_t V);

/* Host: the inverse of the semantic map m (host int64 [S], values in [0, C)) as
 * CSR arrays: row_off (host int64 [C + 1]) and row_pos (host int64 [S]), each
 * row's positions in increasing order.  HARTS_EINVAL if some m[s] is outside
 * [0, C). */
int harts_logprob_rows(const int64_t *m, int64_t S, int64_t C, int64_t *row_off, int64_t *row_pos);

/* ---------------------------------------------------------------- tree causal convolution
 * [blog 4.3] The KDA layer's depthwise causal convolution over the compact
 * rows: a branch's window reaches into its real ancestors' last w - 1 tokens,
 * never into another trajectory, and no row is expanded:
 *     out[t, c] = sum_{j < w} weight[c, j] * x[anc_j(t), c],   anc_0(t) = t,
 * anc_j(t) the row of the token j places before t on the trajectories through
 * t (they share t's prefix), zero before a trajectory's first token.
 *
 * Host: harts_conv_tables builds, from m (host int64 [S], semantic -> compact,
 * as harts_plan_maps returns it) and the trajectory offsets (host int64
 * [n_traj + 1], offsets[0] = 0):
 *   anc: int32 [C][w - 1], anc[t][j - 1] = anc_j(t) or -1;
 *   gather_off: int64 [C + 1]; gather: int64 [C * (w - 1)]: for each row s the
 *     pairs (t, j) with anc_j(t) = s encoded as 8 t + j, in increasing (j, t).
 * HARTS_EINVAL if m is not the map of a prefix tree (a row with two different
 * predecessors), a row is on no trajectory, or w is outside [2, 8].
 */
int harts_conv_tables(const int64_t *m, const int64_t *traj_offsets, int64_t n_traj, int64_t C, int32_t w,
                      int32_t *anc, int64_t *gather_off, int64_t *gather);

/* x: device [C, channels] (dtype bf16 or fp32), rows contiguous, 16-byte aligned;
 * weight: device float32 [channels, w]; anc: device copy of the table above;
 * out: device [C, channels], x's dtype, must not overlap x.  channels a
 * positive multiple of 8; C <= 65535 * 64 (HARTS_ERANGE).  fp32 accumulation. */
int harts_conv_fwd(const void *x, const float *weight, const int32_t *anc, int64_t C, int32_t channels, int32_t w,
                   int32_t dtype, void *out, void *stream);

/* Gradients of L = sum_t <dout[t], out[t]>:
 *   dx[s, c] = weight[c, 0] dout[s, c] + sum over the gather entries (t, j) of s of weight[c, j] dout[t, c]
 *   dweight[c, j] = sum_t dout[t, c] x[anc_j(t), c]   (fixed-order block sums)
 * dx: device [C, channels] in x's dtype, or NULL; dweight: device float32
 * [channels, w], or NULL (then no workspace is needed).
 * workspace: device, >= harts_conv_workspace_size(C, channels, w) bytes. */
size_t harts_conv_workspace_size(int64_t C, int32_t channels, int32_t w);
int harts_conv_bwd(const void *x, const float *weight, const int32_t *anc, const int64_t *gather_off,
                   const int64_t *gather, const void *dout, int64_t C, int32_t channels, int32_t w, int32_t dtype,
                   void *dx, float *dweight, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- tree attention
 * Softmax attention of the hybrid model's full-attention (MLA) layer on compact
 * rows (HARTS, section 4 "MLA execution"; blog section 4.3, MLA paragraph;
 * Figure C.1(c)): a branch's queries read the keys and values of its ancestor
 * prefix and its own earlier rows (bottom-right causal alignment), so a compact
 * row t attends over the rows of its root-to-t path, t included:
 *   o[t, h] = sum_{a in path(t)} softmax_a(scale <q[t, h], k[a, h]>) v[a, h]
 * The ancestor view is read through row-index lists; no key or value row is
 * copied.
 *
 * Host: harts_attn_tables_build derives the paths from m (host int64 [S],
 * semantic -> compact) and the trajectory offsets (host int64 [n_traj + 1]),
 * cuts the rows into fork-free segments and those into query tiles of up to 128
 * rows and key tiles of up to 128 rows.
 * harts_attn_tables_copy fills caller arrays (sizes from harts_attn_info):
 *   qtiles  int32 [n_qtiles][4]   {row0, n, off, base}: query rows row0..row0+n-1,
 *           keys kv_list[off + v] for v < base + n; query row0 + i sees v iff v <= base + i
 *   kv_list int32 [kv_list_len]   per segment: ancestor rows (root first), own rows
 *   ktiles  int32 [n_ktiles][4]   {row0, n, off, nq}: key rows row0..row0+n-1,
 *           queries q_list[off + u] for u < nq; key row0 + j is seen by u iff u >= j
 *   q_list  int32 [q_list_len]    per segment: own rows, rows of every segment below
 *   pos     int32 [C]             position of the row on its trajectories (the RoPE
 *                                 position id of the row), may be NULL
 * Tiles come longest first.  HARTS_EINVAL if m is not the map of a prefix tree
 * (a row with two different prefixes) or a row is on no trajectory; HARTS_ERANGE
 * if a list outgrows int32 offsets. */
typedef struct harts_attn_tables harts_attn_tables;
typedef struct {
  int64_t C, n_segments, n_qtiles, n_ktiles, kv_list_len, q_list_len;
  int64_t pairs;     /* sum over rows of the path length: visible (query, key) pairs per head */
  int32_t max_depth; /* longest path */
} harts_attn_info_t;
int harts_attn_tables_build(const int64_t *m, const int64_t *traj_offsets, int64_t n_traj, int64_t C,
                            harts_attn_tables **out);
int harts_attn_info(const harts_attn_tables *t, harts_attn_info_t *info);
int harts_attn_tables_copy(const harts_attn_tables *t, int32_t *qtiles, int32_t *kv_list, int32_t *ktiles,
                           int32_t *q_list, int32_t *pos);
void harts_attn_tables_free(harts_attn_tables *t);

/* Forward.  q, k: device bf16 [C, H, dqk]; v: device bf16 [C, H, dv]; rows
 * contiguous, 16-byte aligned; (dqk, dv) in {(192, 128), (128, 128), (64, 64)}.
 * qtiles / kv_list: device copies of the tables above.  Outputs: o device bf16
 * [C, H, dv] (must not overlap the inputs); lse device float32 [C, H], the natural
 * log of each softmax denominator (needed by the backward).  P is rounded to bf16
 * for the value product; fp32 accumulation. */
int harts_attn_fwd(const void *q, const void *k, const void *v, const int32_t *qtiles, int64_t n_qtiles,
                   const int32_t *kv_list, int64_t C, int32_t H, int32_t dqk, int32_t dv, float scale, void *o,
                   float *lse, void *stream);

/* Gradients of L = sum_t <dout[t], o[t]> (each compact row counted once):
 *   dq[t] = scale sum_a ds[t, a] k[a],  dk[a] = scale sum_t ds[t, a] q[t],
 *   dv[a] = sum_t p[t, a] dout[t],  ds = p (dout v^T - <dout[t], o[t]>)
 * o, lse: the forward's outputs; dout: device bf16 [C, H, dv]; dq, dk, dv_out:
 * device bf16, shapes of q, k, v (each row written once, no accumulation);
 * workspace: device, >= harts_attn_workspace_size(C, H) bytes.  dq is computed
 * by query tiles, dk and dv by key tiles: no atomics, deterministic. */
size_t harts_attn_workspace_size(int64_t C, int32_t H);
int harts_attn_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                   const int32_t *qtiles, int64_t n_qtiles, const int32_t *kv_list, const int32_t *ktiles,
                   int64_t n_ktiles, const int32_t *q_list, int64_t C, int32_t H, int32_t dqk, int32_t dv,
                   float scale, void *dq, void *dk, void *dv_out, void *workspace, size_t workspace_bytes,
                   void *stream);

/* ---------------------------------------------------------------- MoE router statistics
 * A compact row is routed once; its multiplicity q_c (semantic positions that
 * read row c, sum_c q_c = S; harts_plan_maps returns it) restores the training
 * weights (HARTS blog sections 4.3-4.4; arXiv summary, section 4 "MoE
 * execution"; Figure C.1(d)):
 *   p[c] = softmax(z[c]), lse_c = log sum_e exp z[c, e]
 *   top_c = the k experts with the largest p[c, e] + bias[e] (ties: lower index)
 *   counts[e] = sum_c q_c [e in top_c]      mass[e] = sum_c q_c p[c, e]
 *   losses[0] = L_z = sum_c q_c lse_c^2 / S
 *   losses[1] = L_aux = E / (k S^2) sum_e counts[e] mass[e]
 * logits: device float32 [C, E]; bias: device float32 [E] or NULL (zero);
 * q: device int32 [C]; outputs (device): topk int32 [C, k] (decreasing score),
 * lse float32 [C], counts int32 [E], mass float32 [E], losses float32 [2].
 * E in {64, 128, 256, 512}, k in [1, 8], S >= C; counts are exact integers,
 * mass and losses are fixed-order fp32 sums (run to run identical).
 * workspace: device, >= harts_moe_workspace_size(C, E) bytes. */
size_t harts_moe_workspace_size(int64_t C, int32_t E);
int harts_moe_stats(const float *logits, const float *bias, const int32_t *q, int64_t C, int32_t E, int32_t k,
                    int64_t S, int32_t *topk, float *lse, int32_t *counts, float *mass, float *losses,
                    void *workspace, size_t workspace_bytes, void *stream);
/* Gradient of z_coef L_z + aux_coef L_aux with respect to the logits, the counts
 * of harts_moe_stats held fixed:
 *   dlogits[c, e] = q_c p[c, e] (z_coef 2 lse_c / S + aux_coef E / (k S^2) (counts[e] - <counts, p[c]>))
 * dlogits: device float32 [C, E], must not overlap logits. */
int harts_moe_grad(const float *logits, const int32_t *q, const int32_t *counts, int64_t C, int32_t E, int32_t k,
                   int64_t S, float z_coef, float aux_coef, float *dlogits, void *stream);
/* Expert-bias update from the weighted counts: bias[e] += gamma sign(mean_j counts[j] - counts[e]). */
int harts_moe_bias_update(const int32_t *counts, int32_t E, float gamma, float *bias, void *stream);

/* ---------------------------------------------------------------- kernel timing
 * For benchmarks and profiling.  While enabled, every kernel the library
 * enqueues is bracketed by two HIP events recorded on the same stream (this
 * adds event overhead; keep it off in timed production runs).
 * harts_profile_enable(1) starts a fresh record, (0) stops recording.
 * harts_profile_collect() waits for the recorded events and reports, per
 * kernel name, the number of launches, their summed elapsed time and the
 * summed work units (token-heads processed, replay included; logits rows for
 * the log-prob kernels).  out: host array of max_entries; *n_out receives the
 * number of kernel names recorded (may exceed max_entries).
 */
typedef struct {
  char name[40];
  int64_t launches;
  double total_ms;
  int64_t units;
} harts_profile_entry;

int harts_profile_enable(int32_t on);
int harts_profile_collect(harts_profile_entry *out, int32_t max_entries, int32_t *n_out);

/* ---------------------------------------------------------------- misc */
const char *harts_last_error(void);
/* Library version string. */
const char *harts_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HARTS_H */
