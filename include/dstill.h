/*
 * dstill.h -- C ABI of a gfx950 (MI355X) library for one cycle of one-pass
 * block-diffusion speculative drafting with lossless verification.
 *
 * A cycle is four calls, in this order:
 *
 *   dstill_inject_kv       fuse target hidden features and write them as K/V
 *                          into every draft layer's cache
 *   dstill_block_draft     one forward pass of the drafter over an anchor plus
 *                          gamma masked positions, attending the injected
 *                          context and, bidirectionally, the block itself
 *   dstill_lm_head_argmax  shared LM head with a fused vocabulary-wide
 *                          argmax / log-sum-exp (/ Gumbel-max sampling)
 *   dstill_verify          greedy prefix match or rejection sampling against
 *                          the target's logits; yields tau in [1, gamma+1]
 *
 * Sources (page title, then section):
 *  - "DFlash - Block Diffusion for Flash Speculative Decoding" (review page),
 *    Method / Inference: the fusion H_t = RMSNorm(W_c [H^l1; ...; H^l5]) and
 *    the injection Q_i = W_i^Q H_d, K_i = [W_i^K H_t; W_i^K H_d],
 *    V_i = [W_i^V H_t; W_i^V H_d]; the injected K/V persist across drafting
 *    iterations.  Preliminary: tau in [1, gamma+1] counts the target's token
 *    and L = (T_draft + T_verify) / tau.
 *  - "DStill: Trajectory Consistency Distillation ...", Setup and notation:
 *    blocks of B positions, anchor at 0, masks at 1..B-1, attention
 *    bidirectional inside the block and to the context strictly before the
 *    anchor.  Inference: greedy verification and the standard rejection-
 *    sampling verifier; a correction or bonus token becomes the next anchor.
 *  - "SPOT" (speculative decoding for diffusion targets), Method: D copies of
 *    a block behind one cached prefix, each copy attending the prefix and
 *    itself; a shared Gumbel table couples drafter and verifier draws.
 *
 * Conventions shared by every call:
 *  - Tensor arguments are DEVICE pointers owned by the caller; the library
 *    never allocates, frees or retains them past the call.  Structs
 *    (dstill_config, dstill_weights, dstill_kv, dstill_sample) are HOST
 *    memory and are read during the call only (dstill_create copies them).
 *  - Matrices are row-major.  Weights are [out_features, in_features].
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *    null stream).  Outputs are valid once the caller synchronises the stream.
 *  - Return value: DSTILL_OK (0) or a negative DSTILL_E* code.  Every check
 *    is made on the host BEFORE anything is enqueued, so on error nothing
 *    runs; dstill_last_error() then describes the problem (thread-local).
 *  - Faults in the data itself (an id outside the vocabulary, a context
 *    longer than the planned bound, non-finite logits) never trap: the
 *    kernels clamp and raise a per-sequence flag bit instead.
 *  - `ws` is caller-provided device scratch of at least the size the
 *    matching *_workspace_bytes query returns; it holds no state between
 *    calls.  Calls that share a `ws` buffer must be ordered on one stream.
 */
#ifndef DSTILL_H
#define DSTILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define DSTILL_OK            0
#define DSTILL_EINVAL       -1   /* null pointer or out-of-range scalar        */
#define DSTILL_ESHAPE       -2   /* inconsistent or unsupported sizes          */
#define DSTILL_EUNSUPPORTED -3   /* valid request the library does not handle */
#define DSTILL_EWORKSPACE   -4   /* ws too small (query *_workspace_bytes)     */
#define DSTILL_EHIP         -5   /* a HIP runtime call failed                  */

/* ---- element types ------------------------------------------------------ */
#define DSTILL_F32  0
#define DSTILL_BF16 1

/* ---- LM-head selection modes ------------------------------------------- */
#define DSTILL_HEAD_ARGMAX        0  /* top-1 per row (greedy drafting)       */
#define DSTILL_HEAD_GUMBEL        1  /* argmax(z/T + G): a draw from softmax(z/T) */
#define DSTILL_HEAD_SHARED_GUMBEL 2  /* same, one table G per block slot shared
                                        by all rows of that slot (SPOT)        */

/* ---- verification modes ------------------------------------------------- */
#define DSTILL_VERIFY_GREEDY 0
#define DSTILL_VERIFY_RS     1

/* ---- per-sequence flag bits (out_flags of dstill_verify, flags of
 *      dstill_block_draft) ----------------------------------------------- */
#define DSTILL_FLAG_NEAR_TIE_TARGET 1u  /* a deciding target argmax had a top-2 gap < 1e-5 */
#define DSTILL_FLAG_NEAR_THRESHOLD  2u  /* |p/q - u| < 1e-5 at a deciding accept test     */
#define DSTILL_FLAG_NEAR_TIE_SAMPLE 4u  /* residual / bonus Gumbel-max top-2 gap < 1e-5  */
#define DSTILL_FLAG_ZERO_RESIDUAL   8u  /* max(0, p - q) summed to 0: drew from p instead */
#define DSTILL_FLAG_BAD_INPUT      16u  /* id outside [0, vocab) or non-finite logits   */
#define DSTILL_FLAG_CTX_CLAMPED    32u  /* ctx_len exceeded max_ctx or the cache capacity */

/* Near-tie band used by every flag above. */
#define DSTILL_NEAR 1e-5f

/* Philox stream purposes (counter word 3 = cycle << 8 | purpose). */
#define DSTILL_RNG_DRAFT    0u
#define DSTILL_RNG_ACCEPT   1u
#define DSTILL_RNG_RESIDUAL 2u
#define DSTILL_RNG_SHARED   3u

/* ---- model description -------------------------------------------------- */

/* Drafter geometry: Qwen3-style layers (DStill appendix drafter table), read
 * as pre-norm RMSNorm, grouped-query attention with optional per-head q/k
 * RMSNorm and rotary embedding (rotate-half pairs (i, i + head_dim/2),
 * frequency rope_theta^(-2i/head_dim)), SwiGLU MLP, residual adds, a final
 * RMSNorm and no biases.  `max_block` bounds B = gamma + 1 (at most 16). */
typedef struct {
  int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, mlp, vocab;
  int32_t n_feat_layers, target_hidden;  /* fused feature width F = product */
  int32_t max_block;                     /* 1..16                           */
  int32_t mask_token_id;                 /* embedding row of [MASK]         */
  int32_t qk_norm;                       /* 1 = per-head q/k RMSNorm        */
  int32_t dtype;                         /* DSTILL_F32 or DSTILL_BF16       */
  float rms_eps, rope_theta;
  /* Sliding-window drafter attention (DStill appendix drafter table: SWA of
   * 2048 on the Gemma and Nemotron drafters, "SWA + 1 Full" on one).  With
   * swa_window = W > 0 the block of a sequence with context length S sees
   * the context positions [max(0, S - W), S) and the whole block; layers
   * whose bit is set in full_attn_mask (bit l = layer l) see all of [0, S).
   * 0 = every layer sees the whole context. */
  int32_t swa_window;
  uint32_t full_attn_mask;
} dstill_config;

/* One draft layer; every tensor has the config dtype.
 *   attn_norm [hidden], wqkv [(n_q+2 n_kv) head_dim, hidden] (rows W^Q, W^K,
 *   W^V), q_norm/k_norm [head_dim], wo [hidden, n_q head_dim],
 *   mlp_norm [hidden], w_gate_up [2 mlp, hidden] (rows gate, then up),
 *   w_down [hidden, mlp]. */
typedef struct {
  const void *attn_norm, *wqkv, *q_norm, *k_norm, *wo, *mlp_norm, *w_gate_up, *w_down;
} dstill_layer_weights;

/* Shared frozen embedding [vocab, hidden] and LM head [vocab, hidden] (both
 * reused from the target: DStill, Experimental Setup; DFlash review,
 * Training), the fusion projection W_c [hidden, F] with RMSNorm gain g_fuse
 * [hidden], the final RMSNorm gain g_final [hidden], and `layers`, a HOST
 * array of n_layers entries. */
typedef struct {
  const void *embed, *lm_head, *w_fuse, *g_fuse, *g_final;
  const dstill_layer_weights *layers;
} dstill_weights;

/* Persistent draft KV cache: k[l], v[l] (HOST arrays of n_layers DEVICE
 * pointers) in the config dtype.  k[l] is [max_batch][n_kv_heads][cap][head_dim]
 * (row (b, h, p) is the injected key of context position p of sequence b);
 * v[l] is stored in tiles of 64 positions, d-major inside a tile:
 * [max_batch][n_kv_heads][cap/64][head_dim][64] (element (b, h, p/64, d, p%64)
 * is component d of the injected value of position p), so the attention's
 * P.V product reads each 64-key tile of V^T as one contiguous block.  cap
 * must be a multiple of 64. */
typedef struct {
  void *const *k;
  void *const *v;
  int32_t max_batch, cap;
} dstill_kv;

typedef struct dstill_handle dstill_handle;

/* Validate the config and weight pointers and keep a private copy of both
 * (the weights themselves are not copied: the caller keeps them alive and
 * unchanged while the handle is used).  The handle is immutable, so calls on
 * different streams may share it.  Errors: EINVAL (null), ESHAPE (sizes),
 * EUNSUPPORTED (head_dim not in {64,128}, group size > 16, max_block > 16). */
int dstill_create(const dstill_config *cfg, const dstill_weights *w, dstill_handle **out);
int dstill_destroy(dstill_handle *h);

/* Bytes of ONE K (or V) cache tensor of one layer (cap a multiple of 64). */
int dstill_kv_bytes(const dstill_config *cfg, int32_t max_batch, int32_t cap, size_t *bytes);

/* Upper bounds a caller plans with; every call's workspace need is a
 * function of its actual arguments and never exceeds this query's answer
 * for limits at least as large. */
typedef struct {
  int32_t max_batch;        /* sequences per block_draft call           */
  int32_t max_copies;       /* copies per sequence (SPOT layout)       */
  int32_t max_ctx;          /* largest context length                  */
  int32_t max_inject_rows;  /* rows per inject_kv call                 */
  int32_t max_head_rows;    /* rows per lm_head_argmax call            */
} dstill_limits;
int dstill_workspace_bytes(const dstill_handle *h, const dstill_limits *lim, size_t *bytes);

/* ---- step 1: feature fusion + KV injection ------------------------------
 * DFlash review, Method / Inference (fusion and injection equations).
 * For each row i < n: H_t = RMSNorm(feats[i] . W_c^T) * g_fuse, rounded to the
 * config dtype; then for every layer l, with W_k, W_v the K and V row blocks
 * of that layer's wqkv:
 *   K = rope(k_norm(H_t W_k^T) * g_k, pos[i]),  V = H_t W_v^T,
 * written to kv->k[l] / kv->v[l] at (seq_id[i], head, pos[i]).  Rows whose
 * seq_id is outside [0, kv->max_batch) or pos outside [0, kv->cap) are
 * computed but not written.
 *   feats  [n, n_feat_layers*target_hidden], config dtype (layer-major concat)
 *   seq_id, pos  [n] int32
 * Errors: EINVAL, ESHAPE (n < 0), EWORKSPACE. n == 0 is a no-op. */
int dstill_inject_kv(const dstill_handle *h, const void *feats, const int32_t *seq_id,
                     const int32_t *pos, int32_t n, const dstill_kv *kv,
                     void *ws, size_t ws_bytes, void *stream);

/* ---- step 2: one-pass block draft --------------------------------------
 * DStill, Setup and notation / Inference; DFlash review, Method / Inference.
 * Sequence b has context length S_b = ctx_len[b] (device) and the block sits
 * at positions S_b .. S_b+block-1.  block_tokens [bs][n_copies][block] holds
 * the anchor at slot 0 and mask_token_id (or revealed ids) elsewhere.  Every
 * layer: u = RMSNorm(h)*g_attn; q,k,v = u Wqkv^T; q,k <- rope(norm(.)*g);
 * attention of each query over [cached K/V rows 0..S_b-1 ; the block K/V of
 * the same copy], no mask, scale 1/sqrt(head_dim); h += o W_o^T;
 * h += W_down(silu(W_gate u') * W_up u') with u' = RMSNorm(h)*g_mlp.
 * hidden_out [bs][n_copies][block][hidden] (config dtype) = RMSNorm(h)*g_final.
 *   max_ctx: host bound on every ctx_len (plans the context split); a
 *     ctx_len above min(max_ctx, kv->cap) is clamped and flagged.
 *   flags: optional [bs] uint32 (NULL to skip), DSTILL_FLAG_CTX_CLAMPED and
 *     DSTILL_FLAG_BAD_INPUT (a token id outside [0, vocab), clamped).
 * Errors: EINVAL, ESHAPE (bs > kv->max_batch, block > max_block, ...),
 * EWORKSPACE. */
int dstill_block_draft(const dstill_handle *h, const int32_t *block_tokens,
                       const int32_t *ctx_len, int32_t bs, int32_t block, int32_t n_copies,
                       int32_t max_ctx, const dstill_kv *kv, void *hidden_out,
                       uint32_t *flags, void *ws, size_t ws_bytes, void *stream);

/* ---- step 3: shared LM head with fused vocabulary reduction ------------
 * z = hidden_row . W_lm^T over the whole vocabulary, never stored unless
 * logits_out is given.  Per row: ids = argmax of the score (z, or z/T + G in
 * the Gumbel modes; ties go to the lowest id), zmax = max z, lse =
 * log sum_v exp(z_v / T), zsel = z[ids], gap = score of the winner minus the
 * runner-up.  Gumbel-max over z/T is a draw from softmax(z/T) (DStill,
 * Inference; D-Loop Notation, Eq. 1 factorised proposal).
 * Row addressing: row r is hidden + ((r / rows_per_seq) * seq_stride +
 * r % rows_per_seq) * hidden; it belongs to sequence r / rows_per_seq at
 * slot r % rows_per_seq.  Gumbel noise for (row, v) is Philox4x64-10 element
 * v of stream (purpose DSTILL_RNG_DRAFT, seq, slot, cycle); in SHARED mode
 * the stream is (DSTILL_RNG_SHARED, 0, slot, cycle) for every row.
 * logits_out: NULL or [rows, vocab] fp32 (needed by rejection sampling). */
typedef struct {
  int32_t mode;        /* DSTILL_HEAD_*                  */
  float temperature;   /* > 0; ignored in ARGMAX mode   */
  uint64_t seed;       /* Philox key word 0             */
  uint64_t cycle;      /* counter word 3 = cycle<<8|purpose (cycle < 2^56) */
} dstill_sample;
int dstill_lm_head_argmax(const dstill_handle *h, const void *hidden, int32_t rows,
                          int32_t rows_per_seq, int32_t seq_stride, const dstill_sample *s,
                          int32_t *ids, float *zmax, float *lse, float *zsel, float *gap,
                          float *logits_out, void *ws, size_t ws_bytes, void *stream);

/* ---- step 4: verification -----------------------------------------------
 * DStill, Inference; DFlash review, Preliminary; textbook speculative
 * sampling (Leviathan et al., Chen et al., cited there).
 * Target row k (k = 0..gamma) is the target's distribution for the token
 * after block slot k; draft row k (k < gamma) is the drafter's distribution
 * of draft_ids[k].  With p_k = softmax(target_k / T), q_k = softmax(draft_k / T):
 *  GREEDY: L = number of leading k with draft_ids[k] == argmax target_k;
 *          emit draft_ids[0..L-1], then argmax target_L.
 *  RS:     accept draft k while u_k < p_k(y)/q_k(y), u_k = uniform of
 *          stream (DSTILL_RNG_ACCEPT, b, k, cycle) element 0; at the first
 *          rejection emit the Gumbel-max draw from norm(max(0, p_k - q_k))
 *          (stream (DSTILL_RNG_RESIDUAL, b, k, cycle)); after gamma
 *          acceptances emit the draw from p_gamma (same stream, pos gamma).
 * out_tokens [bs][gamma+1] (-1 after tau), out_tau [bs] = L + 1, out_flags.
 *   draft_lse [bs][gamma] = log sum exp(draft/T) and draft_logits
 *   [bs][gamma][vocab] fp32 are required in RS mode, ignored in GREEDY.
 *   target_logits [bs][gamma+1][vocab] in target_dtype (DSTILL_F32/BF16).
 * Errors: EINVAL, ESHAPE, EWORKSPACE.  No handle needed: model-independent. */
int dstill_verify_workspace_bytes(int32_t bs, int32_t gamma, int32_t vocab, size_t *bytes);
int dstill_verify(int32_t mode, int32_t bs, int32_t gamma, int32_t vocab, float temperature,
                  uint64_t seed, uint64_t cycle, const int32_t *draft_ids,
                  const float *draft_lse, const float *draft_logits,
                  const void *target_logits, int32_t target_dtype, int32_t *out_tokens,
                  int32_t *out_tau, uint32_t *out_flags, void *ws, size_t ws_bytes,
                  void *stream);

/* ---- verification without a caller workspace ------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as dstill_verify, minus ws / ws_bytes: the
 * workspace is a fixed array of DSTILL_NOALLOC_SCRATCH_BYTES inside the
 * library, one per device, held until the process ends.  The call allocates
 * nothing (no hipMalloc / hipFree); its first call on a device looks up that
 * device's array address.  Shapes whose dstill_verify_workspace_bytes exceeds
 * the array are refused with EWORKSPACE before anything is enqueued (4 MiB
 * covers bs up to 6060 at gamma 15, 31772 at gamma 1, at any vocabulary).  Every call
 * on a device shares its array: calls that overlap on one device race, so
 * order them (one stream, or events between streams). */
#define DSTILL_NOALLOC_SCRATCH_BYTES (4u << 20)
int dstill_verify_noalloc(int32_t mode, int32_t bs, int32_t gamma, int32_t vocab,
                          float temperature, uint64_t seed, uint64_t cycle,
                          const int32_t *draft_ids, const float *draft_lse,
                          const float *draft_logits, const void *target_logits,
                          int32_t target_dtype, int32_t *out_tokens, int32_t *out_tau,
                          uint32_t *out_flags, void *stream);

/* ---- D-Loop: looped second draft pass and joint K-branch verification ----
 * D-Loop page, section 3.1 (the prefix score after Eq. (4), Eq. (5)) and
 * section 3.3 (inference: joint verification of K branches).
 *
 * dstill_dloop_branches: from the first pass's head statistics of slots
 * 1..gamma (ids, zmax, lse: [bs][gamma], device), the confidence of each
 * proposed token is c_k = exp(zmax_k - lse_k) (its softmax probability at
 * T = 1, computed in fp64) and each prefix length l = 0..gamma-1 is scored
 * r_l = (c_1 ... c_l)(1 - c_{l+1}) (taken left to right in fp64).  The K
 * largest scores (ties to the smaller l) give the branches, in decreasing
 * order of r: prefix_len [bs][K] int32, score [bs][K] fp64 (NULL to skip),
 * and block_tokens [bs][K][gamma+1] int32 = (anchor[b], ids[b][0..l-1],
 * mask_id, ..., mask_id), ready for dstill_block_draft with n_copies = K
 * (each branch is a copy of the block behind the shared context).
 * Non-finite statistics give unspecified (in-range) lengths.
 * Errors: ESHAPE unless 1 <= K <= gamma <= 63; EINVAL on null pointers. */
int dstill_dloop_branches(int32_t bs, int32_t gamma, int32_t K, const int32_t *anchor,
                          const int32_t *ids, const float *zmax, const float *lse,
                          int32_t mask_id, int32_t *block_tokens, int32_t *prefix_len,
                          double *score, void *stream);

/* dstill_dloop_merge: each branch's proposal (Eq. (5)): out_ids[b][j][k] =
 * first_ids[b][k] for k < prefix_len[b][j], else second_ids[b][j][k]
 * (first_ids [bs][gamma], second_ids and out_ids [bs][K][gamma], int32,
 * device; second_ids are the second pass's head ids of slots 1..gamma).
 * Errors: ESHAPE, EINVAL. */
int dstill_dloop_merge(int32_t bs, int32_t gamma, int32_t K, const int32_t *first_ids,
                       const int32_t *second_ids, const int32_t *prefix_len, int32_t *out_ids,
                       void *stream);

/* dstill_verify_branches: joint greedy verification of K branch proposals
 * per sequence.  Branch j of sequence b has draft_ids [bs][K][gamma] and its
 * own target rows target_logits [bs][K][gamma+1][vocab] (target_dtype
 * DSTILL_F32 or DSTILL_BF16).  Each branch is verified by the GREEDY rule of
 * dstill_verify; the branch with the largest tau (ties to the lowest j) is
 * committed: out_tokens [bs][gamma+1] (-1 after tau), out_tau [bs],
 * out_branch [bs] (NULL to skip); out_flags [bs] is the OR of every branch's
 * flags (a near tie in any branch can change which is longest).
 * Workspace: dstill_verify_branches_workspace_bytes.
 * Errors: ESHAPE, EUNSUPPORTED, EINVAL, EWORKSPACE. */
int dstill_verify_branches_workspace_bytes(int32_t bs, int32_t K, int32_t gamma, int32_t vocab,
                                           size_t *bytes);
int dstill_verify_branches(int32_t bs, int32_t K, int32_t gamma, int32_t vocab,
                           const int32_t *draft_ids, const void *target_logits,
                           int32_t target_dtype, int32_t *out_tokens, int32_t *out_tau,
                           int32_t *out_branch, uint32_t *out_flags, void *ws, size_t ws_bytes,
                           void *stream);

/* ---- SPOT: state-equality verification over a draft tree ------------------
 * SPOT page, section 4 (problem setting; state-equality verification; the
 * coupled-noise match).  A block state is L slots, each a token or mask_id.
 * State 0 of each sequence is the root, states 1..n_states-1 are drafts with
 * parent[b][j] the index of an earlier state.  For every state the caller
 * supplies the target's per-slot head outputs over all L slots (the
 * multi-copy layout with the shared-Gumbel head: ids [bs][n_states][L] =
 * argmax(z/T + G_slot), zmax and lse [bs][n_states][L] at temperature T,
 * gap [bs][n_states][L] or NULL).  A state commits at its masked slot of
 * largest confidence zmax/T - lse (fp64; ties to the lowest slot) the id of
 * that slot; a state with no masked slot commits nothing.  Draft j is
 * accepted iff its parent is accepted and state j equals the parent's state
 * with the parent's commit filled in.  The path from the root follows the
 * lowest accepted child; the round emits the commit of every state on it,
 * the deepest included.
 * Outputs (device): out_n [bs] commits emitted; out_slots, out_tokens
 * [bs][n_states] (slot, token) in order, -1 after out_n; out_state [bs] the
 * deepest accepted state; out_flags [bs]: DSTILL_FLAG_NEAR_TIE_TARGET when a
 * state on the path has its two best confidences within 1e-5,
 * DSTILL_FLAG_NEAR_TIE_SAMPLE when a commit on it has a head gap below 1e-5.
 * Errors: ESHAPE unless 1 <= n_states, L <= 64; EINVAL on null pointers or
 * temperature <= 0. */
int dstill_spot_verify(int32_t bs, int32_t n_states, int32_t L, int32_t mask_id,
                       float temperature, const int32_t *states, const int32_t *parent,
                       const int32_t *ids, const float *zmax, const float *lse, const float *gap,
                       int32_t *out_n, int32_t *out_slots, int32_t *out_tokens,
                       int32_t *out_state, uint32_t *out_flags, void *stream);

/* ---- DStill multi-step refinement: one commit pass --------------------------
 * DStill page, "Multi-step drafting" and the teacher rollout of its appendix.
 * Between drafter passes over a block state tokens [bs][block] (slot 0 the
 * anchor), with kappa [bs][block] the commit pass of each slot (0 for the
 * anchor, -1 while masked): given the head's greedy ids, zmax and lse of
 * slots 1..block-1 on pass t of K ([bs][block-1], device), the
 * n_t = ceil(masked / (K - t + 1)) masked slots of largest confidence
 * max_v softmax(z) (ranked as zmax - lse in fp64, ties to the lower slot)
 * take their ids and kappa = t.  Pass t = K commits every remaining slot.
 * tokens and kappa are updated in place (device).
 * Errors: ESHAPE unless 2 <= block <= 64 and 1 <= t <= K; EINVAL on nulls. */
int dstill_refine_commit(int32_t bs, int32_t block, int32_t t, int32_t K, const int32_t *ids,
                         const float *zmax, const float *lse, int32_t *tokens, int32_t *kappa,
                         void *stream);

/* Message for the last non-zero status returned on this thread. */
const char *dstill_last_error(void);
/* Library ABI version (major * 100 + minor). */
int dstill_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSTILL_H */
