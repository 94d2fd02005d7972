// Internal launch interface between the host dispatcher (api.cpp) and the
// kernels.  Every launcher only enqueues work on the given stream; argument
// validation happens before any of them is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dstill {

// ---- dense projections (gemm.hip) -----------------------------------------
constexpr int GEMM_MAX_GROUPS = 8;
struct GemmArgs {
  const void *X;  // [M, K] activations, row stride ldx (elements)
  long ldx;
  const void *W;  // [N, K] weight rows, row stride ldw (elements)
  long ldw;
  float *out;     // [splits][M][N] fp32 partial sums
  int M, N, K, splits, dtype;
  // Fused SwiGLU (bf16, one split, mlp a multiple of 64): W is gate rows
  // [0, mlp) then up rows [mlp, 2 mlp) (N = 2 mlp) and the product is written
  // as act[M][mlp] = bf16(silu(gate) * up) instead of partial sums.
  void *swiglu_act = nullptr;
  int mlp = 0;
  // Weight groups (bf16 LDS path only): when wg_rows > 0, output rows
  // [g wg_rows, (g + 1) wg_rows) of W are rows 0 .. wg_rows - 1 of wg[g]
  // (N = groups x wg_rows, wg_rows a multiple of 256), so one launch covers
  // row blocks of several weight tensors.  W is ignored.
  const void *wg[GEMM_MAX_GROUPS] = {};
  int wg_rows = 0;
};
// Whether a product can take weight groups (bf16 with depth a multiple of 64).
bool gemm_can_group(int K, int dtype);
// Whether a gate|up product of these sizes takes the fused SwiGLU epilogue:
// bf16, mlp a multiple of 64, and one split already gives every compute unit
// a workgroup (the fusion saves the partial plane and the separate pass).
bool gemm_can_fuse_swiglu(int M, int mlp, int K, int dtype, int num_cu);
void gemm_pick_tile(int M, int *ntw, int *mtw);
int gemm_plan_splits(int M, int N, int K, int dtype, int num_cu);
void launch_gemm(const GemmArgs &a, hipStream_t st);

// ---- per-row and element-wise stages (layer_ops.hip) ------------------------
void launch_draft_prep(const int32_t *tokens, const int32_t *ctx_len, int bs, int per_seq,
                       int vocab, int ctx_limit, int32_t *eff_ctx, int32_t *tok_clamped,
                       uint32_t *flags, hipStream_t st);
void launch_embed(int dtype, const void *embed, const int32_t *tok, int R, int d, float *h,
                  hipStream_t st);
// out = RMSNorm(x) * gain with x = sum of `nsplit` partial planes (+ resid);
// the new residual is written back when write_resid is set.  Scratch: xtmp
// [M, d] fp32 (used when x has nowhere else to live), ssp [M, ceil(d/1024)].
void launch_norm_rows(int dtype, const float *parts, int nsplit, int M, int d, float *resid,
                      int write_resid, const void *gain, float eps, void *out, long out_stride,
                      float *xtmp, float *ssp, hipStream_t st);
// (cos, sin) of the rotary pairs of n rows, [n][dh/2] float2: row r sits at
// pos[r] (injection) or, with pos null, at eff_ctx[r / rows_per_seq] + r % block.
void launch_rope_table(const int32_t *eff_ctx, int rows_per_seq, int block, const int32_t *pos,
                       int n, int dh, float theta, float *tab, hipStream_t st);
void launch_qkv_post(int dtype, const float *parts, int nsplit, int R, int hq, int hkv, int dh,
                     const int32_t *eff_ctx, int rows_per_seq, int block, const void *q_norm,
                     const void *k_norm, int qk_norm, float eps, const float *rope, void *q,
                     void *kb, void *vb, hipStream_t st);
void launch_swiglu(int dtype, const float *parts, int nsplit, int R, int mlp, void *act,
                   hipStream_t st);
// K/V of `layers` draft layers from one partial-plane set: plane columns
// [l * 2 kvd, (l + 1) * 2 kvd) hold layer l's K then V rows (kvd = hkv dh).
struct InjectLayers {
  const void *k_norm[GEMM_MAX_GROUPS];
  void *kc[GEMM_MAX_GROUPS], *vc[GEMM_MAX_GROUPS];
  int layers;
};
void launch_inject_post(int dtype, const float *parts, int nsplit, int n, int hkv, int dh,
                        const int32_t *seq, const int32_t *pos, const InjectLayers &il,
                        int qk_norm, float eps, const float *rope, int max_batch, int cap,
                        hipStream_t st);

// ---- block attention over injected context (attn.hip) --------------------
struct AttnArgs {
  int dtype;
  const void *q;       // [bs*C*B, hq*dh]
  const void *kb;      // [bs*C*B, hkv*dh] block keys
  const void *vb;      // [bs*C][hkv][dh][16] block values, d-major
  const void *kc;      // cache K of this layer [max_batch][hkv][cap][dh]
  const void *vc;      // cache V of this layer [max_batch][hkv][cap/64][dh][64]
  const int32_t *eff_ctx;  // [bs] clamped context lengths
  int bs, C, B, hq, hkv, dh, cap;
  int split;           // context keys per split (multiple of 64)
  int nsplit;          // splits planned for the longest context
  float scale;         // 1/sqrt(dh)
  float *opart;        // [bs*C][hq][nsplit][B][dh]
  float *mlpart;       // [bs*C][hq][nsplit][B][2]  (running max in log2 units, sum)
  void *out;           // [bs*C*B, hq*dh]
  const int *worklist = nullptr;  // optional [nsplit * hkv * bs*C] item order
  // Sliding window over the context: the block sees context positions
  // [S - window, S) (all of [0, S) when window is 0 or S <= window).
  int window = 0;
};
// Item order for launch_attention, longest first (one small kernel; depends
// only on eff_ctx and the split plan, so one list serves every layer).
void launch_attention_worklist(const AttnArgs &a, int *list, hipStream_t st);
void launch_attention(const AttnArgs &a, hipStream_t st);

// ---- LM head with fused vocabulary reduction (lm_head.hip) -----------------
struct HeadPartial {
  float best, second, zbest, zmax, m, s;  // m: max z/T in block, s: sum exp(z/T - m)
  int idx, pad;
};
struct HeadArgs {
  int dtype;
  const void *hidden;
  int rows, rows_per_seq, seq_stride, d, vocab;
  const void *w;       // [vocab, d]
  int mode;
  float temperature;
  uint64_t seed, cycle;
  HeadPartial *part;   // [rows][nvb]
  int nvb;             // vocabulary blocks
  float *logits;       // optional [rows][vocab]
  int32_t *ids;
  float *zmax, *lse, *zsel, *gap;
};
int head_vocab_block();
void launch_lm_head(const HeadArgs &a, hipStream_t st);

// ---- verification (verify.hip) ------------------------------------------
struct VerifyArgs {
  int mode, bs, gamma, vocab, tdtype;
  float temperature;
  uint64_t seed, cycle;
  const int32_t *draft_ids;
  const float *draft_lse;
  const float *draft_logits;
  const void *target;
  int32_t *tokens, *tau;
  uint32_t *flags;
  void *ws;
  int nsplit;          // vocabulary splits per target row
  int nsamp;           // vocabulary splits of the residual / bonus draw
};
// splits of a vocabulary-wide pass over `rows` rows
int verify_plan_splits(int rows, int vocab);
size_t verify_ws_bytes(int bs, int gamma, int nsplit, int nsamp);
void launch_verify(const VerifyArgs &a, hipStream_t st);

// Argument checks, workspace sizing and launch of one verification call
// (api.cpp); the workspace is the caller's or the library's fixed scratch.
int verify_call(int32_t mode, int32_t bs, int32_t gamma, int32_t vocab, float temperature,
                uint64_t seed, uint64_t cycle, const int32_t *draft_ids, const float *draft_lse,
                const float *draft_logits, const void *target_logits, int32_t target_dtype,
                int32_t *out_tokens, int32_t *out_tau, uint32_t *out_flags, void *ws,
                size_t ws_bytes, void *stream);
// Records msg as the thread's last error and returns code.
int api_fail(int code, const char *msg);

// ---- D-Loop second pass (dloop.hip) -----------------------------------------
struct DloopArgs {
  int bs, gamma, K, mask_id;
  const int32_t *anchor;  // [bs]
  const int32_t *ids;     // [bs, gamma] first-pass proposal
  const float *zmax, *lse;  // [bs, gamma] first-pass head statistics
  int32_t *block_tokens;  // [bs, K, gamma + 1]
  int32_t *prefix_len;    // [bs, K]
  double *score;          // [bs, K] or null
};
void launch_dloop_branches(const DloopArgs &a, hipStream_t st);
void launch_dloop_merge(int bs, int gamma, int K, const int32_t *first, const int32_t *second,
                        const int32_t *lens, int32_t *out, hipStream_t st);
void launch_branch_pick(int bs, int K, int gamma, const int32_t *tok, const int32_t *tau,
                        const uint32_t *flags, int32_t *out_tokens, int32_t *out_tau,
                        int32_t *out_branch, uint32_t *out_flags, hipStream_t st);

// ---- SPOT state-equality verification (spot.hip) -------------------------------
struct SpotArgs {
  int bs, n_states, L, mask_id;
  float temperature;
  const int32_t *states;  // [bs, n_states, L]
  const int32_t *parent;  // [bs, n_states]
  const int32_t *ids;     // [bs, n_states, L] per-slot head outputs
  const float *zmax, *lse, *gap;  // gap may be null
  int32_t *out_n, *out_slots, *out_tokens, *out_state;
  uint32_t *out_flags;
};
void launch_spot_verify(const SpotArgs &a, hipStream_t st);

// ---- multi-step refinement (refine.hip) ------------------------------------------
struct RefineArgs {
  int bs, block, t, K;
  const int32_t *ids;       // [bs, block - 1] greedy ids of slots 1..block-1
  const float *zmax, *lse;  // [bs, block - 1]
  int32_t *tokens, *kappa;  // [bs, block], updated in place
};
void launch_refine_commit(const RefineArgs &a, hipStream_t st);

}  // namespace dstill
