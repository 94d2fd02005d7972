// Host side of the C ABI declared in include/dstill.h: argument checks (all
// before anything is enqueued), shape planning (k-splits, context splits,
// vocabulary blocks), carving of the caller's workspace, and the launch
// sequence of each call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dstill.h"
#include "kernels.hpp"

using namespace dstill;

struct dstill_handle {
  dstill_config cfg;
  dstill_weights w;
  std::vector<dstill_layer_weights> layers;
};

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_check(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSTILL_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DSTILL_OK;
}

int elem_bytes(int dtype) { return dtype == DSTILL_BF16 ? 2 : 4; }
int kw_of(int dtype) { return dtype == DSTILL_BF16 ? 32 : 16; }

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

int num_cu() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Sub-allocator over the caller's workspace (256-byte aligned slices).
struct Carver {
  char *base;
  size_t off = 0;
  explicit Carver(void *p) : base((char *)p) {}
  template <typename T> T *take(size_t count) {
    T *p = base ? (T *)(base + off) : nullptr;
    off += a256(count * sizeof(T));
    return p;
  }
};

int qkv_cols(const dstill_config &c) { return (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim; }

// Largest partial-sum plane set any projection of a row block of M rows needs.
size_t gemm_parts_floats(const dstill_config &c, int M, int ncu) {
  const int d = c.hidden, F = c.n_feat_layers * c.target_hidden;
  struct P { int N, K; } ps[] = {{qkv_cols(c), d},
                                 {d, c.n_q_heads * c.head_dim},
                                 {2 * c.mlp, d},
                                 {d, c.mlp},
                                 {d, F},
                                 {2 * c.n_kv_heads * c.head_dim, d},
                                 {2 * c.n_kv_heads * c.head_dim *
                                      std::min(c.n_layers, (int32_t)GEMM_MAX_GROUPS), d}};
  size_t best = 0;
  for (const P &p : ps) {
    const int s = gemm_plan_splits(M, p.N, p.K, c.dtype, ncu);
    best = std::max(best, (size_t)s * M * p.N);
  }
  return best;
}

struct AttnPlan {
  int split, nsplit;
};
// Split of the context keys among attention workgroups, which run two per
// compute unit (slots = 2 ncu).  With ns splits of max_ctx keys per (sequence,
// kv head) pair there are ns * pairs workgroups, and ns = slots / pairs fills
// one round exactly.  When that leaves fewer than four splits per pair (many
// pairs), contexts of different lengths leave one round unbalanced, so ns is
// taken 1.5 times larger and the longest-first work list evens it out.  (On
// the 8B-shaped drafter this beat fixed split lengths: one round for 32 pairs
// of 32K keys and for 72 pairs of 4K, 1.5 rounds for 256 pairs of 1K-8K.)
AttnPlan attn_plan(int max_ctx, int pairs, int ncu) {
  const long slots = 2L * ncu;
  long ns = std::max<long>(1, slots / pairs);
  if (ns < 4) ns = std::max<long>(1, 3 * slots / (2 * pairs));
  long split = ((long)max_ctx + ns - 1) / ns;
  // at most 128 splits (the merge kernel stages one weight per split)
  const long floor_split = std::max<long>(128, ((long)max_ctx + 127) / 128);
  split = (std::max(split, floor_split) + 63) / 64 * 64;
  AttnPlan p;
  p.split = (int)split;
  p.nsplit = std::max(1, (int)(((long)max_ctx + split - 1) / split));
  return p;
}

// Workspace of one block_draft call.
struct DraftWs {
  int32_t *eff_ctx, *tok, *wlist, *wlist_win;
  float *h, *parts, *opart, *mlpart, *ssp, *rope;
  void *u, *q, *kb, *vb, *attn, *act;
};
size_t draft_ws(const dstill_config &c, int bs, int C, int B, AttnPlan ap, int ncu, void *ws,
                DraftWs *out) {
  const int R = bs * C * B, d = c.hidden, eb = elem_bytes(c.dtype);
  const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  Carver cv(ws);
  DraftWs w;
  w.eff_ctx = cv.take<int32_t>(bs);
  w.tok = cv.take<int32_t>(R);
  w.wlist = cv.take<int32_t>((size_t)ap.nsplit * bs * C * c.n_kv_heads);
  w.wlist_win = cv.take<int32_t>((size_t)ap.nsplit * bs * C * c.n_kv_heads);  // windowed layers
  w.h = cv.take<float>((size_t)R * d);
  w.ssp = cv.take<float>((size_t)R * ((d + 1023) / 1024));
  w.rope = cv.take<float>((size_t)R * c.head_dim);  // [R][dh/2] (cos, sin)
  w.u = cv.take<char>((size_t)R * d * eb);
  w.q = cv.take<char>((size_t)R * qd * eb);
  w.kb = cv.take<char>((size_t)R * kvd * eb);
  w.vb = cv.take<char>((size_t)bs * C * kvd * 16 * eb);  // d-major, 16 key slots
  w.attn = cv.take<char>((size_t)R * qd * eb);
  w.act = cv.take<char>((size_t)R * c.mlp * eb);
  w.parts = cv.take<float>(gemm_parts_floats(c, R, ncu));
  const size_t rec = (size_t)bs * C * c.n_q_heads * ap.nsplit * B;
  w.opart = cv.take<float>(rec * c.head_dim);
  w.mlpart = cv.take<float>(rec * 2);
  if (out) *out = w;
  return cv.off;
}

struct InjectWs {
  void *ht;
  float *parts, *xtmp, *ssp, *rope;
};
size_t inject_ws(const dstill_config &c, int n, int ncu, void *ws, InjectWs *out) {
  Carver cv(ws);
  InjectWs w;
  w.ht = cv.take<char>((size_t)n * c.hidden * elem_bytes(c.dtype));
  w.xtmp = cv.take<float>((size_t)n * c.hidden);
  w.ssp = cv.take<float>((size_t)n * ((c.hidden + 1023) / 1024));
  w.rope = cv.take<float>((size_t)n * c.head_dim);  // [n][dh/2] (cos, sin)
  w.parts = cv.take<float>(gemm_parts_floats(c, n, ncu));
  if (out) *out = w;
  return cv.off;
}

size_t head_ws(const dstill_config &c, int rows) {
  const int nvb = (c.vocab + head_vocab_block() - 1) / head_vocab_block();
  return a256((size_t)rows * nvb * sizeof(HeadPartial));
}

int check_config(const dstill_config *c) {
  if (!c) return fail(DSTILL_EINVAL, "config is null");
  if (c->dtype != DSTILL_F32 && c->dtype != DSTILL_BF16)
    return fail(DSTILL_EUNSUPPORTED, "dtype %d is neither DSTILL_F32 nor DSTILL_BF16", c->dtype);
  if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->mlp < 1 ||
      c->vocab < 2 || c->n_feat_layers < 1 || c->target_hidden < 1)
    return fail(DSTILL_ESHAPE, "every model size must be positive (vocab >= 2)");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(DSTILL_EUNSUPPORTED, "head_dim %d: only 64 and 128 are built", c->head_dim);
  if (c->dtype == DSTILL_F32 && c->head_dim != 64)
    return fail(DSTILL_EUNSUPPORTED, "fp32 drafters are built for head_dim 64 only");
  if (c->n_q_heads % c->n_kv_heads)
    return fail(DSTILL_ESHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", c->n_q_heads,
                c->n_kv_heads);
  if (c->swa_window < 0) return fail(DSTILL_ESHAPE, "swa_window %d < 0", c->swa_window);
  if (c->n_q_heads / c->n_kv_heads > 16)
    return fail(DSTILL_EUNSUPPORTED, "GQA group %d exceeds 16", c->n_q_heads / c->n_kv_heads);
  if (c->max_block < 1 || c->max_block > 16)
    return fail(DSTILL_EUNSUPPORTED, "max_block %d outside 1..16", c->max_block);
  if (c->hidden > 8192) return fail(DSTILL_EUNSUPPORTED, "hidden %d exceeds 8192", c->hidden);
  const int kw = kw_of(c->dtype);
  const int F = c->n_feat_layers * c->target_hidden;
  if (c->hidden % kw || c->mlp % kw || F % kw || (c->n_q_heads * c->head_dim) % kw)
    return fail(DSTILL_EUNSUPPORTED,
                "hidden, mlp, fused feature width and n_q_heads*head_dim must be multiples of %d",
                kw);
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab)
    return fail(DSTILL_ESHAPE, "mask_token_id %d outside [0, vocab)", c->mask_token_id);
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 1.f))
    return fail(DSTILL_EINVAL, "rms_eps must be >= 0 and rope_theta > 1");
  return DSTILL_OK;
}

int check_kv(const dstill_handle *h, const dstill_kv *kv) {
  if (!kv || !kv->k || !kv->v) return fail(DSTILL_EINVAL, "kv or its pointer arrays are null");
  if (kv->max_batch < 1 || kv->cap < 1) return fail(DSTILL_ESHAPE, "kv max_batch/cap must be >= 1");
  if (kv->cap % 64) return fail(DSTILL_ESHAPE, "kv cap %d is not a multiple of 64", kv->cap);
  for (int l = 0; l < h->cfg.n_layers; ++l)
    if (!kv->k[l] || !kv->v[l]) return fail(DSTILL_EINVAL, "kv cache of layer %d is null", l);
  return DSTILL_OK;
}

}  // namespace

namespace dstill {

int verify_call(int32_t mode, int32_t bs, int32_t gamma, int32_t vocab, float temperature,
                uint64_t seed, uint64_t cycle, const int32_t *draft_ids, const float *draft_lse,
                const float *draft_logits, const void *target_logits, int32_t target_dtype,
                int32_t *out_tokens, int32_t *out_tau, uint32_t *out_flags, void *ws,
                size_t ws_bytes, void *stream) {
  if (mode != DSTILL_VERIFY_GREEDY && mode != DSTILL_VERIFY_RS)
    return fail(DSTILL_EINVAL, "unknown verify mode %d", mode);
  if (bs < 0 || gamma < 1 || gamma > 63 || vocab < 2)
    return fail(DSTILL_ESHAPE, "need bs >= 0, 1 <= gamma <= 63, vocab >= 2");
  if (target_dtype != DSTILL_F32 && target_dtype != DSTILL_BF16)
    return fail(DSTILL_EUNSUPPORTED, "target_dtype %d", target_dtype);
  if (bs == 0) return DSTILL_OK;
  if (!draft_ids || !target_logits || !out_tokens || !out_tau || !out_flags || !ws)
    return fail(DSTILL_EINVAL, "null tensor argument");
  if (mode == DSTILL_VERIFY_RS) {
    if (!draft_lse || !draft_logits)
      return fail(DSTILL_EINVAL, "rejection sampling needs draft_lse and draft_logits");
    if (!(temperature > 0.f)) return fail(DSTILL_EINVAL, "temperature must be > 0");
  }
  if (cycle >> 56) return fail(DSTILL_EINVAL, "cycle must be < 2^56");
  const int nsplit = verify_plan_splits(bs * (gamma + 1), vocab);
  const int nsamp = verify_plan_splits(bs, vocab);
  const size_t need = verify_ws_bytes(bs, gamma, nsplit, nsamp);
  if (ws_bytes < need) return fail(DSTILL_EWORKSPACE, "verify needs %zu workspace bytes", need);
  VerifyArgs a;
  a.mode = mode; a.bs = bs; a.gamma = gamma; a.vocab = vocab; a.tdtype = target_dtype;
  a.temperature = mode == DSTILL_VERIFY_RS ? temperature : 1.0f;
  a.seed = seed; a.cycle = cycle;
  a.draft_ids = draft_ids; a.draft_lse = draft_lse; a.draft_logits = draft_logits;
  a.target = target_logits;
  a.tokens = out_tokens; a.tau = out_tau; a.flags = out_flags;
  a.ws = ws; a.nsplit = nsplit; a.nsamp = nsamp;
  launch_verify(a, (hipStream_t)stream);
  return hip_check("verify launch");
}

int api_fail(int code, const char *msg) { return fail(code, "%s", msg); }

}  // namespace dstill

extern "C" {

int dstill_version(void) { return 100; }

const char *dstill_last_error(void) { return g_err.c_str(); }

int dstill_create(const dstill_config *cfg, const dstill_weights *w, dstill_handle **out) {
  if (!out) return fail(DSTILL_EINVAL, "out is null");
  *out = nullptr;
  if (int e = check_config(cfg)) return e;
  if (!w || !w->embed || !w->lm_head || !w->w_fuse || !w->g_fuse || !w->g_final || !w->layers)
    return fail(DSTILL_EINVAL, "a shared weight pointer is null");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dstill_layer_weights &L = w->layers[l];
    if (!L.attn_norm || !L.wqkv || !L.wo || !L.mlp_norm || !L.w_gate_up || !L.w_down ||
        (cfg->qk_norm && (!L.q_norm || !L.k_norm)))
      return fail(DSTILL_EINVAL, "a weight pointer of layer %d is null", l);
  }
  dstill_handle *h = new dstill_handle;
  h->cfg = *cfg;
  h->w = *w;
  h->layers.assign(w->layers, w->layers + cfg->n_layers);
  h->w.layers = h->layers.data();
  *out = h;
  return DSTILL_OK;
}

int dstill_destroy(dstill_handle *h) {
  delete h;
  return DSTILL_OK;
}

int dstill_kv_bytes(const dstill_config *cfg, int32_t max_batch, int32_t cap, size_t *bytes) {
  if (int e = check_config(cfg)) return e;
  if (!bytes) return fail(DSTILL_EINVAL, "bytes is null");
  if (max_batch < 1 || cap < 1 || cap % 64)
    return fail(DSTILL_ESHAPE, "max_batch must be >= 1 and cap a positive multiple of 64");
  *bytes = (size_t)max_batch * cfg->n_kv_heads * cap * cfg->head_dim * elem_bytes(cfg->dtype);
  return DSTILL_OK;
}

int dstill_workspace_bytes(const dstill_handle *h, const dstill_limits *lim, size_t *bytes) {
  if (!h || !lim || !bytes) return fail(DSTILL_EINVAL, "null argument");
  if (lim->max_batch < 0 || lim->max_copies < 0 || lim->max_ctx < 0 || lim->max_inject_rows < 0 ||
      lim->max_head_rows < 0)
    return fail(DSTILL_ESHAPE, "limits must be >= 0");
  const dstill_config &c = h->cfg;
  const int ncu = num_cu();
  size_t best = 0;
  // block_draft: every (bs, copies) up to the limits at the largest block
  const int B = c.max_block;
  for (int bs = 1; bs <= lim->max_batch; ++bs)
    for (int C = 1; C <= std::max(1, lim->max_copies); ++C) {
      const int pairs = bs * C * c.n_kv_heads;
      const AttnPlan ap = attn_plan(std::max(1, lim->max_ctx), pairs, ncu);
      // a call with a smaller max_ctx may plan more, shorter splits (never
      // more than 3 ncu / pairs + 1): bound the count
      AttnPlan bound = ap;
      bound.nsplit = std::max(ap.nsplit, std::min((std::max(1, lim->max_ctx) + 127) / 128,
                                                  3 * ncu / pairs + 2));
      best = std::max(best, draft_ws(c, bs, C, B, bound, ncu, nullptr, nullptr));
      // fewer rows per block give other k-split choices
      for (int b2 = 1; b2 < B; ++b2)
        best = std::max(best, draft_ws(c, bs, C, b2, bound, ncu, nullptr, nullptr));
    }
  // every row count: a product's k-split plan can move either way with the
  // row count, so skipping any could under-report (each size costs a few
  // split-plan evaluations: ~50 ms of host time at 65536 rows)
  for (int n = 1; n <= lim->max_inject_rows; ++n)
    best = std::max(best, inject_ws(c, n, ncu, nullptr, nullptr));
  best = std::max(best, head_ws(c, lim->max_head_rows));
  *bytes = best;
  return DSTILL_OK;
}

int dstill_inject_kv(const dstill_handle *h, const void *feats, const int32_t *seq_id,
                     const int32_t *pos, int32_t n, const dstill_kv *kv, void *ws,
                     size_t ws_bytes, void *stream) {
  if (!h) return fail(DSTILL_EINVAL, "handle is null");
  if (n < 0) return fail(DSTILL_ESHAPE, "n = %d < 0", n);
  if (n == 0) return DSTILL_OK;
  if (!feats || !seq_id || !pos) return fail(DSTILL_EINVAL, "feats/seq_id/pos is null");
  if (int e = check_kv(h, kv)) return e;
  if (!ws) return fail(DSTILL_EINVAL, "ws is null");
  const dstill_config &c = h->cfg;
  const int ncu = num_cu();
  const size_t need = inject_ws(c, n, ncu, nullptr, nullptr);
  if (ws_bytes < need) return fail(DSTILL_EWORKSPACE, "inject_kv needs %zu workspace bytes", need);
  InjectWs w;
  inject_ws(c, n, ncu, ws, &w);
  hipStream_t st = (hipStream_t)stream;
  const int d = c.hidden, F = c.n_feat_layers * c.target_hidden;
  const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  const int eb = elem_bytes(c.dtype);

  launch_rope_table(nullptr, 1, 1, pos, n, c.head_dim, c.rope_theta, w.rope, st);
  GemmArgs g;
  g.dtype = c.dtype;
  g.X = feats; g.ldx = F; g.W = h->w.w_fuse; g.ldw = F; g.out = w.parts;
  g.M = n; g.N = d; g.K = F;
  g.splits = gemm_plan_splits(n, d, F, c.dtype, ncu);
  launch_gemm(g, st);
  launch_norm_rows(c.dtype, w.parts, g.splits, n, d, nullptr, 0, h->w.g_fuse, c.rms_eps, w.ht, d,
                   w.xtmp, w.ssp, st);
  // K/V rows of the draft layers: with bf16 weights one product covers up to
  // GEMM_MAX_GROUPS layers (each layer's W^K|W^V rows are one weight group)
  // and one pass scatters all of them; otherwise one product per layer
  const int per = gemm_can_group(d, c.dtype) && (2 * kvd) % 256 == 0 ? GEMM_MAX_GROUPS : 1;
  for (int l0 = 0; l0 < c.n_layers; l0 += per) {
    const int nl = std::min(per, c.n_layers - l0);
    GemmArgs k;
    k.dtype = c.dtype;
    k.X = w.ht; k.ldx = d;
    k.ldw = d; k.out = w.parts; k.M = n; k.N = 2 * kvd * nl; k.K = d;
    InjectLayers il;
    il.layers = nl;
    for (int i = 0; i < nl; ++i) {
      const dstill_layer_weights &L = h->layers[l0 + i];
      const void *wkv = (const char *)L.wqkv + (size_t)qd * d * eb;  // rows W^K then W^V
      if (per > 1) k.wg[i] = wkv;
      else k.W = wkv;
      il.k_norm[i] = L.k_norm;
      il.kc[i] = kv->k[l0 + i];
      il.vc[i] = kv->v[l0 + i];
    }
    if (per > 1) k.wg_rows = 2 * kvd;
    k.splits = gemm_plan_splits(n, k.N, d, c.dtype, ncu);
    launch_gemm(k, st);
    launch_inject_post(c.dtype, w.parts, k.splits, n, c.n_kv_heads, c.head_dim, seq_id, pos, il,
                       c.qk_norm, c.rms_eps, w.rope, kv->max_batch, kv->cap, st);
  }
  return hip_check("inject_kv launch");
}

int dstill_block_draft(const dstill_handle *h, const int32_t *block_tokens,
                       const int32_t *ctx_len, int32_t bs, int32_t block, int32_t n_copies,
                       int32_t max_ctx, const dstill_kv *kv, void *hidden_out, uint32_t *flags,
                       void *ws, size_t ws_bytes, void *stream) {
  if (!h) return fail(DSTILL_EINVAL, "handle is null");
  const dstill_config &c = h->cfg;
  if (bs < 0 || n_copies < 1) return fail(DSTILL_ESHAPE, "bs must be >= 0 and n_copies >= 1");
  if (block < 1 || block > c.max_block)
    return fail(DSTILL_ESHAPE, "block %d outside 1..max_block (%d)", block, c.max_block);
  if (max_ctx < 0) return fail(DSTILL_ESHAPE, "max_ctx %d < 0", max_ctx);
  if (bs == 0) return DSTILL_OK;
  if (!block_tokens || !ctx_len || !hidden_out) return fail(DSTILL_EINVAL, "null tensor argument");
  if (int e = check_kv(h, kv)) return e;
  if (bs > kv->max_batch) return fail(DSTILL_ESHAPE, "bs %d > kv max_batch %d", bs, kv->max_batch);
  if (!ws) return fail(DSTILL_EINVAL, "ws is null");
  const int ncu = num_cu();
  const int ctx_limit = std::min(max_ctx, kv->cap);
  const AttnPlan ap = attn_plan(std::max(1, ctx_limit), bs * n_copies * c.n_kv_heads, ncu);
  const size_t need = draft_ws(c, bs, n_copies, block, ap, ncu, nullptr, nullptr);
  if (ws_bytes < need) return fail(DSTILL_EWORKSPACE, "block_draft needs %zu workspace bytes", need);
  DraftWs w;
  draft_ws(c, bs, n_copies, block, ap, ncu, ws, &w);
  hipStream_t st = (hipStream_t)stream;
  const int R = bs * n_copies * block, d = c.hidden;
  const int qd = c.n_q_heads * c.head_dim, qkvn = qkv_cols(c);

  launch_draft_prep(block_tokens, ctx_len, bs, n_copies * block, c.vocab, ctx_limit, w.eff_ctx,
                    w.tok, flags, st);
  launch_embed(c.dtype, h->w.embed, w.tok, R, d, w.h, st);
  launch_rope_table(w.eff_ctx, n_copies * block, block, nullptr, R, c.head_dim, c.rope_theta,
                    w.rope, st);
  // pre-attention norm of layer 0; later layers get it fused after the MLP
  launch_norm_rows(c.dtype, nullptr, 0, R, d, w.h, 0, h->layers[0].attn_norm, c.rms_eps, w.u, d,
                   nullptr, w.ssp, st);
  AttnArgs a;
  a.dtype = c.dtype;
  a.q = w.q; a.kb = w.kb; a.vb = w.vb;
  a.eff_ctx = w.eff_ctx;
  a.bs = bs; a.C = n_copies; a.B = block;
  a.hq = c.n_q_heads; a.hkv = c.n_kv_heads; a.dh = c.head_dim; a.cap = kv->cap;
  a.split = ap.split; a.nsplit = ap.nsplit;
  a.scale = 1.0f / sqrtf((float)c.head_dim);
  a.opart = w.opart; a.mlpart = w.mlpart; a.out = w.attn;
  launch_attention_worklist(a, w.wlist, st);
  a.worklist = w.wlist;
  // Windowed layers see at most swa_window + 63 keys from the chunk holding
  // the window's first key: they get a split plan of their own for that
  // range (no more splits than the full plan, whose records the workspace
  // holds) and their own work list.
  AttnArgs aw = a;
  aw.window = c.swa_window;
  bool any_window = false;
  for (int l = 0; l < c.n_layers; ++l)
    any_window = any_window || (c.swa_window > 0 && !((c.full_attn_mask >> l) & 1u));
  if (any_window) {
    const int range = std::min(ctx_limit, c.swa_window + 63);
    const AttnPlan apw = attn_plan(std::max(1, range), bs * n_copies * c.n_kv_heads, ncu);
    if (apw.nsplit <= ap.nsplit) {
      aw.split = apw.split;
      aw.nsplit = apw.nsplit;
    }
    launch_attention_worklist(aw, w.wlist_win, st);
    aw.worklist = w.wlist_win;
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const dstill_layer_weights &L = h->layers[l];
    GemmArgs g;
    g.dtype = c.dtype;
    g.X = w.u; g.ldx = d; g.W = L.wqkv; g.ldw = d; g.out = w.parts;
    g.M = R; g.N = qkvn; g.K = d;
    g.splits = gemm_plan_splits(R, qkvn, d, c.dtype, ncu);
    launch_gemm(g, st);
    launch_qkv_post(c.dtype, w.parts, g.splits, R, c.n_q_heads, c.n_kv_heads, c.head_dim,
                    w.eff_ctx, n_copies * block, block, L.q_norm, L.k_norm, c.qk_norm, c.rms_eps,
                    w.rope, w.q, w.kb, w.vb, st);
    const bool windowed = c.swa_window > 0 && !((c.full_attn_mask >> l) & 1u);
    AttnArgs &al = windowed ? aw : a;
    al.kc = kv->k[l]; al.vc = kv->v[l];
    launch_attention(al, st);
    // O projection, then h += o and the pre-MLP norm
    g.X = w.attn; g.ldx = qd; g.W = L.wo; g.ldw = qd; g.N = d; g.K = qd;
    g.splits = gemm_plan_splits(R, d, qd, c.dtype, ncu);
    launch_gemm(g, st);
    launch_norm_rows(c.dtype, w.parts, g.splits, R, d, w.h, 1, L.mlp_norm, c.rms_eps, w.u, d,
                     nullptr, w.ssp, st);
    // gate|up, SwiGLU, down
    g.X = w.u; g.ldx = d; g.W = L.w_gate_up; g.ldw = d; g.N = 2 * c.mlp; g.K = d;
    g.splits = gemm_plan_splits(R, 2 * c.mlp, d, c.dtype, ncu);
    if (gemm_can_fuse_swiglu(R, c.mlp, d, c.dtype, ncu)) {
      g.splits = 1;
      g.swiglu_act = w.act; g.mlp = c.mlp;  // SwiGLU in the product's epilogue
      launch_gemm(g, st);
      g.swiglu_act = nullptr; g.mlp = 0;
    } else {
      launch_gemm(g, st);
      launch_swiglu(c.dtype, w.parts, g.splits, R, c.mlp, w.act, st);
    }
    g.X = w.act; g.ldx = c.mlp; g.W = L.w_down; g.ldw = c.mlp; g.N = d; g.K = c.mlp;
    g.splits = gemm_plan_splits(R, d, c.mlp, c.dtype, ncu);
    launch_gemm(g, st);
    // h += down; then the next layer's pre-attention norm, or the final norm
    const bool last = l + 1 == c.n_layers;
    launch_norm_rows(c.dtype, w.parts, g.splits, R, d, w.h, 1,
                     last ? h->w.g_final : h->layers[l + 1].attn_norm, c.rms_eps,
                     last ? hidden_out : w.u, d, nullptr, w.ssp, st);
  }
  return hip_check("block_draft launch");
}

int dstill_lm_head_argmax(const dstill_handle *h, const void *hidden, int32_t rows,
                          int32_t rows_per_seq, int32_t seq_stride, const dstill_sample *s,
                          int32_t *ids, float *zmax, float *lse, float *zsel, float *gap,
                          float *logits_out, void *ws, size_t ws_bytes, void *stream) {
  if (!h) return fail(DSTILL_EINVAL, "handle is null");
  if (rows < 0) return fail(DSTILL_ESHAPE, "rows %d < 0", rows);
  if (rows == 0) return DSTILL_OK;
  if (!hidden || !ids || !s) return fail(DSTILL_EINVAL, "hidden/ids/sample is null");
  if (rows_per_seq < 1 || seq_stride < rows_per_seq)
    return fail(DSTILL_ESHAPE, "need rows_per_seq >= 1 and seq_stride >= rows_per_seq");
  if (s->mode < DSTILL_HEAD_ARGMAX || s->mode > DSTILL_HEAD_SHARED_GUMBEL)
    return fail(DSTILL_EINVAL, "unknown head mode %d", s->mode);
  if (!(s->temperature > 0.f)) return fail(DSTILL_EINVAL, "temperature must be > 0");
  if (s->cycle >> 56) return fail(DSTILL_EINVAL, "cycle must be < 2^56");
  if (!ws) return fail(DSTILL_EINVAL, "ws is null");
  const dstill_config &c = h->cfg;
  const size_t need = head_ws(c, rows);
  if (ws_bytes < need) return fail(DSTILL_EWORKSPACE, "lm_head_argmax needs %zu workspace bytes", need);
  HeadArgs a;
  a.dtype = c.dtype;
  a.hidden = hidden;
  a.rows = rows; a.rows_per_seq = rows_per_seq; a.seq_stride = seq_stride;
  a.d = c.hidden; a.vocab = c.vocab; a.w = h->w.lm_head;
  a.mode = s->mode; a.temperature = s->temperature; a.seed = s->seed; a.cycle = s->cycle;
  a.part = (HeadPartial *)ws;
  a.nvb = (c.vocab + head_vocab_block() - 1) / head_vocab_block();
  a.logits = logits_out;
  a.ids = ids; a.zmax = zmax; a.lse = lse; a.zsel = zsel; a.gap = gap;
  launch_lm_head(a, (hipStream_t)stream);
  return hip_check("lm_head_argmax launch");
}

int dstill_verify_workspace_bytes(int32_t bs, int32_t gamma, int32_t vocab, size_t *bytes) {
  if (!bytes) return fail(DSTILL_EINVAL, "bytes is null");
  if (bs < 0 || gamma < 1 || gamma > 63 || vocab < 2)
    return fail(DSTILL_ESHAPE, "need bs >= 0, 1 <= gamma <= 63, vocab >= 2");
  *bytes = verify_ws_bytes(bs, gamma, verify_plan_splits(bs * (gamma + 1), vocab),
                           verify_plan_splits(bs, vocab));
  return DSTILL_OK;
}


int dstill_verify(int32_t mode, int32_t bs, int32_t gamma, int32_t vocab, float temperature,
                  uint64_t seed, uint64_t cycle, const int32_t *draft_ids,
                  const float *draft_lse, const float *draft_logits,
                  const void *target_logits, int32_t target_dtype, int32_t *out_tokens,
                  int32_t *out_tau, uint32_t *out_flags, void *ws, size_t ws_bytes,
                  void *stream) {
  return verify_call(mode, bs, gamma, vocab, temperature, seed, cycle, draft_ids, draft_lse,
                     draft_logits, target_logits, target_dtype, out_tokens, out_tau, out_flags,
                     ws, ws_bytes, stream);
}

int dstill_dloop_branches(int32_t bs, int32_t gamma, int32_t K, const int32_t *anchor,
                          const int32_t *ids, const float *zmax, const float *lse,
                          int32_t mask_id, int32_t *block_tokens, int32_t *prefix_len,
                          double *score, void *stream) {
  if (bs < 0 || gamma < 1 || gamma > 63 || K < 1 || K > gamma)
    return fail(DSTILL_ESHAPE, "need bs >= 0, 1 <= gamma <= 63, 1 <= K <= gamma");
  if (bs == 0) return DSTILL_OK;
  if (!anchor || !ids || !zmax || !lse || !block_tokens || !prefix_len)
    return fail(DSTILL_EINVAL, "null tensor argument");
  DloopArgs a;
  a.bs = bs; a.gamma = gamma; a.K = K; a.mask_id = mask_id;
  a.anchor = anchor; a.ids = ids; a.zmax = zmax; a.lse = lse;
  a.block_tokens = block_tokens; a.prefix_len = prefix_len; a.score = score;
  launch_dloop_branches(a, (hipStream_t)stream);
  return hip_check("dloop_branches launch");
}

int dstill_dloop_merge(int32_t bs, int32_t gamma, int32_t K, const int32_t *first_ids,
                       const int32_t *second_ids, const int32_t *prefix_len, int32_t *out_ids,
                       void *stream) {
  if (bs < 0 || gamma < 1 || gamma > 63 || K < 1 || K > 65535)
    return fail(DSTILL_ESHAPE, "need bs >= 0, 1 <= gamma <= 63, 1 <= K <= 65535");
  if (bs == 0) return DSTILL_OK;
  if (!first_ids || !second_ids || !prefix_len || !out_ids)
    return fail(DSTILL_EINVAL, "null tensor argument");
  launch_dloop_merge(bs, gamma, K, first_ids, second_ids, prefix_len, out_ids,
                     (hipStream_t)stream);
  return hip_check("dloop_merge launch");
}

static size_t branch_ws_bytes(int32_t bs, int32_t K, int32_t gamma, int32_t vocab) {
  const long n = (long)bs * K;
  const size_t inner = verify_ws_bytes((int)n, gamma, verify_plan_splits((int)n * (gamma + 1), vocab),
                                       verify_plan_splits((int)n, vocab));
  return a256(inner) + a256((size_t)n * (gamma + 1) * 4) + 2 * a256((size_t)n * 4);
}

int dstill_verify_branches_workspace_bytes(int32_t bs, int32_t K, int32_t gamma, int32_t vocab,
                                           size_t *bytes) {
  if (!bytes) return fail(DSTILL_EINVAL, "bytes is null");
  if (bs < 0 || K < 1 || gamma < 1 || gamma > 63 || vocab < 2 || (long)bs * K > (1L << 24))
    return fail(DSTILL_ESHAPE, "need bs >= 0, K >= 1, 1 <= gamma <= 63, vocab >= 2");
  *bytes = branch_ws_bytes(bs, K, gamma, vocab);
  return DSTILL_OK;
}

int dstill_verify_branches(int32_t bs, int32_t K, int32_t gamma, int32_t vocab,
                           const int32_t *draft_ids, const void *target_logits,
                           int32_t target_dtype, int32_t *out_tokens, int32_t *out_tau,
                           int32_t *out_branch, uint32_t *out_flags, void *ws, size_t ws_bytes,
                           void *stream) {
  if (bs < 0 || K < 1 || gamma < 1 || gamma > 63 || vocab < 2 || (long)bs * K > (1L << 24))
    return fail(DSTILL_ESHAPE, "need bs >= 0, K >= 1, 1 <= gamma <= 63, vocab >= 2");
  if (target_dtype != DSTILL_F32 && target_dtype != DSTILL_BF16)
    return fail(DSTILL_EUNSUPPORTED, "target_dtype %d", target_dtype);
  if (bs == 0) return DSTILL_OK;
  if (!draft_ids || !target_logits || !out_tokens || !out_tau || !out_flags || !ws)
    return fail(DSTILL_EINVAL, "null tensor argument");
  const size_t need = branch_ws_bytes(bs, K, gamma, vocab);
  if (ws_bytes < need)
    return fail(DSTILL_EWORKSPACE, "verify_branches needs %zu workspace bytes", need);
  const int n = bs * K;
  Carver cv(ws);
  const int nsplit = verify_plan_splits(n * (gamma + 1), vocab);
  const int nsamp = verify_plan_splits(n, vocab);
  void *inner = cv.take<char>(verify_ws_bytes(n, gamma, nsplit, nsamp));
  int32_t *tok = cv.take<int32_t>((size_t)n * (gamma + 1));
  int32_t *tau = cv.take<int32_t>(n);
  uint32_t *flg = cv.take<uint32_t>(n);
  hipStream_t st = (hipStream_t)stream;
  // every branch verified as its own sequence, then the longest one kept
  VerifyArgs a;
  a.mode = DSTILL_VERIFY_GREEDY; a.bs = n; a.gamma = gamma; a.vocab = vocab;
  a.tdtype = target_dtype; a.temperature = 1.0f; a.seed = 0; a.cycle = 0;
  a.draft_ids = draft_ids; a.draft_lse = nullptr; a.draft_logits = nullptr;
  a.target = target_logits;
  a.tokens = tok; a.tau = tau; a.flags = flg;
  a.ws = inner; a.nsplit = nsplit; a.nsamp = nsamp;
  launch_verify(a, st);
  launch_branch_pick(bs, K, gamma, tok, tau, flg, out_tokens, out_tau, out_branch, out_flags, st);
  return hip_check("verify_branches launch");
}

int dstill_spot_verify(int32_t bs, int32_t n_states, int32_t L, int32_t mask_id,
                       float temperature, const int32_t *states, const int32_t *parent,
                       const int32_t *ids, const float *zmax, const float *lse, const float *gap,
                       int32_t *out_n, int32_t *out_slots, int32_t *out_tokens,
                       int32_t *out_state, uint32_t *out_flags, void *stream) {
  if (bs < 0 || n_states < 1 || n_states > 64 || L < 1 || L > 64)
    return fail(DSTILL_ESHAPE, "need bs >= 0, 1 <= n_states <= 64, 1 <= L <= 64");
  if (!(temperature > 0.f)) return fail(DSTILL_EINVAL, "temperature must be > 0");
  if (bs == 0) return DSTILL_OK;
  if (!states || !parent || !ids || !zmax || !lse || !out_n || !out_slots || !out_tokens ||
      !out_state || !out_flags)
    return fail(DSTILL_EINVAL, "null tensor argument");
  SpotArgs a;
  a.bs = bs; a.n_states = n_states; a.L = L; a.mask_id = mask_id; a.temperature = temperature;
  a.states = states; a.parent = parent; a.ids = ids; a.zmax = zmax; a.lse = lse; a.gap = gap;
  a.out_n = out_n; a.out_slots = out_slots; a.out_tokens = out_tokens; a.out_state = out_state;
  a.out_flags = out_flags;
  launch_spot_verify(a, (hipStream_t)stream);
  return hip_check("spot_verify launch");
}

int dstill_refine_commit(int32_t bs, int32_t block, int32_t t, int32_t K, const int32_t *ids,
                         const float *zmax, const float *lse, int32_t *tokens, int32_t *kappa,
                         void *stream) {
  if (bs < 0 || block < 2 || block > 64 || K < 1 || t < 1 || t > K)
    return fail(DSTILL_ESHAPE, "need bs >= 0, 2 <= block <= 64, 1 <= t <= K");
  if (bs == 0) return DSTILL_OK;
  if (!ids || !zmax || !lse || !tokens || !kappa)
    return fail(DSTILL_EINVAL, "null tensor argument");
  RefineArgs a;
  a.bs = bs; a.block = block; a.t = t; a.K = K;
  a.ids = ids; a.zmax = zmax; a.lse = lse; a.tokens = tokens; a.kappa = kappa;
  launch_refine_commit(a, (hipStream_t)stream);
  return hip_check("refine_commit launch");
}

}  // extern "C"
