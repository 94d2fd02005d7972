// Host-side argument checks of the C ABI (include/dstill.h), driven from C++
// so the library's host code can be built and run under AddressSanitizer
// and UndefinedBehaviorSanitizer (tests/test_abi_sanitized.py).  Every call
// here fails validation (or is a pure size query) before the library touches
// a device, so no GPU is needed.  Exits 0 when every check holds; a sanitizer
// finding aborts the process.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "dstill.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static dstill_config base_cfg() {
  dstill_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = 2; c.hidden = 512; c.n_q_heads = 8; c.n_kv_heads = 2; c.head_dim = 128;
  c.mlp = 1408; c.vocab = 5003; c.n_feat_layers = 3; c.target_hidden = 384; c.max_block = 16;
  c.mask_token_id = 5002; c.qk_norm = 1; c.dtype = DSTILL_BF16; c.rms_eps = 1e-6f;
  c.rope_theta = 1e6f;
  return c;
}

int main() {
  void *p = reinterpret_cast<void *>(4096);  // never dereferenced: calls fail validation first
  dstill_layer_weights L[2];
  for (auto &l : L) l = {p, p, p, p, p, p, p, p};
  dstill_weights w = {p, p, p, p, p, L};
  dstill_handle *h = nullptr;

  // create: bad configs are refused with a message
  CHECK(dstill_create(nullptr, &w, &h) == DSTILL_EINVAL);
  struct Bad { void (*set)(dstill_config &); int code; } bad[] = {
      {[](dstill_config &c) { c.head_dim = 96; }, DSTILL_EUNSUPPORTED},
      {[](dstill_config &c) { c.n_kv_heads = 3; }, DSTILL_ESHAPE},
      {[](dstill_config &c) { c.max_block = 17; }, DSTILL_EUNSUPPORTED},
      {[](dstill_config &c) { c.dtype = 7; }, DSTILL_EUNSUPPORTED},
      {[](dstill_config &c) { c.mlp = 1400; }, DSTILL_EUNSUPPORTED},
      {[](dstill_config &c) { c.mask_token_id = 5003; }, DSTILL_ESHAPE},
      {[](dstill_config &c) { c.vocab = 1; }, DSTILL_ESHAPE},
  };
  for (const Bad &b : bad) {
    dstill_config c = base_cfg();
    b.set(c);
    CHECK(dstill_create(&c, &w, &h) == b.code);
    CHECK(dstill_last_error() && std::strlen(dstill_last_error()) > 0);
  }
  dstill_layer_weights Lnull[2] = {};
  dstill_weights wnull = {p, p, p, p, p, Lnull};
  dstill_config c = base_cfg();
  CHECK(dstill_create(&c, &wnull, &h) == DSTILL_EINVAL);

  // a valid handle and the size queries
  CHECK(dstill_create(&c, &w, &h) == DSTILL_OK && h != nullptr);
  size_t n = 0;
  CHECK(dstill_kv_bytes(&c, 3, 128, &n) == DSTILL_OK && n == 3u * 2 * 128 * 128 * 2);
  CHECK(dstill_kv_bytes(&c, 3, 104, &n) == DSTILL_ESHAPE);
  dstill_limits lim = {3, 2, 1029, 77, 45};
  CHECK(dstill_workspace_bytes(h, &lim, &n) == DSTILL_OK && n > 0);
  dstill_limits neg = {-1, 0, 0, 0, 0};
  CHECK(dstill_workspace_bytes(h, &neg, &n) == DSTILL_ESHAPE);

  // calls that fail validation enqueue nothing
  void *kvp[2] = {p, p};
  dstill_kv kv = {kvp, kvp, 3, 128};
  dstill_sample s = {DSTILL_HEAD_ARGMAX, 1.0f, 0, 0};
  const int32_t *ip = static_cast<const int32_t *>(p);
  CHECK(dstill_block_draft(h, ip, ip, 4, 16, 1, 50, &kv, p, nullptr, p, 1u << 30, nullptr) ==
        DSTILL_ESHAPE);  // bs > max_batch
  CHECK(dstill_block_draft(h, ip, ip, 2, 17, 1, 50, &kv, p, nullptr, p, 1u << 30, nullptr) ==
        DSTILL_ESHAPE);  // block > max_block
  CHECK(dstill_block_draft(h, ip, ip, 2, 16, 1, 50, &kv, p, nullptr, p, 1, nullptr) ==
        DSTILL_EWORKSPACE);
  dstill_kv kvbad = {kvp, kvp, 3, 100};
  CHECK(dstill_block_draft(h, ip, ip, 2, 16, 1, 50, &kvbad, p, nullptr, p, 1u << 30, nullptr) ==
        DSTILL_ESHAPE);  // cap not a multiple of 64
  int32_t *op = static_cast<int32_t *>(p);
  CHECK(dstill_lm_head_argmax(h, p, 15, 15, 16, &s, op, nullptr, nullptr, nullptr, nullptr,
                              nullptr, p, 8, nullptr) == DSTILL_EWORKSPACE);
  s.temperature = 0.0f;
  CHECK(dstill_lm_head_argmax(h, p, 15, 15, 16, &s, op, nullptr, nullptr, nullptr, nullptr,
                              nullptr, p, 1u << 30, nullptr) == DSTILL_EINVAL);
  CHECK(dstill_inject_kv(h, p, ip, ip, -1, &kv, p, 1u << 30, nullptr) == DSTILL_ESHAPE);
  CHECK(dstill_inject_kv(h, p, ip, ip, 5, &kv, p, 8, nullptr) == DSTILL_EWORKSPACE);
  CHECK(dstill_destroy(h) == DSTILL_OK);

  // verification is model-independent
  CHECK(dstill_verify_workspace_bytes(32, 15, 151936, &n) == DSTILL_OK && n > 0);
  CHECK(dstill_verify_workspace_bytes(32, 64, 151936, &n) == DSTILL_ESHAPE);
  const float *fp = static_cast<const float *>(p);
  uint32_t *up = static_cast<uint32_t *>(p);
  CHECK(dstill_verify(3, 2, 15, 1000, 1.0f, 0, 0, ip, fp, fp, p, 0, op, op, up, p, 1u << 30,
                      nullptr) == DSTILL_EINVAL);  // mode
  CHECK(dstill_verify(DSTILL_VERIFY_RS, 2, 15, 1000, 1.0f, 0, 0, ip, nullptr, nullptr, p, 0, op,
                      op, up, p, 1u << 30, nullptr) == DSTILL_EINVAL);  // RS without q
  CHECK(dstill_verify(DSTILL_VERIFY_GREEDY, 2, 15, 1000, 1.0f, 0, 0, ip, fp, fp, p, 0, op, op,
                      up, p, 16, nullptr) == DSTILL_EWORKSPACE);
  CHECK(dstill_verify(DSTILL_VERIFY_GREEDY, 2, 15, 1000, 1.0f, 0, 0, ip, nullptr, nullptr, p, 5,
                      op, op, up, p, 1u << 30, nullptr) == DSTILL_EUNSUPPORTED);  // dtype
  CHECK(dstill_verify(DSTILL_VERIFY_GREEDY, 0, 15, 1000, 1.0f, 0, 0, ip, fp, fp, p, 0, op, op,
                      up, p, 0, nullptr) == DSTILL_OK);  // empty batch
  CHECK(dstill_verify(DSTILL_VERIFY_GREEDY, 2, 15, 1000, 1.0f, 0, 1ull << 60, ip, fp, fp, p, 0,
                      op, op, up, p, 1u << 30, nullptr) == DSTILL_EINVAL);  // cycle range
  // the no-allocation variant refuses a shape beyond its scratch before any device call
  CHECK(dstill_verify_noalloc(DSTILL_VERIFY_GREEDY, 7000, 15, 151936, 1.0f, 0, 0, ip, nullptr,
                              nullptr, p, DSTILL_F32, op, op, up, nullptr) == DSTILL_EWORKSPACE);
  CHECK(dstill_verify_noalloc(DSTILL_VERIFY_GREEDY, 0, 15, 151936, 1.0f, 0, 0, ip, nullptr,
                              nullptr, p, DSTILL_F32, op, op, up, nullptr) == DSTILL_OK);

  // the small decision kernels' shape checks
  double *dp = static_cast<double *>(p);
  CHECK(dstill_dloop_branches(1, 15, 16, ip, ip, fp, fp, 0, op, op, dp, nullptr) == DSTILL_ESHAPE);
  CHECK(dstill_dloop_merge(1, 64, 4, ip, ip, ip, op, nullptr) == DSTILL_ESHAPE);
  CHECK(dstill_refine_commit(1, 65, 1, 8, ip, fp, fp, op, op, nullptr) == DSTILL_ESHAPE);
  CHECK(dstill_refine_commit(1, 16, 9, 8, ip, fp, fp, op, op, nullptr) == DSTILL_ESHAPE);
  CHECK(dstill_version() == 100);

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("abi checks: all passed\n");
  return 0;
}
