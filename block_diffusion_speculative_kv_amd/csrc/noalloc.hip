// dstill_verify_noalloc: verification for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It is dstill_verify with the workspace
// taken from a fixed device array of DSTILL_NOALLOC_SCRATCH_BYTES in this
// library instead of from the caller.
//
// The array's name is a host-side stand-in on the host, not a device
// address: its address on each device comes from hipGetSymbolAddress, looked
// up once per device (with that device current) on the first call there, and
// only that pointer is handed to the kernels.  Every byte the verification
// kernels read from their workspace is written earlier in the same call (split
// records, target log-sum-exps, per-sequence decisions, sampling records), so
// nothing has to start at zero and no clearing pass is enqueued.  All calls on
// one device share its array: calls that overlap on one device (different
// streams, or different host threads, without ordering between them) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dstill.h"
#include "kernels.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[DSTILL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of this device's copy of the scratch array (null on error,
// with the error recorded).
void *scratch_ptr(int *status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = dstill::api_fail(DSTILL_EHIP, "verify_noalloc: no current device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *status = dstill::api_fail(DSTILL_EHIP, "verify_noalloc: scratch symbol lookup failed");
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int dstill_verify_noalloc(int32_t mode, int32_t bs, int32_t gamma, int32_t vocab,
                                     float temperature, uint64_t seed, uint64_t cycle,
                                     const int32_t *draft_ids, const float *draft_lse,
                                     const float *draft_logits, const void *target_logits,
                                     int32_t target_dtype, int32_t *out_tokens, int32_t *out_tau,
                                     uint32_t *out_flags, void *stream) {
  // the workspace bound is checked before anything touches the device
  if (bs > 0 && gamma >= 1 && gamma <= 63 && vocab >= 2) {
    size_t need = 0;
    if (dstill_verify_workspace_bytes(bs, gamma, vocab, &need) != DSTILL_OK) return DSTILL_ESHAPE;
    if (need > DSTILL_NOALLOC_SCRATCH_BYTES)
      return dstill::api_fail(DSTILL_EWORKSPACE,
                              "verify_noalloc: this shape needs more than the fixed scratch "
                              "(DSTILL_NOALLOC_SCRATCH_BYTES); use dstill_verify");
  }
  int status = DSTILL_OK;
  void *ws = nullptr;
  if (bs > 0) {
    ws = scratch_ptr(&status);
    if (!ws) return status;
  }
  return dstill::verify_call(mode, bs, gamma, vocab, temperature, seed, cycle, draft_ids,
                             draft_lse, draft_logits, target_logits, target_dtype, out_tokens,
                             out_tau, out_flags, ws, DSTILL_NOALLOC_SCRATCH_BYTES, stream);
}
