// sampler_sample_noalloc: sampler_sample with its workspace in a file-scope
// device array instead of a caller buffer, for callers that cannot allocate
// (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Nothing here allocates: the array is part of the library's
// device code object, placed on each GPU when the runtime loads the library
// there, and held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is ever passed to kernels.
#include <mutex>

#include "ts_internal.hpp"

namespace {

constexpr size_t kScratchBytes = TS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

thread_local char g_err[256] = "";

// The device address of this device's copy of `scratch` (nullptr and a
// message on failure).
void* scratch_for(int dev, const char** why) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) return g_scratch[dev];
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr) {
    snprintf(g_err, sizeof(g_err), "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
             hipGetErrorString(e));
    *why = g_err;
    return nullptr;
  }
  g_scratch[dev] = p;
  return p;
}

}  // namespace

namespace ts {
// Records a failure for ts_last_error (defined with the other entry points).
int fail_message(int code, const char* msg);
}  // namespace ts

extern "C" int sampler_sample_noalloc(const float* logits, int64_t rows, int64_t vocab,
                                      int64_t ld_logits, const ts_row_params* params,
                                      int64_t row_offset, int32_t max_logprobs,
                                      int32_t* token_ids, float* token_logprobs,
                                      int32_t* topn_ids, float* topn_logprobs,
                                      int32_t* row_status, void* stream) {
  if (rows < 0 || vocab < 0 || max_logprobs < 0)
    return ts::fail_message(TS_EINVAL, "negative size or max_logprobs");
  if (rows == 0) return TS_OK;
  const size_t need = sampler_workspace_bytes(rows, vocab, max_logprobs);
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "rows=%lld vocab=%lld max_logprobs=%d need a %zu-byte workspace; the built-in "
             "scratch holds %zu (use sampler_sample with a caller workspace)",
             (long long)rows, (long long)vocab, max_logprobs, need, kScratchBytes);
    return ts::fail_message(TS_EUNSUPPORTED, msg);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return ts::fail_message(TS_EHIP, "no current HIP device (or more than 64 devices)");
  const char* why = "";
  void* ws = scratch_for(dev, &why);
  if (!ws) return ts::fail_message(TS_EHIP, why);
  return sampler_sample(logits, rows, vocab, ld_logits, params, row_offset, max_logprobs,
                        token_ids, token_logprobs, topn_ids, topn_logprobs, row_status, ws,
                        kScratchBytes, stream);
}
