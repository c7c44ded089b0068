// Relaxed chain verification without a caller workspace: the per-chunk
// partials live in a fixed device array of this library instead, so the
// call needs no allocation at all (for callers that cannot allocate: code
// under graph capture, tight serving loops, harnesses that forbid it).
//
// The array is a file-scope __device__ symbol.  Its host-side name is only a
// stand-in, so each device's address of it is taken once with
// hipGetSymbolAddress while that device is current, and only that address
// is handed to the kernels.  Every call on one device shares its array:
// calls that overlap on one device (two streams without ordering between
// them) race on it.  The partials need no clearing: each scan workgroup
// writes its own slot before the final pass reads it.
#include <mutex>

#include "../../include/eagle3.h"
#include "common.h"
#include "internal.h"

namespace e3 {
namespace {

constexpr size_t kScratchBytes = EAGLE3_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint4 scratch[kScratchBytes / sizeof(uint4)];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, taken on the first call made with it
// current; NULL if the runtime refuses.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace e3

using namespace e3;

extern "C" {

eagle3_status eagle3_relaxed_accept_noalloc(const int32_t* draft, const float* logits, const uint8_t* relaxed,
                                            int32_t batch, int32_t gamma, int32_t vocab, int32_t topk,
                                            float delta, int32_t* accept_len, int32_t* bonus,
                                            eagle3_stream_t stream) {
  size_t need = 0;
  const eagle3_status st = eagle3_relaxed_accept_workspace_size(batch, gamma, vocab, &need);
  if (st != EAGLE3_OK) return st;
  if (need > kScratchBytes) return EAGLE3_ERR_WORKSPACE;
  void* p = device_scratch();
  if (!p) return EAGLE3_ERR_HIP;
  return eagle3_relaxed_accept(draft, logits, relaxed, batch, gamma, vocab, topk, delta, accept_len, bonus, p,
                               kScratchBytes, stream);
}

}  // extern "C"
