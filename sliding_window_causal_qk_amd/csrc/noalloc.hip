// attn_fwd_noalloc: the forward for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The forward's only scratch buffer -- the per-key logit scales
// of the QK-RMSNorm, fp32 [B, H, T] -- lives in a file-scope device array
// instead of a caller's workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` from the
// library's first use on that device until the process ends.  Its address on a
// device comes from hipGetSymbolAddress with that device current, once per
// device; kernels only ever see that address, never the host-side symbol.
// Every call on one device shares the array: calls that overlap in time on one
// device (two streams, or two host threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/swattn.h"

namespace {
constexpr size_t kScratchBytes = size_t(8) << 20;   // fp32 key scales of B * H * T <= 2^21 rows
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up once).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t attn_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int T,
                     int H, int D, int window, int causal, float eps, void* stream) {
  // Empty problems and problems beyond the scratch size go to attn_fwd with no
  // workspace: it validates every argument first (so a bad argument reports
  // the same status as there), returns ATTN_OK for an empty problem and
  // ATTN_ERR_WORKSPACE for a valid one -- without any HIP call.
  const size_t need = attn_fwd_workspace_bytes(B, T, H, D);
  if (B <= 0 || T <= 0 || H <= 0 || need > kScratchBytes)
    return attn_fwd(q, k, v, o, lse, nullptr, 0, B, T, H, D, window, causal, eps, stream);
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return ATTN_ERR_HIP;
  return attn_fwd(q, k, v, o, lse, ws, kScratchBytes, B, T, H, D, window, causal, eps, stream);
}

}  // extern "C"
