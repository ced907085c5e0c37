// Opt-in per-kernel timing: when enabled, every launch of a selected kernel is
// bracketed by two HIP events recorded on the launch stream; attn_profile_read
// waits for them and sums the elapsed times per kernel.  Disabled (the
// default), the hooks cost one relaxed atomic load per launch.  The events
// themselves cost a few microseconds of GPU time per launch, so a caller
// timing the whole step selects only the kernels it needs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/swattn.h"
#include "profile.h"

namespace swattn {
namespace {

struct Rec {
  int kernel;
  hipEvent_t start, stop;
};

std::atomic<unsigned> g_mask{0u};   // bit i: kernel i is recorded
std::mutex g_mu;
std::vector<Rec> g_recs;
double g_total_ms[kNumKernels];
long long g_count[kNumKernels];

const char* kNames[kNumKernels] = {"fwd_prep", "attn_fwd", "bwd_kscale", "bwd_dkdv", "bwd_dq", "bwd_gate"};
static_assert(kNumKernels <= 32, "one mask bit per kernel");

// fold finished records into the totals; returns false on a HIP error
bool drain() {
  bool ok = true;
  for (Rec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      ok = false;
    } else {
      g_total_ms[r.kernel] += ms;
      g_count[r.kernel] += 1;
    }
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_recs.clear();
  return ok;
}

}  // namespace

ProfToken prof_begin(int kernel, hipStream_t stream) {
  ProfToken t{-1, nullptr, nullptr, stream};
  if (((g_mask.load(std::memory_order_relaxed) >> kernel) & 1u) == 0) return t;
  if (hipEventCreate(&t.start) != hipSuccess) return t;
  if (hipEventCreate(&t.stop) != hipSuccess) {
    (void)hipEventDestroy(t.start);
    return t;
  }
  (void)hipEventRecord(t.start, stream);
  t.kernel = kernel;
  return t;
}

void prof_end(const ProfToken& t) {
  if (t.kernel < 0) return;
  (void)hipEventRecord(t.stop, t.stream);
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back(Rec{t.kernel, t.start, t.stop});
}

}  // namespace swattn

extern "C" {

int attn_profile_enable_mask(unsigned mask) {
  std::lock_guard<std::mutex> lk(swattn::g_mu);
  bool ok = swattn::drain();
  for (int i = 0; i < swattn::kNumKernels; ++i) {
    swattn::g_total_ms[i] = 0.0;
    swattn::g_count[i] = 0;
  }
  swattn::g_mask.store(mask & ((1u << swattn::kNumKernels) - 1u));
  return ok ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_profile_enable(int on) { return attn_profile_enable_mask(on ? ~0u : 0u); }

int attn_profile_read(int kernel, double* total_ms, long long* launches) {
  if (kernel < 0 || kernel >= swattn::kNumKernels || !total_ms || !launches) return ATTN_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(swattn::g_mu);
  bool ok = swattn::drain();
  *total_ms = swattn::g_total_ms[kernel];
  *launches = swattn::g_count[kernel];
  return ok ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_device_info(int device, int* compute_units, int* max_clock_khz) {
  if (!compute_units || !max_clock_khz || device < 0) return ATTN_ERR_INVALID_ARG;
  if (hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, device) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

const char* attn_kernel_name(int kernel) {
  if (kernel < 0 || kernel >= swattn::kNumKernels) return "unknown";
  return swattn::kNames[kernel];
}

}  // extern "C"
