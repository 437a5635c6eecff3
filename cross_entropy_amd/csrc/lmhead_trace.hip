// lmhead_trace.hip -- optional per-kernel tracing of the library's launches.
//
// When enabled, every kernel launch of the library is bracketed by two HIP
// events recorded on the stream the kernel is launched on, and tagged with
// the algorithmic work of that launch (flops and bytes). Reading folds the
// finished records into per-kernel totals (launches, summed duration, summed
// work). Disabled (the default), the hooks cost one atomic load per launch
// and record nothing. This is the one piece of state the library keeps
// across calls; it exists for measurement only.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/lmhead_logps.h"
#include "lmhead_internal.h"

namespace lmh {
namespace {

struct Record {
  int kernel;
  hipEvent_t start, stop;
  double flops, bytes;
};

struct Totals {
  int64_t launches = 0;
  double ms = 0.0, flops = 0.0, bytes = 0.0;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<hipEvent_t> g_pool;
std::vector<Record> g_pending;
Totals g_totals[kNumKernels];
thread_local hipEvent_t t_start = nullptr;

const char* const kNames[kNumKernels] = {
    "fwd_stats_kernel", "fwd_merge_kernel", "bwd_step_kernel", "transpose_kernel", "fill_zero_kernel",
    "pad_rows_kernel", "bwd_step_bf16_kernel",
};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Folds every pending record whose events have completed (waits for them).
void fold_locked() {
  for (Record& r : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      Totals& t = g_totals[r.kernel];
      t.launches += 1;
      t.ms += ms;
      t.flops += r.flops;
      t.bytes += r.bytes;
    }
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_pending.clear();
}

}  // namespace

void trace_begin(hipStream_t stream) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  t_start = take_event();
  if (t_start) (void)hipEventRecord(t_start, stream);
}

void trace_end(int kernel, hipStream_t stream, double flops, double bytes) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!t_start) return;
  hipEvent_t stop = take_event();
  if (!stop) return;
  (void)hipEventRecord(stop, stream);
  g_pending.push_back(Record{kernel, t_start, stop, flops, bytes});
  t_start = nullptr;
}

}  // namespace lmh

extern "C" {

int lmhead_logps_trace_enable(int on) {
  std::lock_guard<std::mutex> lk(lmh::g_mu);
  lmh::fold_locked();
  for (auto& t : lmh::g_totals) t = lmh::Totals{};
  lmh::g_on.store(on != 0);
  return LMH_OK;
}

int lmhead_logps_trace_read(int kernel, int64_t* launches, double* total_ms, double* flops,
                            double* bytes) {
  if (kernel < 0 || kernel >= lmh::kNumKernels) return LMH_ERR_ARGS;
  if (!launches || !total_ms || !flops || !bytes) return LMH_ERR_NULL;
  std::lock_guard<std::mutex> lk(lmh::g_mu);
  lmh::fold_locked();
  const lmh::Totals& t = lmh::g_totals[kernel];
  *launches = t.launches;
  *total_ms = t.ms;
  *flops = t.flops;
  *bytes = t.bytes;
  return LMH_OK;
}

const char* lmhead_logps_trace_kernel_name(int kernel) {
  if (kernel < 0 || kernel >= lmh::kNumKernels) return nullptr;
  return lmh::kNames[kernel];
}

}  // extern "C"
