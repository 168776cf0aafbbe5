// profile.hip -- opt-in per-kernel timing with HIP events (tracing aid).
//
// While enabled, every kernel the library enqueues is bracketed by two HIP
// events recorded on the stream the kernel is launched on; qlora_profile_end
// waits for them and accumulates the elapsed time per kernel name.  Off by
// default: then a launch costs one relaxed atomic load.
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/qlora_profile.h"
#include "qlora_internal.h"

namespace qlora {
namespace {

struct Record {
  const char *name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;
std::vector<std::pair<std::string, std::pair<int64_t, double>>> g_summary;

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

}  // namespace

ProfScope::ProfScope(const char *name, hipStream_t s) : name_(name), stream_(s) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  stop_ = take_event();
  if (start_ && stop_) (void)hipEventRecord(start_, s);
}

ProfScope::~ProfScope() {
  if (!start_ || !stop_) return;
  (void)hipEventRecord(stop_, stream_);
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back({name_, start_, stop_});
}

}  // namespace qlora

using namespace qlora;

extern "C" {

int qlora_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto &r : g_records) {
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
  g_summary.clear();
  g_enabled.store(true);
  return QLORA_OK;
}

int qlora_profile_end(void) {
  g_enabled.store(false);
  std::lock_guard<std::mutex> lk(g_mu);
  std::map<std::string, std::pair<int64_t, double>> acc;
  int status = QLORA_OK;
  for (auto &r : g_records) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      status = QLORA_ERR_HIP;
    auto &e = acc[r.name];
    e.first += 1;
    e.second += ms;
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_records.clear();
  g_summary.assign(acc.begin(), acc.end());
  return status;
}

int qlora_profile_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int)g_summary.size();
}

int qlora_profile_entry(int i, const char **name, int64_t *launches, double *total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int)g_summary.size()) return QLORA_ERR_BAD_SHAPE;
  if (name) *name = g_summary[i].first.c_str();
  if (launches) *launches = g_summary[i].second.first;
  if (total_ms) *total_ms = g_summary[i].second.second;
  return QLORA_OK;
}

int qlora_profile_linear_fwd_bf16w(const uint16_t *W_bf16, int64_t n, int64_t k, const uint16_t *X, int64_t M,
                                   const uint16_t *A, const uint16_t *B, int r, float alpha, uint16_t *Y, float *H_out,
                                   void *ws, size_t ws_bytes, hipStream_t stream) {
  const size_t need = qlora_linear_workspace_bytes(M, n, k, r);
  if (n < 1 || k < 64 || k % 64 != 0 || k >= (int64_t(1) << 22) || M < 0 || r < 1 || r > 128 ||
      (M > 0 && need == 0))
    return QLORA_ERR_BAD_SHAPE;
  if (!(alpha == alpha) || alpha - alpha != 0.f) return QLORA_ERR_BAD_ALPHA;
  if (M == 0) return QLORA_OK;
  const void *ptrs[] = {W_bf16, X, A, B, Y, ws};
  for (const void *ptr : ptrs) {
    if (!ptr) return QLORA_ERR_NULL_ARG;
    if (reinterpret_cast<uintptr_t>(ptr) & 15u) return QLORA_ERR_MISALIGNED;
  }
  if (H_out && (reinterpret_cast<uintptr_t>(H_out) & 15u)) return QLORA_ERR_MISALIGNED;
  if (ws_bytes < need) return QLORA_ERR_WORKSPACE;
  hipError_t e = launch_linear_fwd_bf16w(W_bf16, n, k, M, r, (float)alpha / (float)r, X, A, B, Y, H_out, ws, stream);
  return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP;
}

}  // extern "C"
