// Per-kernel timing: hipEvent pairs recorded around the library's launches on the
// caller's stream while enabled (see qz_timing_enable in include/qz.h).
#include <atomic>
#include <mutex>
#include <vector>

#include "qz_internal.h"

namespace qz {

namespace {

struct Record {
  int kind;
  hipEvent_t b, e;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<Record> g_records;
std::vector<hipEvent_t> g_pool;

const char* const kNames[K_KIND_COUNT] = {
    "hessian_gram_bf16", "hessian_finish", "rfactor_fp64", "gptq_block", "gemm_gptq_trailing",
    "gemm_admm_setup", "gemm_admm_wupdate1", "gemm_admm_wupdate2", "admm_project", "admm_other",
    "grid_rtn", "pack", "eig_prepare", "objective", "ls_gradient", "ls_propose",
    "ls_accept", "order"};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t ev = g_pool.back();
    g_pool.pop_back();
    return ev;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

}  // namespace

ScopedTimer::ScopedTimer(int kind, hipStream_t s) : kind_(kind), s_(s) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  b_ = take_event();
  e_ = take_event();
  if (b_ && e_) (void)hipEventRecord(b_, s_);
}

ScopedTimer::~ScopedTimer() {
  if (!b_ || !e_) return;
  (void)hipEventRecord(e_, s_);
  std::lock_guard<std::mutex> lk(g_mu);
  g_records.push_back({kind_, b_, e_});
}

}  // namespace qz

extern "C" {

int qz_timing_enable(int on) {
  qz::g_on.store(on ? 1 : 0);
  return QZ_OK;
}

int qz_timing_read(int64_t* launches, double* total_ms, int max_kinds, int reset) {
  using namespace qz;
  const int n = max_kinds < K_KIND_COUNT ? (max_kinds < 0 ? 0 : max_kinds) : K_KIND_COUNT;
  int64_t cnt[K_KIND_COUNT] = {};
  double ms[K_KIND_COUNT] = {};
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Record& r : g_records) {
    if (hipEventSynchronize(r.e) != hipSuccess) return fail(QZ_EHIP, "timing: event sync failed");
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.b, r.e) != hipSuccess) return fail(QZ_EHIP, "timing: elapsed failed");
    cnt[r.kind] += 1;
    ms[r.kind] += t;
  }
  for (int k = 0; k < n; ++k) {
    if (launches) launches[k] = cnt[k];
    if (total_ms) total_ms[k] = ms[k];
  }
  if (reset) {
    for (const Record& r : g_records) {
      g_pool.push_back(r.b);
      g_pool.push_back(r.e);
    }
    g_records.clear();
  }
  return K_KIND_COUNT;
}

const char* qz_timing_kind_name(int kind) {
  if (kind < 0 || kind >= qz::K_KIND_COUNT) return "";
  return qz::kNames[kind];
}

}  // extern "C"
