// Optional per-kernel timing for benchmarks. Off by default; while enabled
// (hstu_profile_begin .. hstu_profile_end) every launch of the library is
// bracketed by a pair of HIP events recorded on the caller's stream, and
// hstu_profile_end waits for them and sums the elapsed times per kernel.
// Intended for one host thread driving the library at a time.
#include <mutex>
#include <vector>

#include "../../include/hstu_attn.h"
#include "internal.h"

namespace hstu {

namespace {

struct Rec {
  int id;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_enabled = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

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

const char* const kNames[kNumKernelIds] = {"prep", "fwd", "bwd_pre", "bwd",
                                           "dq", "fill", "linear", "layernorm_gate",
                                           "bucketize", "fp8_linear", "fp8_quantize", "dq_ds",
                                           "rab_reduce"};

}  // namespace

void prof_before(int id, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled) return;
  Rec r{id, take_event(), take_event()};
  if (!r.a || !r.b) return;
  hipEventRecord(r.a, s);
  g_recs.push_back(r);
}

void prof_after(int id, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled || g_recs.empty() || g_recs.back().id != id) return;
  hipEventRecord(g_recs.back().b, s);
}

}  // namespace hstu

using namespace hstu;

extern "C" {

HSTU_API hstu_status hstu_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Rec& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_enabled = true;
  return HSTU_OK;
}

HSTU_API hstu_status hstu_profile_end(int32_t n, double* total_ms, int32_t* counts) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_enabled = false;
  if (n < 0 || (n > 0 && (!total_ms || !counts))) return HSTU_EINVAL;
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.0;
    counts[i] = 0;
  }
  hstu_status st = HSTU_OK;
  for (const Rec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = HSTU_EHIP;
    } else if (r.id < n) {
      total_ms[r.id] += ms;
      counts[r.id] += 1;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return st;
}

HSTU_API const char* hstu_kernel_name(int32_t id) {
  return (id >= 0 && id < kNumKernelIds) ? kNames[id] : "";
}

HSTU_API int32_t hstu_kernel_count(void) { return kNumKernelIds; }

}  // extern "C"
