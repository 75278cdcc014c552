// Launch timing of the dense dequant-MFMA kernels with HIP events on the launch
// stream.  Off by default; when on, every launch carries a start and a stop event that
// the dispatch itself records (hipExtLaunchKernelGGL), so the elapsed time is the
// kernel's own, and msq_timing_collect aggregates it with the algorithmic flops per
// kernel name.
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/msq.h"
#include "internal.hpp"

namespace msq {
namespace {

struct Rec {
  char name[48];
  double flops, bytes;
  hipEvent_t a, b;
};

std::mutex g_mu;
int g_on = 0;  // 0 off, 1 every launch, 2 launches with flops only
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
hipError_t g_err = hipSuccess;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  // No system-scope fence when the event is recorded: a timing event only needs the
  // timestamp, and the fence (cache writeback) would be counted in the kernel's time.
  hipEvent_t e = nullptr;
  const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
  if (err != hipSuccess && g_err == hipSuccess) g_err = err;
  return err == hipSuccess ? e : nullptr;
}

}  // namespace

bool timing_on() { return g_on != 0; }
bool timing_wants(double flops) { return g_on == 1 || (g_on == 2 && flops > 0.0); }

int timing_begin(const char* name, double flops, double bytes, hipEvent_t* start, hipEvent_t* stop) {
  *start = *stop = nullptr;
  if (!g_on || (g_on == 2 && !(flops > 0.0))) return -1;
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r;
  snprintf(r.name, sizeof(r.name), "%s", name);
  r.flops = flops;
  r.bytes = bytes;
  r.a = take_event();
  r.b = take_event();
  if (!r.a || !r.b) {
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
    return -1;
  }
  g_recs.push_back(r);
  *start = r.a;
  *stop = r.b;
  return (int)g_recs.size() - 1;
}

}  // namespace msq

using namespace msq;

extern "C" {

int msq_timing_enable(int on) {
  if (on < 0 || on > 2) return set_error(MSQ_E_INVAL, "msq_timing_enable: on = %d (0, 1 or 2)", on);
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on;
  return MSQ_OK;
}

int msq_timing_reserve(int events) {
  if (events < 0) return set_error(MSQ_E_INVAL, "msq_timing_reserve: events = %d", events);
  std::lock_guard<std::mutex> lk(g_mu);
  while ((int)g_pool.size() < events) {
    hipEvent_t e = nullptr;
    const hipError_t err = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (err != hipSuccess) return hip_error(err, "msq_timing_reserve: hipEventCreateWithFlags");
    g_pool.push_back(e);
  }
  return MSQ_OK;
}

int msq_timing_collect(msq_kernel_timing* out, int max, int* n_out) {
  if (!n_out || (max > 0 && !out)) return set_error(MSQ_E_INVAL, "msq_timing_collect: null pointer");
  std::lock_guard<std::mutex> lk(g_mu);
  std::vector<msq_kernel_timing> agg;
  hipError_t err = g_err;
  for (const Rec& r : g_recs) {
    float ms = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess && err == hipSuccess) err = e;
    size_t i = 0;
    while (i < agg.size() && strcmp(agg[i].name, r.name) != 0) ++i;
    if (i == agg.size()) {
      msq_kernel_timing t;
      memset(&t, 0, sizeof(t));
      strncpy(t.name, r.name, sizeof(t.name) - 1);
      agg.push_back(t);
    }
    agg[i].launches++;
    agg[i].total_ms += ms;
    agg[i].total_flops += r.flops;
    agg[i].total_bytes += r.bytes;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  g_err = hipSuccess;
  *n_out = (int)agg.size();
  for (int i = 0; i < max && i < (int)agg.size(); ++i) out[i] = agg[i];
  return err == hipSuccess ? MSQ_OK : hip_error(err, "msq_timing_collect");
}

}  // extern "C"
