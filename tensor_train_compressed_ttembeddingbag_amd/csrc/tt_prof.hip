// tt_prof.hip -- optional per-kernel timing: while enabled, every kernel the
// library enqueues is launched with a pair of HIP events that its own dispatch
// records at the kernel's start and end (hipExtLaunchKernelGGL); tt_profile_read
// waits for the events and sums the elapsed times.
#include <mutex>
#include <vector>

#include "tt_internal.h"

namespace ttb {
namespace {

struct Rec {
  int id;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_pending;
std::vector<hipEvent_t> g_pool;
double g_ms[K_COUNT] = {0};
long long g_n[K_COUNT] = {0};

const char *g_names[K_COUNT] = {"k_route_coop", "k_route_a", "k_route_b", "k_route_c",
                                "k_fwd", "k_bwd", "k_seg", "k_cache_lookup",
                                "k_yinit", "k_zero", "k_dmerge", "k_dsplit", "k_dapply",
                                "k_dd_frag", "k_dd_gu", "k_meta"};

hipEvent_t take() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain() {
  for (Rec &r : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      g_ms[r.id] += ms;
      g_n[r.id] += 1;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_pending.clear();
}

}  // namespace

void prof_events(int id, hipEvent_t *start, hipEvent_t *stop) {
  *start = *stop = nullptr;
  if (!g_on) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t a = take(), b = take();
  if (!a || !b) return;
  *start = a;
  *stop = b;
  g_pending.push_back({id, a, b});
  if (g_pending.size() > 4096) drain();
}

}  // namespace ttb

extern "C" {

int tt_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(ttb::g_mu);
  ttb::drain();
  for (int i = 0; i < ttb::K_COUNT; ++i) {
    ttb::g_ms[i] = 0.0;
    ttb::g_n[i] = 0;
  }
  ttb::g_on = on != 0;
  return TT_OK;
}

int tt_profile_read(int kernel_id, double *total_ms, int64_t *launches) {
  if (kernel_id < 0 || kernel_id >= ttb::K_COUNT || !total_ms || !launches) return TT_EINVAL;
  std::lock_guard<std::mutex> lk(ttb::g_mu);
  ttb::drain();
  *total_ms = ttb::g_ms[kernel_id];
  *launches = ttb::g_n[kernel_id];
  return TT_OK;
}

const char *tt_profile_kernel_name(int kernel_id) {
  if (kernel_id < 0 || kernel_id >= ttb::K_COUNT) return nullptr;
  return ttb::g_names[kernel_id];
}

}  // extern "C"

extern "C" int tt_profile_num_kernels(void) { return ttb::K_COUNT; }
