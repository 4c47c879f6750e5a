// Event bracketing of kernel launches, linked only into the timing build
// (libqlora_nf4_timing.so, every source compiled with QLORA_KERNEL_TIMING).
// The product library has none of this state.
#include "../kernels.h"

namespace {
struct ProfState {
  bool on = false;
  int cap = 0, n = 0;
  uint32_t mask = 0xFFFFFFFFu;
  hipEvent_t *ev = nullptr;
  int *kid = nullptr;
};
ProfState g_prof;

void destroy_events(int count) {
  for (int i = 0; i < count; ++i) (void)hipEventDestroy(g_prof.ev[i]);
  delete[] g_prof.ev;
  delete[] g_prof.kid;
  g_prof = ProfState{};
}
}  // namespace

int ql_prof_begin(int kernel_id, hipStream_t st) {
  if (!g_prof.on || g_prof.n >= g_prof.cap || !((g_prof.mask >> kernel_id) & 1u)) return -1;
  const int s = g_prof.n++;
  g_prof.kid[s] = kernel_id;
  (void)hipEventRecord(g_prof.ev[2 * s], st);
  return s;
}

void ql_prof_end(int slot, hipStream_t st) {
  if (slot >= 0) (void)hipEventRecord(g_prof.ev[2 * slot + 1], st);
}

extern "C" {

qlora_status qlora_profile_release(void) {
  destroy_events(2 * g_prof.cap);
  return QLORA_OK;
}

qlora_status qlora_profile_begin(int32_t cap, uint32_t mask) {
  if (cap < 1) return QLORA_ERR_INVALID_ARG;
  if (g_prof.cap != cap) {
    qlora_profile_release();
    g_prof.ev = new hipEvent_t[2 * cap];
    g_prof.kid = new int[cap];
    for (int i = 0; i < 2 * cap; ++i) {
      if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) {
        (void)hipGetLastError();
        destroy_events(i);   // the events created so far, and both arrays
        return QLORA_ERR_HIP;
      }
    }
    g_prof.cap = cap;
  }
  g_prof.n = 0;
  g_prof.mask = mask ? mask : 0xFFFFFFFFu;
  g_prof.on = true;
  return QLORA_OK;
}

qlora_status qlora_profile_end(void) {
  g_prof.on = false;
  return QLORA_OK;
}

qlora_status qlora_profile_query(int32_t kernel_id, int32_t *count, double *total_ms) {
  if (!count || !total_ms) return QLORA_ERR_INVALID_ARG;
  *count = 0;
  *total_ms = 0.0;
  for (int s = 0; s < g_prof.n; ++s) {
    if (g_prof.kid[s] != kernel_id) continue;
    if (hipEventSynchronize(g_prof.ev[2 * s + 1]) != hipSuccess) return QLORA_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, g_prof.ev[2 * s], g_prof.ev[2 * s + 1]) != hipSuccess)
      return QLORA_ERR_HIP;
    *count += 1;
    *total_ms += ms;
  }
  return QLORA_OK;
}

}  // extern "C"
