// qlora_linear_fwd_noalloc: the forward for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its scratch is a file-scope device array of fixed size instead
// of a caller workspace; every call on a device shares that device's copy.
#include <atomic>

#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = QLORA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per device, held until the process ends. In host code the name
// is only a stand-in: kernels get the device address from the table below.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device ordinal (0 = not looked up yet).
// Two threads racing on the first call store the same value.
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

qlora_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return QLORA_ERR_HIP;
  }
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return QLORA_ERR_HIP;
    }
    a = (uintptr_t)p;
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *out = (void *)a;
  return QLORA_OK;
}

}  // namespace

extern "C" qlora_status qlora_linear_fwd_noalloc(const qlora_nf4_weight *w, const uint16_t *X,
                                                 int64_t M, const uint16_t *A, const uint16_t *B,
                                                 int32_t r, float lora_alpha, uint16_t *Y,
                                                 float *H_save, void *stream) {
  // size check first, on the host: nothing is looked up or launched for a
  // call whose scratch would not fit
  if (!w) return QLORA_ERR_INVALID_ARG;
  const size_t need = qlora_workspace_bytes(QLORA_OP_FWD, w->d, w->k, M, r, w->double_quant);
  if (need == (size_t)-1) {
    if (M < 1 || r < 1) return QLORA_ERR_INVALID_ARG;
    return QLORA_ERR_UNSUPPORTED;
  }
  if (need > kScratchBytes) return QLORA_ERR_WORKSPACE;
  void *ws = nullptr;
  const qlora_status s = scratch_of_current_device(&ws);
  if (s != QLORA_OK) return s;
  return qlora_linear_fwd(w, X, M, A, B, r, lora_alpha, Y, H_save, ws, kScratchBytes, stream);
}
