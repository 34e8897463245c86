// dvssq_linear_decode_noalloc: the decode call for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Instead of a caller workspace it uses `scratch`, one
// file-scope device array of kScratchBytes per GPU, which the code object
// holds from load until the process ends.  Its device address on each GPU is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is handed to the kernels: in host code the array's
// name is a host-side stand-in, not a device address.  Nothing here allocates.
#include <stdint.h>

#include <atomic>

#include "dvssq_internal.h"

namespace dvssq {

namespace {

constexpr int64_t kScratchBytes = int64_t(32) << 20;   // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void *> g_scratch[kMaxDevices];

// Device address of this GPU's scratch array, looked up on the first call on
// the device (the current device).  nullptr on a HIP error.
void *scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

// Workspace regions of one call inside the scratch array: the layout of a
// workspace sized for exactly this M (prefill regions scale with M_max).
WsLayout call_layout(const dvssq_layout &L, int32_t M) {
  dvssq_layout Lm = L;
  Lm.M_max = M;
  return ws_layout(Lm);
}

}  // namespace

}  // namespace dvssq

using namespace dvssq;

extern "C" int dvssq_linear_decode_noalloc(const dvssq_layout *L, const void *blob, const void *x, void *y,
                                           int32_t M, uint32_t flags, void *stream) {
  int rc = decode_check_args(L, blob, x, y, M, flags);
  if (rc != DVSSQ_OK) return rc;
  const WsLayout W = call_layout(*L, M);
  int64_t need = 0;
  decode_dispatch(*L, W, blob, x, y, M, nullptr, flags, nullptr, &need, true);
  if (need > kScratchBytes) return DVSSQ_EUNSUPPORTED;
  void *ws = scratch_ptr();
  if (ws == nullptr) return DVSSQ_EHIP;
  return decode_dispatch(*L, W, blob, x, y, M, ws, flags, static_cast<hipStream_t>(stream), nullptr, false);
}
