// moe_nvfp4_forward_noalloc: the whole layer with no workspace argument and no allocation, for
// callers that cannot allocate (code under HIP graph capture, tight serving loops, hosts that forbid
// hipMalloc).  The workspace moe_nvfp4_forward takes from the caller lives here in one file-scope
// device array of MOE_NOALLOC_SCRATCH_BYTES, which every GPU the library runs on holds until the
// process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device with hipGetSymbolAddress, with that device current, and only that
// address is ever passed to a kernel.  Each device holds its own copy of the array at its own
// address.  The forward needs no part of its workspace to start at zero (every buffer is written
// before it is read, and its counters are cleared by its own first kernel), so nothing is cleared
// between calls.  Calls on one device share the array:
// two calls that overlap in time on one device race.
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up yet)

// Device address of this device's copy of `scratch` (looked up on the first call on the device).
moe_status_t scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status_t moe_nvfp4_forward_noalloc(const moe_nvfp4_layer_t* layer, const uint16_t* x, int32_t T,
                                                  uint16_t* out, const moe_forward_aux_t* aux, void* stream) {
  // shapes first, then the size: a layer whose workspace exceeds the array is refused before any
  // device call (MOE_ERR_WORKSPACE_TOO_SMALL)
  if (moe_status_t st = moe_validate_forward(layer, T, kScratchBytes, nullptr)) return st;
  if (T == 0) return MOE_OK;
  void* ws = nullptr;
  if (moe_status_t st = scratch_on_current_device(&ws)) return st;
  return moe_nvfp4_forward(layer, x, T, out, ws, kScratchBytes, aux, stream);
}
