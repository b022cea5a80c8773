// ttt_la_forward_noalloc: ttt_la_forward with the library's own device
// scratch instead of a caller workspace, for callers that cannot allocate
// device memory.  The scratch is a file-scope device array of fixed size; each
// GPU holds its own copy (at its own address) from the first use on that
// device until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ttt_la.h"

namespace {

constexpr size_t kScratchBytes = TTT_LA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Device scratch shared by every allocation-free call on a device.  In host code this name is only a
// stand-in for the symbol: its device address comes from hipGetSymbolAddress (per device).
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per device.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TTT_LA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TTT_LA_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return TTT_LA_OK;
}

}  // namespace

extern "C" int ttt_la_forward_noalloc(const void* Q, const void* K, const void* V, const float* eta,
                                      const float* W0, int64_t chunk, int32_t mode, const ttt_la_desc* desc,
                                      void* O, float* W_out, void* stream) {
  // ttt_la_workspace_bytes is 0 for invalid arguments too: ttt_la_forward then reports them
  const size_t need = ttt_la_workspace_bytes(desc, chunk, mode);
  if (need > kScratchBytes) return TTT_LA_ERR_SCRATCH;
  if (need == 0) return ttt_la_forward(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, nullptr, 0, stream);
  void* ws = nullptr;
  const int st = scratch_ptr(&ws);
  if (st != TTT_LA_OK) return st;
  return ttt_la_forward(Q, K, V, eta, W0, chunk, mode, desc, O, W_out, ws, kScratchBytes, stream);
}
