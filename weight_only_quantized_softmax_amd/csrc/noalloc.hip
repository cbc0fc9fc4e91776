// qmoe_forward_noalloc: the whole forward with its intermediates in a fixed device array of
// the library instead of a caller-given workspace, for callers that cannot allocate (code
// under graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ object: each GPU the library runs on holds its own
// copy, at its own address, from the library's load on that GPU until the process ends. In
// host code the array's name is only a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress (on the first call on that device, with the
// device current) and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "qmoe.h"

namespace {

static_assert(QMOE_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte pieces");

static __device__ __align__(256) unsigned char scratch[QMOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of this GPU's copy of the array, taken once per device.
qmoe_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return qmoe::fail_with(QMOE_ERR_DEVICE, "hipGetDevice failed", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return qmoe::fail_with(QMOE_ERR_UNSUPPORTED, "device index beyond the library's table", "");
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return qmoe::fail_with(QMOE_ERR_DEVICE, "hipGetSymbolAddress of the scratch array failed",
                             hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return QMOE_OK;
}

}  // namespace

extern "C" qmoe_status qmoe_forward_noalloc(const qmoe_params* p, const void* input,
                                            const void* router_logits, qmoe_stack fc1,
                                            qmoe_stack fc2, qmoe_stack fc3,
                                            const void* shared_output, void* output,
                                            void* stream) {
  const qmoe_status v = qmoe_validate(p);
  if (v != QMOE_OK) return v;
  if (p->num_tokens == 0) return QMOE_OK;
  const size_t need = qmoe_workspace_size(p);
  if (need > QMOE_NOALLOC_SCRATCH_BYTES)
    return qmoe::fail_with(QMOE_ERR_UNSUPPORTED,
                           "these shapes need more intermediate memory than the fixed array "
                           "holds (qmoe_workspace_size > QMOE_NOALLOC_SCRATCH_BYTES); use "
                           "qmoe_forward with a workspace",
                           "");
  void* ws = nullptr;
  const qmoe_status s = scratch_address(&ws);
  if (s != QMOE_OK) return s;
  // nothing in the forward needs its intermediates to start at zero: every piece is written
  // before it is read, within the same call
  return qmoe_forward(p, input, router_logits, fc1, fc2, fc3, shared_output, output, ws,
                      QMOE_NOALLOC_SCRATCH_BYTES, stream);
}
