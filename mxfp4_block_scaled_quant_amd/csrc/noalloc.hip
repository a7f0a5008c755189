// mxfp4_linear_noalloc (include/mxfp4.h): mxfp4_linear without a caller
// workspace and without any allocation, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops).  The
// quantised activations go to a fixed-size array in the library's own device
// memory, `scratch`, one per GPU (each GPU that runs the library holds it
// until the process ends).  Every call on a GPU shares that GPU's array:
// calls that overlap in time on one GPU (other streams) race.  The array
// keeps the last call's contents; nothing in it needs to start at zero (each
// call writes every byte it reads).
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/mxfp4.h"
#include "mxfp4_launch.h"

namespace mxfp4 {
namespace {

// 32 MiB: the quantised activations (ceil(M/16) * (ceil(K/128) KiB +
// ceil(K/512) * 256 bytes)) of up to M = 4400 at K = 14336, M = 12336 at
// K = 5120.
constexpr size_t kScratchBytes = size_t(32) << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// The array's device address on each device ordinal (0: not yet looked up).
// In host code `scratch` names a host-side stand-in, not device memory: only
// the address hipGetSymbolAddress returns, with that device current, is.
std::atomic<uintptr_t> g_scratch_addr[64];

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return MXFP4_ERR_DEVICE;
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MXFP4_ERR_DEVICE;
    a = (uintptr_t)ptr;
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *out = (void*)a;
  return MXFP4_OK;
}

}  // namespace
}  // namespace mxfp4

using namespace mxfp4;

extern "C" int mxfp4_linear_noalloc(const void* x, int64_t ldx, const void* w_pre, const void* ws_pre,
                                    const void* bias, void* out, int64_t ldo, int out_dtype, int64_t M,
                                    int64_t N, int64_t K, void* stream) {
  int st = linear_check(x, ldx, w_pre, ws_pre, bias, out, ldo, out_dtype, M, N, K);
  if (st) return st;
  const size_t need = linear_act_bytes(M, N, K);
  if (need > kScratchBytes) return MXFP4_ERR_WORKSPACE;
  if (M == 0) return MXFP4_OK;
  int cus = 0;
  st = device_cus(&cus);
  if (st) return st;
  void* ws = nullptr;
  if (need) {
    st = scratch_address(&ws);
    if (st) return st;
  }
  return linear_run(x, ldx, w_pre, ws_pre, bias, out, ldo, out_dtype, M, N, K, ws, kScratchBytes, false, cus,
                    (hipStream_t)stream);
}
