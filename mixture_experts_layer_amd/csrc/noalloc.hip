// moe_permute_noalloc: token dispatch with its scratch in a device array of the library,
// for callers that cannot allocate device memory (code under HIP graph capture, serving
// loops that forbid allocation).
//
// The dispatch metadata of moe_permute (Transformer Engine guide "Mixture of Experts",
// section "Token dispatch") needs per-chunk expert histograms and row bases. Here they live
// in `scratch`, a file-scope device array of kNoAllocScratchBytes (4 MiB) that each GPU the
// library runs on holds until the process ends. Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol): the device address is taken
// once per device with hipGetSymbolAddress, with that device current, and kept per device.
// Every call on one GPU shares that GPU's array, so calls that overlap on one GPU (two
// streams, or a captured graph replayed while an eager call runs) race on it. The kernels
// overwrite every scratch value they later read, so nothing has to start at zero.
#include <mutex>

#include "internal.h"

namespace moe {

namespace {

constexpr size_t kNoAllocScratchBytes = 4u << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device

// Device address of this device's `scratch` (looked up on the first call per device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t permute_noalloc_scratch_limit() { return kNoAllocScratchBytes; }

hipError_t launch_permute_noalloc(const void* x, const int32_t* topk_idx, int T, int H, int E,
                                  int k, int out_dtype, void* xp, float* xp_scale,
                                  int32_t* offsets, int32_t* row_of, int32_t* src_of,
                                  hipStream_t s) {
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return e;
  e = launch_dispatch_meta(topk_idx, T, E, k, offsets, row_of, src_of, ws, s);
  if (e != hipSuccess) return e;
  if (out_dtype == MOE_BF16) return launch_scatter_rows(x, row_of, nullptr, T, H, k, xp, s);
  return launch_scatter_rows_fp8(x, row_of, T, H, k, (uint8_t*)xp, xp_scale, s);
}

}  // namespace moe
