// rfp2_moe_gemm without a caller workspace: the prompt-batch routed-expert
// product of rfp2_moe_gemm (same sort and product kernels), with the sorted
// slots kept in a device array owned by the library, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// symbol); the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.  Every call on a
// GPU uses that GPU's copy, so calls that overlap in time on one GPU race on
// it.  The sort writes every entry the product reads (offsets and tile
// numbers of every expert, the slots of every routed expert), so nothing has
// to be cleared between calls.
#include <mutex>

#include "rfp2_internal.h"

namespace rfp2 {

namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

}  // namespace

// Device address of the current device's scratch array (looked up on the
// first call on that device).
hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_moe_gemm_noalloc(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                   const int32_t* ids, int64_t T, int64_t top_k,
                                   const int8_t* q, const float* d, float* y, int32_t* err,
                                   hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_moe_gemm(w, E, N, K, ids, T, top_k, q, d, y, err, ws, stream);
}

}  // namespace rfp2
