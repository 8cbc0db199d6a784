// Measurement helper: the plainest kernel that reads a buffer from HBM.
// Each thread XORs the 16-byte pieces it visits (consecutive threads read
// consecutive pieces, grid-stride, 2048 workgroups of 256 threads) and
// stores its XOR only when it equals the caller's `magic` word, so every
// load is live but the kernel ends without a reduction or a store (a
// per-workgroup XOR reduction through LDS and a barrier added ~0.65 us at
// 26 MB).  Its time for a given byte count is what any kernel reading that
// many bytes can hope for on this GPU: launch, ramp-up and the memory system
// included.  Of the forms measured at 26 MB (1024 .. 8192 workgroups, 256 ..
// 1024 threads, 1 .. 16 loads in flight per lane, one contiguous chunk per
// workgroup, direct-to-LDS loads) none was faster.
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

constexpr int kCeilThreads = 256;

__global__ __launch_bounds__(kCeilThreads) void read_ceiling_kernel(const uint4* __restrict__ buf,
                                                                    int64_t pieces,
                                                                    uint32_t magic,
                                                                    uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kCeilThreads;
  const int64_t gid = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = gid; i < pieces; i += stride) {
    const uint4 v = buf[i];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == magic) out[gid] = x;
}

}  // namespace

hipError_t launch_read_ceiling(const uint8_t* buf, int64_t bytes, uint32_t magic, uint32_t* out,
                               hipStream_t stream) {
  const int64_t pieces = bytes / 16;
  const int64_t need = (pieces + kCeilThreads - 1) / kCeilThreads;
  const uint32_t grid = (uint32_t)std::max<int64_t>(1, std::min<int64_t>(need, kReadCeilingGrid));
  hipLaunchKernelGGL(read_ceiling_kernel, dim3(grid), dim3(kCeilThreads), 0, stream,
                     reinterpret_cast<const uint4*>(buf), pieces, magic, out);
  return hipGetLastError();
}

}  // namespace rfp2
