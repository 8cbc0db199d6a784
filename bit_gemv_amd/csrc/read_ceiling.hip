// Measurement helper: the plainest kernel that reads a buffer from HBM.
// Each thread XORs the 16-byte pieces it visits (consecutive threads read
// consecutive pieces, grid-stride), and one lane per workgroup stores the
// workgroup's XOR, so the loads cannot be dropped.  Its time for a given
// byte count is what any kernel reading that many bytes can hope for on
// this GPU: launch, ramp-up and the memory system included.
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

constexpr int kCeilThreads = 256;

__global__ __launch_bounds__(kCeilThreads) void read_ceiling_kernel(const uint4* __restrict__ buf,
                                                                    int64_t pieces,
                                                                    uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kCeilThreads;
  uint4 acc = make_uint4(0u, 0u, 0u, 0u);
  for (int64_t i = (int64_t)blockIdx.x * kCeilThreads + threadIdx.x; i < pieces; i += stride) {
    const uint4 v = buf[i];
    acc.x ^= v.x;
    acc.y ^= v.y;
    acc.z ^= v.z;
    acc.w ^= v.w;
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o, 64);
  __shared__ uint32_t wave_x[kCeilThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kCeilThreads / 64; ++w) t ^= wave_x[w];
    out[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_read_ceiling(const uint8_t* buf, int64_t bytes, uint32_t* out,
                               hipStream_t stream) {
  const int64_t pieces = bytes / 16;
  const int64_t need = (pieces + kCeilThreads - 1) / kCeilThreads;
  const uint32_t grid = (uint32_t)std::max<int64_t>(1, std::min<int64_t>(need, kReadCeilingGrid));
  hipLaunchKernelGGL(read_ceiling_kernel, dim3(grid), dim3(kCeilThreads), 0, stream,
                     reinterpret_cast<const uint4*>(buf), pieces, out);
  return hipGetLastError();
}

}  // namespace rfp2
