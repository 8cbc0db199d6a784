// Inspection kernels: they expose the int8 lanes, the decoded scales and the
// int32 half sums that the product kernels compute internally, using the
// same device functions (expand_half, the fp8 scale convert, transpose_half,
// half_dot), so those intermediates can be compared bit for bit with a
// reference ("ROCmFP2 codebook research report", "03 · Runtime").
#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

__device__ __forceinline__ void load_block(const uint8_t* w, int64_t blk,
                                           uint32_t& c0, uint32_t& c1,
                                           uint32_t& sc) {
  const uint16_t* src = reinterpret_cast<const uint16_t*>(w + blk * 10);
  c0 = (uint32_t)src[0] | ((uint32_t)src[1] << 16);
  c1 = (uint32_t)src[2] | ((uint32_t)src[3] << 16);
  sc = (uint32_t)src[4];                  // scale pair in bytes 0, 1
}

__global__ __launch_bounds__(256) void debug_decode_kernel(
    const uint8_t* __restrict__ w, int64_t nblocks, uint32_t* __restrict__ codes,
    float* __restrict__ scales) {
  const float fix = scale_fix();
  for (int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x; blk < nblocks;
       blk += (int64_t)gridDim.x * 256) {
    uint32_t c[2], sc;
    load_block(w, blk, c[0], c[1], sc);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t W[4];
      expand_half(c[h], W);
      // weight 4j+i of the half is byte j of W[i]; rebuild natural order
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = __builtin_amdgcn_perm(W[1], W[0], 0x00000400u + 0x0101u * j);
        const uint32_t hi = __builtin_amdgcn_perm(W[3], W[2], 0x00000400u + 0x0101u * j);
        codes[blk * 8 + h * 4 + j] = (lo & 0xFFFFu) | (hi << 16);
      }
    }
    const float nan = __builtin_nanf("");
    scales[blk * 2 + 0] = scale_byte_bad(sc & 0xFFu) ? nan : fp8_byte<0>(sc) * fix;
    scales[blk * 2 + 1] = scale_byte_bad(sc >> 8) ? nan : fp8_byte<1>(sc) * fix;
  }
}

__global__ __launch_bounds__(256) void debug_half_dots_kernel(
    const uint8_t* __restrict__ w, int64_t N, int64_t nb,
    const uint32_t* __restrict__ q, int64_t M, int32_t* __restrict__ sums) {
  const int64_t total = M * N * nb;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / (N * nb);
    const int64_t rest = idx - m * N * nb;     // = n * nb + b
    const int64_t b = rest % nb;
    uint32_t c[2], sc;
    load_block(w, rest, c[0], c[1], sc);
    const uint32_t* qa = q + (m * nb + b) * 8;  // 32 int8 = 8 words
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t W[4], A[4];
      expand_half(c[h], W);
      const uint32_t X[4] = {qa[4 * h + 0], qa[4 * h + 1], qa[4 * h + 2], qa[4 * h + 3]};
      transpose_half(X, A);
      sums[idx * 2 + h] = half_dot(W, A);
    }
  }
}

}  // namespace

hipError_t launch_debug_decode(const uint8_t* w, int64_t N, int64_t K,
                               int8_t* codes, float* scales, hipStream_t stream) {
  const int64_t nblocks = N * (K / 32);
  const int64_t grid = std::min<int64_t>((nblocks + 255) / 256, kMaxGrid);
  hipLaunchKernelGGL(debug_decode_kernel, dim3((uint32_t)grid), dim3(256), 0, stream,
                     w, nblocks, reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_debug_half_dots(const uint8_t* w, int64_t N, int64_t K,
                                  const int8_t* q, int64_t M, int32_t* sums,
                                  hipStream_t stream) {
  const int64_t nb = K / 32;
  const int64_t total = M * N * nb;
  const int64_t grid = std::min<int64_t>((total + 255) / 256, kMaxGrid);
  hipLaunchKernelGGL(debug_half_dots_kernel, dim3((uint32_t)grid), dim3(256), 0, stream,
                     w, N, nb, reinterpret_cast<const uint32_t*>(q), M, sums);
  return hipGetLastError();
}

}  // namespace rfp2
