// Quantizers: fp32 activations -> int8 + one fp32 scale per 32 values, and
// fp32 weights -> ROCmFP2 blocks ("ROCmFP2 codebook research report",
// "02 · Quantization" and "03 · Runtime").
#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {

// ---------------------------------------------------------------------------
// Activations.  Eight lanes own one 32-value block, four values each (one
// 16-byte load per lane, one 4-byte store of the four int8 results).  The
// block maximum is combined across the eight lanes with xor shuffles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void quantize_acts_kernel(
    const float4* __restrict__ a, int64_t nblocks, uint32_t* __restrict__ q,
    float* __restrict__ d) {
  // grid-stride over whole workgroups so that the eight lanes of a block
  // always run the same iterations
  for (int64_t base = (int64_t)blockIdx.x * 256; base < nblocks * 8;
       base += (int64_t)gridDim.x * 256) {
  const int64_t tid = base + threadIdx.x;
  const int64_t blk = tid >> 3;
  const bool valid = blk < nblocks;
  const float4 v = valid ? a[tid] : make_float4(0.f, 0.f, 0.f, 0.f);
  float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
  int finite = isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w);
#pragma unroll
  for (int off = 4; off >= 1; off >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    finite &= __shfl_xor(finite, off, 64);
  }
  float scale = __fdiv_rn(amax, 127.0f);
  uint32_t packed = 0;
  if (!finite) {
    scale = __builtin_nanf("");
  } else if (scale != 0.0f) {
    const float vals[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float r = roundf(__fdiv_rn(vals[i], scale));   // halves away from zero
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      packed |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * i);
    }
  }
  if (valid) {
    q[tid] = packed;
    if ((tid & 7) == 0) d[blk] = scale;
  }
  }
}

hipError_t launch_quantize_acts(const float* a, int64_t M, int64_t K, int8_t* q,
                                float* d, hipStream_t stream) {
  const int64_t nblocks = M * (K / 32);
  const int64_t threads = nblocks * 8;
  const int64_t grid = std::min<int64_t>((threads + 255) / 256, kMaxGrid);
  hipLaunchKernelGGL(quantize_acts_kernel, dim3((uint32_t)grid), dim3(256), 0,
                     stream, reinterpret_cast<const float4*>(a), nblocks,
                     reinterpret_cast<uint32_t*>(q), d);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weights.  One thread owns one 32-weight block (two halves).  For each half
// every legal scale byte is tried; the squared error is summed in fp64 in
// index order with one rounding per operation (no fused multiply-add), so the
// chosen byte is reproducible bit for bit.  The winner is the least error;
// among equal errors the byte nearest the start byte (nearest scale to
// max|x|/4, lower on a tie), lower side first.
// ---------------------------------------------------------------------------
//
// With an importance vector (imp != null: the importance of each of the
// half's 16 input channels) the error of a candidate is
// sum_i wt_i * (x_i - xhat_i)^2 with wt_i = imp_i * sqrt(sigma^2 + x_i^2) and
// sigma^2 the mean of x^2 over the half ("05 · Completed experiment"; the page
// leaves sigma undefined).  The weights are computed once per half, every
// step rounded once (fp64 sqrt is correctly rounded), in the same order as
// the plain error, so the choice is reproducible bit for bit as well.
__device__ void search_half(const float* x, const float* imp, uint32_t& code_word,
                            uint32_t& byte) {
#pragma clang fp contract(off)
  double xs[16];
  double amax = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    xs[i] = (double)x[i];
    amax = fmax(amax, fabs(xs[i]));
  }
  double wt[16];
  if (imp) {
    double s2 = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s2 = s2 + xs[i] * xs[i];
    const double sigma2 = s2 / 16.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) wt[i] = (double)imp[i] * sqrt(sigma2 + xs[i] * xs[i]);
  }
  const double target = amax * 0.25;
  int start = 0;
  double best_dist = fabs(ue4m3_f64(0) - target);
  for (int b = 1; b <= 0x7E; ++b) {
    const double dist = fabs(ue4m3_f64(b) - target);
    if (dist < best_dist) { best_dist = dist; start = b; }
  }
  double best = __builtin_inf();
  int best_b = start, best_rank = 1 << 30;
  for (int b = 0; b <= 0x7E; ++b) {
    const double s = ue4m3_f64(b);
    const double lim = 2.5 * s;
    double sse = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double level = fabs(xs[i]) > lim ? 4.0 : 1.0;
      const double xh = (xs[i] < 0.0 ? -level : level) * s;
      const double e = xs[i] - xh;
      double t = e * e;
      if (imp) t = wt[i] * t;
      sse = sse + t;
    }
    const int rank = b < start ? 2 * (start - b) - 1 : 2 * (b - start);
    if (sse < best || (sse == best && rank < best_rank)) {
      best = sse; best_b = b; best_rank = rank;
    }
  }
  const double lim = 2.5 * ue4m3_f64(best_b);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool outer = fabs(xs[i]) > lim;
    const uint32_t c = xs[i] < 0.0 ? (outer ? 0u : 1u) : (outer ? 3u : 2u);
    w |= c << (2 * i);       // weight i: byte i/4, bits 2(i%4)
  }
  code_word = w;
  byte = (uint32_t)best_b;
}

// imp: null, or the importance of each of the K input channels; block blk
// covers columns 32*(blk % blocks_per_row) .. +31.
__global__ __launch_bounds__(128) void quantize_weights_kernel(
    const float* __restrict__ x, int64_t nblocks, int64_t blocks_per_row,
    const float* __restrict__ imp, uint16_t* __restrict__ w) {
  for (int64_t blk = (int64_t)blockIdx.x * 128 + threadIdx.x; blk < nblocks;
       blk += (int64_t)gridDim.x * 128) {
  float v[32];
  const float* src = x + blk * 32;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = src[i];
  const float* ib = imp ? imp + (blk % blocks_per_row) * 32 : nullptr;
  uint32_t c0, c1, e0, e1;
  search_half(v, ib, c0, e0);
  search_half(v + 16, ib ? ib + 16 : nullptr, c1, e1);
  uint16_t* dst = w + blk * 5;      // 10 bytes, 2-byte aligned
  dst[0] = (uint16_t)(c0 & 0xFFFFu);
  dst[1] = (uint16_t)(c0 >> 16);
  dst[2] = (uint16_t)(c1 & 0xFFFFu);
  dst[3] = (uint16_t)(c1 >> 16);
  dst[4] = (uint16_t)(e0 | (e1 << 8));
  }
}

hipError_t launch_quantize_weights(const float* x, int64_t N, int64_t K,
                                   const float* imp, uint8_t* w, hipStream_t stream) {
  const int64_t nblocks = N * (K / 32);
  const int64_t grid = std::min<int64_t>((nblocks + 127) / 128, kMaxGrid);
  hipLaunchKernelGGL(quantize_weights_kernel, dim3((uint32_t)grid), dim3(128),
                     0, stream, x, nblocks, K / 32, imp, reinterpret_cast<uint16_t*>(w));
  return hipGetLastError();
}

}  // namespace rfp2
