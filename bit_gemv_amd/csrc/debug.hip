// Inspection kernels: they expose the int8 lanes, the decoded scales, the
// int32 half sums and the fp16 weights that the product kernels compute
// internally, by calling the products' own device functions on the same
// register layouts, so that those intermediates can be compared bit for bit
// with a reference ("ROCmFP2 codebook research report", "03 · Runtime":
// SPREAD / PERMUTE turn each code byte into four int8 lanes, DOT4 sums each
// 16-weight half in int32, the scales are applied afterwards).
//
//   * GEMV decode (rfp2_debug_decode, rfp2_debug_half_dots): the block
//     stream is cut into 80-byte groups of 8 blocks, as the GEMV's lanes hold
//     them, and every block is decoded by decode_block (the 64-bit selector
//     shifts of expand_block, the funnel shift for the odd blocks that start
//     at byte 2 of a dword, the packed fp8 convert of both scales) and summed
//     by block_half_sums against activations transposed as the GEMV stages
//     them.
//   * GEMV matrix-core half sums (rfp2_debug_half_sums_mf): the same blocks
//     summed by half_sums_mf, the 4x4x4 int8 matrix-core form of two to eight
//     columns, with its lane layout: quads of lanes are four rows at one
//     group, each lane supplies one column's activations.
//   * fp16 decode (rfp2_debug_decode_f16): pairs of blocks, as the fp16
//     matrix-core kernels load them, decoded by decode_pair_block_f16 (the
//     dense prompt-batch kernel) or decode_half (the routed kernel).
#include "f16_decode.h"
#include "gemv_kernel.h"
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

using gemv_detail::block_half_sums;
using gemv_detail::decode_block;
using gemv_detail::half_sums_mf;
using gemv_detail::v4i;

// `n` dwords of the block stream starting at byte `off` (a multiple of 2),
// read as 16-bit pieces (the stream is only 2-byte aligned here); bytes at or
// past `end` read as zero.
template <int n>
__device__ __forceinline__ void load_dwords(const uint8_t* w, int64_t off, int64_t end,
                                            uint32_t (&dw)[n]) {
  const uint16_t* src = reinterpret_cast<const uint16_t*>(w + off);
#pragma unroll
  for (int i = 0; i < n; ++i) {
    const uint32_t lo = off + 4 * i < end ? src[2 * i] : 0u;
    const uint32_t hi = off + 4 * i + 2 < end ? src[2 * i + 1] : 0u;
    dw[i] = lo | (hi << 16);
  }
}

// Weight 4j+i of a half is byte j of W[i] (expand_half's lane order): the
// four natural-order dwords of the half.
__device__ __forceinline__ void natural_order(const uint32_t (&W)[4], uint32_t* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t lo = __builtin_amdgcn_perm(W[1], W[0], 0x00000400u + 0x0101u * j);
    const uint32_t hi = __builtin_amdgcn_perm(W[3], W[2], 0x00000400u + 0x0101u * j);
    out[j] = (lo & 0xFFFFu) | (hi << 16);
  }
}

__global__ __launch_bounds__(256) void debug_decode_kernel(
    const uint8_t* __restrict__ w, int64_t nblocks, uint32_t* __restrict__ codes,
    float* __restrict__ scales) {
  const float fix = scale_fix();
  const float nan = __builtin_nanf("");
  const int64_t ngroups = (nblocks + 7) / 8;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < ngroups;
       g += (int64_t)gridDim.x * 256) {
    uint32_t dw[20];
    load_dwords(w, g * 80, nblocks * 10, dw);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const int64_t blk = g * 8 + jb;
      if (blk >= nblocks) break;
      uint32_t W0[4], W1[4], sc;
      float s0, s1;
      decode_block(dw, jb, W0, W1, s0, s1, sc);
      natural_order(W0, codes + blk * 8);
      natural_order(W1, codes + blk * 8 + 4);
      // the GEMV's flags: the top bit of each byte of the pair marks
      // 0x80..0xFF (0x7F is NaN through the convert itself)
      const uint32_t flags = (jb & 1) ? sc >> 16 : sc;
      scales[blk * 2 + 0] = (flags & 0x80u) ? nan : s0 * fix;
      scales[blk * 2 + 1] = (flags & 0x8000u) ? nan : s1 * fix;
    }
  }
}

__global__ __launch_bounds__(256) void debug_half_dots_kernel(
    const uint8_t* __restrict__ w, int64_t nblocks, int64_t nb,
    const uint32_t* __restrict__ q, int64_t M, int32_t* __restrict__ sums) {
  const int64_t ngroups = (nblocks + 7) / 8;
  const int64_t total = M * ngroups;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / ngroups;
    const int64_t g = idx - m * ngroups;
    uint32_t dw[20];
    load_dwords(w, g * 80, nblocks * 10, dw);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const int64_t blk = g * 8 + jb;           // = n * nb + b
      if (blk >= nblocks) break;
      uint32_t W0[4], W1[4], sc;
      float s0, s1;
      decode_block(dw, jb, W0, W1, s0, s1, sc);
      // the block's 32 int8 activations of column m, each half transposed
      // into the lane order of the expanded weights (as the GEMV stages them)
      const uint32_t* qa = q + (m * nb + blk % nb) * 8;
      const uint32_t X0[4] = {qa[0], qa[1], qa[2], qa[3]};
      const uint32_t X1[4] = {qa[4], qa[5], qa[6], qa[7]};
      uint32_t T0[4], T1[4];
      transpose_half(X0, T0);
      transpose_half(X1, T1);
      int32_t S0, S1;
      block_half_sums(W0, W1, make_uint4(T0[0], T0[1], T0[2], T0[3]),
                      make_uint4(T1[0], T1[1], T1[2], T1[3]), S0, S1);
      sums[(m * nblocks + blk) * 2 + 0] = S0;
      sums[(m * nblocks + blk) * 2 + 1] = S1;
    }
  }
}

// Quads of four rows at one 8-block group (rows 4r..4r+3 of the matrix,
// group g of each row) against quads of four columns (4c..4c+3), the lane
// layout of the GEMV's matrix-core form: lane 4u+i of a wave holds row 4r+i
// of quad u as the B operand and column 4c+i as the A operand, and receives
// its row's sums for columns 4c..4c+3.  Sixteen quads per wave and
// iteration; every lane runs every iteration (a quad past the end recomputes
// the last one, and a row or column past the end re-reads the last one;
// neither stores).  Requires nb % 8 == 0.
__global__ __launch_bounds__(256) void debug_half_sums_mf_kernel(
    const uint8_t* __restrict__ w, int64_t N, int64_t nb, const uint32_t* __restrict__ q,
    int64_t M, int32_t* __restrict__ sums) {
  const int lane = threadIdx.x & 63;
  const int i = lane & 3;
  const int64_t row_quads = (N + 3) / 4, col_quads = (M + 3) / 4, groups = nb / 8;
  const int64_t nquads = col_quads * row_quads * groups;
  const int64_t waves = (int64_t)gridDim.x * 4;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  for (int64_t base = wave * 16; base < nquads; base += waves * 16) {   // uniform per wave
    const int64_t mine = base + (lane >> 2);
    const bool store = mine < nquads;
    const int64_t Q = store ? mine : nquads - 1;
    const int64_t g = Q % groups, rest = Q / groups;
    const int64_t r4 = rest % row_quads, c4 = rest / row_quads;
    const int64_t n = 4 * r4 + i;
    const int64_t nr = n < N ? n : N - 1;
    const int64_t ma = 4 * c4 + i < M ? 4 * c4 + i : M - 1;
    uint32_t dw[20];
    load_dwords(w, (nr * nb + 8 * g) * 10, N * nb * 10, dw);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      const int64_t b = 8 * g + jb;
      uint32_t W0[4], W1[4], sc;
      float s0, s1;
      decode_block(dw, jb, W0, W1, s0, s1, sc);
      const uint32_t* qa = q + (ma * nb + b) * 8;
      const uint32_t X0[4] = {qa[0], qa[1], qa[2], qa[3]};
      const uint32_t X1[4] = {qa[4], qa[5], qa[6], qa[7]};
      uint32_t T0[4], T1[4];
      transpose_half(X0, T0);
      transpose_half(X1, T1);
      // half 0 from the product's biased start (the int32 pattern of fp32
      // 1.5 * 2^23), the bias taken off again in integer arithmetic
      constexpr int kBias = 0x4B400000;
      const v4i S0 = half_sums_mf(W0, make_uint4(T0[0], T0[1], T0[2], T0[3]),
                                  v4i{kBias, kBias, kBias, kBias}) -
                     v4i{kBias, kBias, kBias, kBias};
      const v4i S1 = half_sums_mf(W1, make_uint4(T1[0], T1[1], T1[2], T1[3]));
      if (store && n < N) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = 4 * c4 + j;
          if (m < M) {
            sums[((m * N + n) * nb + b) * 2 + 0] = S0[j];
            sums[((m * N + n) * nb + b) * 2 + 1] = S1[j];
          }
        }
      }
    }
  }
}

// fp16 bits of the 16 weights of one half, in natural order, from 8 dwords
// in the k order of expand_half_f16.
__device__ __forceinline__ void store_half_f16(const uint32_t (&o)[8], uint16_t* out) {
#pragma unroll
  for (int e = 0; e < 16; ++e)
    out[f16_weight_of(e)] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
}

__global__ __launch_bounds__(256) void debug_decode_f16_kernel(
    const uint8_t* __restrict__ w, int64_t nblocks, int form, uint16_t* __restrict__ out) {
  const int64_t npairs = (nblocks + 1) / 2;
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < npairs;
       p += (int64_t)gridDim.x * 256) {
    uint32_t wd[5];
    load_dwords(w, p * 20, nblocks * 10, wd);
    const int nblk = 2 * p + 1 < nblocks ? 2 : 1;
    if (form == 0) {
      for (int blk = 0; blk < nblk; ++blk) {
        uint32_t h0[8], h1[8];
        decode_pair_block_f16(wd, blk, h0, h1);
        store_half_f16(h0, out + (2 * p + blk) * 32);
        store_half_f16(h1, out + (2 * p + blk) * 32 + 16);
      }
    } else {
      const WPair wp{wd[0], wd[1], wd[2], wd[3], wd[4]};
      for (int kh = 0; kh < 2; ++kh) {
        v8h a0, a1;
        uint32_t o[8];
        decode_half<0>(wp, kh, a0, a1);
        const uint4 x0 = __builtin_bit_cast(uint4, a0), x1 = __builtin_bit_cast(uint4, a1);
        o[0] = x0.x; o[1] = x0.y; o[2] = x0.z; o[3] = x0.w;
        o[4] = x1.x; o[5] = x1.y; o[6] = x1.z; o[7] = x1.w;
        store_half_f16(o, out + (2 * p) * 32 + 16 * kh);
        if (nblk == 2) {
          decode_half<1>(wp, kh, a0, a1);
          const uint4 y0 = __builtin_bit_cast(uint4, a0), y1 = __builtin_bit_cast(uint4, a1);
          o[0] = y0.x; o[1] = y0.y; o[2] = y0.z; o[3] = y0.w;
          o[4] = y1.x; o[5] = y1.y; o[6] = y1.z; o[7] = y1.w;
          store_half_f16(o, out + (2 * p + 1) * 32 + 16 * kh);
        }
      }
    }
  }
}

int64_t grid_for(int64_t items) {
  return std::max<int64_t>(1, std::min<int64_t>((items + 255) / 256, kMaxGrid));
}

}  // namespace

hipError_t launch_debug_decode(const uint8_t* w, int64_t N, int64_t K,
                               int8_t* codes, float* scales, hipStream_t stream) {
  const int64_t nblocks = N * (K / 32);
  hipLaunchKernelGGL(debug_decode_kernel, dim3((uint32_t)grid_for((nblocks + 7) / 8)), dim3(256),
                     0, stream, w, nblocks, reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_debug_half_dots(const uint8_t* w, int64_t N, int64_t K,
                                  const int8_t* q, int64_t M, int32_t* sums,
                                  hipStream_t stream) {
  const int64_t nb = K / 32;
  const int64_t nblocks = N * nb;
  hipLaunchKernelGGL(debug_half_dots_kernel, dim3((uint32_t)grid_for(M * ((nblocks + 7) / 8))),
                     dim3(256), 0, stream, w, nblocks, nb,
                     reinterpret_cast<const uint32_t*>(q), M, sums);
  return hipGetLastError();
}

hipError_t launch_debug_half_sums_mf(const uint8_t* w, int64_t N, int64_t K,
                                     const int8_t* q, int64_t M, int32_t* sums,
                                     hipStream_t stream) {
  const int64_t nb = K / 32;
  const int64_t quads = ((M + 3) / 4) * ((N + 3) / 4) * (nb / 8);
  // 64 quads per 256-thread workgroup and iteration
  hipLaunchKernelGGL(debug_half_sums_mf_kernel, dim3((uint32_t)grid_for(quads * 4)), dim3(256),
                     0, stream, w, N, nb, reinterpret_cast<const uint32_t*>(q), M, sums);
  return hipGetLastError();
}

hipError_t launch_debug_decode_f16(const uint8_t* w, int64_t N, int64_t K, int form,
                                   uint16_t* out, hipStream_t stream) {
  const int64_t nblocks = N * (K / 32);
  hipLaunchKernelGGL(debug_decode_f16_kernel, dim3((uint32_t)grid_for((nblocks + 1) / 2)),
                     dim3(256), 0, stream, w, nblocks, form, out);
  return hipGetLastError();
}

}  // namespace rfp2
