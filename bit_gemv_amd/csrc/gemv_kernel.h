// Kernel template of the ROCmFP2 GEMV (see gemv.hip for the design).
#pragma once

#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {
namespace gemv_detail {


constexpr int kWaves = 4;            // waves per workgroup
constexpr int kRecord = 76;          // LDS dwords per (column, group)
constexpr int kMaxLdsBytes = 65536;  // LDS budget per workgroup
constexpr int kMaxGroupsPerTile = 8;

// Decode one 80-byte group held in registers and accumulate its product with
// M activation columns.  `act` points at the LDS record of column 0 for this
// group; columns are `col_stride` dwords apart.
template <int M>
__device__ __forceinline__ void group_product(const uint32_t (&dw)[20],
                                              const uint32_t* act, int col_stride,
                                              float (&acc)[M], uint32_t& bad_lo,
                                              uint32_t& bad_hi) {
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) {
    // block jb occupies bytes 10*jb .. 10*jb+9 of the group
    const int o = (10 * jb) / 4;
    uint32_t c0, c1, sc;
    if ((jb & 1) == 0) {          // starts on a dword: codes dw[o], dw[o+1]
      c0 = dw[o];
      c1 = dw[o + 1];
    } else {                       // starts at byte 2 of dw[o]
      c0 = __builtin_amdgcn_alignbit(dw[o + 1], dw[o], 16);
      c1 = __builtin_amdgcn_alignbit(dw[o + 2], dw[o + 1], 16);
    }
    sc = dw[o + 2];               // scale pair: bytes 0,1 (even) or 2,3 (odd)
    uint32_t W0[4], W1[4];
    expand_half(c0, W0);
    expand_half(c1, W1);
    float s0, s1;
    if ((jb & 1) == 0) {
      s0 = fp8_byte<0>(sc);
      s1 = fp8_byte<1>(sc);
      bad_lo |= scale_pair_bad<0>(sc);
    } else {
      s0 = fp8_byte<2>(sc);
      s1 = fp8_byte<3>(sc);
      bad_hi |= scale_pair_bad<1>(sc);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t* a = act + m * col_stride + jb * 8;
      const uint4 A0 = *reinterpret_cast<const uint4*>(a);
      const uint4 A1 = *reinterpret_cast<const uint4*>(a + 4);
      const float dm = __uint_as_float(act[m * col_stride + 64 + jb]);
      const uint32_t a0[4] = {A0.x, A0.y, A0.z, A0.w};
      const uint32_t a1[4] = {A1.x, A1.y, A1.z, A1.w};
      const int32_t S0 = half_dot(W0, a0);
      const int32_t S1 = half_dot(W1, a1);
      acc[m] = fmaf(dm, fmaf(s1, (float)S1, s0 * (float)S0), acc[m]);
    }
  }
}

template <int JT>
__device__ __forceinline__ void load_groups(uint32_t (&buf)[JT][20],
                                            const uint4* row_ptr, int t, int j0,
                                            int L, bool active) {
#pragma unroll
  for (int jj = 0; jj < JT; ++jj) {
    const int g = t + (j0 + jj) * L;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (active) v = row_ptr[g * 5 + k];
      buf[jj][4 * k + 0] = v.x;
      buf[jj][4 * k + 1] = v.y;
      buf[jj][4 * k + 2] = v.z;
      buf[jj][4 * k + 3] = v.w;
    }
  }
}

// M activation columns; JT groups loaded per tile; MOE selects the expert
// of blockIdx.y through ids[].
template <int M, int JT, bool MOE>
__global__ __launch_bounds__(256) void gemv_kernel(
    const uint8_t* __restrict__ w, int N, int K, const int8_t* __restrict__ q,
    const float* __restrict__ d, float* __restrict__ y, int lshift, int J,
    const int32_t* __restrict__ ids, int E, int32_t* __restrict__ err) {
  extern __shared__ uint32_t lds[];
  const int G = K >> 8;
  const int L = 1 << lshift;
  const int S = 64 >> lshift;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane >> lshift;
  const int t = lane & (L - 1);
  const int row = blockIdx.x * (kWaves * S) + wave * S + slot;
  const int64_t row_bytes = (int64_t)G * 80;

  const uint8_t* wb = w;
  float* yb = y;
  bool id_ok = true;
  if (MOE) {
    const int e = ids[blockIdx.y];
    id_ok = e >= 0 && e < E;
    wb = w + (int64_t)(id_ok ? e : 0) * (int64_t)N * row_bytes;
    yb = y + (int64_t)blockIdx.y * N;
  }
  const bool active = id_ok && row < N;
  const uint4* row_ptr =
      reinterpret_cast<const uint4*>(wb + (int64_t)(active ? row : 0) * row_bytes);

  // first tile of weights goes out before the activation staging
  uint32_t buf[JT][20];
  load_groups<JT>(buf, row_ptr, t, 0, L, active);

  // stage activations: one half (16 bytes) per thread per step
  const int halves_per_col = K >> 4;
  for (int h = threadIdx.x; h < M * halves_per_col; h += 256) {
    const int m = h / halves_per_col;
    const int hk = h - m * halves_per_col;
    const uint4 x = reinterpret_cast<const uint4*>(q + (int64_t)m * K)[hk];
    const uint32_t X[4] = {x.x, x.y, x.z, x.w};
    uint32_t A[4];
    transpose_half(X, A);
    const int b = hk >> 1;
    uint32_t* dst = lds + (m * G + (b >> 3)) * kRecord + (b & 7) * 8 + (hk & 1) * 4;
    *reinterpret_cast<uint4*>(dst) = make_uint4(A[0], A[1], A[2], A[3]);
  }
  const int nb = K >> 5;
  for (int i = threadIdx.x; i < M * nb; i += 256) {
    const int m = i / nb;
    const int b = i - m * nb;
    lds[(m * G + (b >> 3)) * kRecord + 64 + (b & 7)] =
        __float_as_uint(d[(int64_t)m * nb + b]);
  }
  __syncthreads();

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  uint32_t bad_lo = 0, bad_hi = 0;
  const int col_stride = G * kRecord;
  for (int j0 = 0; j0 < J; j0 += JT) {
    if (j0 > 0) load_groups<JT>(buf, row_ptr, t, j0, L, active);
#pragma unroll
    for (int jj = 0; jj < JT; ++jj) {
      const int g = t + (j0 + jj) * L;
      group_product<M>(buf[jj], lds + g * kRecord, col_stride, acc, bad_lo, bad_hi);
    }
  }

  const float fix = scale_fix();
  const bool bad = scale_flags_set<0>(bad_lo) || scale_flags_set<1>(bad_hi);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = bad ? __builtin_nanf("") : acc[m];
    for (int off = 1; off < L; off <<= 1) v += __shfl_xor(v, off, 64);
    acc[m] = v * fix;
  }
  if (t == 0 && row < N) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      yb[(int64_t)m * N + row] = id_ok ? acc[m] : __builtin_nanf("");
  }
  if (MOE && !id_ok && blockIdx.x == 0 && threadIdx.x == 0 && err != nullptr)
    err[0] = 1;
}

using GemvFn = void (*)(const uint8_t*, int, int, const int8_t*, const float*,
                        float*, int, int, const int32_t*, int, int32_t*);

template <int M, bool MOE>
GemvFn pick_tile(int jt) {
  switch (jt) {
    case 1: return gemv_kernel<M, 1, MOE>;
    case 2: return gemv_kernel<M, 2, MOE>;
    case 3: return gemv_kernel<M, 3, MOE>;
    case 4: return gemv_kernel<M, 4, MOE>;
    case 5: return gemv_kernel<M, 5, MOE>;
    case 6: return gemv_kernel<M, 6, MOE>;
    case 7: return gemv_kernel<M, 7, MOE>;
    default: return gemv_kernel<M, 8, MOE>;
  }
}

}  // namespace gemv_detail
}  // namespace rfp2
