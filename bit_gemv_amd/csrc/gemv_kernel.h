// Kernel template of the ROCmFP2 GEMV (the design notes are in gemv.hip).
#pragma once

#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {
namespace gemv_detail {

constexpr int kRecord = 76;          // LDS dwords per (column, 8-block group)
constexpr int kMaxLdsBytes = 65536;  // LDS budget per workgroup
constexpr int kMaxWaves = 8;         // waves per workgroup (each owns a K slice)

struct Params {
  const uint8_t* w;
  int N, K;
  const int8_t* q;
  const float* d;
  float* y;
  int lshift;      // log2(lanes that share a row inside one wave)
  int wk;          // waves per workgroup: the row's groups are split among them
  int J;           // groups per lane
  const int32_t* ids;   // routed experts (MoE form) or null
  int E;
  int32_t* err;
};

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
    uint32_t c0, c1;
    if ((jb & 1) == 0) {          // starts on a dword: codes dw[o], dw[o+1]
      c0 = dw[o];
      c1 = dw[o + 1];
    } else {                       // starts at byte 2 of dw[o]
      c0 = __builtin_amdgcn_alignbit(dw[o + 1], dw[o], 16);
      c1 = __builtin_amdgcn_alignbit(dw[o + 2], dw[o + 1], 16);
    }
    const uint32_t sc = dw[o + 2];   // scale pair: bytes 0,1 (even) or 2,3 (odd)
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

// A wave's chunk of weights is its S = 64/L rows x L consecutive groups
// (80*L bytes per row) = 320 16-byte pieces, fetched with fully coalesced
// direct-to-LDS loads (global_load_lds_dwordx4: lane l of instruction k
// stores piece 64k + l at LDS dst + 16*(64k + l)).  Piece c belongs to row
// c / (5L) and sits 16*(c % (5L)) bytes into that row's segment, so lane l
// later finds its own group -- row slot l / L, group l % L -- as the 80
// contiguous LDS bytes at dst + 80*l.  The five per-lane byte offsets do not
// depend on which chunk is loaded and are computed once.  Pieces of rows past
// the end are fetched from the last row instead (the data is never used), so
// every chunk is exactly five load instructions and `vmcnt` counts chunks.
struct ChunkOffsets {
  int off[5];
};

__device__ __forceinline__ ChunkOffsets chunk_offsets(int lane, int lshift,
                                                      int row0, int N,
                                                      int row_bytes) {
  ChunkOffsets o;
  const int seg = 5 << lshift;                 // 16-byte pieces per row segment
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    const int c = 64 * k + lane;
    const int r = (c >> lshift) / 5;
    const int col = c - r * seg;
    const int rr = min(r, N - 1 - row0);       // clamp rows past the end
    o.off[k] = rr * row_bytes + col * 16;
  }
  return o;
}

__device__ __forceinline__ void load_chunk(const uint8_t* base, const ChunkOffsets& o,
                                           uint32_t* dst) {
#pragma unroll
  for (int k = 0; k < 5; ++k)
    __builtin_amdgcn_global_load_lds(base + o.off[k], dst + 256 * k, 16, 0, 0);
}

// Wait until at most 5*ahead weight loads (= `ahead` chunks) are outstanding.
__device__ __forceinline__ void wait_chunks(int ahead) {
  switch (ahead) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
  }
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// One workgroup = p.wk waves x 64 lanes computes S = 64 / L rows.  Inside a
// wave, L lanes share a row (lane t of row slot `slot`); across the waves of
// the workgroup the row's G = K/256 groups are split: in step j the wave
// covers groups (j * wk + wave) * L .. + L - 1, lane t taking one of them.
// A wave keeps up to JT chunks in flight in an LDS ring and computes chunk j
// as soon as it has landed.  Each wave stages the activations of its own
// groups, so no workgroup barrier precedes the products; one barrier
// precedes the final cross-wave sum.  M activation columns; MOE selects the
// weight matrix through ids[blockIdx.y].
template <int M, int JT, bool MOE>
__global__ __launch_bounds__(512) void gemv_kernel(Params p) {
  extern __shared__ uint32_t lds[];
  const int K = p.K, N = p.N;
  const int ls = p.lshift;
  const int L = 1 << ls;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = lane >> ls;
  const int t = lane & (L - 1);
  const int row0 = blockIdx.x * (64 >> ls);
  const int row = row0 + slot;
  const int row_bytes = (K >> 8) * 80;

  const uint8_t* wb = p.w;
  float* yb = p.y;
  bool id_ok = true;
  if (MOE) {
    const int e = p.ids[blockIdx.y];
    id_ok = e >= 0 && e < p.E;
    wb = p.w + (int64_t)(id_ok ? e : 0) * (int64_t)N * row_bytes;
    yb = p.y + (int64_t)blockIdx.y * N;
  }
  wb += (int64_t)row0 * row_bytes;

  // per-wave LDS: JT chunk buffers of 1280 dwords, then the activation
  // records of this wave's groups (M columns x J*L groups)
  const int ag = p.J << ls;                     // activation groups of the wave
  const int wave_dwords = JT * 1280 + M * ag * kRecord;
  uint32_t* wlds = lds + wave * wave_dwords;
  uint32_t* alds = wlds + JT * 1280;
  const int step = p.wk << ls;                  // groups between a wave's steps

  // Activation loads go out first: they hit L2 and, since a wave's loads
  // complete in issue order, queuing them behind the weights would hold the
  // staging until the weights had arrived.  Item h = (column m, local group
  // lgl = j*L + t', half b); its global group is (j*wk + wave)*L + t'.
  const int n_halves = M * ag * 16;
  const int n_scales = M * ag * 8;
  const int nb = K >> 5;
  auto group_of = [&](int lgl) {
    return (((lgl >> ls) * p.wk + wave) << ls) + (lgl & (L - 1));
  };
  uint4 x0 = make_uint4(0u, 0u, 0u, 0u);
  float d0 = 0.0f;
  int rec0 = 0, drec0 = 0;
  {
    const int m = M == 1 ? 0 : lane / (ag * 16);
    const int r = lane - m * ag * 16;
    const int lgl = r >> 4;
    if (lane < n_halves) {
      x0 = reinterpret_cast<const uint4*>(p.q + (int64_t)m * K)[group_of(lgl) * 16 + (r & 15)];
      rec0 = (m * ag + lgl) * kRecord + ((r & 15) >> 1) * 8 + (r & 1) * 4;
    }
    const int md = M == 1 ? 0 : lane / (ag * 8);
    const int rd = lane - md * ag * 8;
    if (lane < n_scales) {
      d0 = p.d[(int64_t)md * nb + group_of(rd >> 3) * 8 + (rd & 7)];
      drec0 = (md * ag + (rd >> 3)) * kRecord + 64 + (rd & 7);
    }
  }

  // weights: the first JT chunks
  const ChunkOffsets co = chunk_offsets(lane, ls, row0, N, row_bytes);
#pragma unroll
  for (int j = 0; j < JT; ++j)                 // J is a multiple of JT
    load_chunk(wb + (int64_t)((j * p.wk + wave) << ls) * 80, co, wlds + j * 1280);

  // stage this wave's activations, transposed within each half
  for (int h = lane; h < n_halves; h += 64) {
    uint4 x = x0;
    int rec = rec0;
    if (h != lane) {
      const int m = M == 1 ? 0 : h / (ag * 16);
      const int r = h - m * ag * 16;
      x = reinterpret_cast<const uint4*>(p.q + (int64_t)m * K)[group_of(r >> 4) * 16 + (r & 15)];
      rec = (m * ag + (r >> 4)) * kRecord + ((r & 15) >> 1) * 8 + (r & 1) * 4;
    }
    const uint32_t X[4] = {x.x, x.y, x.z, x.w};
    uint32_t A[4];
    transpose_half(X, A);
    *reinterpret_cast<uint4*>(alds + rec) = make_uint4(A[0], A[1], A[2], A[3]);
  }
  for (int i = lane; i < n_scales; i += 64) {
    float v = d0;
    int rec = drec0;
    if (i != lane) {
      const int m = M == 1 ? 0 : i / (ag * 8);
      const int r = i - m * ag * 8;
      v = p.d[(int64_t)m * nb + group_of(r >> 3) * 8 + (r & 7)];
      rec = (m * ag + (r >> 3)) * kRecord + 64 + (r & 7);
    }
    alds[rec] = __float_as_uint(v);
  }

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  uint32_t bad_lo = 0, bad_hi = 0;
  const int col_stride = ag * kRecord;
  for (int j = 0; j < p.J; ++j) {
    const int buf_i = JT == 1 ? 0 : j % JT;
    wait_chunks(min(JT, p.J - j) - 1);          // chunk j has landed
    __builtin_amdgcn_wave_barrier();
    uint32_t buf[20];
    const uint4* src = reinterpret_cast<const uint4*>(wlds + buf_i * 1280 + 20 * lane);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const uint4 v = src[k];
      buf[4 * k + 0] = v.x;
      buf[4 * k + 1] = v.y;
      buf[4 * k + 2] = v.z;
      buf[4 * k + 3] = v.w;
    }
    wait_lds();                     // chunk j is in registers, the activations
    __builtin_amdgcn_wave_barrier();  // are staged: the buffer can be reused
    if (j + JT < p.J)
      load_chunk(wb + (int64_t)((((j + JT) * p.wk) + wave) << ls) * 80, co,
                 wlds + buf_i * 1280);
    group_product<M>(buf, alds + ((j << ls) + t) * kRecord, col_stride, acc, bad_lo, bad_hi);
  }

  // row sum: xor shuffles over the L lanes of the row, then over the waves
  const bool bad = scale_flags_set<0>(bad_lo) || scale_flags_set<1>(bad_hi);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = bad ? __builtin_nanf("") : acc[m];
    for (int off = 1; off < L; off <<= 1) v += __shfl_xor(v, off, 64);
    acc[m] = v;
  }
  const int S = 64 >> ls;
  if (p.wk > 1) {
    float* red = reinterpret_cast<float*>(lds + p.wk * wave_dwords);
    if (t == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) red[(wave * S + slot) * M + m] = acc[m];
    }
    __syncthreads();
    if (wave == 0 && t == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float v = red[slot * M + m];
        for (int wv = 1; wv < p.wk; ++wv) v += red[(wv * S + slot) * M + m];
        acc[m] = v;
      }
    }
  }
  if (wave == 0 && t == 0 && row < N) {
    const float fix = scale_fix();
#pragma unroll
    for (int m = 0; m < M; ++m)
      yb[(int64_t)m * N + row] = id_ok ? acc[m] * fix : __builtin_nanf("");
  }
  if (MOE && !id_ok && blockIdx.x == 0 && threadIdx.x == 0 && p.err != nullptr)
    p.err[0] = 1;
}

using GemvFn = void (*)(Params);

constexpr int kMaxChunksInFlight = 4;

template <int M, bool MOE>
GemvFn pick(int jt) {
  switch (jt) {
    case 1: return gemv_kernel<M, 1, MOE>;
    case 2: return gemv_kernel<M, 2, MOE>;
    case 3: return gemv_kernel<M, 3, MOE>;
    default: return gemv_kernel<M, 4, MOE>;
  }
}

}  // namespace gemv_detail
}  // namespace rfp2
