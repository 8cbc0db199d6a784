// ROCmFP2 GEMV for a few activation columns, and its routed-expert form.
//
// Method ("ROCmFP2 codebook research report", "03 · Runtime"): every code
// byte is expanded once into four int8 lanes, each 16-weight half is dotted
// with the int8 activations into an int32 sum, and only then are the two
// weight scales and the activation scale applied,
//   y += d_a * (s_0 * S_0 + s_1 * S_1).
// The multi-column form ("Why AMD-friendly does not mean always faster")
// expands a block once and reuses it for every activation column.
//
// gfx950 mapping
//   * The stored matrix is one contiguous stream of 10-byte blocks.  K is a
//     multiple of 256, so a row is a whole number of 80-byte groups (8 blocks,
//     five 16-byte loads).  A lane owns whole groups: no block straddles two
//     lanes and every load is a 16-byte vector load.
//   * L lanes share a row, L being the largest power of two (<= 64) dividing
//     the G = K/256 groups of a row; each lane takes J = G/L groups (group
//     t + L*j for lane t).  A wave covers 64/L rows, so all 64 lanes work and
//     the row sum is a log2(L)-step xor-shuffle reduction.
//   * The loads of a lane's groups are issued before the workgroup stages the
//     activations, so HBM latency overlaps the staging.
//   * Activations are staged once per workgroup in LDS, transposed within
//     each half to the lane order of the expanded weights (see expand_half),
//     together with the per-block activation scales.  One 76-dword record per
//     (column, group): 64 dwords of activations, 8 scales, 4 dwords of pad so
//     that lanes reading neighbouring groups hit different LDS banks.
#include "gemv_kernel.h"

namespace rfp2 {

namespace gemv_detail {
GemvFn pick_m1(int jt);
GemvFn pick_m2(int jt);
GemvFn pick_m3(int jt);
GemvFn pick_m4(int jt);
GemvFn pick_m5(int jt);
GemvFn pick_m6(int jt);
GemvFn pick_m7(int jt);
GemvFn pick_m8(int jt);
}  // namespace gemv_detail

namespace {

using namespace gemv_detail;

GemvFn pick_kernel(int M, int jt) {
  switch (M) {
    case 1: return pick_m1(jt);
    case 2: return pick_m2(jt);
    case 3: return pick_m3(jt);
    case 4: return pick_m4(jt);
    case 5: return pick_m5(jt);
    case 6: return pick_m6(jt);
    case 7: return pick_m7(jt);
    default: return pick_m8(jt);
  }
}

struct Geometry {
  int lshift;   // log2 of lanes per row
  int J;        // groups per lane
  int jt;       // groups per load tile (divides J)
  int rows_per_wg;
};

Geometry geometry(int64_t K) {
  const int G = (int)(K / 256);
  int lshift = 0;
  while (lshift < 6 && (G % (2 << lshift)) == 0) ++lshift;
  Geometry g;
  g.lshift = lshift;
  g.J = G >> lshift;
  g.jt = 1;
  for (int c = kMaxGroupsPerTile; c >= 1; --c)
    if (g.J % c == 0) { g.jt = c; break; }
  g.rows_per_wg = kWaves * (64 >> lshift);
  return g;
}

}  // namespace

hipError_t launch_gemv(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream) {
  const Geometry g = geometry(K);
  const int G = (int)(K / 256);
  const int per_col_lds = G * kRecord * 4;
  const int cols_per_launch = std::max(1, std::min<int>((int)M, kMaxLdsBytes / per_col_lds));
  const dim3 grid((uint32_t)((N + g.rows_per_wg - 1) / g.rows_per_wg));
  for (int64_t m0 = 0; m0 < M; m0 += cols_per_launch) {
    const int mc = (int)std::min<int64_t>(cols_per_launch, M - m0);
    GemvFn fn = pick_kernel(mc, g.jt);
    hipLaunchKernelGGL(fn, grid, dim3(256), (size_t)mc * per_col_lds, stream, w,
                       (int)N, (int)K, q + m0 * K, d + m0 * (K / 32), y + m0 * N,
                       g.lshift, g.J, (const int32_t*)nullptr, 0, (int32_t*)nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                           const int32_t* ids, int64_t top_k, const int8_t* q,
                           const float* d, float* y, int32_t* err,
                           hipStream_t stream) {
  const Geometry g = geometry(K);
  const int G = (int)(K / 256);
  const dim3 grid((uint32_t)((N + g.rows_per_wg - 1) / g.rows_per_wg), (uint32_t)top_k);
  GemvFn fn = pick_tile<1, true>(g.jt);
  hipLaunchKernelGGL(fn, grid, dim3(256), (size_t)G * kRecord * 4, stream, w,
                     (int)N, (int)K, q, d, y, g.lshift, g.J, ids, (int)E, err);
  return hipGetLastError();
}

}  // namespace rfp2
