// ROCmFP2 x int8 GEMM on the i8 matrix cores (prompt batches).
//
// Method ("ROCmFP2 codebook research report", "03 · Runtime", applied to a
// tile of activation columns): the stored blocks are expanded to int8 once
// per tile and reused by every token of the tile; each 16-weight half gives
// an int32 partial per (token, row); the two weight scales and the token's
// activation scale are applied to the partials,
//   y[m,n] += d[m,b] * (s0[n,b] * P0[m,n] + s1[n,b] * P1[m,n]).
//
// gfx950 mapping
//   * v_mfma_i32_32x32x16_i8: one instruction is exactly one 16-weight half
//     (K = 16) of a 32 x 32 (token x row) tile, so every int32 partial is a
//     per-half sum and no weight scale is mixed into another.
//   * Workgroup tile 128 tokens x 128 rows, four waves of 64 x 64 (2 x 2
//     MFMA tiles); K advances 128 weights (4 blocks) per LDS stage.
//   * Weights are expanded in registers (expand_half) and written to LDS as
//     int8 in the lane order of expand_half; activations are staged with the
//     same within-half permutation (transpose_half), so the dot product over
//     each half is unchanged.  Row strides of 136 bytes keep the 8-byte LDS
//     operand reads of 32 lanes on distinct banks.
#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;          // tokens per workgroup tile
constexpr int BN = 128;          // weight rows per workgroup tile
constexpr int BKB = 4;           // blocks (of 32 weights) per LDS stage
constexpr int kStride = BKB * 32 + 8;   // LDS bytes per row of a stage (136)

struct __align__(16) GemmSmem {
  int8_t wq[BN * kStride];       // expanded weights, permuted within halves
  int8_t aq[BM * kStride];       // activations, same permutation
  float ws[BN][BKB * 2];         // weight scale per (row, half)
  float ad[BKB][BM];             // activation scale per (block, token)
};

__global__ __launch_bounds__(256) void gemm_kernel(
    const uint8_t* __restrict__ w, int N, int K, const int8_t* __restrict__ q,
    const float* __restrict__ d, int M, float* __restrict__ y, int m_tiles) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // consecutive workgroups walk the token tiles of one row tile, so a row
  // tile's weights are expanded by neighbouring workgroups close in time
  const int mt = blockIdx.x % m_tiles;
  const int nt = blockIdx.x / m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int64_t row_bytes = (int64_t)(K / 32) * 10;
  const int nb = K / 32;

  const v16i zero = {};
  float facc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) facc[i][j][r] = 0.0f;

  // staging roles
  const int wrow = tid >> 1;          // weight row within the tile
  const int wpair = tid & 1;          // blocks 2*wpair, 2*wpair+1 of the stage
  const bool wrow_ok = n0 + wrow < N;
  const int arow = tid >> 1;          // token within the tile
  const int ahalf = tid & 1;          // 64-byte half of the stage's 128 bytes
  const bool arow_ok = m0 + arow < M;

  for (int kb = 0; kb < nb; kb += BKB) {
    // ---- weights: two blocks (20 bytes, dword aligned) per thread
    {
      uint32_t D[5] = {0u, 0u, 0u, 0u, 0u};
      if (wrow_ok) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(
            w + (int64_t)(n0 + wrow) * row_bytes + (int64_t)(kb + 2 * wpair) * 10);
#pragma unroll
        for (int i = 0; i < 5; ++i) D[i] = src[i];
      }
      const uint32_t codes[4] = {D[0], D[1], __builtin_amdgcn_alignbit(D[3], D[2], 16),
                                 __builtin_amdgcn_alignbit(D[4], D[3], 16)};
#pragma unroll
      for (int h = 0; h < 4; ++h) {   // halves of the two blocks
        uint32_t W[4];
        expand_half(codes[h], W);
        int8_t* dst = sm.wq + wrow * kStride + (2 * wpair) * 32 + h * 16;
        *reinterpret_cast<uint2*>(dst) = make_uint2(W[0], W[1]);
        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(W[2], W[3]);
      }
      const float nan = __builtin_nanf("");
      const bool bad0 = scale_flags_set<0>(scale_pair_bad<0>(D[2]));
      const bool bad1 = scale_flags_set<1>(scale_pair_bad<1>(D[4]));
      sm.ws[wrow][4 * wpair + 0] = bad0 ? nan : fp8_byte<0>(D[2]);
      sm.ws[wrow][4 * wpair + 1] = bad0 ? nan : fp8_byte<1>(D[2]);
      sm.ws[wrow][4 * wpair + 2] = bad1 ? nan : fp8_byte<2>(D[4]);
      sm.ws[wrow][4 * wpair + 3] = bad1 ? nan : fp8_byte<3>(D[4]);
    }
    // ---- activations: four halves (64 bytes) per thread
    {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (arow_ok)
          x = *reinterpret_cast<const uint4*>(q + (int64_t)(m0 + arow) * K +
                                              (int64_t)kb * 32 + ahalf * 64 + i * 16);
        const uint32_t X[4] = {x.x, x.y, x.z, x.w};
        uint32_t A[4];
        transpose_half(X, A);
        int8_t* dst = sm.aq + arow * kStride + ahalf * 64 + i * 16;
        *reinterpret_cast<uint2*>(dst) = make_uint2(A[0], A[1]);
        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(A[2], A[3]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int idx = tid * 2 + i;          // 512 = BKB * BM scales
        const int blk = idx / BM, m = idx % BM;
        sm.ad[blk][m] = (m0 + m < M) ? d[(int64_t)(m0 + m) * nb + kb + blk] : 0.0f;
      }
    }
    __syncthreads();

    // ---- matrix cores: per block, two halves, 2 x 2 tiles per wave
    const int koff_lane = 8 * (lane >> 5);
#pragma unroll
    for (int blk = 0; blk < BKB; ++blk) {
      v16i P[2][2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int koff = blk * 32 + h * 16 + koff_lane;
        long a[2], b[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          a[t] = *reinterpret_cast<const long*>(
              sm.aq + (wm * 64 + t * 32 + (lane & 31)) * kStride + koff);
          b[t] = *reinterpret_cast<const long*>(
              sm.wq + (wn * 64 + t * 32 + (lane & 31)) * kStride + koff);
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            P[h][tm][tn] = __builtin_amdgcn_mfma_i32_32x32x16_i8(
                a[tm], b[tn], zero, 0, 0, 0);
      }
      // rescale: lane holds row n = lane % 32 of each tile and tokens
      // (r % 4) + 8 * (r / 4) + 4 * (lane / 32), r = 0..15
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const int n = wn * 64 + tn * 32 + (lane & 31);
        const float s0 = sm.ws[n][2 * blk];
        const float s1 = sm.ws[n][2 * blk + 1];
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float4 dv = *reinterpret_cast<const float4*>(
                &sm.ad[blk][wm * 64 + tm * 32 + 8 * p + 4 * (lane >> 5)]);
            const float dd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * p + e;
              const float t = fmaf(s1, (float)P[1][tm][tn][r],
                                   s0 * (float)P[0][tm][tn][r]);
              facc[tm][tn][r] = fmaf(dd[e], t, facc[tm][tn][r]);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  const float fix = scale_fix();
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int n = n0 + wn * 64 + tn * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + tm * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
        if (m < M) y[(int64_t)m * N + n] = facc[tm][tn][r] * fix;
      }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream) {
  const int m_tiles = (int)((M + BM - 1) / BM);
  const int n_tiles = (int)((N + BN - 1) / BN);
  hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)(m_tiles * n_tiles)), dim3(256), 0,
                     stream, w, (int)N, (int)K, q, d, (int)M, y, m_tiles);
  return hipGetLastError();
}

}  // namespace rfp2
