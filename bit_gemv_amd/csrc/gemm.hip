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
//     MFMA tiles); K advances 128 weights (4 blocks) per LDS stage.  Two LDS
//     buffers: while the waves compute stage s, the global loads of stage s+1
//     are already in registers; one barrier per stage.  Two workgroups per
//     CU.
//   * Weights are expanded in registers (expand_half) and written to LDS as
//     int8 in the lane order of expand_half; activations are staged with the
//     same within-half permutation (transpose_half), so the dot product over
//     each half is unchanged.  Row strides of 136 bytes keep the 8-byte LDS
//     operand reads of 32 lanes on distinct banks.
//   * The fp32 rescale of every (token, row, block) is vector-ALU work that
//     no MFMA shape removes: per-half weight scales and per-block activation
//     scales both vary along K.  It, not the matrix cores, bounds this
//     kernel.  Four instructions instead of five: the first half's partial
//     is accumulated onto the int32 bit pattern of 1.5 * 2^23, so the result
//     read as fp32 is exactly 1.5 * 2^23 + P0 (|P0| <= 16 * 4 * 127 < 2^22),
//     and s0 * P0 = fma(s0, that, -1.5 * 2^23 * s0) in one instruction,
//     exact (s0 has at most 4 significant bits, s0 * P0 at most 17) -- the
//     same value as the convert and multiply it replaces, so the outputs
//     are unchanged; then one convert of P1, fma(s1, P1, s0 * P0), and the
//     fma with the activation scale.
//   * Workgroup -> tile order is XCD-aware: the hardware deals workgroups to
//     the 8 XCDs round-robin, so consecutive tiles are given to workgroups
//     that land on the same XCD, and the token tiles of one row tile run
//     next to each other and share that XCD's L2 for the weights.
#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;          // tokens per workgroup tile
constexpr int BN = 128;          // weight rows per workgroup tile
constexpr int BKB = 4;           // blocks (of 32 weights) per LDS stage
constexpr int kStride = BKB * 32 + 8;   // LDS bytes per row of a stage (136)
constexpr int kXcds = 8;

struct __align__(16) Stage {
  int8_t wq[BN * kStride];       // expanded weights, permuted within halves
  int8_t aq[BM * kStride];       // activations, same permutation
  float ws[BN][BKB * 2];         // weight scale per (row, half)
  float ad[BKB][BM];             // activation scale per (block, token)
};

struct Prefetch {
  uint32_t wd[5];                // two blocks of one weight row
  uint4 a[4];                    // 64 bytes of one token's activations
  float d[2];                    // two activation scales
};

__device__ __forceinline__ void fetch(Prefetch& f, const uint8_t* __restrict__ w,
                                      const int8_t* __restrict__ q,
                                      const float* __restrict__ d, int64_t row_bytes,
                                      int K, int nb, int kb, int tid, int n0, int m0,
                                      int N, int M) {
  const int wrow = tid >> 1, wpair = tid & 1;
  // rows / tokens past the end read row / token 0 (never stored)
  const int n = n0 + wrow < N ? n0 + wrow : 0;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(
      w + (int64_t)n * row_bytes + (int64_t)(kb + 2 * wpair) * 10);
#pragma unroll
  for (int i = 0; i < 5; ++i) f.wd[i] = src[i];
  const int arow = tid >> 1, ahalf = tid & 1;
  const int m = m0 + arow < M ? m0 + arow : 0;
  const uint4* asrc = reinterpret_cast<const uint4*>(q + (int64_t)m * K + (int64_t)kb * 32 +
                                                     ahalf * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = asrc[i];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid * 2 + i;        // 512 = BKB * BM scales
    const int blk = idx / BM, mm = idx % BM;
    const int mr = m0 + mm < M ? m0 + mm : 0;
    f.d[i] = d[(int64_t)mr * nb + kb + blk];
  }
}

__device__ __forceinline__ void stage_to_lds(const Prefetch& f, Stage& st, int tid) {
  const int wrow = tid >> 1, wpair = tid & 1;
  const uint32_t codes[4] = {f.wd[0], f.wd[1], __builtin_amdgcn_alignbit(f.wd[3], f.wd[2], 16),
                             __builtin_amdgcn_alignbit(f.wd[4], f.wd[3], 16)};
#pragma unroll
  for (int h = 0; h < 4; ++h) {   // the four halves of the two blocks
    uint32_t W[4];
    expand_half(codes[h], W);
    int8_t* dst = st.wq + wrow * kStride + (2 * wpair) * 32 + h * 16;
    *reinterpret_cast<uint2*>(dst) = make_uint2(W[0], W[1]);
    *reinterpret_cast<uint2*>(dst + 8) = make_uint2(W[2], W[3]);
  }
  // an illegal scale byte in a block makes both of its scales NaN (bit-or
  // with a quiet NaN pattern: no branch)
  const uint32_t nan0 = scale_flags_set<0>(scale_pair_bad<0>(f.wd[2])) ? 0x7FC00000u : 0u;
  const uint32_t nan1 = scale_flags_set<1>(scale_pair_bad<1>(f.wd[4])) ? 0x7FC00000u : 0u;
  float4 s;
  s.x = __uint_as_float(__float_as_uint(fp8_byte<0>(f.wd[2])) | nan0);
  s.y = __uint_as_float(__float_as_uint(fp8_byte<1>(f.wd[2])) | nan0);
  s.z = __uint_as_float(__float_as_uint(fp8_byte<2>(f.wd[4])) | nan1);
  s.w = __uint_as_float(__float_as_uint(fp8_byte<3>(f.wd[4])) | nan1);
  *reinterpret_cast<float4*>(&st.ws[wrow][4 * wpair]) = s;

  const int arow = tid >> 1, ahalf = tid & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t X[4] = {f.a[i].x, f.a[i].y, f.a[i].z, f.a[i].w};
    uint32_t A[4];
    transpose_half(X, A);
    int8_t* dst = st.aq + arow * kStride + ahalf * 64 + i * 16;
    *reinterpret_cast<uint2*>(dst) = make_uint2(A[0], A[1]);
    *reinterpret_cast<uint2*>(dst + 8) = make_uint2(A[2], A[3]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int idx = tid * 2 + i;
    st.ad[idx / BM][idx % BM] = f.d[i];
  }
}

__global__ __launch_bounds__(256, 2) void gemm_kernel(
    const uint8_t* __restrict__ w, int N, int K, const int8_t* __restrict__ q,
    const float* __restrict__ d, int M, float* __restrict__ y, int m_tiles,
    int tiles) {
  __shared__ Stage sm[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // XCD-aware order: workgroup b runs on XCD b % 8; give XCD x the
  // consecutive tiles x*per, x*per+1, ... (token tiles of a row tile first)
  int tile = blockIdx.x;
  if (tiles % kXcds == 0) tile = (blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
  const int mt = tile % m_tiles;
  const int nt = tile / m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int64_t row_bytes = (int64_t)(K / 32) * 10;
  const int nb = K / 32;
  const int stages = nb / BKB;

  float facc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) facc[i][j][r] = 0.0f;

  // the accumulator start of the first half's partials: fp32 1.5 * 2^23
  v16i kBias;
#pragma unroll
  for (int r = 0; r < 16; ++r) kBias[r] = 0x4B400000;
  Prefetch f;
  fetch(f, w, q, d, row_bytes, K, nb, 0, tid, n0, m0, N, M);
  const int koff_lane = 8 * (lane >> 5);
  for (int s = 0; s < stages; ++s) {
    Stage& st = sm[s & 1];
    stage_to_lds(f, st, tid);
    if (s + 1 < stages) fetch(f, w, q, d, row_bytes, K, nb, (s + 1) * BKB, tid, n0, m0, N, M);
    __syncthreads();

#pragma unroll
    for (int blk = 0; blk < BKB; ++blk) {
      long a[2][2];                 // [half][tm]
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
          a[h][tm] = *reinterpret_cast<const long*>(
              st.aq + (wm * 64 + tm * 32 + (lane & 31)) * kStride + blk * 32 + h * 16 +
              koff_lane);
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const int n = wn * 64 + tn * 32 + (lane & 31);
        const long b0 = *reinterpret_cast<const long*>(st.wq + n * kStride + blk * 32 + koff_lane);
        const long b1 =
            *reinterpret_cast<const long*>(st.wq + n * kStride + blk * 32 + 16 + koff_lane);
        const float2 sc = *reinterpret_cast<const float2*>(&st.ws[n][2 * blk]);
        const float nb0 = -12582912.0f * sc.x;
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) {
          const v16i P0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[0][tm], b0, kBias, 0, 0, 0);
          const v16i P1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(a[1][tm], b1, v16i{}, 0, 0, 0);
          // lane holds row n of the tile and tokens
          // (r % 4) + 8 * (r / 4) + 4 * (lane / 32), r = 0..15
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const float4 dv = *reinterpret_cast<const float4*>(
                &st.ad[blk][wm * 64 + tm * 32 + 8 * p + 4 * (lane >> 5)]);
            const float dd[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * p + e;
              const float t = fmaf(sc.y, (float)P1[r], fmaf(sc.x, __int_as_float(P0[r]), nb0));
              facc[tm][tn][r] = fmaf(dd[e], t, facc[tm][tn][r]);
            }
          }
        }
      }
    }
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

// Inspection of the GEMM's decode (rfp2_debug_decode_i8): the two blocks of
// pair p of the flat block stream, loaded and decoded exactly as
// stage_to_lds decodes a thread's pair (the second block funnel-shifted out
// of the dwords), written in natural weight order.
__global__ __launch_bounds__(256) void debug_decode_i8_kernel(
    const uint8_t* __restrict__ w, int64_t nblocks, uint32_t* __restrict__ codes,
    float* __restrict__ scales) {
  const float fix = scale_fix();
  for (int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x; p < (nblocks + 1) / 2;
       p += (int64_t)gridDim.x * 256) {
    // the 20-byte pair as 16-bit pieces (the stream is only 2-byte aligned
    // here); bytes past the end read as zero
    const uint16_t* src = reinterpret_cast<const uint16_t*>(w + p * 20);
    const int64_t end = nblocks * 10;
    Prefetch f;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int64_t off = p * 20 + 4 * i;
      f.wd[i] = (off < end ? (uint32_t)src[2 * i] : 0u) |
                ((off + 2 < end ? (uint32_t)src[2 * i + 1] : 0u) << 16);
    }
    const uint32_t cw[4] = {f.wd[0], f.wd[1], __builtin_amdgcn_alignbit(f.wd[3], f.wd[2], 16),
                            __builtin_amdgcn_alignbit(f.wd[4], f.wd[3], 16)};
    const float nan = __builtin_nanf("");
    const bool bad0 = scale_flags_set<0>(scale_pair_bad<0>(f.wd[2]));
    const bool bad1 = scale_flags_set<1>(scale_pair_bad<1>(f.wd[4]));
    const float sv[4] = {bad0 ? nan : fp8_byte<0>(f.wd[2]) * fix,
                         bad0 ? nan : fp8_byte<1>(f.wd[2]) * fix,
                         bad1 ? nan : fp8_byte<2>(f.wd[4]) * fix,
                         bad1 ? nan : fp8_byte<3>(f.wd[4]) * fix};
#pragma unroll
    for (int h = 0; h < 4; ++h) {              // the four halves of the pair
      const int64_t blk = 2 * p + (h >> 1);
      if (blk >= nblocks) break;
      uint32_t W[4];
      expand_half(cw[h], W);
      // weight 4j+i of the half is byte j of W[i]
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = __builtin_amdgcn_perm(W[1], W[0], 0x00000400u + 0x0101u * j);
        const uint32_t hi = __builtin_amdgcn_perm(W[3], W[2], 0x00000400u + 0x0101u * j);
        codes[blk * 8 + (h & 1) * 4 + j] = (lo & 0xFFFFu) | (hi << 16);
      }
      scales[blk * 2 + (h & 1)] = sv[h];
    }
  }
}

}  // namespace

hipError_t launch_debug_decode_i8(const uint8_t* w, int64_t N, int64_t K, int8_t* codes,
                                  float* scales, hipStream_t stream) {
  const int64_t npairs = (N * (K / 32) + 1) / 2;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((npairs + 255) / 256, kMaxGrid));
  hipLaunchKernelGGL(debug_decode_i8_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, w,
                     N * (K / 32), reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream) {
  const int m_tiles = (int)((M + BM - 1) / BM);
  const int n_tiles = (int)((N + BN - 1) / BN);
  const int tiles = m_tiles * n_tiles;
  hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)tiles), dim3(256), 0, stream, w, (int)N,
                     (int)K, q, d, (int)M, y, m_tiles, tiles);
  return hipGetLastError();
}

}  // namespace rfp2
