// ROCmFP2 x int8 GEMM on the fp16 matrix cores, with exact operands.
//
// Same product as gemm.hip ("ROCmFP2 codebook research report", "03 ·
// Runtime": int8 activations, weights = level x UE4M3 scale of their half,
// activation scale applied per 32-block), computed in a different order:
//   * every reconstructed weight level*s (|level| in {1, 4}, s a UE4M3 value
//     with at most 4 significant bits between 2^-10 and 224) and every int8
//     activation is exactly an fp16 number, and every product is exact in
//     fp32;
//   * so the per-half weight scales go into the operands, and one fp16 MFMA
//     pair (K = 16 each) gives the whole 32-weight block's sum
//     C = s0 * S0 + s1 * S1 directly in fp32 -- exactly, unless the two
//     halves' scales are more than 2^10 apart, where it rounds once;
//   * the epilogue per (token, row, block) is one FMA, y += d * C, against
//     two int->fp32 converts and three FMAs for the int32 per-half partials.
// The rescale, not the matrix cores, bounds the int8 path; here the two are
// of the same order.
//
// gfx950 mapping: workgroup tile 128 tokens x 128 rows, four waves of 64 x 64
// (2 x 2 tiles of v_mfma_f32_32x32x16_f16), K stage of 2 blocks, two LDS
// buffers with register prefetch of the next stage, XCD-aware tile order
// (as gemm.hip).  Within each 16-weight half the k order in LDS is
// 0,4, 1,5, 2,6, 3,7, 8,12, 9,13, 10,14, 11,15 for weights and activations
// alike (the order the decode produces cheaply); a dot product over the half
// does not depend on it.
#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BKB = 2;                          // blocks per LDS stage
constexpr int kRowBytes = BKB * 32 * 2 + 16;    // fp16 row of a stage + pad (144)
constexpr int kXcds = 8;

struct __align__(16) StageF16 {
  uint8_t wh[BN * kRowBytes];      // fp16 weights (level * scale)
  uint8_t ah[BM * kRowBytes];      // fp16 activations
  float ad[BKB][BM];               // activation scale per (block, token)
};

struct PrefetchF16 {
  uint32_t wd[5];                  // the 20-byte block pair holding this thread's block
  uint4 a[2];                      // 32 int8 activations
  float d;
};

// fp16 bit patterns of [-4s, -s] (lo) and [s, 4s] (hi) for one half, from
// its scale byte (s via the hardware fp8 convert and the fix-up power of two;
// an illegal byte gives NaN).
template <int BYTE>
__device__ __forceinline__ void half_table(uint32_t word, bool bad, float fix,
                                           uint32_t& lo, uint32_t& hi) {
  const float s = bad ? __builtin_nanf("") : fp8_byte<BYTE>(word) * fix;
  const _Float16 h1 = (_Float16)s;
  const _Float16 h4 = (_Float16)(4.0f * s);
  const uint32_t b1 = __builtin_bit_cast(uint16_t, h1);
  const uint32_t b4 = __builtin_bit_cast(uint16_t, h4);
  hi = b1 | (b4 << 16);
  lo = (b4 ^ 0x8000u) | ((b1 ^ 0x8000u) << 16);
}

// Expand the 16 codes of one half (X) to 8 dwords of fp16 pairs in the k
// order 0,4, 1,5, 2,6, 3,7, 8,12, 9,13, 10,14, 11,15.  D_i = 2*code of
// weights i, 4+i, 8+i, 12+i (one byte each); a byte permute turns D_i into
// the byte selectors (2c, 2c+1) of two fp16 lanes, a second one looks them
// up in the 8-byte table [-4s, -s, s, 4s].
__device__ __forceinline__ void expand_half_f16(uint32_t X, uint32_t lo, uint32_t hi,
                                                uint32_t (&out)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t D = (i == 0 ? (X << 1) : (X >> (2 * i - 1))) & 0x06060606u;
    const uint32_t D1 = D | 0x01010101u;
    const uint32_t sel_lo = __builtin_amdgcn_perm(D1, D, 0x05010400u);
    const uint32_t sel_hi = __builtin_amdgcn_perm(D1, D, 0x07030602u);
    out[i] = __builtin_amdgcn_perm(hi, lo, sel_lo);
    out[4 + i] = __builtin_amdgcn_perm(hi, lo, sel_hi);
  }
}

__device__ __forceinline__ uint32_t pack_f16(int a, int b) {
  const uint32_t x = __builtin_bit_cast(uint16_t, (_Float16)a);
  const uint32_t y = __builtin_bit_cast(uint16_t, (_Float16)b);
  return x | (y << 16);
}

// 16 int8 activations of one half (natural order, 4 words) -> 8 dwords of
// fp16 pairs in the same k order as expand_half_f16.
__device__ __forceinline__ void act_half_f16(const uint32_t (&X)[4], uint32_t (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 8 * j;
    out[j] = pack_f16((int)(int8_t)(X[0] >> s), (int)(int8_t)(X[1] >> s));
    out[4 + j] = pack_f16((int)(int8_t)(X[2] >> s), (int)(int8_t)(X[3] >> s));
  }
}

__device__ __forceinline__ void fetch(PrefetchF16& f, const uint8_t* __restrict__ w,
                                      const int8_t* __restrict__ q,
                                      const float* __restrict__ d, int64_t row_bytes,
                                      int K, int nb, int kb, int tid, int n0, int m0,
                                      int N, int M) {
  // thread -> (weight row tid / 2, block tid % 2 of the stage); both threads
  // of a row load the dword-aligned 20-byte pair of blocks
  const int wrow = tid >> 1;
  const int n = n0 + wrow < N ? n0 + wrow : 0;   // rows past the end read row 0
  const uint32_t* src =
      reinterpret_cast<const uint32_t*>(w + (int64_t)n * row_bytes + (int64_t)kb * 10);
#pragma unroll
  for (int i = 0; i < 5; ++i) f.wd[i] = src[i];
  // thread -> (token tid / 2, 32-byte block tid % 2 of the stage)
  const int arow = tid >> 1, ablk = tid & 1;
  const int m = m0 + arow < M ? m0 + arow : 0;
  const uint4* asrc =
      reinterpret_cast<const uint4*>(q + (int64_t)m * K + (int64_t)(kb + ablk) * 32);
  f.a[0] = asrc[0];
  f.a[1] = asrc[1];
  f.d = d[(int64_t)m * nb + kb + ablk];
}

__device__ __forceinline__ void stage_to_lds(const PrefetchF16& f, StageF16& st, int tid,
                                             float fix) {
  const int wrow = tid >> 1, blk = tid & 1;
  uint32_t c0, c1, sc;
  if (blk == 0) {
    c0 = f.wd[0];
    c1 = f.wd[1];
    sc = f.wd[2];
  } else {
    c0 = __builtin_amdgcn_alignbit(f.wd[3], f.wd[2], 16);
    c1 = __builtin_amdgcn_alignbit(f.wd[4], f.wd[3], 16);
    sc = f.wd[4] >> 16;
  }
  const bool bad = scale_flags_set<0>(scale_pair_bad<0>(sc));
  uint32_t lo0, hi0, lo1, hi1;
  half_table<0>(sc, bad, fix, lo0, hi0);
  half_table<1>(sc, bad, fix, lo1, hi1);
  uint32_t h0[8], h1[8];
  expand_half_f16(c0, lo0, hi0, h0);
  expand_half_f16(c1, lo1, hi1, h1);
  uint4* dst = reinterpret_cast<uint4*>(st.wh + wrow * kRowBytes + blk * 64);
  dst[0] = make_uint4(h0[0], h0[1], h0[2], h0[3]);
  dst[1] = make_uint4(h0[4], h0[5], h0[6], h0[7]);
  dst[2] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
  dst[3] = make_uint4(h1[4], h1[5], h1[6], h1[7]);

  const int arow = tid >> 1, ablk = tid & 1;
  uint4* adst = reinterpret_cast<uint4*>(st.ah + arow * kRowBytes + ablk * 64);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t X[4] = {f.a[h].x, f.a[h].y, f.a[h].z, f.a[h].w};
    uint32_t o[8];
    act_half_f16(X, o);
    adst[2 * h] = make_uint4(o[0], o[1], o[2], o[3]);
    adst[2 * h + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
  st.ad[ablk][arow] = f.d;
}

__global__ __launch_bounds__(256, 2) void gemm_f16_kernel(
    const uint8_t* __restrict__ w, int N, int K, const int8_t* __restrict__ q,
    const float* __restrict__ d, int M, float* __restrict__ y, int m_tiles,
    int tiles) {
  __shared__ StageF16 sm[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  int tile = blockIdx.x;
  if (tiles % kXcds == 0) tile = (blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
  const int mt = tile % m_tiles;
  const int nt = tile / m_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int64_t row_bytes = (int64_t)(K / 32) * 10;
  const int nb = K / 32;
  const int stages = nb / BKB;
  const float fix = scale_fix();

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  PrefetchF16 f;
  fetch(f, w, q, d, row_bytes, K, nb, 0, tid, n0, m0, N, M);
  const int koff = 16 * (lane >> 5);            // bytes: 8 fp16 per lane half
  for (int s = 0; s < stages; ++s) {
    StageF16& st = sm[s & 1];
    stage_to_lds(f, st, tid, fix);
    if (s + 1 < stages) fetch(f, w, q, d, row_bytes, K, nb, (s + 1) * BKB, tid, n0, m0, N, M);
    __syncthreads();

#pragma unroll
    for (int blk = 0; blk < BKB; ++blk) {
      v8h a[2][2], b[2][2];                     // [half][tile]
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          a[h][t] = *reinterpret_cast<const v8h*>(
              st.ah + (wm * 64 + t * 32 + (lane & 31)) * kRowBytes + blk * 64 + h * 32 + koff);
          b[h][t] = *reinterpret_cast<const v8h*>(
              st.wh + (wn * 64 + t * 32 + (lane & 31)) * kRowBytes + blk * 64 + h * 32 + koff);
        }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        float dd[16];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float4 dv = *reinterpret_cast<const float4*>(
              &st.ad[blk][wm * 64 + tm * 32 + 8 * p + 4 * (lane >> 5)]);
          dd[4 * p + 0] = dv.x;
          dd[4 * p + 1] = dv.y;
          dd[4 * p + 2] = dv.z;
          dd[4 * p + 3] = dv.w;
        }
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          v16f c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0][tm], b[0][tn], v16f{}, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[1][tm], b[1][tn], c, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[tm][tn][r] = fmaf(dd[r], c[r], acc[tm][tn][r]);
        }
      }
    }
  }

#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      const int n = n0 + wn * 64 + tn * 32 + (lane & 31);
      if (n >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + tm * 32 + (r & 3) + 8 * (r >> 2) + 4 * (lane >> 5);
        if (m < M) y[(int64_t)m * N + n] = acc[tm][tn][r];
      }
    }
}

}  // namespace

hipError_t launch_gemm_f16(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                           const float* d, int64_t M, float* y, hipStream_t stream) {
  const int m_tiles = (int)((M + BM - 1) / BM);
  const int n_tiles = (int)((N + BN - 1) / BN);
  const int tiles = m_tiles * n_tiles;
  hipLaunchKernelGGL(gemm_f16_kernel, dim3((uint32_t)tiles), dim3(256), 0, stream, w,
                     (int)N, (int)K, q, d, (int)M, y, m_tiles, tiles);
  return hipGetLastError();
}

}  // namespace rfp2
