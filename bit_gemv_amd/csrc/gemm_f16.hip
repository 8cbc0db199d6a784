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
  // bit-or with a quiet NaN pattern instead of a select: no branch
  const float s = __uint_as_float(__float_as_uint(fp8_byte<BYTE>(word) * fix) |
                                  (bad ? 0x7FC00000u : 0u));
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

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Two int8 activations -> one dword of two exact fp16 values.  The byte
// permute places a0 and a1 (raw two's-complement bytes) in the low byte of
// each 16-bit lane; flipping bit 7 gives a + 128 in 0..255, and setting the
// exponent bits 0x6400 makes that the fp16 number 1024 + a + 128 (fp16 has
// unit spacing on [1024, 2048)); one packed subtraction of 1152 leaves a,
// exactly.
__device__ __forceinline__ uint32_t act_pair_f16(uint32_t X0, uint32_t X1, int j) {
  const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
  const uint32_t t = (__builtin_amdgcn_perm(X1, X0, sel) ^ 0x00800080u) | 0x64006400u;
  const h2 v = __builtin_bit_cast(h2, t) - h2{(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, v);
}

// 16 int8 activations of one half (natural order, 4 words) -> 8 dwords of
// fp16 pairs in the same k order as expand_half_f16.
__device__ __forceinline__ void act_half_f16(const uint32_t (&X)[4], uint32_t (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = act_pair_f16(X[0], X[1], j);
    out[4 + j] = act_pair_f16(X[2], X[3], j);
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
  // block 0 of the pair is dwords 0..2 (scales in the low half of dword 2),
  // block 1 starts 16 bits into dword 2; selects and funnel shifts, no branch
  const uint32_t sh = 16u * (uint32_t)blk;
  const uint32_t c0 = __builtin_amdgcn_alignbit(f.wd[3], blk ? f.wd[2] : f.wd[0], sh);
  const uint32_t c1 = __builtin_amdgcn_alignbit(f.wd[4], blk ? f.wd[3] : f.wd[1], sh);
  const uint32_t sc = (blk ? f.wd[4] : f.wd[2]) >> sh;
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

// Block sums of the stage in sm for this wave's 64 x 64 (row x token) tile,
// rescaled by the activation scales and added to acc.  MFMA operand A is the
// weights (i = row), B the activations (j = token), so every lane holds one
// token's column of each 32 x 32 tile and the activation scale of a block is
// one register per tile.
__device__ __forceinline__ void compute_stage(const StageF16& st, int lane, int wm, int wn,
                                              v16f (&acc)[2][2]) {
  const int koff = 16 * (lane >> 5);            // bytes: 8 fp16 per lane half
#pragma unroll
  for (int blk = 0; blk < BKB; ++blk) {
    v8h a[2][2], b[2][2];                       // [half][tile]
    float dd[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        a[h][t] = *reinterpret_cast<const v8h*>(
            st.wh + (wn * 64 + t * 32 + (lane & 31)) * kRowBytes + blk * 64 + h * 32 + koff);
        b[h][t] = *reinterpret_cast<const v8h*>(
            st.ah + (wm * 64 + t * 32 + (lane & 31)) * kRowBytes + blk * 64 + h * 32 + koff);
      }
      dd[t] = st.ad[blk][wm * 64 + t * 32 + (lane & 31)];
    }
    // all four tiles' block sums first, then the rescale, so that the FMAs
    // of a tile do not wait on the matrix-core latency of that same tile
    v16f c[2][2];
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int tm = 0; tm < 2; ++tm) {
        c[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[0][tn], b[0][tm], v16f{}, 0, 0, 0);
        c[tn][tm] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[1][tn], b[1][tm], c[tn][tm], 0, 0, 0);
      }
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tn][tm][r] = fmaf(dd[tm], c[tn][tm][r], acc[tn][tm][r]);
  }
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

  v16f acc[2][2];                               // [row tile][token tile]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  // Software pipeline: iteration s computes stage s from one LDS buffer while
  // it expands stage s+1 (already in registers) into the other buffer and
  // loads stage s+2 from memory; a single barrier ends the iteration.  The
  // buffer written in iteration s was last read in iteration s-1, before the
  // barrier that ended it.  The loop body has no branch (the last stage is
  // peeled off and the load of a stage past the end re-reads the last one),
  // so the matrix-core and vector work of an iteration can be interleaved.
  PrefetchF16 f;
  fetch(f, w, q, d, row_bytes, K, nb, 0, tid, n0, m0, N, M);
  stage_to_lds(f, sm[0], tid, fix);
  fetch(f, w, q, d, row_bytes, K, nb, stages > 1 ? BKB : 0, tid, n0, m0, N, M);
  __syncthreads();
  for (int s = 0; s + 1 < stages; ++s) {
    compute_stage(sm[s & 1], lane, wm, wn, acc);
    stage_to_lds(f, sm[(s + 1) & 1], tid, fix);
    const int next = s + 2 < stages ? s + 2 : stages - 1;
    fetch(f, w, q, d, row_bytes, K, nb, next * BKB, tid, n0, m0, N, M);
    __syncthreads();
  }
  compute_stage(sm[(stages - 1) & 1], lane, wm, wn, acc);

  // lane -> token m, register r -> row n; rows n..n+3 of a register group are
  // contiguous in y, so whole groups go out as one 16-byte store
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
#pragma unroll
  for (int tn = 0; tn < 2; ++tn)
#pragma unroll
    for (int tm = 0; tm < 2; ++tm) {
      const int m = m0 + wm * 64 + tm * 32 + (lane & 31);
      if (m >= M) continue;
      float* yr = y + (int64_t)m * N;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 64 + tn * 32 + 8 * g + 4 * (lane >> 5);
        const v16f& v = acc[tn][tm];
        if (vec && n + 3 < N) {
          *reinterpret_cast<float4*>(yr + n) =
              make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) yr[n + e] = v[4 * g + e];
        }
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
