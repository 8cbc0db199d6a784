// fp16 decode of ROCmFP2 blocks for the fp16 matrix-core products
// (rfp2_gemm_f16's dense kernel and rfp2_moe_gemm's routed kernel), shared
// with the inspection kernels so that they expose exactly what the products
// compute.
//
// "ROCmFP2 codebook research report", "02 · Quantization": a weight is its
// level (-4, -1, +1, +4) times the UE4M3 scale of its half.  Every such
// product (at most 4 significant bits, 2^-10 .. 896) and every int8
// activation is exactly an fp16 number.
#pragma once

#include "rfp2_device.h"

namespace rfp2 {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));

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

// Dense form: block blk (0 or 1) of the dword-aligned 20-byte pair of blocks
// wd[0..4], both halves expanded to fp16 in the k order of expand_half_f16.
// Block 0 of the pair is dwords 0..2 (scales in the low half of dword 2),
// block 1 starts 16 bits into dword 2; selects and funnel shifts, no branch.
// An illegal scale byte in the block makes both of its halves NaN.
__device__ __forceinline__ void decode_pair_block_f16(const uint32_t (&wd)[5], int blk, float fix,
                                                      uint32_t (&h0)[8], uint32_t (&h1)[8]) {
  const uint32_t sh = 16u * (uint32_t)blk;
  const uint32_t c0 = __builtin_amdgcn_alignbit(wd[3], blk ? wd[2] : wd[0], sh);
  const uint32_t c1 = __builtin_amdgcn_alignbit(wd[4], blk ? wd[3] : wd[1], sh);
  const uint32_t sc = (blk ? wd[4] : wd[2]) >> sh;
  const bool bad = scale_flags_set<0>(scale_pair_bad<0>(sc));
  uint32_t lo0, hi0, lo1, hi1;
  half_table<0>(sc, bad, fix, lo0, hi0);
  half_table<1>(sc, bad, fix, lo1, hi1);
  expand_half_f16(c0, lo0, hi0, h0);
  expand_half_f16(c1, lo1, hi1, h1);
}

// The 20-byte pair of blocks (2p, 2p + 1) of one weight row (named fields:
// no indexing, which would put them in scratch memory).
struct WPair {
  uint32_t d0, d1, d2, d3, d4;
};

// Routed form: this lane's half (kh) of block ODD of a pair, decoded to the
// two MFMA A operands (steps 0 and 1) of the block: a0 holds the half's k
// order positions 0..7, a1 positions 8..15.
template <int ODD>
__device__ __forceinline__ void decode_half(const WPair& w, int kh, float fix, v8h& a0,
                                            v8h& a1) {
  uint32_t x0, x1, sc;
  if constexpr (ODD) {
    x0 = __builtin_amdgcn_alignbit(w.d3, w.d2, 16);
    x1 = __builtin_amdgcn_alignbit(w.d4, w.d3, 16);
    sc = w.d4 >> 16;
  } else {
    x0 = w.d0;
    x1 = w.d1;
    sc = w.d2 & 0xFFFFu;
  }
  const bool bad = scale_flags_set<0>(scale_pair_bad<0>(sc));
  const uint32_t X = kh ? x1 : x0;
  uint32_t lo, hi;
  half_table<0>(kh ? sc >> 8 : sc, bad, fix, lo, hi);
  uint32_t o[8];
  expand_half_f16(X, lo, hi, o);
  a0 = __builtin_bit_cast(v8h, make_uint4(o[0], o[1], o[2], o[3]));
  a1 = __builtin_bit_cast(v8h, make_uint4(o[4], o[5], o[6], o[7]));
}

}  // namespace rfp2
