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

// The fp16 lookup table of one half, from its UE4M3 scale byte (byte BYTE of
// `word`).  h: fp16(s) in its low 16 bits, from gfx950's scaled fp8 -> fp16
// convert (OCP E4M3FN of the byte is 2s; a scale of 0.5, a power of two, is
// applied exactly); checked over every byte at every byte position.  T: the
// high bytes of -4s, -s, s, 4s (bytes 0..3, indexed by the 2-bit code),
// from fp16(4s) (the same convert with a scale of 2) and fp16(s) plus the
// sign bits.  All four values have the low byte of fp16(s): 4s only moves
// the exponent, the sign bit is in the high byte, and every level times a
// legal scale is a normal fp16 number or zero.  A block with an illegal
// scale byte (flagged in `bad`) gets NaN high bytes in every entry.
// (The converts write the low 16 bits of their result and keep the high ones
// of the value passed in; only the low two bytes are used, so the scale word
// itself is passed and no register has to be cleared first.)
template <int BYTE>
__device__ __forceinline__ void half_table(uint32_t word, bool bad, uint32_t& h, uint32_t& T) {
  typedef _Float16 h2v __attribute__((ext_vector_type(2)));
  const h2v keep = __builtin_bit_cast(h2v, word);
  h = __builtin_bit_cast(uint32_t,
                         __builtin_amdgcn_cvt_scalef32_f16_fp8(keep, (int)word, 0.5f, BYTE, false));
  const uint32_t h4 = __builtin_bit_cast(
      uint32_t, __builtin_amdgcn_cvt_scalef32_f16_fp8(keep, (int)word, 2.0f, BYTE, false));
  // v_perm: selector bytes 0..3 pick from the second source, 4..7 from the first
  T = __builtin_amdgcn_perm(h4, h, 0x05010105u) | 0x00008080u;
  T = bad ? 0x7E7E7E7Eu : T;
}

// Expand the 16 codes of one half (X: byte j = weights 4j..4j+3, two bits
// each) to 8 dwords of fp16 pairs: dword 2f holds weights f and 8+f, dword
// 2f+1 weights 4+f and 12+f (f = 0..3).  A dword's byte selector carries the
// two codes in bytes 1 and 3 and, in bytes 0 and 2, the index (4) of h's
// byte 0, the low byte shared by all four levels; one byte permute then
// builds both fp16 values.  The codes of field f of bytes 1, 3 are X >> 2f;
// those of bytes 0, 2 are X << (8 - 2f): both halves of the 64-bit pair
// (X : X << 8) shifted right by 2f (bits of X that enter the low word's top
// lie above bit 25, outside the mask).
// (x & 0x03000300) | 0x00040004 in one instruction; the compiler emits an
// AND and an OR for it, as both constants are literals.
__device__ __forceinline__ uint32_t code_selector(uint32_t x) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(0x03000300u), "v"(0x00040004u));
  return r;
}

__device__ __forceinline__ void expand_half_f16(uint32_t X, uint32_t h, uint32_t T,
                                                uint32_t (&out)[8]) {
  const uint64_t V = ((uint64_t)X << 32) | (uint64_t)(X << 8);
  const uint64_t S[4] = {V, shr64<2>(V), shr64<4>(V), shr64<6>(V)};
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const uint32_t lo = code_selector((uint32_t)S[f]);
    const uint32_t hi = code_selector((uint32_t)(S[f] >> 32));
    out[2 * f] = __builtin_amdgcn_perm(h, T, lo);
    out[2 * f + 1] = __builtin_amdgcn_perm(h, T, hi);
  }
}

// Position e (0..15) of expand_half_f16's output (dword e / 2, low fp16 for
// even e) holds weight f16_weight_of(e) of the half.
__device__ __forceinline__ int f16_weight_of(int e) {
  return (e >> 2) + 8 * (e & 1) + 4 * ((e >> 1) & 1);
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// Two int8 activations -> one dword of two exact fp16 values: byte j of Xa
// (low) and byte j of Xb (high).  The byte permute places them (raw two's
// complement) in the low byte of each 16-bit lane with a zero high byte;
// flipping bit 7 gives a + 128 in 0..255 and setting the exponent bits
// 0x6400 makes that the fp16 number 1024 + a + 128 (fp16 has unit spacing on
// [1024, 2048)): one XOR with 0x64806480 does both, as the high bytes are
// zero.  One packed subtraction of 1152 leaves a, exactly.
__device__ __forceinline__ uint32_t act_pair_f16(uint32_t Xa, uint32_t Xb, int j) {
  const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
  const uint32_t t = __builtin_amdgcn_perm(Xb, Xa, sel) ^ 0x64806480u;
  const h2 v = __builtin_bit_cast(h2, t) - h2{(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(uint32_t, v);
}

// 16 int8 activations of one half (natural order, 4 words) -> 8 dwords of
// fp16 pairs in the order of expand_half_f16 (dword 2f: activations f, 8+f;
// dword 2f+1: 4+f, 12+f).
__device__ __forceinline__ void act_half_f16(const uint32_t (&X)[4], uint32_t (&out)[8]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    out[2 * f] = act_pair_f16(X[0], X[2], f);
    out[2 * f + 1] = act_pair_f16(X[1], X[3], f);
  }
}

// Dense form: block blk (0 or 1) of the dword-aligned 20-byte pair of blocks
// wd[0..4], both halves expanded to fp16 in the order of expand_half_f16.
// Block 0 of the pair is dwords 0..2 (scales in the low half of dword 2),
// block 1 starts 16 bits into dword 2; selects and funnel shifts, no branch.
// An illegal scale byte in the block makes both of its halves NaN.
__device__ __forceinline__ void decode_pair_block_f16(const uint32_t (&wd)[5], int blk,
                                                      uint32_t (&h0)[8], uint32_t (&h1)[8]) {
  const uint32_t sh = 16u * (uint32_t)blk;
  const uint32_t c0 = __builtin_amdgcn_alignbit(wd[3], blk ? wd[2] : wd[0], sh);
  const uint32_t c1 = __builtin_amdgcn_alignbit(wd[4], blk ? wd[3] : wd[1], sh);
  const uint32_t sc = (blk ? wd[4] : wd[2]) >> sh;
  const bool bad = scale_flags_set<0>(scale_pair_bad<0>(sc));
  uint32_t f0, t0, f1, t1;
  half_table<0>(sc, bad, f0, t0);
  half_table<1>(sc, bad, f1, t1);
  expand_half_f16(c0, f0, t0, h0);
  expand_half_f16(c1, f1, t1, h1);
}

// The 20-byte pair of blocks (2p, 2p + 1) of one weight row (named fields:
// no indexing, which would put them in scratch memory).
struct WPair {
  uint32_t d0, d1, d2, d3, d4;
};

// Routed form: this lane's half (kh) of block ODD of a pair, decoded to the
// two MFMA A operands (steps 0 and 1) of the block: a0 holds positions 0..7
// of expand_half_f16's order, a1 positions 8..15.
template <int ODD>
__device__ __forceinline__ void decode_half(const WPair& w, int kh, v8h& a0, v8h& a1) {
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
  uint32_t h, T;
  half_table<0>(sc >> (8 * kh), bad, h, T);
  uint32_t o[8];
  expand_half_f16(X, h, T, o);
  a0 = __builtin_bit_cast(v8h, make_uint4(o[0], o[1], o[2], o[3]));
  a1 = __builtin_bit_cast(v8h, make_uint4(o[4], o[5], o[6], o[7]));
}

}  // namespace rfp2
