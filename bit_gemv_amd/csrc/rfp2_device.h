// Device building blocks shared by every ROCmFP2 kernel of this library
// (gfx950 / CDNA4, wave64).
//
// Format and arithmetic: "ROCmFP2 codebook research report" (llm.ciru.ai),
//   "01 · Storage"      block = 8 code bytes (weight 4j+i in bits 2i..2i+1 of
//                       byte j) + scale byte of weights 0..15 + scale byte of
//                       weights 16..31;
//   "02 · Quantization" codes 00/01/10/11 -> -4/-1/+1/+4; UE4M3 scale bytes;
//   "03 · Runtime"      byte -> four int8 lanes through a byte permute of the
//                       four-level constant, four-lane int8 dot into int32 per
//                       half, scales applied after the integer sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rfp2 {

// The four levels -4, -1, +1, +4 as the bytes of one word: a byte selector
// equal to the 2-bit code picks the level.
constexpr uint32_t kLevels = 0x0401FFFCu;
constexpr uint32_t kLow2 = 0x03030303u;

// Expand the four code bytes of one 16-weight half (X: byte j = weights
// 4j..4j+3) into four int8x4 words.  Word i holds the weights i, 4+i, 8+i and
// 12+i in its bytes 0..3: shifting X right by 2i and keeping the low two bits
// of every byte gives four selectors at once, and one byte permute turns them
// into levels.  Activations are fed in the same lane order (see
// transpose_half), so no weight ever has to be moved into natural order.
__device__ __forceinline__ void expand_half(uint32_t X, uint32_t (&W)[4]) {
  W[0] = __builtin_amdgcn_perm(kLevels, kLevels, X & kLow2);
  W[1] = __builtin_amdgcn_perm(kLevels, kLevels, (X >> 2) & kLow2);
  W[2] = __builtin_amdgcn_perm(kLevels, kLevels, (X >> 4) & kLow2);
  W[3] = __builtin_amdgcn_perm(kLevels, kLevels, (X >> 6) & kLow2);
}

// Both halves of one block at once: C0, C1 are the two halves' code words.
// The shifts by 2, 4 and 6 are taken on the 64-bit pair C1:C0, one
// instruction for both halves (bits of C1 that enter the top of the low
// word are above every byte's low two bits and are masked off).  The compiler
// splits a 64-bit shift whose halves are used separately into two 32-bit
// ones, so the shift is written as asm.
template <int N>
__device__ __forceinline__ uint64_t shr64(uint64_t x) {
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "I"(N), "v"(x));
  return r;
}
__device__ __forceinline__ void expand_block(uint32_t C0, uint32_t C1, uint32_t (&W0)[4],
                                             uint32_t (&W1)[4]) {
  const uint64_t C = ((uint64_t)C1 << 32) | C0;
  W0[0] = __builtin_amdgcn_perm(kLevels, kLevels, C0 & kLow2);
  W1[0] = __builtin_amdgcn_perm(kLevels, kLevels, C1 & kLow2);
  const uint64_t S2 = shr64<2>(C), S4 = shr64<4>(C), S6 = shr64<6>(C);
  W0[1] = __builtin_amdgcn_perm(kLevels, kLevels, (uint32_t)S2 & kLow2);
  W1[1] = __builtin_amdgcn_perm(kLevels, kLevels, (uint32_t)(S2 >> 32) & kLow2);
  W0[2] = __builtin_amdgcn_perm(kLevels, kLevels, (uint32_t)S4 & kLow2);
  W1[2] = __builtin_amdgcn_perm(kLevels, kLevels, (uint32_t)(S4 >> 32) & kLow2);
  W0[3] = __builtin_amdgcn_perm(kLevels, kLevels, (uint32_t)S6 & kLow2);
  W1[3] = __builtin_amdgcn_perm(kLevels, kLevels, (uint32_t)(S6 >> 32) & kLow2);
}

// 4x4 byte transpose of the 16 int8 activations of one half: X[j] holds
// a[4j..4j+3] in natural order; A[i] = (a[i], a[4+i], a[8+i], a[12+i]), the
// lane order expand_half produces for the weights.
__device__ __forceinline__ void transpose_half(const uint32_t (&X)[4],
                                               uint32_t (&A)[4]) {
  // v_perm: selector byte 0..3 picks from the second source, 4..7 from the first
  const uint32_t lo01 = __builtin_amdgcn_perm(X[1], X[0], 0x05010400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(X[1], X[0], 0x07030602u);
  const uint32_t lo23 = __builtin_amdgcn_perm(X[3], X[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(X[3], X[2], 0x07030602u);
  A[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  A[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  A[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  A[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// First dot of a chain: v_dot4_i32_i8 with an inline-constant zero
// accumulator (the builtin with a zero accumulator becomes a v_mov of zero
// plus the accumulating dot4c form: one extra VALU op per chain).
__device__ __forceinline__ int32_t dot4_from_zero(uint32_t a, uint32_t b) {
  int32_t r;
  asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// int32 sum of one 16-weight half: four 4-lane int8 dot products.
__device__ __forceinline__ int32_t half_dot(const uint32_t (&W)[4],
                                            const uint32_t* A) {
  int32_t s = dot4_from_zero(W[0], A[0]);
  s = __builtin_amdgcn_sdot4((int)W[1], (int)A[1], s, false);
  s = __builtin_amdgcn_sdot4((int)W[2], (int)A[2], s, false);
  s = __builtin_amdgcn_sdot4((int)W[3], (int)A[3], s, false);
  return s;
}

// ---------------------------------------------------------------------------
// UE4M3 scale bytes.
//
// A legal byte b = E:M (E = b >> 3, M = b & 7) is M * 2^-10 for E == 0 and
// (8 + M) * 2^(E - 11) otherwise.  That is the E4M3 layout with exponent bias
// 8, so the hardware fp8 -> fp32 convert of the same byte gives the scale
// times a fixed power of two (1 for a bias-8 convert, 2 for the OCP bias-7
// convert).  The kernels convert with the hardware instruction (one op per
// scale, exact) and multiply the finished sums by `scale_fix()`, computed
// once per thread from the convert of 0x38 (scale 0.5).  A byte outside
// 0x00..0x7E is flagged by `scale_pair_bad` and turns the result into NaN.
// ---------------------------------------------------------------------------
template <int BYTE>
__device__ __forceinline__ float fp8_byte(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, BYTE);
}

// Bytes 0,1 (HI = false) or 2,3 (HI = true) of `word` as two fp8 values.
template <bool HI>
__device__ __forceinline__ float2 fp8_pair(uint32_t word) {
  typedef float v2f __attribute__((ext_vector_type(2)));
  const v2f v = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
  return make_float2(v.x, v.y);
}

__device__ __forceinline__ float scale_fix() {
  return fp8_byte<0>(0x38u) > 0.75f ? 0.5f : 1.0f;
}

// Bits 7 / 15 (pair in the low half) of the result are set when a byte of
// the pair is 0x7F or above.  Adding 1 to each byte turns 0x7F into 0x80; the
// OR with the bytes themselves catches 0x80..0xFF.  For a pair in the high
// half (bytes 2, 3) use HI = 1: the flags then sit in bits 23 / 31.
template <int HI>
__device__ __forceinline__ uint32_t scale_pair_bad(uint32_t word) {
  return word | (word + (HI ? 0x01010000u : 0x00000101u));
}
template <int HI>
__device__ __forceinline__ bool scale_flags_set(uint32_t acc) {
  return (acc & (HI ? 0x80800000u : 0x00008080u)) != 0u;
}

// One scale byte (0..255) is illegal when it is 0x7F or above.
__device__ __forceinline__ bool scale_byte_bad(uint32_t b) {
  return ((b | (b + 1u)) & 0x80u) != 0u;
}

// Rounding-exact decode used by the weight quantizer (fp64).
__device__ __forceinline__ double ue4m3_f64(int b) {
  const int E = b >> 3, M = b & 7;
  return E == 0 ? (double)M * 0x1p-10 : ldexp((double)(8 + M), E - 11);
}

}  // namespace rfp2
