// Kernel template of the ROCmFP2 GEMV (the design notes are in gemv.hip).
#pragma once

#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {
namespace gemv_detail {

// Activations of one (column, 8-block group) in LDS: 16 pieces of 16 bytes
// (each the 16 int8 of one half, transposed) and one pad piece, so that the
// L lanes of a row, which read L consecutive groups, hit different banks.
constexpr int kGroupPieces = 17;
constexpr int kGroupDwords = 4 * kGroupPieces;
constexpr int kMaxLdsBytes = 65536;  // LDS budget per workgroup (dense GEMV)
constexpr int kMaxLdsBytesPerBlock = 163840;  // gfx950: 160 KiB per workgroup
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
  const int32_t* ids;   // routed experts (MoE form) or null: one per slot
  int E;
  int32_t* err;
  int top_k;            // MoE form: slots per token (slot s belongs to token s / top_k)
  int S;                // MoE form: number of slots
  const float* a;       // fp32 activations (quantizing form) or null
  int8_t* qo;           // quantizing form: q and d written by workgroup 0
  float* dout;
};

// Decode block jb (0..7) of an 80-byte group held in registers: the eight
// int8x4 words of its two halves (expand_block's lane order), both scales
// from one packed fp8 convert (each the UE4M3 value times scale_fix()'s
// inverse), and the dword holding its scale pair (bytes 0,1 for an even
// block, 2,3 for an odd one), whose top bits flag bytes 0x80..0xFF.  gfx950
// converts OCP E4M3FN, where byte 0x7F is NaN, so that byte poisons the
// products by itself.
__device__ __forceinline__ void decode_block(const uint32_t (&dw)[20], int jb,
                                             uint32_t (&W0)[4], uint32_t (&W1)[4],
                                             float& s0, float& s1, uint32_t& sc) {
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
  sc = dw[o + 2];
  expand_block(c0, c1, W0, W1);
  const float2 sp = (jb & 1) ? fp8_pair<true>(sc) : fp8_pair<false>(sc);
  s0 = sp.x;
  s1 = sp.y;
}

// The int32 sums of a block's two halves against one column's activations
// (each half's 16 int8 in the lane order of the expanded weights).
__device__ __forceinline__ void block_half_sums(const uint32_t (&W0)[4], const uint32_t (&W1)[4],
                                                const uint4& A0, const uint4& A1, int32_t& S0,
                                                int32_t& S1) {
  const uint32_t a0[4] = {A0.x, A0.y, A0.z, A0.w};
  const uint32_t a1[4] = {A1.x, A1.y, A1.z, A1.w};
  S0 = half_dot(W0, a0);
  S1 = half_dot(W1, a1);
}

// Block jb of the group against the M columns; acts(m, A0, A1, d) supplies
// column m's activations (two words of 16 int8) and block scale.  Bytes
// 0x80..0xFF of the scale pair are OR-ed into bad_* (bits 7/15 for an even
// block, 23/31 for an odd one).
template <int M, typename Acts>
__device__ __forceinline__ void block_product(const uint32_t (&dw)[20], int jb, Acts acts,
                                              float (&acc)[M], uint32_t& bad_lo,
                                              uint32_t& bad_hi, int ncols) {
  uint32_t W0[4], W1[4], sc;
  float s0, s1;
  decode_block(dw, jb, W0, W1, s0, s1, sc);
  if ((jb & 1) == 0)
    bad_lo |= sc;
  else
    bad_hi |= sc;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (m >= ncols) break;                  // (uniform) unused columns of a group
    uint4 A0, A1;
    float dm;
    acts(m, A0, A1, dm);
    int32_t S0, S1;
    block_half_sums(W0, W1, A0, A1, S0, S1);
    acc[m] = fmaf(dm, fmaf(s1, (float)S1, s0 * (float)S0), acc[m]);
  }
}

// Decode one 80-byte group held in registers and accumulate its product with
// M activation columns.  `act` points at the LDS activations of column 0 for
// this group and `dact` at its 8 block scales; columns are `act_stride` and
// `d_stride` dwords apart.  With AHEAD a block's activations are read from
// LDS one block ahead of its products, so that their latency hides behind
// the previous block's vector work (dense product at 16384 x 5120: M = 1, 2,
// 3, 4 take 2.5, 5.5, 5 and 7 % less time); otherwise each block reads its
// activations where it uses them.  The extra registers cost waves per SIMD:
// the dense M = 8 product was 15 % slower with it, the routed-token product
// (128 experts of 1536 x 4096, top-8) 14 % at T = 2 and 30 % at T = 4.
template <int M, bool AHEAD>
__device__ __forceinline__ void group_product(const uint32_t (&dw)[20],
                                              const uint32_t* act, int act_stride,
                                              const float* dact, int d_stride,
                                              float (&acc)[M], uint32_t& bad_lo,
                                              uint32_t& bad_hi, int ncols = M) {
  auto load = [&](int jb, int m, uint4& A0, uint4& A1, float& dm) {
    const uint32_t* a = act + m * act_stride + jb * 8;
    A0 = *reinterpret_cast<const uint4*>(a);
    A1 = *reinterpret_cast<const uint4*>(a + 4);
    dm = dact[m * d_stride + jb];
  };
  if constexpr (AHEAD) {
    uint4 nA0[M], nA1[M];
    float nd[M];
    auto fetch = [&](int jb) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (m >= ncols) break;
        load(jb, m, nA0[m], nA1[m], nd[m]);
      }
    };
    fetch(0);
#pragma unroll
    for (int jb = 0; jb < 8; ++jb) {
      uint4 A0[M], A1[M];
      float dd[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        A0[m] = nA0[m];
        A1[m] = nA1[m];
        dd[m] = nd[m];
      }
      if (jb < 7) fetch(jb + 1);
      block_product<M>(dw, jb, [&](int m, uint4& a0, uint4& a1, float& dm) {
        a0 = A0[m];
        a1 = A1[m];
        dm = dd[m];
      }, acc, bad_lo, bad_hi, ncols);
    }
  } else {
#pragma unroll
    for (int jb = 0; jb < 8; ++jb)
      block_product<M>(dw, jb, [&](int m, uint4& a0, uint4& a1, float& dm) {
        load(jb, m, a0, a1, dm);
      }, acc, bad_lo, bad_hi, ncols);
  }
}

// Matrix-core form of group_product for two to eight columns.  The int32 half
// sums come from v_mfma_i32_4x4x4_16b_i8 instead of the lane's own dot4
// chains: the instruction is sixteen independent 4x4x4 products, one per
// quad of lanes (lanes 4q..4q+3); in quad q, lane 4q+i supplies row i of A
// (four int8 along k) and lane 4q+j column j of B, and lane 4q+j receives
// D[i][j] in its register i.  Here the four lanes of a quad are four weight
// rows at the same group, B is each lane's own expanded weight word, and A
// is column i's activation word (lane 4q+i reads column i), so lane 4q+j
// gets its own row's sums for all four columns, one per register.  Four
// steps over the words i = 0..3 of a half (weights i, 4+i, 8+i, 12+i, the
// activations transposed to match) accumulate the half's int32 sum: the
// same integers as half_dot, so the outputs are bit for bit those of
// group_product.  `act0` points at this lane's column's activations of the
// group (column lane % 4), `act1` at those of column 4 + lane % 4 (five to
// eight columns: a second quad of columns, a second set of products), and
// `dact` at the group's block scales laid out [block][column] with four or
// eight column slots per block.  Column slots past M compute unused sums.
typedef int v4i __attribute__((ext_vector_type(4)));

// `start` is the accumulator's initial value (zero, or the bias below).
__device__ __forceinline__ v4i half_sums_mf(const uint32_t (&W)[4], const uint4& A,
                                            v4i start = v4i{0, 0, 0, 0}) {
  v4i s = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A.x, (int)W[0], start, 0, 0, 0);
  s = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A.y, (int)W[1], s, 0, 0, 0);
  s = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A.z, (int)W[2], s, 0, 0, 0);
  s = __builtin_amdgcn_mfma_i32_4x4x4i8((int)A.w, (int)W[3], s, 0, 0, 0);
  return s;
}

// NQL: quads of column slots per block in the scale array (may exceed the
// quads this call computes: a routed group of at most four columns in a
// launch for more runs the first quad only).
template <int M, int NQL = (M + 3) / 4>
__device__ __forceinline__ void group_product_mf(const uint32_t (&dw)[20], const uint32_t* act0,
                                                 const uint32_t* act1, const float* dact,
                                                 float (&acc)[M], uint32_t& bad_lo,
                                                 uint32_t& bad_hi) {
  static_assert(M >= 2 && M <= 8, "one or two quads of columns");
  constexpr int NQ = (M + 3) / 4;         // quads of columns: act0 = columns 0..3, act1 4..7
  static_assert(NQL >= NQ, "the scale array holds every computed quad");
  const uint32_t* act[2] = {act0, act1};
  auto load = [&](int jb, uint4 (&A0)[NQ], uint4 (&A1)[NQ], float4 (&d4)[NQ]) {
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      A0[u] = *reinterpret_cast<const uint4*>(act[u] + jb * 8);
      A1[u] = *reinterpret_cast<const uint4*>(act[u] + jb * 8 + 4);
      d4[u] = *reinterpret_cast<const float4*>(dact + (jb * NQL + u) * 4);
    }
  };
  // a block's activations are read one block ahead of its products
  uint4 nA0[NQ], nA1[NQ];
  float4 nd[NQ];
  load(0, nA0, nA1, nd);
#pragma unroll
  for (int jb = 0; jb < 8; ++jb) {
    uint4 A0[NQ], A1[NQ];
    float4 d4[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      A0[u] = nA0[u];
      A1[u] = nA1[u];
      d4[u] = nd[u];
    }
    if (jb < 7) load(jb + 1, nA0, nA1, nd);
    uint32_t W0[4], W1[4], sc;
    float s0, s1;
    decode_block(dw, jb, W0, W1, s0, s1, sc);
    if ((jb & 1) == 0)
      bad_lo |= sc;
    else
      bad_hi |= sc;
    // half 0's sums start from the int32 bit pattern of fp32 1.5 * 2^23, so
    // read as fp32 they are exactly 1.5 * 2^23 + S0 (|S0| <= 16 * 4 * 127 <
    // 2^22) and s0 * S0 = fma(s0, that, -1.5 * 2^23 * s0) is one exact
    // instruction (s0 has at most 4 significant bits, s0 * S0 at most 17):
    // the value the convert and the multiply give, one instruction fewer
    v4i S0[NQ], S1[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      S0[u] = half_sums_mf(W0, A0[u], v4i{0x4B400000, 0x4B400000, 0x4B400000, 0x4B400000});
      S1[u] = half_sums_mf(W1, A1[u]);
    }
    const float nb0 = -12582912.0f * s0;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int u = m >> 2, i = m & 3;
      const float dm = i == 0 ? d4[u].x : i == 1 ? d4[u].y : i == 2 ? d4[u].z : d4[u].w;
      acc[m] = fmaf(dm, fmaf(s1, (float)S1[u][i], fmaf(s0, __int_as_float(S0[u][i]), nb0)),
                    acc[m]);
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
    o.off[k] = (int)__umul24((uint32_t)rr, (uint32_t)row_bytes) + col * 16;  // both < 2^24
  }
  return o;
}

// Direct-to-LDS loads, written as inline asm so that every wait on them is
// the kernel's own: the compiler cannot tell which LDS bytes such a load
// writes, so for its own form of the instruction it waits for all of them to
// land before any LDS access and before using any earlier global load --
// which would hold every weight read behind the activation staging and keep
// the chunk ring from overlapping loads with compute.  Lane l of a 16-byte
// load writes LDS bytes [m0 + 16 l, m0 + 16 l + 16); of a 4-byte load,
// [m0 + 4 l, m0 + 4 l + 4).  m0 must be wave-uniform.  No global load in
// this kernel is visible to the compiler, so it inserts no vmcnt wait of its
// own; the s_nop covers the m0-write -> LDS-DMA hazard.  m0 is a register
// the compiler reserves and sets right before each of its own uses (it
// ignores it in a clobber list); nothing else in this kernel reads it.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(m0v) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t m0v) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(base), "s"(m0v) : "memory");
}

// Byte address of an LDS location (the form m0 takes), made wave-uniform.
__device__ __forceinline__ uint32_t lds_m0(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// One chunk: five 16-byte loads into the 5 KB at LDS byte address m0v.
__device__ __forceinline__ void load_chunk(const uint8_t* base, const ChunkOffsets& o,
                                           uint32_t m0v) {
#pragma unroll
  for (int k = 0; k < 5; ++k) dma16(base, (uint32_t)o.off[k], m0v + 1024 * k);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Quantizing form: the lane's 16 fp32 activations (64 bytes at abase + aoff)
// into registers, a workgroup barrier (every wave's activation loads are
// then queued ahead of the workgroup's weight loads: a compute unit returns
// vector loads in order, so an activation load, an L2 hit, issued after other
// waves' weight loads waits for their HBM data; one token at 16384 x 5120,
// 4096 x 4096, 4096 x 14336, 512 x 2048, alternating timings: 8.32, 4.29,
// 7.52, 4.03 -> 8.11, 4.07, 7.08, 3.88 us), then one weight chunk (as
// load_chunk), then a wait for the activations only.  One asm statement, so
// that the registers the loads fill are not touched before the wait (the
// outputs are early-clobber: no input shares a register with them while the
// loads are in flight).  Every wave of the workgroup runs it exactly once.
__device__ __forceinline__ void load_acts_and_chunk(const float* abase, uint32_t aoff,
                                                    const uint8_t* wbase, const ChunkOffsets& o,
                                                    uint32_t m0v, v4f (&x)[4]) {
  asm volatile(
      "global_load_dwordx4 %0, %4, %5\n\t"
      "global_load_dwordx4 %1, %4, %5 offset:16\n\t"
      "global_load_dwordx4 %2, %4, %5 offset:32\n\t"
      "global_load_dwordx4 %3, %4, %5 offset:48\n\t"
      "s_barrier\n\t"
      "s_mov_b32 m0, %11\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %12\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, %12\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, %12\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, %12\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, %12\n\t"
      "s_waitcnt vmcnt(5)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(aoff), "s"(abase), "v"(o.off[0]), "v"(o.off[1]), "v"(o.off[2]), "v"(o.off[3]),
        "v"(o.off[4]), "s"(m0v), "s"(wbase)
      : "memory");
}

// The same for two halves per lane: 2 x 16 fp32 activations at abase + aoff0
// and abase + aoff1, the barrier, then the weight chunk, then a wait for the
// activations.
__device__ __forceinline__ void load_acts2_and_chunk(const float* abase, uint32_t aoff0,
                                                     uint32_t aoff1, const uint8_t* wbase,
                                                     const ChunkOffsets& o, uint32_t m0v,
                                                     v4f (&x)[4], v4f (&z)[4]) {
  asm volatile(
      "global_load_dwordx4 %0, %8, %10\n\t"
      "global_load_dwordx4 %1, %8, %10 offset:16\n\t"
      "global_load_dwordx4 %2, %8, %10 offset:32\n\t"
      "global_load_dwordx4 %3, %8, %10 offset:48\n\t"
      "global_load_dwordx4 %4, %9, %10\n\t"
      "global_load_dwordx4 %5, %9, %10 offset:16\n\t"
      "global_load_dwordx4 %6, %9, %10 offset:32\n\t"
      "global_load_dwordx4 %7, %9, %10 offset:48\n\t"
      "s_barrier\n\t"
      "s_mov_b32 m0, %16\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, %17\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, %17\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %13, %17\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %14, %17\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %15, %17\n\t"
      "s_waitcnt vmcnt(5)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(z[0]), "=&v"(z[1]),
        "=&v"(z[2]), "=&v"(z[3])
      : "v"(aoff0), "v"(aoff1), "s"(abase), "v"(o.off[0]), "v"(o.off[1]), "v"(o.off[2]),
        "v"(o.off[3]), "v"(o.off[4]), "s"(m0v), "s"(wbase)
      : "memory");
}

// The routed quantizing form splits the above in two, so that the expert id
// (a scalar load, on which the weight address depends) is awaited only once
// the activation loads are out: first the activation loads alone, then --
// the expert known -- the barrier, the weight chunk and the wait for the
// activations.  The registers the first asm fills are in-out operands of
// the second, so nothing reads them in between.
__device__ __forceinline__ void load_acts(const float* abase, uint32_t aoff, v4f (&x)[4]) {
  asm volatile(
      "global_load_dwordx4 %0, %4, %5\n\t"
      "global_load_dwordx4 %1, %4, %5 offset:16\n\t"
      "global_load_dwordx4 %2, %4, %5 offset:32\n\t"
      "global_load_dwordx4 %3, %4, %5 offset:48"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(aoff), "s"(abase)
      : "memory");
}
__device__ __forceinline__ void load_acts2(const float* abase, uint32_t aoff0, uint32_t aoff1,
                                           v4f (&x)[4], v4f (&z)[4]) {
  asm volatile(
      "global_load_dwordx4 %0, %8, %10\n\t"
      "global_load_dwordx4 %1, %8, %10 offset:16\n\t"
      "global_load_dwordx4 %2, %8, %10 offset:32\n\t"
      "global_load_dwordx4 %3, %8, %10 offset:48\n\t"
      "global_load_dwordx4 %4, %9, %10\n\t"
      "global_load_dwordx4 %5, %9, %10 offset:16\n\t"
      "global_load_dwordx4 %6, %9, %10 offset:32\n\t"
      "global_load_dwordx4 %7, %9, %10 offset:48"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(z[0]), "=&v"(z[1]),
        "=&v"(z[2]), "=&v"(z[3])
      : "v"(aoff0), "v"(aoff1), "s"(abase)
      : "memory");
}
__device__ __forceinline__ void chunk_after_acts(const uint8_t* wbase, const ChunkOffsets& o,
                                                 uint32_t m0v, v4f (&x)[4]) {
  asm volatile(
      "s_barrier\n\t"
      "s_mov_b32 m0, %9\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, %10\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %5, %10\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %6, %10\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %7, %10\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, %10\n\t"
      "s_waitcnt vmcnt(5)"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
      : "v"(o.off[0]), "v"(o.off[1]), "v"(o.off[2]), "v"(o.off[3]), "v"(o.off[4]), "s"(m0v),
        "s"(wbase)
      : "memory");
}
__device__ __forceinline__ void chunk_after_acts2(const uint8_t* wbase, const ChunkOffsets& o,
                                                  uint32_t m0v, v4f (&x)[4], v4f (&z)[4]) {
  asm volatile(
      "s_barrier\n\t"
      "s_mov_b32 m0, %13\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %8, %14\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %9, %14\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %10, %14\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %11, %14\n\t"
      "s_add_u32 m0, m0, 0x400\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %12, %14\n\t"
      "s_waitcnt vmcnt(5)"
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(z[0]), "+v"(z[1]), "+v"(z[2]),
        "+v"(z[3])
      : "v"(o.off[0]), "v"(o.off[1]), "v"(o.off[2]), "v"(o.off[3]), "v"(o.off[4]), "s"(m0v),
        "s"(wbase)
      : "memory");
}

// Quantize the 16 fp32 activations of one half in place of the separate
// activation kernel, with its exact arithmetic: the block's max |a| comes
// from this lane and its partner (the other half of the block, lane ^ 1),
// d = fl32(max / 127) (IEEE division), q = roundf(fl32(a / d)) (halves away
// from zero), d = NaN and q = 0 for a block with a non-finite value, q = 0
// when d = 0, q clamped to +-127.  For a normal d, |a / d| <= 127 * (1 +
// 2^-23) and the clamp never acts; a subnormal d keeps fewer significant
// bits, and a / d reaches up to ~190 when max |a| is below ~2.2e-41.
//   * fl32(a / d) is replaced by t = a * rcp(d); adding 1.5 * 2^23 rounds t
//     to the nearest integer k and leaves k's two's-complement low byte in
//     the low byte of the sum.  Error budget, with |a / d| <= 127 * (1 +
//     2^-23) < 127.00002: rcp is within one ulp (relative error <= 2^-23), so
//     the exact product a * rcp(d) is within 127.00002 * 2^-23 < 1.52e-5 of
//     a / d; rounding the product (the compiler may instead fuse it into the
//     add) moves it by at most half an ulp at 127, 3.9e-6; and fl32(a / d)
//     is within 3.9e-6 of a / d.  So |t - fl32(a / d)| < 2.3e-5 and, when
//     |t - k| < 0.49997 = 0.5 - 3e-5, fl32(a / d) lies strictly within 0.5 of
//     k: k is roundf(fl32(a / d)).
//   * Otherwise (t within 3e-5 of a half-integer), or when d is subnormal,
//     the lane redoes its values with the IEEE division, the clamp and
//     roundf.
// A receives q packed four per dword in the lane order of the expanded
// weights (A[i] = q[i], q[4+i], q[8+i], q[12+i]: packing in that order costs
// the same as packing in natural order and saves the transpose); returns d.
__device__ __forceinline__ uint32_t pack_low_bytes(uint32_t b0, uint32_t b1, uint32_t b2,
                                                   uint32_t b3) {
  // v_perm: selector bytes 0..3 pick from the second source, 4..7 from the
  // first, 0x0C gives zero
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0C0C0400u);
  const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000C0Cu);
  return lo | hi;
}

// max(|x|, |y|, |z|), NaN when any of them is NaN (IEEE 754-2019 maximum;
// the older three-input max drops a quiet NaN operand).
__device__ __forceinline__ float maximum3_abs(float x, float y, float z) {
  float r;
  asm("v_maximum3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(x), "v"(y), "v"(z));
  return r;
}

__device__ __forceinline__ float quantize_half(const v4f (&x)[4], uint32_t (&A)[4]) {
  constexpr float kMagic = 12582912.0f;          // 1.5 * 2^23
  float v[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i] = x[i].x;
    v[4 * i + 1] = x[i].y;
    v[4 * i + 2] = x[i].z;
    v[4 * i + 3] = x[i].w;
  }
  // max |a| with the NaN-propagating three-input maximum (a NaN anywhere
  // gives NaN), then as a bit pattern, where NaN and Inf sort above every
  // finite value, so the same max decides finiteness
  float am = maximum3_abs(v[0], v[1], v[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) am = maximum3_abs(am, v[i], v[i + 1]);
  am = maximum3_abs(am, v[15], v[15]);
  uint32_t amb = __float_as_uint(am);
  amb = max(amb, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amb, 0xB1, 0xF, 0xF, false));
  A[0] = A[1] = A[2] = A[3] = 0u;
  if (amb >= 0x7F800000u) return __builtin_nanf("");
  const float dv = __fdiv_rn(__uint_as_float(amb), 127.0f);
  if (dv == 0.0f) return dv;
  const float inv = __builtin_amdgcn_rcpf(dv);
  bool need_exact = dv < 1.17549435e-38f;
  uint32_t u[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float t = v[i] * inv;
    const float s = t + kMagic;                  // rounds t to an integer
    need_exact |= fabsf(t - (s - kMagic)) > 0.49997f;
    u[i] = __float_as_uint(s);
  }
  if (need_exact) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      u[i] = __float_as_uint(roundf(fminf(fmaxf(__fdiv_rn(v[i], dv), -127.0f), 127.0f)) + kMagic);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) A[i] = pack_low_bytes(u[i], u[4 + i], u[8 + i], u[12 + i]);
  return dv;
}

// Sum of v over the L consecutive lanes of a row (L a power of two); every
// lane of the row receives it.  Up to 16 lanes the steps are DPP moves fused
// into the adds (quad permutes, then half-row and row mirrors: after each
// step all lanes of a 2^i-lane group hold the same value, so a mirror adds
// the partner group's sum); wider rows finish with cross-row shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_sum(float v, int L) {
  if (L >= 2) v += dpp_move<0xB1>(v);     // quad_perm [1,0,3,2]
  if (L >= 4) v += dpp_move<0x4E>(v);     // quad_perm [2,3,0,1]
  if (L >= 8) v += dpp_move<0x141>(v);    // row_half_mirror
  if (L >= 16) v += dpp_move<0x140>(v);   // row_mirror
  if (L >= 32) v += __shfl_xor(v, 16, 64);
  if (L >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// The same for the matrix-core lane order, where the L lanes of a row are 4
// apart (lane bits 2 .. 2 + log2 L): the sum lands in the row's lane t = 0
// (the other lanes hold partial sums).  Row shifts by 4 and 8 inside each
// 16-lane row, then lane shuffles; each step adds the partner group that
// lies above, so the summation tree is row_sum's.
__device__ __forceinline__ float row_sum_mf(float v, int L) {
  if (L >= 2) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104,
                                                               0xF, 0xF, false));  // row_shl:4
  if (L >= 4) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x108,
                                                               0xF, 0xF, false));  // row_shl:8
  if (L >= 8) v += __shfl_down(v, 16, 64);
  if (L >= 16) v += __shfl_down(v, 32, 64);
  return v;
}

// Wait until at most 5*ahead loads (= `ahead` chunks) are outstanding.
__device__ __forceinline__ void wait_chunks(int ahead) {
  switch (ahead) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(20)" ::: "memory"); break;
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
// weight matrix through ids[blockIdx.y].  QH > 0: the quantizing form, each
// lane quantizing QH (1 or 2) halves of the wave's activation slice.  MF:
// the matrix-core form of two to eight columns (group_product_mf), in which
// the four lanes of a quad are four rows at the same group: lane =
// (slot / 4) * 4L + t * 4 + slot % 4, so it needs L <= 16.  A routed group
// with fewer columns than M computes the missing ones from a repeat of its
// last column and does not store them.
template <int M, int JT, bool MOE, int QH, bool MF = false>
__global__ __launch_bounds__(512) void gemv_kernel(Params p) {
  constexpr bool QA = QH > 0;
  static_assert(QH >= 0 && QH <= 2, "one or two halves per lane");
  static_assert(!QA || (M == 1 && JT == 1), "the quantizing form is one column, one chunk");
  static_assert(!MF || (M >= 2 && M <= 8 && !QA), "matrix-core form: 2..8 columns");
  extern __shared__ uint32_t lds[];
  const int K = p.K, N = p.N;
  const int ls = p.lshift;
  const int L = 1 << ls;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = MF ? (lane & 3) | ((lane >> (2 + ls)) << 2) : lane >> ls;
  const int t = MF ? (lane >> 2) & (L - 1) : lane & (L - 1);
  const int row0 = blockIdx.x * (64 >> ls);
  const int row = row0 + slot;
  const int row_bytes = (K >> 8) * 80;

  const uint8_t* wb = p.w;
  bool id_ok = true;
  // Column m of this workgroup reads token col_tok[m] and writes y row
  // col_out[m].  Dense form: column m is token m.  MoE form: blockIdx.y is
  // a slot; with M > 1 (several tokens) the slots routed to the same expert
  // are grouped, so the expert's rows are decoded once for all of them: the
  // workgroup of the first slot of every run of M same-expert slots (in slot
  // order) computes that run, the others exit at once.  Unused columns of a
  // shorter run are skipped.
  int ncols = M;
  int col_tok[M], col_out[M];
#pragma unroll
  for (int m = 0; m < M; ++m) col_tok[m] = col_out[m] = m;
  int e = 0;                                    // the slot's expert (MoE form)
  if (MOE) {
    const int s0 = blockIdx.y;
    e = p.ids[s0];
    col_tok[0] = s0 / p.top_k;
    col_out[0] = s0;
    if (M > 1) {
      // one ballot covers the slots (S <= 64): which of them use expert e
      const int v = lane < p.S ? p.ids[lane] : ~e;
      uint64_t mask = __ballot(v == e);
      const uint64_t below = (uint64_t(1) << s0) - 1;
      if (__popcll(mask & below) % M) return;   // uniform: the whole workgroup
      mask &= ~below;
      ncols = min(__popcll(mask), M);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        if (m < ncols) {
          const int u = __ffsll((long long)mask) - 1;
          col_out[m] = u;
          col_tok[m] = u / p.top_k;
          mask &= mask - 1;
        } else {
          col_out[m] = col_out[m - 1];
          col_tok[m] = col_tok[m - 1];
        }
      }
    }
    // the expert selects the weight matrix (the quantizing form does this
    // once its activation loads are out, below)
    if constexpr (!QA) {
      id_ok = e >= 0 && e < p.E;
      wb = p.w + (int64_t)(id_ok ? e : 0) * (int64_t)N * row_bytes;
    }
  }
  if constexpr (!(MOE && QA)) wb += (int64_t)row0 * row_bytes;

  // per-wave LDS: JT chunk buffers of 1280 dwords, then this wave's
  // activations (M columns x ag = J*L groups of kGroupPieces pieces) and
  // their block scales (8 per group), each rounded up to whole 64-lane loads
  const int ag = p.J << ls;                     // activation groups of the wave
  const int n_pieces = M * ag * kGroupPieces;
  constexpr int MD = MF ? 4 * ((M + 3) / 4) : M;   // column slots of the scale array
  const int n_scales = MD * ag * 8;
  const int act_rounds = (n_pieces + 63) >> 6;
  const int d_rounds = (n_scales + 63) >> 6;
  // The routed matrix-core form carves the activations exactly (the last
  // load round only partly used) and keeps the cross-wave partial sums in the
  // chunk ring, which takes a four-token workgroup (4 waves, 4 groups each)
  // from 45 KB to 39 KB: four per compute unit instead of three (128 experts
  // of 1536 x 4096, top-8, four tokens: 13.05 -> 12.27 us with half of the
  // experts shared, 18.82 -> 17.08 us with none; the dense form, whose
  // workgroups all fit anyway, lost 2 % with it).
  constexpr bool EXACT = MF && MOE;
  const int act_dwords = EXACT ? n_pieces * 4 : act_rounds * 256;
  const int wave_dwords = JT * 1280 + act_dwords + d_rounds * 64;
  // what this workgroup actually loads and transposes (a short MoE group
  // stages only its own columns; the LDS carving above is for M)
  const int use_pieces = ncols * ag * kGroupPieces;
  const int use_scales = (MF ? MD : ncols) * ag * 8;
  const int use_act_rounds = (use_pieces + 63) >> 6;
  const int use_d_rounds = (use_scales + 63) >> 6;
  uint32_t* wlds = lds + wave * wave_dwords;
  uint32_t* alds = wlds + JT * 1280;
  float* dlds = reinterpret_cast<float*>(alds + act_dwords);
  const int nb = K >> 5;
  // (24-bit multiplies, full rate: every index here is below 2^24, K below 2^16)
  auto group_of = [&](int lgl) {
    return (int)((__umul24((uint32_t)(lgl >> ls), (uint32_t)p.wk) + wave) << ls) +
           (lgl & (L - 1));
  };
  // token of a lane-dependent column index: lane c of tok_lanes holds
  // col_tok[c], read back with a lane shuffle (no indexed register array,
  // which the compiler would place in scratch memory)
  int tok_lanes = col_tok[0];
#pragma unroll
  for (int c = 1; c < M; ++c) tok_lanes = lane == c ? col_tok[c] : tok_lanes;
  // (dense, up to four columns: column m is token m; the shuffle is kept for
  // more columns, where dropping it moved the five-column kernel from 119 to
  // 129 registers, one wave per SIMD fewer, 19 % slower for eight columns)
  auto token_of = [&](int m) {
    return (!MOE && M <= 4) ? m : M == 1 ? col_tok[0] : __shfl(tok_lanes, m, 64);
  };

  // The weight offsets are pure arithmetic: done first, they are ready when
  // the loads go out.
  const ChunkOffsets co = chunk_offsets(lane, ls, row0, N, row_bytes);

  const uint32_t ring_m0 = lds_m0(wlds);
  if constexpr (QA) {
    // Quantizing form: lane l of the wave takes halves l, l + 64, ... (QH of
    // them) of the wave's slice (ag*16 <= 64 * QH halves; lanes past the end
    // repeat the last half and write nothing), loads their fp32 activations
    // and the weight chunk in one go, quantizes while the weights stream, and
    // writes each int8 half (in the lane order of the expanded weights) and
    // its block scale to the same LDS slots the loaded form uses.  Workgroup
    // 0 also writes q and d out.  A block's two halves sit in lanes 2k and
    // 2k + 1 of the same round, which share the block maximum.
    const int n_halves = ag * 16;
    int hs[QH], aoffs[QH];
#pragma unroll
    for (int r = 0; r < QH; ++r) {
      hs[r] = min(lane + 64 * r, n_halves - 1);
      aoffs[r] = (group_of(hs[r] >> 4) * 256 + (hs[r] & 15) * 16) * 4;
    }
    v4f x[QH][4];
    if constexpr (MOE) {
      // the expert id is awaited after the activation loads are issued (its
      // scalar load's latency then overlaps theirs); the empty asm keeps
      // every use of it below the first asm
      if constexpr (QH == 1)
        load_acts(p.a, (uint32_t)aoffs[0], x[0]);
      else
        load_acts2(p.a, (uint32_t)aoffs[0], (uint32_t)aoffs[QH - 1], x[0], x[QH - 1]);
      asm volatile("" : "+s"(e));
      id_ok = e >= 0 && e < p.E;
      wb = p.w + (int64_t)(id_ok ? e : 0) * (int64_t)N * row_bytes + (int64_t)row0 * row_bytes;
      if constexpr (QH == 1)
        chunk_after_acts(wb + (int64_t)(wave << ls) * 80, co, ring_m0, x[0]);
      else
        chunk_after_acts2(wb + (int64_t)(wave << ls) * 80, co, ring_m0, x[0], x[QH - 1]);
    } else if constexpr (QH == 1) {
      load_acts_and_chunk(p.a, (uint32_t)aoffs[0], wb + (int64_t)(wave << ls) * 80, co,
                          ring_m0, x[0]);
    } else {
      load_acts2_and_chunk(p.a, (uint32_t)aoffs[0], (uint32_t)aoffs[QH - 1],
                           wb + (int64_t)(wave << ls) * 80, co, ring_m0, x[0], x[QH - 1]);
    }
#pragma unroll
    for (int r = 0; r < QH; ++r) {
      uint32_t A[4];
      const float dv = quantize_half(x[r], A);
      const int lgl = hs[r] >> 4, piece = hs[r] & 15;
      if (lane + 64 * r < n_halves) {
        reinterpret_cast<uint4*>(alds)[lgl * kGroupPieces + piece] =
            make_uint4(A[0], A[1], A[2], A[3]);
        if ((piece & 1) == 0) dlds[lgl * 8 + (piece >> 1)] = dv;
        if (blockIdx.x == 0 && (!MOE || blockIdx.y == 0)) {
          const int grp = group_of(lgl);
          uint32_t X[4];                 // the transpose is its own inverse
          transpose_half(A, X);
          reinterpret_cast<uint4*>(p.qo)[grp * 16 + piece] = make_uint4(X[0], X[1], X[2], X[3]);
          if ((piece & 1) == 0) p.dout[grp * 8 + (piece >> 1)] = dv;
        }
      }
    }
  } else {
    // The activations and their scales are loaded straight into place (they
    // hit L2), then the first JT weight chunks.  Loads complete in issue order,
    // so once no more than the 5*JT weight loads are outstanding the
    // activations have landed.  LDS piece p holds piece p % 17 of local group
    // g = p / 17 (column m = g / ag, local group lgl = g % ag, whose global
    // group is (j*wk + wave)*L + t' for lgl = j*L + t'); pad pieces and the
    // rounding slack re-read the first piece.
    {
      const uint32_t m0 = lds_m0(alds);
      // the wave's groups per column, ag = J * L: column of a local group g
      // by a shift when ag is a power of two (uniform), else as a float
      // quotient, exact for g < 2^21 ((g + 1/2) / ag is at least 1 / (2 ag)
      // from an integer; the reciprocal, within one ulp, and the rounded
      // product move it by less than 1.5 * 2^-23 of itself)
      const bool ag_pow2 = (ag & (ag - 1)) == 0;
      const int ag_shift = __builtin_ctz(ag);
      const float inv_ag = __builtin_amdgcn_rcpf((float)ag);
      auto col_of = [&](int g) {
        return M == 1 ? 0 : ag_pow2 ? g >> ag_shift : (int)(((float)g + 0.5f) * inv_ag);
      };
      // round r loads LDS piece pc = 64 r + lane: g = pc / 17 and
      // piece = pc % 17 are stepped from round to round (64 = 3 * 17 + 13)
      int g = (lane * 241) >> 12;                 // lane / 17 for lane < 64
      int piece = lane - kGroupPieces * g;
      for (int r = 0; r < use_act_rounds; ++r) {
        const bool used = piece < 16 && g < ncols * ag;
        const int gu = used ? g : 0;
        const int m = col_of(gu);
        const int lgl = gu - (int)__umul24((uint32_t)m, (uint32_t)ag);
        // the token lookup is a lane shuffle: every lane must take part (a
        // lane left out of it reads as 0 to the others)
        const int tok = token_of(m);
        const uint32_t off =
            used ? __umul24((uint32_t)tok, (uint32_t)K) + (uint32_t)((group_of(lgl) * 16 + piece) * 16)
                 : 0u;
        if (!EXACT || 64 * r + lane < n_pieces) dma16(p.q, off, m0 + 1024 * r);
        piece += 64 - 3 * kGroupPieces;
        g += 3;
        if (piece >= kGroupPieces) {
          piece -= kGroupPieces;
          ++g;
        }
      }
      const uint32_t m0d = lds_m0(dlds);
      for (int r = 0; r < use_d_rounds; ++r) {
        const int i = min(64 * r + lane, use_scales - 1);
        if constexpr (MF) {
          // [group][block][column slot]; slots past the last column re-read it
          constexpr int kMDs = MD == 8 ? 3 : 2;
          const int m = min(i & (MD - 1), ncols - 1);
          dma4(p.d,
               4 * (__umul24((uint32_t)token_of(m), (uint32_t)nb) +
                    (uint32_t)(group_of(i >> (kMDs + 3)) * 8 + ((i >> kMDs) & 7))),
               m0d + 256 * r);
        } else {
          const int gi = i >> 3;
          const int m = col_of(gi);
          const int lgl = gi - (int)__umul24((uint32_t)m, (uint32_t)ag);
          dma4(p.d,
               4 * (__umul24((uint32_t)token_of(m), (uint32_t)nb) +
                    (uint32_t)(group_of(lgl) * 8 + (i & 7))),
               m0d + 256 * r);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < JT; ++j)                 // J is a multiple of JT
      load_chunk(wb + (int64_t)((j * p.wk + wave) << ls) * 80, co, ring_m0 + 5120 * j);
    wait_chunks(JT);

    // transpose each half's 16 activations in place into the lane order of
    // the expanded weights: every piece the loads above wrote (pad pieces and
    // the rounding slack hold copies of a first piece that nothing reads),
    // two rounds at a time so that their LDS reads overlap
    {
      uint4* const base = reinterpret_cast<uint4*>(alds);
      auto transpose_piece = [&](const uint4& x) {
        const uint32_t X[4] = {x.x, x.y, x.z, x.w};
        uint32_t A[4];
        transpose_half(X, A);
        return make_uint4(A[0], A[1], A[2], A[3]);
      };
      for (int r = 0; r < use_act_rounds; r += 2) {
        const int pc0 = 64 * r + lane, pc1 = pc0 + 64;
        const bool ok0 = !EXACT || pc0 < n_pieces;
        const bool ok1 = r + 1 < use_act_rounds && (!EXACT || pc1 < n_pieces);
        uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
        if (ok0) x0 = base[pc0];
        if (ok1) x1 = base[pc1];
        if (ok0) base[pc0] = transpose_piece(x0);
        if (ok1) base[pc1] = transpose_piece(x1);
      }
    }
  }

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  uint32_t bad_lo = 0, bad_hi = 0;
  const int act_stride = ag * kGroupDwords;
  for (int j = 0; j < p.J; ++j) {
    const int buf_i = JT == 1 ? 0 : j % JT;
    wait_chunks(min(JT, p.J - j) - 1);          // chunk j has landed
    __builtin_amdgcn_wave_barrier();
    uint32_t buf[20];
    // this lane's group: row slot `slot`, group t of the row's segment
    const int gl = MF ? slot * L + t : lane;
    const uint4* src = reinterpret_cast<const uint4*>(wlds + buf_i * 1280 + 20 * gl);
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
                 ring_m0 + 5120 * buf_i);
    const int lgl = (j << ls) + t;
    if constexpr (MF) {
      const uint32_t* act0 = alds + min(lane & 3, ncols - 1) * act_stride + lgl * kGroupDwords;
      const uint32_t* act1 = alds + min(4 + (lane & 3), ncols - 1) * act_stride +
                             lgl * kGroupDwords;
      if constexpr (MOE && M > 4) {
        // (uniform) a routed group of at most four columns: one quad of products
        if (ncols <= 4) {
          float(&acc4)[4] = *reinterpret_cast<float(*)[4]>(acc);
          group_product_mf<4, 2>(buf, act0, act1, dlds + lgl * 8 * MD, acc4, bad_lo, bad_hi);
        } else {
          group_product_mf<M>(buf, act0, act1, dlds + lgl * 8 * MD, acc, bad_lo, bad_hi);
        }
      } else {
        group_product_mf<M>(buf, act0, act1, dlds + lgl * 8 * MD, acc, bad_lo, bad_hi);
      }
    }
    else
      group_product<M, (M <= 4) && (!MOE || M == 1)>(buf, alds + lgl * kGroupDwords, act_stride,
                                                    dlds + lgl * 8, ag * 8, acc, bad_lo, bad_hi,
                                                    ncols);
  }

  // row sum: xor shuffles over the L lanes of the row, then over the waves
  const bool bad = scale_flags_set<0>(bad_lo) || scale_flags_set<1>(bad_hi);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float v = bad ? __builtin_nanf("") : acc[m];
    acc[m] = MF ? row_sum_mf(v, L) : row_sum(v, L);
  }
  const int S = 64 >> ls;
  if (p.wk > 1) {
    // wave wv's sums at red + wv * red_stride (EXACT: the start of the
    // wave's own chunk ring, free once its last chunk is read)
    float* red = reinterpret_cast<float*>(EXACT ? lds : lds + p.wk * wave_dwords);
    const int red_stride = EXACT ? wave_dwords : S * M;
    if (t == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) red[wave * red_stride + slot * M + m] = acc[m];
    }
    __syncthreads();
    if (wave == 0 && t == 0) {
      // every partial is read before any is added, so the LDS latency is
      // paid once, not once per wave and column (a loop over the waves
      // waited for each read: ~0.9 us of a 16384 x 5120, M = 4 product);
      // the reads for waves past wk re-read wave wk - 1 and are not added.
      // The sum runs over the waves in order, as before.
      float part[kMaxWaves][M];
#pragma unroll
      for (int wv = 0; wv < kMaxWaves; ++wv) {
        const int src = min(wv, p.wk - 1) * red_stride + slot * M;
#pragma unroll
        for (int m = 0; m < M; ++m) part[wv][m] = red[src + m];
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float v = part[0][m];
#pragma unroll
        for (int wv = 1; wv < kMaxWaves; ++wv)
          if (wv < p.wk) v += part[wv][m];
        acc[m] = v;
      }
    }
  }
  if (wave == 0 && t == 0 && row < N) {
    const float fix = scale_fix();
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (m < ncols)
        p.y[(int64_t)col_out[m] * N + row] = id_ok ? acc[m] * fix : __builtin_nanf("");
  }
  if (MOE && !id_ok && blockIdx.x == 0 && threadIdx.x == 0 && p.err != nullptr)
    p.err[0] = 1;
}

using GemvFn = void (*)(Params);

constexpr int kMaxChunksInFlight = 4;

template <int M, bool MOE, bool MF = false>
GemvFn pick(int jt) {
  switch (jt) {
    case 1: return gemv_kernel<M, 1, MOE, 0, MF>;
    case 2: return gemv_kernel<M, 2, MOE, 0, MF>;
    case 3: return gemv_kernel<M, 3, MOE, 0, MF>;
    default: return gemv_kernel<M, 4, MOE, 0, MF>;
  }
}

}  // namespace gemv_detail
}  // namespace rfp2
