// ROCmFP2 x int8 GEMM on the i8 matrix cores (prompt batches).
//
// Method ("ROCmFP2 codebook research report", "03 · Runtime", applied to a
// tile of activation columns): the stored blocks are expanded to int8 once
// per tile and reused by every token of the tile; the integer dot products
// are rescaled by the weight scales and the token's activation scale,
//   y[m,n] += d[m,b] * (s0[n,b] * P0[m,n] + s1[n,b] * P1[m,n]),
// P_h the int32 sum over half h of block b.
//
// Folded operands.  A legal UE4M3 scale byte is s = mu * 2^(x - 11) with x =
// max(E, 1) and mu = 8 + M (mu = M when E = 0), at most 4 bits.  For a block
// with x_lo = min(x0, x1),
//   s0 * P0 + s1 * P1 = 2^(x_lo - 11) * sum_k a_k * (level_k * c_h),
//   c_h = mu_h * 2^(x_h - x_lo),
// an integer dot product with one power-of-two scale.  When the halves'
// exponents differ by at most 2, |level * c| <= 4 * 60 = 240: one
// v_mfma_i32_16x16x64_i8 takes it whole, its 64 k being the block's 32
// activations twice against two int8 operands wA + wB (a weight whose c is
// 32..60 is split into two equal parts).  That replaces the two per-half
// partials and the per-half scales of the direct form.
//   Blocks whose exponents differ by 3 or more (0.4 % of the blocks of the
// synthetic weights) keep their halves apart: wA = the half of larger
// exponent (level * mu), wB = the other one, each with its own power-of-two
// scale.  A 16-row tile holding such a block in a stage takes the split
// path: one more MFMA (wA alone) and three more instructions per output.
//
// Rescale: the int32 sum accumulates onto the bits of 1.5 * 2^23, so read as
// fp32 it is 1.5 * 2^23 + P exactly (|P| <= 32 * 127 * 240 < 2^22), and
// fma(x, s, -1.5 * 2^23 * s) = s * P exactly (s a power of two); then
// fma(d, ., acc).  Two instructions per (token, row, block): the vector ALU
// work that bounds this kernel (the matrix cores are far from busy).
//
// gfx950 mapping
//   * Workgroup tile 112 rows x 256 tokens, eight waves (two per SIMD), one
//     workgroup per CU; wave w owns tokens 32w..32w+31 (two 16-token MFMA
//     tiles) and all seven 16-row tiles, so the decoded weights in LDS serve
//     all eight waves.  (For 512 x 14336 this is 2 x 128 = 256 workgroups.)
//   * MFMA operand A = activations (i = token), B = weights (j = row): lane
//     l holds row l % 16 of each tile and tokens 4 (l / 16) + r in its
//     registers r, so the row scales are one register per tile and the
//     activation scales one 16-byte LDS read per token tile.
//   * Stages of 2 blocks in two LDS buffers; the global loads of stage s + 3
//     are in flight while stage s is computed and stage s + 1 is staged; one
//     barrier per stage.
//   * Weights are expanded in registers (the per-half level table scaled by
//     the multiplier, looked up by byte permutes) into the lane order of
//     expand_half; activations are staged with the same within-half
//     permutation (transpose_half), so each dot product is unchanged.
//   * Workgroup -> tile order is XCD-aware: the hardware deals workgroups to
//     the 8 XCDs round-robin, so consecutive tiles (the token tiles of one
//     row tile first) are given to workgroups on the same XCD and share its
//     L2 for the weights.
#include "rfp2_device.h"
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kRowTiles = 7;                // 16-row MFMA tiles per workgroup
constexpr int BN = 16 * kRowTiles;          // 112 weight rows per workgroup
constexpr int kWaves = 8;
constexpr int BM = 32 * kWaves;             // 256 tokens per workgroup
constexpr int KB = 2;                       // blocks per LDS stage
constexpr int kWRow = KB * 64 + 16;         // LDS bytes per weight row of a stage (144)
constexpr int kARow = KB * 32 + 16;         // LDS bytes per token row of a stage (80)
constexpr int kDecoders = 56;               // decoding lanes in each of waves 0..3
constexpr int kXcds = 8;
constexpr int kBiasBits = 0x4B400000;       // fp32 1.5 * 2^23
constexpr float kNegBias = -12582912.0f;

// The staged form of one block of one row.
struct Folded {
  uint32_t wa[2][4], wb[2][4];  // [half][word], expand_half lane order
  float2 sm;                    // (s, -1.5*2^23*s); s < 0 (or NaN): split path
  float4 sg;                    // (sA, -1.5*2^23*sA, sB, -1.5*2^23*sB)
};

// Bytes [-4c, -c, c, 4c] (code 0..3 -> level * c), 0 <= c <= 31.
__device__ __forceinline__ uint32_t level_table(uint32_t c) {
  const uint32_t pos = __umul24(c, 0x10004u); // 16-bit lanes (4c, c)
  const v2s n = v2s{0, 0} - __builtin_bit_cast(v2s, pos);
  return __builtin_amdgcn_perm(pos, __builtin_bit_cast(uint32_t, n), 0x04060200u);
}

__device__ __forceinline__ float pow2_scale(int x) {    // 2^(x - 11), 1 <= x <= 31
  return __int_as_float((x + 116) << 23);
}

// Fold one block: C0, C1 the two halves' code words, sc = e0 | e1 << 8.
__device__ __forceinline__ void fold_block(uint32_t C0, uint32_t C1, uint32_t sc,
                                           Folded& f) {
  const int e0 = sc & 0xFF, e1 = (sc >> 8) & 0xFF;
  const int x0 = max(e0 >> 3, 1), x1 = max(e1 >> 3, 1);
  const int mu0 = e0 + 8 - 8 * x0, mu1 = e1 + 8 - 8 * x1;
  const int xl = min(x0, x1), xh = max(x0, x1);
  const bool near = xh - xl <= 2;
  const int c0 = near ? mu0 << (x0 - xl) : mu0;
  const int c1 = near ? mu1 << (x1 - xl) : mu1;
  // near: c > 31 only for c = 4 mu (exponent step 2), split into two 2 mu
  const int h0 = c0 > 31 ? c0 >> 1 : c0, h1 = c1 > 31 ? c1 >> 1 : c1;
  const bool top0 = x0 > x1;                // apart: half 0 has the larger exponent
  const int a0 = near ? h0 : (top0 ? c0 : 0), b0 = near ? c0 - h0 : (top0 ? 0 : c0);
  const int a1 = near ? h1 : (top0 ? 0 : c1), b1 = near ? c1 - h1 : (top0 ? c1 : 0);
  const uint32_t tA0 = level_table(a0), tB0 = level_table(b0);
  const uint32_t tA1 = level_table(a1), tB1 = level_table(b1);
  // selectors: byte j of word i = code of weight 4j + i (as expand_block)
  const uint64_t C = ((uint64_t)C1 << 32) | C0;
  const uint64_t S2 = shr64<2>(C), S4 = shr64<4>(C), S6 = shr64<6>(C);
  const uint32_t sel[2][4] = {
      {C0 & kLow2, (uint32_t)S2 & kLow2, (uint32_t)S4 & kLow2, (uint32_t)S6 & kLow2},
      {C1 & kLow2, (uint32_t)(S2 >> 32) & kLow2, (uint32_t)(S4 >> 32) & kLow2,
       (uint32_t)(S6 >> 32) & kLow2}};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.wa[0][i] = __builtin_amdgcn_perm(tA0, tA0, sel[0][i]);
    f.wb[0][i] = __builtin_amdgcn_perm(tB0, tB0, sel[0][i]);
    f.wa[1][i] = __builtin_amdgcn_perm(tA1, tA1, sel[1][i]);
    f.wb[1][i] = __builtin_amdgcn_perm(tB1, tB1, sel[1][i]);
  }
  const bool bad = scale_byte_bad(e0) || scale_byte_bad(e1);
  const float nan = __builtin_nanf("");
  const float sl = bad ? nan : pow2_scale(xl);
  const float sa = bad ? nan : (near ? sl : pow2_scale(xh));
  f.sg = make_float4(sa, kNegBias * sa, sl, kNegBias * sl);
  f.sm = make_float2(near ? sl : -sl, kNegBias * sl);
}

// Block `blk` (0 or 1) of a dword-aligned 20-byte pair of blocks.
__device__ __forceinline__ void fold_pair_member(const uint32_t (&wd)[5], int blk, Folded& f) {
  const uint32_t C0 = blk ? __builtin_amdgcn_alignbit(wd[3], wd[2], 16) : wd[0];
  const uint32_t C1 = blk ? __builtin_amdgcn_alignbit(wd[4], wd[3], 16) : wd[1];
  const uint32_t sc = blk ? wd[4] >> 16 : wd[2] & 0xFFFFu;
  fold_block(C0, C1, sc, f);
}

struct __align__(16) Stage {
  uint8_t w[BN * kWRow];        // row r, block b: [wA h0 | wA h1 | wB h0 | wB h1]
  uint8_t a[BM * kARow];        // token t, block b: [h0 | h1], transposed halves
  float2 sm[KB][BN];
  float4 sg[KB][BN];
  float d[KB][BM];
};

struct Prefetch {
  uint32_t wd[5];               // the decoded row's 20-byte pair (decoding lanes)
  uint4 a0, a1;                 // one block of one token's activations
  float d;
};

struct Roles {
  bool dec;                     // this lane decodes (row drow, block dblk)
  int drow, dblk;
  const uint8_t* w;             // decoded row
  int atok, ablk;               // staged (token, block)
  const int8_t* q;
  const float* d;
};

__device__ __forceinline__ void fetch(Prefetch& f, const Roles& r, int kb) {
  if (r.dec) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(r.w + (int64_t)kb * 10);
#pragma unroll
    for (int i = 0; i < 5; ++i) f.wd[i] = src[i];
  }
  const uint4* asrc = reinterpret_cast<const uint4*>(r.q + (int64_t)kb * 32);
  f.a0 = asrc[0];
  f.a1 = asrc[1];
  f.d = r.d[kb];
}

__device__ __forceinline__ void stage_to_lds(const Prefetch& f, Stage& st, const Roles& r,
                                             uint32_t* split) {
  if (r.dec) {
    Folded fb;
    fold_pair_member(f.wd, r.dblk, fb);
    // the row tile of a block whose halves stay apart (or NaN) takes the
    // split path: one bit per (block, row tile)
    if (!(fb.sm.x > 0.0f)) atomicOr(&split[r.dblk], 1u << (r.drow >> 4));
    uint4* dst = reinterpret_cast<uint4*>(st.w + r.drow * kWRow + r.dblk * 64);
    dst[0] = make_uint4(fb.wa[0][0], fb.wa[0][1], fb.wa[0][2], fb.wa[0][3]);
    dst[1] = make_uint4(fb.wa[1][0], fb.wa[1][1], fb.wa[1][2], fb.wa[1][3]);
    dst[2] = make_uint4(fb.wb[0][0], fb.wb[0][1], fb.wb[0][2], fb.wb[0][3]);
    dst[3] = make_uint4(fb.wb[1][0], fb.wb[1][1], fb.wb[1][2], fb.wb[1][3]);
    st.sm[r.dblk][r.drow] = fb.sm;
    st.sg[r.dblk][r.drow] = fb.sg;
  }
  uint32_t A0[4], A1[4];
  {
    const uint32_t X0[4] = {f.a0.x, f.a0.y, f.a0.z, f.a0.w};
    const uint32_t X1[4] = {f.a1.x, f.a1.y, f.a1.z, f.a1.w};
    transpose_half(X0, A0);
    transpose_half(X1, A1);
  }
  uint4* adst = reinterpret_cast<uint4*>(st.a + r.atok * kARow + r.ablk * 32);
  adst[0] = make_uint4(A0[0], A0[1], A0[2], A0[3]);
  adst[1] = make_uint4(A1[0], A1[1], A1[2], A1[3]);
  st.d[r.ablk][r.atok] = f.d;
}

// y += d * u for one row tile, u the tile's block sums times their scales.
__device__ __forceinline__ void accumulate(const v4f (&dv)[2], const float (&u)[2][4],
                                           v4f (&acc)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(dv[t][r], u[t][r], acc[t][r]);
}

// Folded form: P = 1.5*2^23 + the block's sum, u = s * sum (exact).
__device__ __forceinline__ void folded_sums(const v4i (&P)[2], float2 s, float (&u)[2][4]) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) u[t][r] = fmaf(__int_as_float(P[t][r]), s.x, s.y);
}

// Split form for a tile with a block whose halves stay apart (or an illegal
// scale byte: NaN): wA's part recomputed alone, u = sA * PA + sB * PB.
__device__ __forceinline__ void split_sums(const Stage& st, int blk, int rt, int g, int li,
                                           const v4i& bias, const v4i (&a)[2],
                                           const v4i (&P)[2], float (&u)[2][4]) {
  const float4 sg = st.sg[blk][16 * rt + li];
  const v4i b = *reinterpret_cast<const v4i*>(st.w + (16 * rt + li) * kWRow + blk * 64 + 16 * g);
  const v4i bA = g < 2 ? b : v4i{0, 0, 0, 0};     // lane groups 2, 3 hold wB
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const v4i PA = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], bA, bias, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      u[t][r] = fmaf((float)(P[t][r] - PA[r]), sg.z, fmaf(__int_as_float(PA[r]), sg.x, sg.y));
  }
}

// The stage's block sums for this wave's 112 rows x 32 tokens, rescaled and
// added to acc[row tile][token tile].  A block's LDS operands are all read
// first (one wait per block instead of one per tile), then the tiles are
// software-pipelined (the MFMAs of tile rt + 1 are issued before tile rt is
// rescaled).  Every tile takes the folded form first; a tile that needs the
// split form (s <= 0 or NaN on one of its rows, rare; the staging lanes set
// its bit in `split`, one scalar test per tile instead of a vector compare:
// 111.9 -> 109.5 us) has its u recomputed in a branch that touches nothing
// else, so the accumulators never meet a branch (where the compiler would
// copy them).
__device__ __forceinline__ void compute_stage(const Stage& st, const uint32_t* split, int wave,
                                              int lane, const v4i& bias,
                                              v4f (&acc)[kRowTiles][2]) {
  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int blk = 0; blk < KB; ++blk) {
    const uint32_t tiles_split = __builtin_amdgcn_readfirstlane(split[blk]);
    v4i a[2], b[kRowTiles];
    v4f dv[2];
    float2 s[kRowTiles];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tok = 32 * wave + 16 * t;
      a[t] = *reinterpret_cast<const v4i*>(st.a + (tok + li) * kARow + blk * 32 + 16 * (g & 1));
      dv[t] = *reinterpret_cast<const v4f*>(&st.d[blk][tok + 4 * g]);
    }
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      b[rt] = *reinterpret_cast<const v4i*>(st.w + (16 * rt + li) * kWRow + blk * 64 + 16 * g);
      s[rt] = st.sm[blk][16 * rt + li];
    }
    v4i P[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) P[0][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b[0], bias, 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      if (rt + 1 < kRowTiles) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          P[(rt + 1) & 1][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], b[rt + 1], bias, 0, 0, 0);
      }
      float u[2][4];
      folded_sums(P[rt & 1], s[rt], u);
      if (__builtin_expect((tiles_split >> rt) & 1u, 0))
        split_sums(st, blk, rt, g, li, bias, a, P[rt & 1], u);
      accumulate(dv, u, acc[rt]);
      // keep the update here: sunk to the end of the block, the seven
      // tiles' u would all be live at once
      asm volatile("" : "+v"(acc[rt][0]), "+v"(acc[rt][1]));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

__global__ __launch_bounds__(512) void gemm_kernel(
    const uint8_t* __restrict__ w, int N, int K, const int8_t* __restrict__ q,
    const float* __restrict__ d, int M, float* __restrict__ y, int m_tiles, int tiles) {
  __shared__ Stage sm[2];
  // split-path flags of stage s in slot s % 4: set while staging (iteration
  // s - 1), read while computing (iteration s), cleared in iteration s + 2;
  // barriers separate all three
  __shared__ uint32_t split[4][KB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int tile = blockIdx.x;
  if (tiles % kXcds == 0) tile = (blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
  const int m0 = (tile % m_tiles) * BM;
  const int n0 = (tile / m_tiles) * BN;
  const int nb = K / 32;
  const int64_t row_bytes = (int64_t)nb * 10;
  const int stages = nb / KB;

  // rows / tokens past the end read row N-1 / token M-1 (never stored)
  Roles ro;
  {
    // two consecutive lanes take the two blocks of one row / token (their
    // global loads then cover whole 20- and 64-byte pieces; mapping
    // consecutive lanes to consecutive rows and tokens removed a quarter of
    // the LDS bank conflicts of the stores but cost 2 and 8 us)
    const int di = kDecoders * wave + lane;
    ro.dec = wave < 4 && lane < kDecoders;
    ro.drow = di >> 1;
    ro.dblk = di & 1;
    ro.w = w + (int64_t)min(n0 + ro.drow, N - 1) * row_bytes;
    ro.atok = tid >> 1;
    ro.ablk = tid & 1;
    const int64_t tok = min(m0 + ro.atok, M - 1);
    ro.q = q + tok * K + ro.ablk * 32;
    ro.d = d + tok * nb + ro.ablk;
  }

  v4f acc[kRowTiles][2];
#pragma unroll
  for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // the MFMA accumulator start, held in registers (as a constant the
  // compiler rebuilds it from scalar registers before every MFMA)
  v4i bias = {kBiasBits, kBiasBits, kBiasBits, kBiasBits};
  asm volatile("" : "+v"(bias));

  // Global loads run two stages ahead: f0 holds even stages, f1 odd ones
  // (the stage count K / 64 is a multiple of 4).  Iteration s computes
  // stage s, stages s + 1 from the set loaded two iterations earlier and
  // reloads that set with stage s + 3 (past the end: the last stage again).
  if (tid < 4 * KB) split[tid / KB][tid % KB] = 0u;
  __syncthreads();
  Prefetch f0, f1;
  fetch(f0, ro, 0);
  fetch(f1, ro, KB);
  stage_to_lds(f0, sm[0], ro, split[0]);
  fetch(f0, ro, 2 * KB);
  __syncthreads();
  const int last = (stages - 1) * KB;
#define RFP2_GEMM_STEP(S, FN, COMPUTE_FIRST)                                   \
  {                                                                             \
    if (COMPUTE_FIRST) compute_stage(sm[(S) & 1], split[(S) & 3], wave, lane, bias, acc); \
    stage_to_lds(FN, sm[((S) + 1) & 1], ro, split[((S) + 1) & 3]);              \
    fetch(FN, ro, min(((S) + 3) * KB, last));                                   \
    if (!(COMPUTE_FIRST)) compute_stage(sm[(S) & 1], split[(S) & 3], wave, lane, bias, acc); \
    if (tid < KB) split[((S) + 2) & 3][tid] = 0u;                               \
    __syncthreads();                                                            \
  }
  // Waves 0..3 compute a stage and then stage the next one; waves 4..7 do
  // it the other way round, so that the two waves of a SIMD are out of
  // phase: one reads its LDS operands while the other computes (120.8 ->
  // 113.4 us on 512 x 14336 x 4096; waves 0..3, the decoding ones, staging
  // first: 117.7 us).  Two copies of the loop, so that the accumulators
  // never meet a branch.  (Loads one stage ahead instead of two: 113.9 us
  // against 111.1 us.)
  if (wave < 4) {
    for (int s = 0; s + 2 < stages; s += 2) {
      RFP2_GEMM_STEP(s, f1, true)
      RFP2_GEMM_STEP(s + 1, f0, true)
    }
  } else {
    for (int s = 0; s + 2 < stages; s += 2) {
      RFP2_GEMM_STEP(s, f1, false)
      RFP2_GEMM_STEP(s + 1, f0, false)
    }
  }
#undef RFP2_GEMM_STEP
  // the last two stages: stage s = stages - 2 computes and stages the last
  {
    const int s = stages - 2;
    compute_stage(sm[s & 1], split[s & 3], wave, lane, bias, acc);
    stage_to_lds(f1, sm[(s + 1) & 1], ro, split[(s + 1) & 3]);
    __syncthreads();
  }
  compute_stage(sm[(stages - 1) & 1], split[(stages - 1) & 3], wave, lane, bias, acc);

  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int n = n0 + 16 * rt + li;
    if (n >= N) continue;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 32 * wave + 16 * t + 4 * g + r;
        if (m < M) y[(int64_t)m * N + n] = acc[rt][t][r];
      }
  }
}

// Inspection of the GEMM's decode (rfp2_debug_decode_i8): block 2p + j of
// the flat block stream is folded from its 20-byte pair exactly as a
// staging lane folds member j of the pair it loaded, and written out in
// natural weight order with its scales.
__global__ __launch_bounds__(256) void debug_decode_i8_kernel(
    const uint8_t* __restrict__ w, int64_t nblocks, int8_t* __restrict__ wa_out,
    int8_t* __restrict__ wb_out, float* __restrict__ s_out) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nblocks;
       i += (int64_t)gridDim.x * 256) {
    // the 20-byte pair as 16-bit pieces (the stream is only 2-byte aligned
    // here); bytes past the end read as zero
    const int64_t p = i >> 1;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(w + p * 20);
    const int64_t end = nblocks * 10;
    uint32_t wd[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) {
      const int64_t off = p * 20 + 4 * k;
      wd[k] = (off < end ? (uint32_t)src[2 * k] : 0u) |
              ((off + 2 < end ? (uint32_t)src[2 * k + 1] : 0u) << 16);
    }
    Folded f;
    fold_pair_member(wd, (int)(i & 1), f);
    // weight 4j + c of a half is byte j of word c
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sel = 0x0C0C0C00u + (uint32_t)j;   // byte j of each word to byte 0
        uint32_t va = 0, vb = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          va |= (__builtin_amdgcn_perm(0u, f.wa[h][c], sel) & 0xFFu) << (8 * c);
          vb |= (__builtin_amdgcn_perm(0u, f.wb[h][c], sel) & 0xFFu) << (8 * c);
        }
        *reinterpret_cast<uint32_t*>(wa_out + i * 32 + 16 * h + 4 * j) = va;
        *reinterpret_cast<uint32_t*>(wb_out + i * 32 + 16 * h + 4 * j) = vb;
      }
    float* so = s_out + i * 6;
    so[0] = f.sm.x;
    so[1] = f.sm.y;
    so[2] = f.sg.x;
    so[3] = f.sg.y;
    so[4] = f.sg.z;
    so[5] = f.sg.w;
  }
}

}  // namespace

hipError_t launch_debug_decode_i8(const uint8_t* w, int64_t N, int64_t K, int8_t* wa,
                                  int8_t* wb, float* scales, hipStream_t stream) {
  const int64_t nblocks = N * (K / 32);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>((nblocks + 255) / 256, kMaxGrid));
  hipLaunchKernelGGL(debug_decode_i8_kernel, dim3((uint32_t)grid), dim3(256), 0, stream, w,
                     nblocks, wa, wb, scales);
  return hipGetLastError();
}

hipError_t launch_gemm(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream) {
  const int m_tiles = (int)((M + BM - 1) / BM);
  const int n_tiles = (int)((N + BN - 1) / BN);
  const int tiles = m_tiles * n_tiles;
  hipLaunchKernelGGL(gemm_kernel, dim3((uint32_t)tiles), dim3(512), 0, stream, w, (int)N,
                     (int)K, q, d, (int)M, y, m_tiles, tiles);
  return hipGetLastError();
}

}  // namespace rfp2
