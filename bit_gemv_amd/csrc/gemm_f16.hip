// ROCmFP2 x int8 GEMM on the fp16 matrix cores, with exact operands.
//
// Same product as gemm.hip ("ROCmFP2 codebook research report", "03 ·
// Runtime": int8 activations, weights = level x UE4M3 scale of their half,
// activation scale applied per 32-block), computed in a different order:
//   * every reconstructed weight level*s (|level| in {1, 4}, s a UE4M3 value
//     with at most 4 significant bits between 2^-10 and 224) and every int8
//     activation is exactly an fp16 number, and every product is exact in
//     fp32;
//   * so the per-half weight scales go into the operands, and the matrix
//     core gives the whole 32-weight block's sum C = s0 * S0 + s1 * S1
//     directly in fp32 (one v_mfma_f32_16x16x32_f16 in the dense kernel, a
//     pair of v_mfma_f32_32x32x16_f16 in the routed one).  It is exact, in
//     any summation order, while the two halves' scale exponents (E, with
//     E = 0 counted as 1) differ by at most 7: every partial sum is an
//     integer multiple of the smaller scale's unit below
//     15 * 8128 * (1 + 2^7) < 2^24.  With a wider split the core's fp32
//     accumulation may round, each step within 2^-24 of the running sum;
//   * the epilogue per (token, row, block) is one FMA, y += d * C, against
//     two for the int8 path's integer block sum (its power-of-two weight
//     scale and the activation scale, gemm.hip).
// The rescale, not the matrix cores, bounds the int8 path; here the two are
// of the same order.
//
// gfx950 mapping: the dense kernel is laid out as gemm.hip (112 x 256 tiles,
// eight waves, one workgroup per compute unit, 16 x 16 MFMA tiles, K stages
// of 2 blocks in two LDS buffers with register prefetch, XCD-aware tile
// order); its 128 x 128 predecessor with 32 x 32 tiles and 448 workgroups
// (two per compute unit where they fit) took 107.0 us against 97.8 us on
// 512 x 14336 x 4096 (alternating timings).  The routed form (tokens sorted by expert, a prompt batch
// through the routed experts) has a kernel of its own below
// (moe_gemm_kernel): 64-token tiles, each inside one expert's slots, with
// the weights decoded straight into registers.  Within each 16-weight half
// the k order in LDS is 0,8, 4,12, 1,9, 5,13, 2,10, 6,14, 3,11, 7,15 for
// weights and activations alike (the order in which one byte permute per
// pair of weights decodes them); a dot product over the half does not
// depend on it.
#include "f16_decode.h"
#include "rfp2_internal.h"

#include <climits>

namespace rfp2 {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;

// Dense product: workgroup tile 112 rows x 256 tokens, eight waves (two per
// SIMD), one workgroup per compute unit (2 x 128 = 256 workgroups on 512 x
// 14336); wave w owns tokens 32w..32w+31 (two 16-token MFMA tiles) and all
// seven 16-row tiles.  One v_mfma_f32_16x16x32_f16 is one whole block of one
// 16 x 16 tile: operand A = the activations (i = token), B = the weights
// (j = row), so lane l holds row l % 16 and tokens 4 (l / 16) + r, and a
// block's activation scales are one 16-byte LDS read per token tile.
constexpr int kRowTiles = 7;
constexpr int BN = 16 * kRowTiles;              // 112 weight rows
constexpr int kWaves = 8;
constexpr int BM = 32 * kWaves;                 // 256 tokens
constexpr int BKB = 2;                          // blocks per LDS stage
constexpr int kRowBytes = BKB * 64 + 16;        // fp16 row of a stage + pad (144)
constexpr int kDecoders = 56;                   // decoding lanes in each of waves 0..3

struct __align__(16) StageF16 {
  uint8_t wh[BN * kRowBytes];      // fp16 weights (level * scale), row r, block b at r*144 + 64b
  uint8_t ah[BM * kRowBytes];      // fp16 activations, same layout
  float ad[BKB][BM];               // activation scale per (block, token)
};

struct PrefetchF16 {
  uint32_t wd[5];                  // the 20-byte block pair holding the decoded block
  uint4 a[2];                      // 32 int8 activations
  float d;
};

// What a thread stages: block dblk of weight row drow (lanes 0..55 of waves
// 0..3; two consecutive lanes take the two blocks of one row) and block
// ablk of token atok (every thread).  Rows / tokens past the end re-read
// row N-1 / token M-1 (never stored).
struct RolesF16 {
  bool dec;
  int drow, dblk, atok, ablk;
  const uint8_t* w;
  const int8_t* q;
  const float* d;
};

__device__ __forceinline__ void fetch(PrefetchF16& f, const RolesF16& r, int kb) {
  if (r.dec) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(r.w + (int64_t)kb * 10);
#pragma unroll
    for (int i = 0; i < 5; ++i) f.wd[i] = src[i];
  }
  const uint4* asrc = reinterpret_cast<const uint4*>(r.q + (int64_t)kb * 32);
  f.a[0] = asrc[0];
  f.a[1] = asrc[1];
  f.d = r.d[kb];
}

__device__ __forceinline__ void stage_to_lds(const PrefetchF16& f, StageF16& st,
                                             const RolesF16& r) {
  if (r.dec) {
    uint32_t h0[8], h1[8];
    decode_pair_block_f16(f.wd, r.dblk, h0, h1);
    uint4* dst = reinterpret_cast<uint4*>(st.wh + r.drow * kRowBytes + r.dblk * 64);
    dst[0] = make_uint4(h0[0], h0[1], h0[2], h0[3]);
    dst[1] = make_uint4(h0[4], h0[5], h0[6], h0[7]);
    dst[2] = make_uint4(h1[0], h1[1], h1[2], h1[3]);
    dst[3] = make_uint4(h1[4], h1[5], h1[6], h1[7]);
  }
  uint4* adst = reinterpret_cast<uint4*>(st.ah + r.atok * kRowBytes + r.ablk * 64);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t X[4] = {f.a[h].x, f.a[h].y, f.a[h].z, f.a[h].w};
    uint32_t o[8];
    act_half_f16(X, o);
    adst[2 * h] = make_uint4(o[0], o[1], o[2], o[3]);
    adst[2 * h + 1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
  st.ad[r.ablk][r.atok] = f.d;
}

// Block sums of the stage for this wave's 112 rows x 32 tokens, rescaled by
// the activation scales and added to acc[row tile][token tile].  A block's
// LDS operands are all read before its first product (one wait per block),
// and the row tiles are software-pipelined (the products of tile rt + 1 are
// issued before tile rt is rescaled).
__device__ __forceinline__ void compute_stage(const StageF16& st, int wave, int lane,
                                              v4f (&acc)[kRowTiles][2]) {
  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int blk = 0; blk < BKB; ++blk) {
    v8h a[2], b[kRowTiles];
    v4f dv[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int tok = 32 * wave + 16 * t;
      a[t] = *reinterpret_cast<const v8h*>(st.ah + (tok + li) * kRowBytes + blk * 64 + 16 * g);
      dv[t] = *reinterpret_cast<const v4f*>(&st.ad[blk][tok + 4 * g]);
    }
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt)
      b[rt] = *reinterpret_cast<const v8h*>(st.wh + (16 * rt + li) * kRowBytes + blk * 64 + 16 * g);
    v4f c[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t) c[0][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], b[0], v4f{}, 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      if (rt + 1 < kRowTiles) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
          c[(rt + 1) & 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], b[rt + 1], v4f{}, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[rt][t][r] = fmaf(dv[t][r], c[rt & 1][t][r], acc[rt][t][r]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct GemmF16Params {
  const uint8_t* w;   // dense: [N] rows; routed: E experts of [N] rows
  int N, K;
  const int8_t* q;
  const float* d;
  float* y;
  // dense product
  int M, m_tiles, tiles;
  // routed product (tokens sorted by expert): expert e's slots are
  // order[offsets[e] .. offsets[e+1]); its 64-token tiles are numbered from
  // tile_start[e]; tile_start[E] tiles in all
  const int32_t* offsets;
  const int32_t* tile_start;
  const int32_t* order;
  int E, top_k, n_tiles;
};

// Expert owning routed tile i: the last e with tile_start[e] <= i (the array
// is non-decreasing; an expert with no slots has an empty range).  Two
// wave-wide probes of at most 64 entries each (E + 1 <= 64 * 64).
__device__ __forceinline__ int expert_of_tile(const int32_t* tile_start, int E, int i,
                                              int lane) {
  const int chunk = (E + 64) >> 6;              // ceil((E + 1) / 64)
  int idx = lane * chunk;
  int v = idx <= E ? tile_start[idx] : INT_MAX;
  const int seg = 63 - __clzll(__ballot(v <= i));   // lane 0 always qualifies
  idx = seg * chunk + lane;
  v = (lane < chunk && idx <= E) ? tile_start[idx] : INT_MAX;
  return seg * chunk + (63 - __clzll(__ballot(v <= i)));
}

// Exclusive prefix sum over the 64 lanes of a wave; `total` gets the sum.
__device__ __forceinline__ int wave_exclusive_sum(int v, int lane, int& total) {
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(inc, d);
    if (lane >= d) inc += u;
  }
  total = __shfl(inc, 63);
  return inc - v;
}

// Slots of expert e (0 when e >= E): offsets has E + 1 entries.
__device__ __forceinline__ int expert_slots(const int32_t* offsets, int E, int e) {
  return offsets[min(e + 1, E)] - offsets[min(e, E)];
}

constexpr int kRankedExperts = 256;             // tile_of_rank: C <= 4

// Long tiles (more than 32 slots) and short ones among the experts
// lane + 64 j, j < C (C = ceil(E / 64) <= 4): expert e with n slots has
// (n + 31) / 64 long tiles and ceil(n / 64) in all.  Consecutive lanes read
// consecutive offsets, and every load is issued before the first is used.

__device__ __forceinline__ void lane_tiles(const int32_t* offsets, int E, int lane, int C,
                                           int& hs, int& ls) {
  int n[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) n[j] = j < C ? expert_slots(offsets, E, 64 * j + lane) : 0;
  hs = 0;
  ls = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int h = (n[j] + 31) >> 6;
    hs += h;
    ls += ((n[j] + 63) >> 6) - h;
  }
}

// Routed tile of rank i.  A tile of more than 32 slots runs two 32-token
// MFMA tiles (twice the matrix-core and rescale work of a smaller one), so
// ranks 0 .. H-1 are the tiles of more than 32 slots (an expert's full
// tiles, then its last tile if that holds more than 32 slots) and ranks
// H .. the experts' last tiles of 1 .. 32 slots.  Workgroups start in rank
// order: the long tiles start first and the short ones fill in behind them,
// instead of two long tiles meeting on one compute unit at the end.  Within
// each kind the order is lane-major over the experts lane + 64 j: one
// wave-wide scan of the lanes' counts finds the lane holding rank i, a
// second over that lane's experts (at most 4) the expert.  For E <= 256
// only: with more experts each wave's loads of the counts (two per 64
// experts) took longer than the reordering gained (2048 experts of 256 x 512
// with one slot each: 62 -> 93 us), and tiles keep the sort's order there.
// -> e, and t, the tile's index among the expert's ceil(n / 64) tiles (the
// count tile_start holds); e = -1 only for a rank past the last tile.
__device__ __forceinline__ void tile_of_rank(const int32_t* offsets, int E, int i, int lane,
                                             int& e_out, int& t_out) {
  const int C = (E + 63) >> 6;
  int hs, ls;
  lane_tiles(offsets, E, lane, C, hs, ls);
  int H, L;
  const int hbase = wave_exclusive_sum(hs, lane, H);
  const int lbase = wave_exclusive_sum(ls, lane, L);
  const bool heavy = i < H;                     // uniform
  const int tgt = heavy ? i : i - H;
  const int base = heavy ? hbase : lbase;
  const int cnt = heavy ? hs : ls;
  const uint64_t hit = __ballot(cnt > 0 && tgt >= base && tgt < base + cnt);
  const int src = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
  const int B = __shfl(base, src);
  int c = 0, h = 0;
  if (lane < C) {
    const int n = expert_slots(offsets, E, src + 64 * lane);
    h = (n + 31) >> 6;
    c = heavy ? h : ((n + 63) >> 6) - h;
  }
  int all;
  const int ex = B + wave_exclusive_sum(c, lane, all);
  const uint64_t hit2 = __ballot(c > 0 && tgt >= ex && tgt < ex + c);
  if (hit == 0 || hit2 == 0) {
    e_out = -1;
    t_out = 0;
    return;
  }
  const int jj = __ffsll((unsigned long long)hit2) - 1;
  e_out = src + 64 * jj;
  t_out = heavy ? tgt - __shfl(ex, jj) : __shfl(h, jj);
}

__global__ __launch_bounds__(512) void gemm_f16_kernel(GemmF16Params p) {
  __shared__ StageF16 sm[2];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int N = p.N, K = p.K;
  const int64_t row_bytes = (int64_t)(K / 32) * 10;
  const int nb = K / 32;
  const int stages = nb / BKB;

  // tile -> (tokens, rows): XCD-aware order over (m, n) tiles as in gemm.hip
  int tile = blockIdx.x;
  if (p.tiles % kXcds == 0)
    tile = (blockIdx.x % kXcds) * (p.tiles / kXcds) + blockIdx.x / kXcds;
  const int m0 = (tile % p.m_tiles) * BM;
  const int n0 = (tile / p.m_tiles) * BN;

  RolesF16 ro;
  {
    const int di = kDecoders * wave + lane;
    ro.dec = wave < 4 && lane < kDecoders;
    ro.drow = di >> 1;
    ro.dblk = di & 1;
    ro.w = p.w + (int64_t)min(n0 + ro.drow, N - 1) * row_bytes;
    ro.atok = tid >> 1;
    ro.ablk = tid & 1;
    const int64_t tok = min(m0 + ro.atok, p.M - 1);
    ro.q = p.q + tok * K + ro.ablk * 32;
    ro.d = p.d + tok * nb + ro.ablk;
  }

  v4f acc[kRowTiles][2];
#pragma unroll
  for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Software pipeline: iteration s computes stage s from one LDS buffer,
  // then stages s + 1 (already in registers) into the other and loads s + 2
  // from memory; one barrier per stage.
  PrefetchF16 f;
  fetch(f, ro, 0);
  stage_to_lds(f, sm[0], ro);
  fetch(f, ro, stages > 1 ? BKB : 0);
  __syncthreads();
  // Waves 0..3 compute a stage and then stage the next one; waves 4..7 do it
  // the other way round, so that the two waves of a SIMD are out of phase
  // (97.9 -> 93.4 us on 512 x 14336 x 4096).  Two copies of the loop, so
  // that the accumulators never meet a branch.
  if (wave < 4) {
    for (int s = 0; s + 1 < stages; ++s) {
      compute_stage(sm[s & 1], wave, lane, acc);
      stage_to_lds(f, sm[(s + 1) & 1], ro);
      fetch(f, ro, (s + 2 < stages ? s + 2 : stages - 1) * BKB);
      __syncthreads();
    }
  } else {
    for (int s = 0; s + 1 < stages; ++s) {
      stage_to_lds(f, sm[(s + 1) & 1], ro);
      fetch(f, ro, (s + 2 < stages ? s + 2 : stages - 1) * BKB);
      compute_stage(sm[s & 1], wave, lane, acc);
      __syncthreads();
    }
  }
  compute_stage(sm[(stages - 1) & 1], wave, lane, acc);

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
        if (m < p.M) p.y[(int64_t)m * N + n] = acc[rt][t][r];
      }
  }
}

// ---------------------------------------------------------------------------
// Routed product (tokens sorted by expert).  A routed tile holds few tokens
// (~32 per expert in a 512-token prompt), so the dense layout above would
// move every decoded weight through LDS for little reuse.  Here each wave
// owns 32 weight rows and decodes its MFMA operand A straight into
// registers; only the activations go through LDS.  One 16-k MFMA step takes
// eight weights of each half of a block (lanes 0-31: half 0, lanes 32-63:
// half 1), so a lane decodes one half: the halves' scales are folded into
// the operand, and the step's sum over both halves is still the block's
// sum.  The activations are laid out to match: for token m and block b the
// LDS row holds, per step j, half 0's eight values then half 1's.

// Twelve waves of 32 rows: 384 rows per workgroup, one workgroup per compute
// unit (161 registers, three waves per SIMD).  A token tile's activations
// are staged once per 384 rows instead of once per 128 (the former
// four-wave workgroups): 179.7 -> 158.8 us on the 512-token workload
// (alternating timings), outputs bit-identical.
constexpr int kMoeWaves = 12;
constexpr int kMoeRows = 32 * kMoeWaves;      // weight rows per workgroup
constexpr int kMoeTokens = 64;                // slots per tile: two 32-token MFMA tiles
constexpr int kMoeKB = 8;                     // blocks per activation stage
constexpr int kMoeActRow = kMoeKB * 64 + 16;  // fp16 bytes of one token's stage (+ pad)

struct __align__(16) MoeStage {
  uint8_t ah[kMoeTokens * kMoeActRow];
  float ad[kMoeKB][kMoeTokens];
};

// A stage's 8 blocks of one weight row are 80 contiguous bytes, 16-byte
// aligned (a row is a whole number of 80-byte groups): five 16-byte loads.
// Pair p of blocks (2p, 2p + 1) is dwords 5p .. 5p + 4 of them.
__device__ __forceinline__ void load_quad(uint4& x, const uint8_t* row, int kb, int k) {
  x = reinterpret_cast<const uint4*>(row + (int64_t)kb * 10)[k];
}
__device__ __forceinline__ WPair pair0(const uint4 (&W)[5]) { return {W[0].x, W[0].y, W[0].z, W[0].w, W[1].x}; }
__device__ __forceinline__ WPair pair1(const uint4 (&W)[5]) { return {W[1].y, W[1].z, W[1].w, W[2].x, W[2].y}; }
__device__ __forceinline__ WPair pair2(const uint4 (&W)[5]) { return {W[2].z, W[2].w, W[3].x, W[3].y, W[3].z}; }
__device__ __forceinline__ WPair pair3(const uint4 (&W)[5]) { return {W[3].w, W[4].x, W[4].y, W[4].z, W[4].w}; }

// One block of a stage's activations for one thread: token t % 64, block
// t / 64 (threads 0..511); in a tile of at most 32 slots, token t % 32 and
// block t / 32 (threads 0..255).  Staging the tile's real tokens only
// halves those tiles' conversion work.
struct ActBlock {
  uint4 q0, q1;
  float d0;
};

__device__ __forceinline__ void load_act(ActBlock& a, const int8_t* qrow, const float* drow,
                                         int kb) {
  const uint4* src = reinterpret_cast<const uint4*>(qrow + (int64_t)kb * 32);
  a.q0 = src[0];
  a.q1 = src[1];
  a.d0 = drow[kb];
}

__device__ __forceinline__ void store_act_block(uint4 lo_half, uint4 hi_half, float d,
                                                MoeStage& st, int m, int b) {
  uint8_t* row = st.ah + m * kMoeActRow + b * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 v = h ? hi_half : lo_half;
    const uint32_t X[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[8];
    act_half_f16(X, o);
    // step 0 takes values o[0..3] of both halves, step 1 values o[4..7]
    *reinterpret_cast<uint4*>(row + h * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4*>(row + 32 + h * 16) = make_uint4(o[4], o[5], o[6], o[7]);
  }
  st.ad[b][m] = d;
}

// Block b of the stage: this lane's B operands (both steps) and activation
// scale in each token tile (the second only when the tile holds more than 32
// slots), read from LDS one block ahead of their products.
struct MoeB {
  v8h b0[2], b1[2];
  float dd[2];
};

__device__ __forceinline__ void moe_b(const MoeStage& st, int b, int lane, bool two, MoeB& o) {
  const int kh = lane >> 5;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1 && !two) break;
    const int m = t * 32 + (lane & 31);
    const uint8_t* row = st.ah + m * kMoeActRow + b * 64 + kh * 16;
    o.b0[t] = *reinterpret_cast<const v8h*>(row);
    o.b1[t] = *reinterpret_cast<const v8h*>(row + 32);
    o.dd[t] = st.ad[b][m];
  }
}

// The block's sums (two 16-k steps) in each token tile ...
__device__ __forceinline__ void moe_mma(v8h a0, v8h a1, const MoeB& B, bool two, v16f (&c)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1 && !two) break;
    c[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, B.b0[t], v16f{}, 0, 0, 0);
    c[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, B.b1[t], c[t], 0, 0, 0);
  }
}

// ... rescaled by the activation scale and added to acc.
__device__ __forceinline__ void moe_scale(const MoeB& B, const v16f (&c)[2], bool two,
                                          v16f (&acc)[2]) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t == 1 && !two) break;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = fmaf(B.dd[t], c[t][r], acc[t][r]);
  }
}

__global__ __launch_bounds__(64 * kMoeWaves) void moe_gemm_kernel(GemmF16Params p) {
  __shared__ MoeStage sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kh = lane >> 5;
  const int N = p.N, K = p.K;
  const int64_t row_bytes = (int64_t)(K / 32) * 10;
  const int nb = K / 32;
  const int nst = nb / kMoeKB;                  // K % 256 == 0

  // token tile of rank i runs on XCD i % 8 with all of its row tiles (its
  // gathered activations stay in that XCD's L2), tiles of more than 32 slots
  // first up to 256 experts; workgroups past the last tile leave
  const int x = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
  const int i = kXcds * (k / p.n_tiles) + x;
  if (i >= p.tile_start[p.E]) return;
  int e, t;
  if (p.E <= kRankedExperts) {
    tile_of_rank(p.offsets, p.E, i, lane, e, t);
    if (e < 0) return;                          // uniform
  } else {
    e = expert_of_tile(p.tile_start, p.E, i, lane);
    t = i - p.tile_start[e];
  }
  const int start = p.offsets[e] + t * kMoeTokens;
  const int rows = min(kMoeTokens, p.offsets[e + 1] - start);
  const int n0 = (k % p.n_tiles) * kMoeRows;
  const bool two = rows > 32;                   // uniform

  // this lane's weight row; this thread's activation token and blocks
  const int n = n0 + wave * 32 + (lane & 31);
  const uint8_t* wrow = p.w + (int64_t)e * N * row_bytes + (int64_t)(n < N ? n : 0) * row_bytes;
  // (consecutive lanes take consecutive tokens: their 16-byte LDS stores,
  // 528 bytes apart, fall on distinct banks).  A tile of at most 32 slots
  // stages only its first 32 token rows.  Whole waves stage or idle.
  const bool act_on = tid < (two ? 8 * 64 : 8 * 32);
  const int am = two ? tid & 63 : tid & 31;
  const int ab = act_on ? (two ? tid >> 6 : tid >> 5) : 0;
  const int token = p.order[start + min(am, rows - 1)] / p.top_k;
  const int8_t* qrow = p.q + (int64_t)token * K + ab * 32;
  const float* drow = p.d + (int64_t)token * nb + ab;

  v16f acc[2] = {v16f{}, v16f{}};
  uint4 W[5];                                   // the stage's 80 bytes of this row
#pragma unroll
  for (int k = 0; k < 5; ++k) load_quad(W[k], wrow, 0, k);
  ActBlock ap;

  // Per stage: this stage's activations (loaded during the previous one) go
  // into LDS between two barriers and the next stage's are loaded; then the
  // 8 blocks, software-pipelined: block b's products are issued, then block
  // b + 1's B operands are read and its A operands decoded while they run,
  // then block b is rescaled (its products are only read once the next
  // block's decode has covered their latency).  The B operands alternate
  // between two named sets, so that no block copies them, and a scheduling
  // barrier per block keeps the compiler from hoisting further (without it
  // the kernel took 256 registers and spilled).  One copy of the loop per
  // tile kind (one or two 32-token MFMA tiles), so that no block branches on
  // it: with a branch per block the compiler copied the 32 accumulator
  // registers back and forth around it.
#define RFP2_MOE_STEP(TWO, b, BC, BN, NEXT)                     \
    moe_mma(a0, a1, BC, TWO, c);                                \
    if ((b) < kMoeKB - 1) moe_b(sm, (b) + 1, lane, TWO, BN);    \
    NEXT;                                                       \
    moe_scale(BC, c, TWO, acc);                                 \
    __builtin_amdgcn_sched_barrier(0);
#define RFP2_MOE_LOOP(TWO)                                                           \
  if (act_on) load_act(ap, qrow, drow, 0);                                           \
  for (int s = 0; s < nst; ++s) {                                                    \
    const int kb_next = min(s + 1, nst - 1) * kMoeKB;   /* past the end: re-read */  \
    __syncthreads();                          /* every wave is done with sm */       \
    if (act_on) {                                                                    \
      store_act_block(ap.q0, ap.q1, ap.d0, sm, am, ab);                              \
      load_act(ap, qrow, drow, kb_next);                                             \
    }                                                                                \
    __syncthreads();                                                                 \
    MoeB bx, by;                                                                     \
    v16f c[2];                                                                       \
    v8h a0, a1;                                                                      \
    moe_b(sm, 0, lane, TWO, bx);                                                     \
    decode_half<0>(pair0(W), kh, a0, a1);                                            \
    RFP2_MOE_STEP(TWO, 0, bx, by, decode_half<1>(pair0(W), kh, a0, a1); load_quad(W[0], wrow, kb_next, 0)) \
    RFP2_MOE_STEP(TWO, 1, by, bx, decode_half<0>(pair1(W), kh, a0, a1))             \
    RFP2_MOE_STEP(TWO, 2, bx, by, decode_half<1>(pair1(W), kh, a0, a1); load_quad(W[1], wrow, kb_next, 1)) \
    RFP2_MOE_STEP(TWO, 3, by, bx, decode_half<0>(pair2(W), kh, a0, a1))             \
    RFP2_MOE_STEP(TWO, 4, bx, by, decode_half<1>(pair2(W), kh, a0, a1); load_quad(W[2], wrow, kb_next, 2)) \
    RFP2_MOE_STEP(TWO, 5, by, bx, decode_half<0>(pair3(W), kh, a0, a1))             \
    RFP2_MOE_STEP(TWO, 6, bx, by, decode_half<1>(pair3(W), kh, a0, a1); load_quad(W[3], wrow, kb_next, 3); load_quad(W[4], wrow, kb_next, 4)) \
    RFP2_MOE_STEP(TWO, 7, by, bx, (void)0)                                          \
  }
  if (two) {
    RFP2_MOE_LOOP(true)
  } else {
    RFP2_MOE_LOOP(false)
  }
#undef RFP2_MOE_LOOP
#undef RFP2_MOE_STEP

  // lane -> token, register r -> row; rows n..n+3 of a register group are
  // contiguous in y, so whole groups go out as one 16-byte store
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int m = t * 32 + (lane & 31);
    if (m >= rows) continue;
    float* yr = p.y + (int64_t)p.order[start + m] * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nn = n0 + wave * 32 + 8 * g + 4 * kh;
      const v16f& v = acc[t];
      if (vec && nn + 3 < N) {
        *reinterpret_cast<float4*>(yr + nn) =
            make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (nn + q < N) yr[nn + q] = v[4 * g + q];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f16(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                           const float* d, int64_t M, float* y, hipStream_t stream) {
  GemmF16Params p{};
  p.w = w; p.N = (int)N; p.K = (int)K; p.q = q; p.d = d; p.y = y; p.M = (int)M;
  p.m_tiles = (int)((M + BM - 1) / BM);
  const int n_tiles = (int)((N + BN - 1) / BN);
  p.tiles = p.m_tiles * n_tiles;
  hipLaunchKernelGGL(gemm_f16_kernel, dim3((uint32_t)p.tiles), dim3(512), 0, stream, p);
  return hipGetLastError();
}

int moe_gemm_tile_tokens() { return kMoeTokens; }

// Workgroups of the routed product: every row tile of the most token tiles
// any routing of S slots over E experts can need (at most one partly filled
// tile per expert that has slots), rounded up to whole rounds of the XCDs.
int64_t moe_gemm_max_grid(int64_t E, int64_t N, int64_t S) {
  const int64_t max_tiles = (S + kMoeTokens - 1) / kMoeTokens + std::min<int64_t>(E, S);
  const int64_t per_xcd = (max_tiles + kXcds - 1) / kXcds;
  return (int64_t)kXcds * ((N + kMoeRows - 1) / kMoeRows) * per_xcd;
}

// Routed product over slots already sorted by expert (offsets, tile_start,
// order as written by the sort kernel with tile rows = moe_gemm_tile_tokens()).
hipError_t launch_moe_gemm_sorted(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                  const int32_t* offsets, const int32_t* tile_start,
                                  const int32_t* order, int64_t S, int64_t top_k,
                                  const int8_t* q, const float* d, float* y,
                                  hipStream_t stream) {
  GemmF16Params p{};
  p.w = w; p.N = (int)N; p.K = (int)K; p.q = q; p.d = d; p.y = y;
  p.offsets = offsets; p.tile_start = tile_start; p.order = order;
  p.E = (int)E; p.top_k = (int)top_k;
  p.n_tiles = (int)((N + kMoeRows - 1) / kMoeRows);
  const int64_t grid = moe_gemm_max_grid(E, N, S);
  hipLaunchKernelGGL(moe_gemm_kernel, dim3((uint32_t)grid), dim3(64 * kMoeWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace rfp2
