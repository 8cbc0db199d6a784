// ROCmFP2 GEMV for a few activation columns, and its routed-expert form.
//
// Method ("ROCmFP2 codebook research report", "03 · Runtime"): every code
// byte is expanded once into four int8 lanes, each 16-weight half is dotted
// with the int8 activations into an int32 sum, and only then are the two
// weight scales and the activation scale applied,
//   y += d_a * (s_0 * S_0 + s_1 * S_1).
// The multi-column form ("Why AMD-friendly does not mean always faster")
// expands a block once and reuses it for every activation column.
//
// gfx950 mapping
//   * The stored matrix is one contiguous stream of 10-byte blocks.  K is a
//     multiple of 256, so a row is a whole number of 80-byte groups (8 blocks,
//     five 16-byte pieces).  A lane owns whole groups: no block straddles two
//     lanes.
//   * A workgroup of wk waves computes S = 64/L rows.  Inside a wave, L lanes
//     (a power of two) share a row; across the waves the row's G = K/256
//     groups are split, so G = L * wk * J with J groups per lane (usually 1).
//     Splitting K over waves, rather than giving one wave many groups per
//     lane, keeps several waves per SIMD: while one wave decodes, the others'
//     loads are in flight.  The row sum is a log2(L)-step xor shuffle inside
//     the wave, then one LDS pass across the waves.
//   * Weights move HBM -> LDS with direct loads (global_load_lds_dwordx4) in
//     which consecutive lanes fetch consecutive 16-byte pieces, so every load
//     instruction touches whole cache lines; each lane then reads its 80-byte
//     group from LDS (conflict-free: lanes are 20 dwords apart).  Loading the
//     80 bytes per lane straight into registers instead spreads each
//     instruction over ~40 cache lines and was measured ~1.3x slower.
//   * Every global load is a direct-to-LDS load issued as inline asm, with
//     explicit vmcnt waits: the activations of the wave's groups and their
//     scales first (L2 hits), then the first chunk(s) of weights; the wave
//     waits only for the activations, transposes them in place, and the
//     weights keep streaming.  The next chunk (J > 1) is requested as soon as
//     the current one is in registers.  (The compiler's own form of these
//     loads makes it wait for all of them before any LDS access.)
//   * Activations sit in LDS as 17 pieces of 16 bytes per (column, group):
//     16 halves, each transposed to the lane order of the expanded weights
//     (see expand_half), and one pad piece so that the lanes of a row, which
//     read neighbouring groups, hit different banks.  The per-block scales
//     sit in an array of their own.
//   * Two to eight columns (dense, or a routed group of several tokens)
//     take the int32 half sums from the matrix cores instead of dot4 chains:
//     v_mfma_i32_4x4x4_16b_i8 is sixteen 4x4x4 products, one per quad of
//     lanes, so a quad holds four rows at the same group (their expanded
//     weight words as B) and one column's activations per lane (as A), and
//     each lane receives its row's half sums for four columns (a second set
//     of products for columns 4..7).  The integers are those of the dot4
//     chains, so the outputs are those of the dot4 form; the vector work per
//     block and column drops from 13 instructions to about 4 (16384 x 5120:
//     M = 2, 3, 4 from 10.1, 12.9, 14.0 us to 9.6, 10.2, 11.6 us; M = 8 from
//     25.3 us in two launches to 15.4 us in one).

#include "gemv_kernel.h"

#include <atomic>
#include <cstdlib>

namespace rfp2 {

namespace gemv_detail {
GemvFn pick_m1(int jt);
GemvFn pick_moe_tokens(int T, bool mf);   // gemv_moe.hip
GemvFn pick_m2(int jt);
GemvFn pick_m3(int jt);
GemvFn pick_m4(int jt);
GemvFn pick_m5(int jt);
GemvFn pick_m6(int jt);
GemvFn pick_m7(int jt);
GemvFn pick_m8(int jt);
GemvFn pick_m2_mf(int jt);
GemvFn pick_m3_mf(int jt);
GemvFn pick_m4_mf(int jt);
GemvFn pick_m5_mf(int jt);
GemvFn pick_m6_mf(int jt);
GemvFn pick_m7_mf(int jt);
GemvFn pick_m8_mf(int jt);
}  // namespace gemv_detail

namespace {

using namespace gemv_detail;

GemvFn pick_kernel(int M, int jt) {
  switch (M) {
    case 1: return pick_m1(jt);
    case 2: return pick_m2(jt);
    case 3: return pick_m3(jt);
    case 4: return pick_m4(jt);
    case 5: return pick_m5(jt);
    case 6: return pick_m6(jt);
    case 7: return pick_m7(jt);
    default: return pick_m8(jt);
  }
}

// The matrix-core form (two to eight columns; a quad of lanes is four rows
// at one group, so at most 16 lanes per row).
bool use_mf(int M, int lshift) { return M >= 2 && M <= 8 && lshift <= 4; }

GemvFn pick_mf(int M, int jt) {
  switch (M) {
    case 2: return pick_m2_mf(jt);
    case 3: return pick_m3_mf(jt);
    case 4: return pick_m4_mf(jt);
    case 5: return pick_m5_mf(jt);
    case 6: return pick_m6_mf(jt);
    case 7: return pick_m7_mf(jt);
    default: return pick_m8_mf(jt);
  }
}

struct Geometry {
  int lshift;   // log2 of lanes per row inside a wave
  int wk;       // waves per workgroup
  int J;        // groups per lane
  int jt;       // chunks in flight per wave (divides J)
  int rows;     // rows per workgroup
};

// Choose how a row's G = K/256 groups are spread: G = L * wk * J.  Measured
// on MI355X over every legal split (M = 1, 2, 4, 8; K = 2048..5120; 512 to
// 16384 rows):
//   * one group per lane for a single column (the most waves in flight);
//     two for several columns (the decode and the per-lane set-up are shared
//     by more products) when that still leaves >= 512 workgroups, else one;
//     the nearest J when the target does not divide;
//   * about four waves per workgroup (order 4, 5, 3, 6, 2, 8, 7, 1);
//   * then the most rows per workgroup (activations shared by more rows);
//   * one chunk in flight per wave: the next is requested as soon as the
//     current one is in registers, and a deeper ring costs more LDS than it
//     hides latency.
constexpr int64_t kMinWorkgroupsForJ2 = 512;
// wave slots of a compute unit the matrix-core GEMV's workgroups can use:
// five waves per SIMD up to four columns (86 registers), four beyond
int64_t wave_slots_per_cu(int M) { return M <= 4 ? 20 : 16; }

struct AnySplit {
  bool operator()(const Geometry&) const { return true; }
};

// max_ag: the most groups a wave may cover (J * L), for forms that need it;
// ok: a further condition on the split
template <typename Ok = AnySplit>
Geometry pick_geometry(int64_t K, int j_target, int max_ag = 1 << 30, Ok ok = Ok{}) {
  static constexpr int kWaveRank[kMaxWaves + 1] = {99, 7, 4, 2, 0, 1, 3, 6, 5};
  const int G = (int)(K / 256);
  Geometry best{};
  int64_t best_key = INT64_MAX;
  for (int ls = 0; ls <= 6; ++ls) {
    const int L = 1 << ls;
    if (G % L) continue;
    for (int wk = 1; wk <= kMaxWaves; ++wk) {
      if ((G / L) % wk) continue;
      const int J = G / L / wk;
      if ((J << ls) > max_ag) continue;
      if (!ok(Geometry{ls, wk, J, 1, 64 >> ls})) continue;
      // smaller is better: distance from the target J (ties: fewer groups),
      // then the wave-count rank, then fewer lanes per row (more rows)
      const int64_t key = ((int64_t)std::abs(J - j_target) << 32) |
                          ((int64_t)std::min(J, 0xFFFF) << 16) |
                          ((int64_t)kWaveRank[wk] << 8) | ls;
      if (key < best_key) {
        best_key = key;
        best = Geometry{ls, wk, J, 1, 64 >> ls};
      }
    }
  }
  return best;
}

// rows_total: the rows the launch covers (N, or N per expert times top_k)
Geometry geometry(int64_t K, int64_t M, int64_t rows_total) {
  if (M >= 2) {
    const Geometry g = pick_geometry(K, 2);
    if ((rows_total + g.rows - 1) / g.rows >= kMinWorkgroupsForJ2) return g;
  }
  return pick_geometry(K, 1);
}

// Per wave: jt chunk buffers, the activations (kGroupPieces 16-byte pieces
// per column and group) and their scales (four column slots per block in the
// matrix-core form), each rounded up to whole 64-lane loads; then the
// cross-wave partial sums.  The routed matrix-core form (exact) carves the
// activations exactly and keeps the partial sums in the chunk buffers.  Must
// match the carving in gemv_kernel.
size_t lds_bytes(int M, const Geometry& g, bool mf = false, bool exact = false) {
  const size_t ag = (size_t)g.J << g.lshift;
  const size_t act_rounds = (M * ag * kGroupPieces + 63) / 64;
  const size_t act_dwords = exact ? M * ag * kGroupPieces * 4 : act_rounds * 256;
  const size_t d_rounds = ((mf ? 4 * ((M + 3) / 4) : M) * ag * 8 + 63) / 64;
  const size_t per_wave = (size_t)g.jt * 1280 + act_dwords + d_rounds * 64;
  return (g.wk * per_wave + (exact ? 0 : (size_t)g.wk * g.rows * M)) * 4;
}

int compute_units();

// Two to four dense columns (the matrix-core form): the one-column rule's
// split as long as all of its workgroups fit on the chip at once (LDS over
// the workgroups a compute unit holds), else the first of these that does:
// one lane per row and four waves (64 rows per workgroup) if that gives
// every compute unit a workgroup, one group per lane, the split with J
// nearest 2.  A launch that needs two rounds of workgroups loses 7-60 %
// (alternating same-box timings, M = 4: 32768 x 4096 14.57 -> 13.58 us,
// 14336 x 4096 10.10 -> 8.44, 18432 x 7168 27.92 -> 17.64, 4096 x 14336
// 23.43 -> 9.64).  Where the usual split fits, it stays: one lane per row
// instead was 8 % slower at 16384 x 4096 and within 2 % at 16384 x 5120
// and 28672 x 4096.
// Whether every workgroup of an M-column launch with split g is resident at
// once (LDS and wave slots over the workgroups a compute unit holds).
bool fits_one_round(int M, const Geometry& g, int64_t rows_total) {
  const size_t lds = lds_bytes(M, g, use_mf(M, g.lshift));
  if (lds > (size_t)kMaxLdsBytesPerBlock) return false;
  const int64_t per_cu = std::max<int64_t>(
      1, std::min<int64_t>((int64_t)kMaxLdsBytesPerBlock / (int64_t)lds,
                           wave_slots_per_cu(M) / g.wk));
  return (rows_total + g.rows - 1) / g.rows <= compute_units() * per_cu;
}

Geometry columns_geometry(int64_t K, int M, int64_t rows_total) {
  const int64_t cus = compute_units();
  auto one_round = [&](const Geometry& g) { return fits_one_round(M, g, rows_total); };
  auto workgroups = [&](const Geometry& g) { return (rows_total + g.rows - 1) / g.rows; };
  const Geometry g2 = pick_geometry(K, 2);
  if (workgroups(g2) >= kMinWorkgroupsForJ2) {
    if (one_round(g2)) return g2;
  } else {
    const Geometry g1 = pick_geometry(K, 1);
    if (one_round(g1)) return g1;
  }
  const int G = (int)(K / 256);
  if (G % 4 == 0) {
    const Geometry g{0, 4, G / 4, 1, 64};
    if (workgroups(g) >= cus && one_round(g)) return g;
  }
  const Geometry g1 = pick_geometry(K, 1);
  if (one_round(g1)) return g1;
  const Geometry g = pick_geometry(K, 2, 1 << 30, one_round);
  return g.wk > 0 ? g : g1;
}

int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

// Each launch reads the whole matrix once, so the M columns should go
// through as few launches as possible.  Two to eight columns run the
// matrix-core form, all of them in one launch whenever some split of K lets
// every workgroup of that launch be resident at once, else in launches of as
// many columns as allow it.  (Before the matrix-core form took five to eight
// columns, the dot4 kernel ran up to seven in one launch when their LDS fit
// one round -- at 16384 x 5120 M = 6 and 7 took 18.6 and 20.7 us against
// 22.4 and 24.5 us as 5+1 and 6+1 columns -- and eight as 5+3, 27.3 us
// against 33.1 us in one launch, whose 157-register waves left one
// workgroup per compute unit.)  Without a matrix-core split (more than 16
// lanes per row): launches of as many dot4 columns as fit 64 KiB, or one
// round.
hipError_t launch_gemv(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream) {
  auto launch = [&](int64_t m0, int mc, const Geometry& g, bool mf) {
    const dim3 grid((uint32_t)((N + g.rows - 1) / g.rows));
    Params p{w, (int)N, (int)K, q + m0 * K, d + m0 * (K / 32), y + m0 * N,
             g.lshift, g.wk, g.J, nullptr, 0, nullptr, 1, 0, nullptr, nullptr, nullptr};
    hipLaunchKernelGGL(mf ? pick_mf(mc, g.jt) : pick_kernel(mc, g.jt), grid, dim3(64 * g.wk),
                       lds_bytes(mc, g, mf), stream, p);
    return hipGetLastError();
  };
  if (M >= 2 && M <= 8) {
    int cols = (int)M;
    Geometry g = columns_geometry(K, cols, N);
    while (cols > 2 && !(use_mf(cols, g.lshift) && fits_one_round(cols, g, N)))
      g = columns_geometry(K, --cols, N);
    if (use_mf(cols, g.lshift)) {
      for (int64_t m0 = 0; m0 < M; m0 += cols) {
        const int mc = (int)std::min<int64_t>(cols, M - m0);
        if (mc >= 2) {
          const Geometry gc = mc == cols ? g : columns_geometry(K, mc, N);
          if (use_mf(mc, gc.lshift)) {
            const hipError_t e = launch(m0, mc, gc, true);
            if (e != hipSuccess) return e;
            continue;
          }
        }
        const hipError_t e = launch(m0, mc, geometry(K, mc, N), false);
        if (e != hipSuccess) return e;
      }
      return hipSuccess;
    }
  }
  const Geometry g = geometry(K, M, N);
  const int64_t cus = compute_units();
  const int64_t grid = (N + g.rows - 1) / g.rows;
  const int64_t share = (grid + cus - 1) / cus;
  const size_t one_round = (size_t)kMaxLdsBytesPerBlock / share;
  size_t cap = kMaxLdsBytes;
  if (M <= 7 && lds_bytes((int)M, g) <= one_round) cap = std::max(cap, one_round);
  int cols = (int)M;
  while (cols > 1 && lds_bytes(cols, g) > cap) --cols;
  for (int64_t m0 = 0; m0 < M; m0 += cols) {
    const int mc = (int)std::min<int64_t>(cols, M - m0);
    const hipError_t e = launch(m0, mc, g, false);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                           const int32_t* ids, int64_t top_k, const int8_t* q,
                           const float* d, float* y, int32_t* err,
                           hipStream_t stream) {
  const Geometry g = geometry(K, 1, N * top_k);
  const dim3 grid((uint32_t)((N + g.rows - 1) / g.rows), (uint32_t)top_k);
  Params p{w, (int)N, (int)K, q, d, y, g.lshift, g.wk, g.J, ids, (int)E, err,
           (int)top_k, (int)top_k, nullptr, nullptr, nullptr};
  const GemvFn fn = pick<1, true>(g.jt);
  hipLaunchKernelGGL(fn, grid, dim3(64 * g.wk), lds_bytes(1, g), stream, p);
  return hipGetLastError();
}

// Several tokens, each routed to top_k experts: slot s = t * top_k + j.  The
// slots routed to one expert are computed together (one decode of the
// expert's rows for up to T tokens).  A group of T columns stages T times
// the activations of one, so the lanes take more groups each (J near T/2,
// at least 2): a workgroup then covers more rows and shares its staged
// activations among them.  Measured on 128 experts of 1536x4096, top-8,
// T = 2, 4, 8 with half of each token's experts shared with the token
// before: J = T/2 beats one group per lane by 2-40% (T = 8 takes 70 KB of
// LDS).  Where T columns cannot fit one workgroup's LDS even at J = 1 (the
// staged activations alone take ~1.19 * T * K bytes) the tokens are done in
// chunks, each a launch of its own.
namespace {
Geometry tokens_geometry(int64_t K, int T) {
  for (int j = std::max(2, T / 2);; --j) {
    const Geometry g = pick_geometry(K, j);
    const bool mf = use_mf(T, g.lshift);
    if (j == 1 || lds_bytes(T, g, mf, mf) <= (size_t)kMaxLdsBytesPerBlock)
      return g;
  }
}
}  // namespace

hipError_t launch_moe_gemv_tokens(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                  const int32_t* ids, int64_t T, int64_t top_k,
                                  const int8_t* q, const float* d, float* y, int32_t* err,
                                  hipStream_t stream) {
  int cols = (int)T;
  Geometry g = tokens_geometry(K, cols);
  while (cols > 1 &&
         lds_bytes(cols, g, use_mf(cols, g.lshift), use_mf(cols, g.lshift)) >
             (size_t)kMaxLdsBytesPerBlock)
    g = tokens_geometry(K, --cols);
  const int64_t nb = K / 32;
  for (int64_t t0 = 0; t0 < T; t0 += cols) {
    const int tc = (int)std::min<int64_t>(cols, T - t0);
    const int32_t* ids_c = ids + t0 * top_k;
    float* y_c = y + t0 * top_k * N;
    hipError_t e;
    if (tc == 1) {
      e = launch_moe_gemv(w, E, N, K, ids_c, top_k, q + t0 * K, d + t0 * nb, y_c, err, stream);
    } else {
      const Geometry gc = tc == cols ? g : tokens_geometry(K, tc);
      const dim3 grid((uint32_t)((N + gc.rows - 1) / gc.rows), (uint32_t)(tc * top_k));
      Params p{w, (int)N, (int)K, q + t0 * K, d + t0 * nb, y_c, gc.lshift, gc.wk, gc.J,
               ids_c, (int)E, err, (int)top_k, (int)(tc * top_k), nullptr, nullptr, nullptr};
      const bool mf = use_mf(tc, gc.lshift);
      hipLaunchKernelGGL(gemv_detail::pick_moe_tokens(tc, mf), grid, dim3(64 * gc.wk),
                         lds_bytes(tc, gc, mf, mf), stream, p);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// One token: quantize the activations inside the product kernel when every
// wave's slice is at most 4 groups (64 halves, one per lane; J*L <= 4) and
// the call reads at most 128 MiB of weights, or in the cases below, else the
// separate quantization kernel followed by the product.  q and d are
// written either way.  Every
// wave of the fused kernel quantizes its own slice (about a fifth of its
// vector work), which pays for the second launch it saves only while the
// launch is a large part of the call: one-token steps at K = 5120 took 8.0 /
// 14.7 / 24.0 / 33.7 / 46.0 us fused against 9.9 / 15.3 / 23.9 / 33.3 /
// 43.0 us as two launches at 25, 50, 100, 150 and 200 MiB of weights.
// Where the one-column geometry gives the waves wider slices (K = 6144 and
// 8192: 8 groups on 3 or 4 waves), the fused launch takes the best geometry
// with at most 4 groups per wave instead (6 or 8 waves) up to 64 MiB: at
// K = 8192 and 5, 10, 20, 40, 60 MiB of weights 4.8 / 5.2 / 7.5 / 12.0 /
// 17.6 us against 6.4 / 7.5 / 9.0 / 13.6 / 17.6 us as two launches, within
// 2 % either way from 50 to 80 MiB.  Wider still (K = 10240 ... 16384), each
// lane quantizes two halves (8 groups per wave) up to 64 MiB: with two groups
// per lane and 4 lanes per row (16 rows per workgroup, so each workgroup's
// quantization serves twice the rows of a one-group split) when that still
// gives every compute unit a workgroup, else with one group per lane (8
// rows).  Against two launches: K = 14336 at 17.5 / 35 / 61 MiB 7.4 / 11.2
// / 19.3 us against 9.1 / 14.0 / 20.3 us; K = 16384 at 20 / 40 / 60 MiB 7.6 /
// 12.0 / 16.5 us against 10.7 / 15.6 / 21.1 us; with 2048 rows (128
// workgroups of 16 rows) the 8-row split is 11-13 % faster than the 16-row
// one.
constexpr int64_t kMaxFusedWeightBytes = int64_t(128) << 20;
constexpr int64_t kMaxFusedOwnGeometryBytes = int64_t(64) << 20;
constexpr int64_t kMaxFusedTwoHalvesBytes = int64_t(64) << 20;
constexpr int kMaxFusedGroups = 4;        // one half per lane
constexpr int kMaxFusedGroups2 = 8;       // two halves per lane

// Halves per lane of the one quantizing launch for a one-token call (g set),
// or 0 when the call runs the two kernels.
int quant_geometry(int64_t K, int64_t rows_total, int64_t weight_bytes, Geometry& g) {
  g = geometry(K, 1, rows_total);
  if (g.jt != 1) return 0;
  const int ag = g.J << g.lshift;
  if (ag <= kMaxFusedGroups) return weight_bytes <= kMaxFusedWeightBytes ? 1 : 0;
  Geometry f = pick_geometry(K, 1, kMaxFusedGroups);
  if (f.wk > 0) {
    if (weight_bytes > kMaxFusedOwnGeometryBytes) return 0;
    g = f;
    return 1;
  }
  if (weight_bytes > kMaxFusedTwoHalvesBytes) return 0;
  f = pick_geometry(K, 2, kMaxFusedGroups2);
  if (f.wk > 0 && (rows_total + f.rows - 1) / f.rows >= compute_units()) {
    g = f;
    return 2;
  }
  if (ag <= kMaxFusedGroups2) return 2;
  f = pick_geometry(K, 1, kMaxFusedGroups2);
  if (f.wk == 0) return 0;                // no split gives every wave <= 8 groups
  g = f;
  return 2;
}

hipError_t launch_quant_gemv(const uint8_t* w, int64_t N, int64_t K, const float* a,
                             int8_t* q, float* d, float* y, hipStream_t stream) {
  Geometry g;
  const int qh = quant_geometry(K, N, N * (K / 32) * 10, g);
  if (qh == 0) {
    const hipError_t e = launch_quantize_acts(a, 1, K, q, d, stream);
    if (e != hipSuccess) return e;
    return launch_gemv(w, N, K, q, d, 1, y, stream);
  }
  const dim3 grid((uint32_t)((N + g.rows - 1) / g.rows));
  Params p{w, (int)N, (int)K, q, d, y, g.lshift, g.wk, g.J, nullptr, 0, nullptr, 1, 0,
           a, q, d};
  const GemvFn fn = qh == 1 ? gemv_kernel<1, 1, false, 1> : gemv_kernel<1, 1, false, 2>;
  hipLaunchKernelGGL(fn, grid, dim3(64 * g.wk), lds_bytes(1, g), stream, p);
  return hipGetLastError();
}

hipError_t launch_quant_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                 const int32_t* ids, int64_t top_k, const float* a,
                                 int8_t* q, float* d, float* y, int32_t* err,
                                 hipStream_t stream) {
  Geometry g;
  const int qh = quant_geometry(K, N * top_k, top_k * N * (K / 32) * 10, g);
  if (qh == 0) {
    const hipError_t e = launch_quantize_acts(a, 1, K, q, d, stream);
    if (e != hipSuccess) return e;
    return launch_moe_gemv(w, E, N, K, ids, top_k, q, d, y, err, stream);
  }
  const dim3 grid((uint32_t)((N + g.rows - 1) / g.rows), (uint32_t)top_k);
  Params p{w, (int)N, (int)K, q, d, y, g.lshift, g.wk, g.J, ids, (int)E, err, (int)top_k,
           (int)top_k, a, q, d};
  const GemvFn fn = qh == 1 ? gemv_kernel<1, 1, true, 1> : gemv_kernel<1, 1, true, 2>;
  hipLaunchKernelGGL(fn, grid, dim3(64 * g.wk), lds_bytes(1, g), stream, p);
  return hipGetLastError();
}

}  // namespace rfp2
