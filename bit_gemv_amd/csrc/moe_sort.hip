// Routed slots grouped by expert: the token order of a prompt batch through
// the routed experts ("ROCmFP2 codebook research report", "04 · Measured
// evidence" and "07 · Recipe decision": the method pays off on large expert
// tensors where prefill dominates, and a prefill product wants each expert's
// tokens together).
//
// Slot s = t * top_k + j carries expert ids[s].  The result lists, for every
// expert in turn, its slots in increasing slot order (slots whose id is not
// in [0, E) are left out): expert e's slots are order[offsets[e] ..
// offsets[e+1]).  With tile_rows > 0 the kernel also numbers the tiles of
// tile_rows slots that a grouped product cuts each expert's slots into:
// expert e owns tiles tile_start[e] .. tile_start[e+1] - 1.
//
// One workgroup of 256 threads (the slot lists of a prompt batch are a few
// thousand entries).  Wave w owns a contiguous chunk of the slots and a row
// of per-expert counters in LDS: it counts its chunk, one block-wide scan
// turns the counters into each (expert, wave) pair's first position (expert
// major, wave minor: the stable order), and each wave then places its chunk.
// Inside a 64-slot group a slot's rank among the group's earlier slots of
// the same expert comes from a per-(wave, expert) 64-bit lane mask in LDS:
// every lane ORs in its own bit and reads the mask back, so the cost does not
// grow with the number of distinct experts in the group.  The waves never
// wait for each other while counting or placing.
#include "rfp2_internal.h"

namespace rfp2 {

namespace {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kRegGroups = 16;                  // 64-slot groups a wave keeps in registers

// Ids of up to kRegGroups consecutive 64-slot groups of [base, hi), one per
// lane and group, all loads issued before any is used (-1 past the end).
__device__ __forceinline__ void load_groups(const int32_t* __restrict__ ids, int base, int hi,
                                            int lane, int (&ev)[kRegGroups]) {
#pragma unroll
  for (int i = 0; i < kRegGroups; ++i) {
    const int s = base + 64 * i + lane;
    ev[i] = s < hi ? ids[s] : -1;
  }
}

// Position of each lane's slot among the wave's slots of the same expert so
// far.  `run` holds the wave's running count per expert, `mask` one zeroed
// 64-bit word per expert.  The lanes of one expert find each other through
// its mask word; the lowest of them advances the running count and clears
// the word.  (A wave's LDS operations complete in issue order, so every OR
// lands before the read-back and every read before the clear.)
__device__ __forceinline__ int place_in_wave(int e, bool valid, int lane, int* run,
                                             unsigned long long* mask) {
  int at = 0, rank = 0;
  if (valid) {
    atomicOr(&mask[e], 1ull << lane);
    __builtin_amdgcn_wave_barrier();
    const unsigned long long same = mask[e];
    at = run[e];
    __builtin_amdgcn_wave_barrier();
    rank = __popcll(same & ((1ull << lane) - 1));
    if (rank == 0) {
      run[e] = at + __popcll(same);
      mask[e] = 0;
    }
  }
  return at + rank;
}

__global__ __launch_bounds__(kSortThreads) void moe_sort_kernel(
    const int32_t* __restrict__ ids, int S, int E, int tile_rows,
    int32_t* __restrict__ offsets, int32_t* __restrict__ tile_start,
    int32_t* __restrict__ order, int32_t* __restrict__ err, float* __restrict__ y, int N) {
  // [kSortWaves][E] lane masks, then [kSortWaves][E] counts / cursors
  extern __shared__ unsigned long long smem[];
  __shared__ int wave_total[2][kSortWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  unsigned long long* masks = smem + wave * E;
  int* cnt = reinterpret_cast<int*>(smem + kSortWaves * E);
  int* mine = cnt + wave * E;                   // this wave's counters
  // wave w's slots: [w * chunk, min((w + 1) * chunk, S)), chunk a multiple of 64
  const int chunk = ((S + kSortWaves * 64 - 1) / (kSortWaves * 64)) * 64;
  const int lo = min(wave * chunk, S), hi = min(lo + chunk, S);
  const bool in_regs = chunk <= kRegGroups * 64;   // uniform over the workgroup

  for (int i = tid; i < kSortWaves * E; i += kSortThreads) {
    smem[i] = 0;
    cnt[i] = 0;
  }
  __syncthreads();

  // pass 1: count per (wave, expert); with in_regs the ids and each slot's
  // position inside its wave's slots of that expert stay in registers
  int ev[kRegGroups], pos[kRegGroups];
#pragma unroll
  for (int i = 0; i < kRegGroups; ++i) ev[i] = -1;   // an empty chunk places nothing
  bool bad = false;
  for (int base = lo; base < hi; base += kRegGroups * 64) {
    load_groups(ids, base, hi, lane, ev);
#pragma unroll
    for (int i = 0; i < kRegGroups; ++i) {
      const int s = base + 64 * i + lane;
      const bool valid = ev[i] >= 0 && ev[i] < E;
      if (!valid && s < hi) {
        bad = true;
        if (y != nullptr)                    // a bad slot's output row is NaN
          for (int n = 0; n < N; ++n) y[(int64_t)s * N + n] = __builtin_nanf("");
      }
      pos[i] = place_in_wave(ev[i], valid, lane, mine, masks);
    }
  }
  if (bad && err != nullptr) err[0] = 1;
  __syncthreads();

  // totals per expert and an exclusive scan over the experts (thread t owns
  // the experts t * per .. t * per + per - 1); each (expert, wave) counter
  // then becomes that pair's first position: expert major, wave minor, the
  // stable order
  const int per = (E + kSortThreads - 1) / kSortThreads;
  const int e_lo = min(tid * per, E), e_hi = min(e_lo + per, E);
  int a = 0, b = 0;
  for (int e = e_lo; e < e_hi; ++e) {
    int c = 0;
    for (int w = 0; w < kSortWaves; ++w) c += cnt[w * E + e];
    a += c;
    b += tile_rows > 0 ? (c + tile_rows - 1) / tile_rows : 0;
  }
  const int own_a = a, own_b = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int xa = __shfl_up(a, o, 64), xb = __shfl_up(b, o, 64);
    if (lane >= o) {
      a += xa;
      b += xb;
    }
  }
  if (lane == 63) {
    wave_total[0][wave] = a;
    wave_total[1][wave] = b;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    a += wave_total[0][w];
    b += wave_total[1][w];
  }
  int sa = a - own_a, sb = b - own_b;           // exclusive starts
  for (int e = e_lo; e < e_hi; ++e) {
    offsets[e] = sa;
    if (tile_start != nullptr) tile_start[e] = sb;
    int c = 0;
    for (int w = 0; w < kSortWaves; ++w) {
      const int cw = cnt[w * E + e];
      cnt[w * E + e] = sa + c;
      c += cw;
    }
    sa += c;
    sb += tile_rows > 0 ? (c + tile_rows - 1) / tile_rows : 0;
  }
  if (tid == kSortThreads - 1) {                // inclusive totals
    offsets[E] = a;
    if (tile_start != nullptr) tile_start[E] = b;
  }
  __syncthreads();

  // pass 2: store each slot at its expert's first position for this wave
  // plus its place among the wave's slots of that expert
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kRegGroups; ++i) {
      const int s = lo + 64 * i + lane;
      if (ev[i] >= 0 && ev[i] < E) order[mine[ev[i]] + pos[i]] = s;
    }
  } else {                                      // long chunks: ranks recomputed
    for (int base = lo; base < hi; base += kRegGroups * 64) {
      load_groups(ids, base, hi, lane, ev);
#pragma unroll
      for (int i = 0; i < kRegGroups; ++i) {
        const bool valid = ev[i] >= 0 && ev[i] < E;
        const int p = place_in_wave(ev[i], valid, lane, mine, masks);
        if (valid) order[p] = base + 64 * i + lane;
      }
    }
  }
}

}  // namespace

hipError_t launch_moe_sort(const int32_t* ids, int64_t S, int64_t E, int64_t tile_rows,
                           int32_t* offsets, int32_t* tile_start, int32_t* order,
                           int32_t* err, float* y, int64_t N, hipStream_t stream) {
  // lane masks (8 bytes) and counters (4 bytes) per wave and expert
  const size_t lds = (size_t)kSortWaves * E * 12;
  hipLaunchKernelGGL(moe_sort_kernel, dim3(1), dim3(kSortThreads), lds, stream, ids, (int)S,
                     (int)E, (int)tile_rows, offsets, tile_start, order, err, y, (int)N);
  return hipGetLastError();
}

// Workspace of the grouped routed product: offsets [E+1], tile_start [E+1]
// and order [S], int32 each.
size_t moe_gemm_workspace_bytes(int64_t E, int64_t S) {
  const size_t b = 4 * (size_t)(2 * (E + 1) + S);
  return (b + 255) & ~size_t(255);
}

hipError_t launch_moe_gemm(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                           const int32_t* ids, int64_t T, int64_t top_k, const int8_t* q,
                           const float* d, float* y, int32_t* err, void* workspace,
                           hipStream_t stream) {
  const int64_t S = T * top_k;
  int32_t* offsets = static_cast<int32_t*>(workspace);
  int32_t* tile_start = offsets + (E + 1);
  int32_t* order = tile_start + (E + 1);
  const hipError_t e = launch_moe_sort(ids, S, E, moe_gemm_tile_tokens(), offsets,
                                       tile_start, order, err, y, N, stream);
  if (e != hipSuccess) return e;
  return launch_moe_gemm_sorted(w, E, N, K, offsets, tile_start, order, S, top_k, q, d, y,
                                stream);
}

}  // namespace rfp2
