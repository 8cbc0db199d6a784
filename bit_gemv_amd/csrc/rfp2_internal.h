// Launchers behind the C ABI.  Arguments have been validated by the caller
// (rfp2_abi.hip); each launcher only sizes the grid and enqueues kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace rfp2 {

constexpr int64_t kMaxGrid = 1 << 20;   // workgroups per launch (grid-stride beyond)
constexpr int kMaxSortExperts = 2048;   // experts of a grouped (sorted) routed product
constexpr int kReadCeilingGrid = 2048;  // workgroups of the read helper (256 threads each)
constexpr size_t kNoallocScratchBytes = size_t(1) << 20;  // library-owned workspace per GPU

hipError_t launch_quantize_acts(const float* a, int64_t M, int64_t K, int8_t* q,
                                float* d, hipStream_t stream);
hipError_t launch_quantize_weights(const float* x, int64_t N, int64_t K,
                                   const float* imp, uint8_t* w, hipStream_t stream);
hipError_t launch_gemv(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream);
hipError_t launch_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                           const int32_t* ids, int64_t top_k, const int8_t* q,
                           const float* d, float* y, int32_t* err,
                           hipStream_t stream);
hipError_t launch_moe_gemv_tokens(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                  const int32_t* ids, int64_t T, int64_t top_k,
                                  const int8_t* q, const float* d, float* y, int32_t* err,
                                  hipStream_t stream);
hipError_t launch_quant_gemv(const uint8_t* w, int64_t N, int64_t K, const float* a,
                             int8_t* q, float* d, float* y, hipStream_t stream);
hipError_t launch_quant_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                 const int32_t* ids, int64_t top_k, const float* a,
                                 int8_t* q, float* d, float* y, int32_t* err,
                                 hipStream_t stream);
hipError_t launch_gemm(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                       const float* d, int64_t M, float* y, hipStream_t stream);
hipError_t launch_gemm_f16(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                           const float* d, int64_t M, float* y, hipStream_t stream);
hipError_t launch_moe_sort(const int32_t* ids, int64_t S, int64_t E, int64_t tile_rows,
                           int32_t* offsets, int32_t* tile_start, int32_t* order,
                           int32_t* err, float* y, int64_t N, hipStream_t stream);
int moe_gemm_tile_tokens();
hipError_t launch_moe_gemm_sorted(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                  const int32_t* offsets, const int32_t* tile_start,
                                  const int32_t* order, int64_t S, int64_t top_k,
                                  const int8_t* q, const float* d, float* y,
                                  hipStream_t stream);
size_t moe_gemm_workspace_bytes(int64_t E, int64_t S);
int64_t moe_gemm_max_grid(int64_t E, int64_t N, int64_t S);
hipError_t launch_moe_gemm(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                           const int32_t* ids, int64_t T, int64_t top_k, const int8_t* q,
                           const float* d, float* y, int32_t* err, void* workspace,
                           hipStream_t stream);
hipError_t launch_moe_gemm_noalloc(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                   const int32_t* ids, int64_t T, int64_t top_k,
                                   const int8_t* q, const float* d, float* y, int32_t* err,
                                   hipStream_t stream);
hipError_t launch_read_ceiling(const uint8_t* buf, int64_t bytes, uint32_t magic, uint32_t* out,
                               hipStream_t stream);
hipError_t launch_debug_decode(const uint8_t* w, int64_t N, int64_t K,
                               int8_t* codes, float* scales, hipStream_t stream);
hipError_t launch_debug_half_dots(const uint8_t* w, int64_t N, int64_t K,
                                  const int8_t* q, int64_t M, int32_t* sums,
                                  hipStream_t stream);
hipError_t launch_debug_half_sums_mf(const uint8_t* w, int64_t N, int64_t K,
                                     const int8_t* q, int64_t M, int32_t* sums,
                                     hipStream_t stream);
hipError_t launch_debug_decode_i8(const uint8_t* w, int64_t N, int64_t K, int8_t* wa,
                                  int8_t* wb, float* scales, hipStream_t stream);
hipError_t launch_debug_decode_f16(const uint8_t* w, int64_t N, int64_t K, int form,
                                   uint16_t* out, hipStream_t stream);

}  // namespace rfp2
