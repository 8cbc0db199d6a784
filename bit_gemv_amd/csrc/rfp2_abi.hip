// C ABI of the library (declared in include/rfp2.h).  Every entry point checks
// its arguments on the host and returns a status before anything is enqueued;
// no HIP call is made for a rejected call.
#include "rfp2.h"
#include "rfp2_internal.h"

namespace {

constexpr int64_t kMaxRows = int64_t(1) << 30;     // row and token counts
constexpr int64_t kMaxGemvK = 32768;               // staged activations fit LDS
constexpr int64_t kMaxSortSlots = int64_t(1) << 24;  // routed slots of one sort

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

rfp2_status from_hip(hipError_t e) {
  return e == hipSuccess ? RFP2_OK : RFP2_E_LAUNCH;
}

bool product_k_ok(int64_t K) {
  return K >= 256 && K % 256 == 0 && K <= kMaxGemvK;
}

}  // namespace

extern "C" {

int rfp2_abi_version(void) { return RFP2_ABI_VERSION; }

const char* rfp2_status_string(int status) {
  switch (status) {
    case RFP2_OK: return "ok";
    case RFP2_E_NULL: return "a required pointer is null";
    case RFP2_E_SHAPE: return "a size is out of range for this call";
    case RFP2_E_ALIGN: return "a pointer is not aligned as this call requires";
    case RFP2_E_LAUNCH: return "the HIP runtime reported an error for the launch";
    default: return "unknown status";
  }
}

rfp2_status rfp2_quantize_acts(const float* a, int64_t M, int64_t K, int8_t* q,
                               float* d, hipStream_t stream) {
  if (!a || !q || !d) return RFP2_E_NULL;
  if (M < 1 || M > kMaxRows || K < 32 || K % 32 != 0 || K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  if (!aligned(a, 16) || !aligned(q, 4) || !aligned(d, 4)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_quantize_acts(a, M, K, q, d, stream));
}

rfp2_status rfp2_quantize_weights(const float* x, int64_t N, int64_t K,
                                  uint8_t* w, hipStream_t stream) {
  if (!x || !w) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || K < 32 || K % 32 != 0 || K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  if (!aligned(x, 4) || !aligned(w, 2)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_quantize_weights(x, N, K, nullptr, w, stream));
}

rfp2_status rfp2_quantize_weights_imatrix(const float* x, int64_t N, int64_t K,
                                          const float* importance, uint8_t* w,
                                          hipStream_t stream) {
  if (!x || !importance || !w) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || K < 32 || K % 32 != 0 || K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  if (!aligned(x, 4) || !aligned(importance, 4) || !aligned(w, 2)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_quantize_weights(x, N, K, importance, w, stream));
}

rfp2_status rfp2_gemv(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                      const float* d, int64_t M, float* y, hipStream_t stream) {
  if (!w || !q || !d || !y) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || M < 1 || M > RFP2_GEMV_MAX_M || !product_k_ok(K))
    return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_gemv(w, N, K, q, d, M, y, stream));
}

rfp2_status rfp2_gemm(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                      const float* d, int64_t M, float* y, hipStream_t stream) {
  if (!w || !q || !d || !y) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || M < 1 || M > kMaxRows || K < 256 || K % 256 != 0 ||
      K > (int64_t(1) << 24))
    return RFP2_E_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) > (int64_t(1) << 31) - 1)
    return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_gemm(w, N, K, q, d, M, y, stream));
}

rfp2_status rfp2_gemm_f16(const uint8_t* w, int64_t N, int64_t K, const int8_t* q,
                          const float* d, int64_t M, float* y, hipStream_t stream) {
  if (!w || !q || !d || !y) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || M < 1 || M > kMaxRows || K < 256 || K % 256 != 0 ||
      K > (int64_t(1) << 24))
    return RFP2_E_SHAPE;
  if (((M + 127) / 128) * ((N + 127) / 128) > (int64_t(1) << 31) - 1)
    return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_gemm_f16(w, N, K, q, d, M, y, stream));
}

rfp2_status rfp2_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                          const int32_t* ids, int64_t top_k, const int8_t* q,
                          const float* d, float* y, int32_t* err,
                          hipStream_t stream) {
  if (!w || !ids || !q || !d || !y) return RFP2_E_NULL;
  if (E < 1 || E > kMaxRows || N < 1 || N > kMaxRows || top_k < 1 ||
      top_k > 65535 || !product_k_ok(K))
    return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4) ||
      !aligned(ids, 4) || (err && !aligned(err, 4)))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_moe_gemv(w, E, N, K, ids, top_k, q, d, y, err, stream));
}

rfp2_status rfp2_moe_gemv_tokens(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                 const int32_t* ids, int64_t T, int64_t top_k,
                                 const int8_t* q, const float* d, float* y, int32_t* err,
                                 hipStream_t stream) {
  if (!w || !ids || !q || !d || !y) return RFP2_E_NULL;
  if (E < 1 || E > kMaxRows || N < 1 || N > kMaxRows || T < 1 || T > RFP2_GEMV_MAX_M ||
      top_k < 1 || T * top_k > 64 || !product_k_ok(K))
    return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4) ||
      !aligned(ids, 4) || (err && !aligned(err, 4)))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(
      rfp2::launch_moe_gemv_tokens(w, E, N, K, ids, T, top_k, q, d, y, err, stream));
}

rfp2_status rfp2_moe_sort(const int32_t* ids, int64_t S, int64_t E, int32_t* offsets,
                          int32_t* order, int32_t* err, hipStream_t stream) {
  if (!ids || !offsets || !order) return RFP2_E_NULL;
  if (S < 1 || S > kMaxSortSlots || E < 1 || E > rfp2::kMaxSortExperts) return RFP2_E_SHAPE;
  if (!aligned(ids, 4) || !aligned(offsets, 4) || !aligned(order, 4) ||
      (err && !aligned(err, 4)))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_moe_sort(ids, S, E, 0, offsets, nullptr, order, err, nullptr,
                                        0, stream));
}

size_t rfp2_moe_gemm_workspace_bytes(int64_t E, int64_t T, int64_t top_k) {
  if (E < 1 || E > rfp2::kMaxSortExperts || T < 1 || top_k < 1 || T > kMaxSortSlots ||
      top_k > kMaxSortSlots || T * top_k > kMaxSortSlots)
    return 0;
  return rfp2::moe_gemm_workspace_bytes(E, T * top_k);
}

rfp2_status rfp2_moe_gemm(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                          const int32_t* ids, int64_t T, int64_t top_k, const int8_t* q,
                          const float* d, float* y, int32_t* err, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (!w || !ids || !q || !d || !y || !workspace) return RFP2_E_NULL;
  const size_t need = rfp2_moe_gemm_workspace_bytes(E, T, top_k);
  if (need == 0 || N < 1 || N > kMaxRows || K < 256 || K % 256 != 0 ||
      K > (int64_t(1) << 24) || workspace_bytes < need)
    return RFP2_E_SHAPE;
  if (rfp2::moe_gemm_max_grid(E, N, T * top_k) > (int64_t(1) << 31) - 1) return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4) ||
      !aligned(ids, 4) || !aligned(workspace, 256) || (err && !aligned(err, 4)))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_moe_gemm(w, E, N, K, ids, T, top_k, q, d, y, err, workspace,
                                        stream));
}

static_assert(RFP2_MOE_GEMM_NOALLOC_MAX_BYTES == rfp2::kNoallocScratchBytes,
              "the header's limit is the size of the library's scratch array");

rfp2_status rfp2_moe_gemm_noalloc(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                  const int32_t* ids, int64_t T, int64_t top_k,
                                  const int8_t* q, const float* d, float* y, int32_t* err,
                                  hipStream_t stream) {
  if (!w || !ids || !q || !d || !y) return RFP2_E_NULL;
  const size_t need = rfp2_moe_gemm_workspace_bytes(E, T, top_k);
  if (need == 0 || need > RFP2_MOE_GEMM_NOALLOC_MAX_BYTES || N < 1 || N > kMaxRows ||
      K < 256 || K % 256 != 0 || K > (int64_t(1) << 24))
    return RFP2_E_SHAPE;
  if (rfp2::moe_gemm_max_grid(E, N, T * top_k) > (int64_t(1) << 31) - 1) return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(d, 4) || !aligned(y, 4) ||
      !aligned(ids, 4) || (err && !aligned(err, 4)))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(
      rfp2::launch_moe_gemm_noalloc(w, E, N, K, ids, T, top_k, q, d, y, err, stream));
}

rfp2_status rfp2_read_ceiling(const uint8_t* buf, int64_t bytes, uint32_t magic, uint32_t* out,
                              hipStream_t stream) {
  if (!buf || !out) return RFP2_E_NULL;
  if (bytes < 16 || bytes % 16 != 0) return RFP2_E_SHAPE;
  if (!aligned(buf, 16) || !aligned(out, 4)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_read_ceiling(buf, bytes, magic, out, stream));
}

rfp2_status rfp2_quant_gemv(const uint8_t* w, int64_t N, int64_t K, const float* a,
                            int8_t* q, float* d, float* y, hipStream_t stream) {
  if (!w || !a || !q || !d || !y) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || !product_k_ok(K)) return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(a, 16) || !aligned(q, 16) || !aligned(d, 4) ||
      !aligned(y, 4))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_quant_gemv(w, N, K, a, q, d, y, stream));
}

rfp2_status rfp2_quant_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                const int32_t* ids, int64_t top_k, const float* a,
                                int8_t* q, float* d, float* y, int32_t* err,
                                hipStream_t stream) {
  if (!w || !ids || !a || !q || !d || !y) return RFP2_E_NULL;
  if (E < 1 || E > kMaxRows || N < 1 || N > kMaxRows || top_k < 1 ||
      top_k > 65535 || !product_k_ok(K))
    return RFP2_E_SHAPE;
  if (!aligned(w, 16) || !aligned(a, 16) || !aligned(q, 16) || !aligned(d, 4) ||
      !aligned(y, 4) || !aligned(ids, 4) || (err && !aligned(err, 4)))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(
      rfp2::launch_quant_moe_gemv(w, E, N, K, ids, top_k, a, q, d, y, err, stream));
}

rfp2_status rfp2_debug_decode(const uint8_t* w, int64_t N, int64_t K,
                              int8_t* codes_out, float* scales_out,
                              hipStream_t stream) {
  if (!w || !codes_out || !scales_out) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || K < 32 || K % 32 != 0 || K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  if (!aligned(w, 2) || !aligned(codes_out, 4) || !aligned(scales_out, 4))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_debug_decode(w, N, K, codes_out, scales_out, stream));
}

rfp2_status rfp2_debug_half_dots(const uint8_t* w, int64_t N, int64_t K,
                                 const int8_t* q, int64_t M, int32_t* sums_out,
                                 hipStream_t stream) {
  if (!w || !q || !sums_out) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || M < 1 || M > kMaxRows || K < 32 || K % 32 != 0 ||
      K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  // M * N * (K / 32) half-sum pairs are indexed in 64 bits: keep it below 2^40
  if (N * (K / 32) > (int64_t(1) << 40) / M) return RFP2_E_SHAPE;
  if (!aligned(w, 2) || !aligned(q, 4) || !aligned(sums_out, 4)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_debug_half_dots(w, N, K, q, M, sums_out, stream));
}

rfp2_status rfp2_debug_half_sums_mf(const uint8_t* w, int64_t N, int64_t K,
                                    const int8_t* q, int64_t M, int32_t* sums_out,
                                    hipStream_t stream) {
  if (!w || !q || !sums_out) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || M < 1 || M > kMaxRows || K < 256 || K % 256 != 0 ||
      K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  if (N * (K / 32) > (int64_t(1) << 40) / M) return RFP2_E_SHAPE;
  if (!aligned(w, 2) || !aligned(q, 4) || !aligned(sums_out, 4)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_debug_half_sums_mf(w, N, K, q, M, sums_out, stream));
}

rfp2_status rfp2_debug_decode_f16(const uint8_t* w, int64_t N, int64_t K, int form,
                                  uint16_t* h_out, hipStream_t stream) {
  if (!w || !h_out) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || K < 32 || K % 32 != 0 || K > (int64_t(1) << 30) ||
      (form != 0 && form != 1))
    return RFP2_E_SHAPE;
  if (!aligned(w, 2) || !aligned(h_out, 2)) return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_debug_decode_f16(w, N, K, form, h_out, stream));
}

rfp2_status rfp2_debug_decode_i8(const uint8_t* w, int64_t N, int64_t K, int8_t* wa_out,
                                 int8_t* wb_out, float* scales_out, hipStream_t stream) {
  if (!w || !wa_out || !wb_out || !scales_out) return RFP2_E_NULL;
  if (N < 1 || N > kMaxRows || K < 32 || K % 32 != 0 || K > (int64_t(1) << 30))
    return RFP2_E_SHAPE;
  if (!aligned(w, 2) || !aligned(wa_out, 4) || !aligned(wb_out, 4) || !aligned(scales_out, 4))
    return RFP2_E_ALIGN;
  (void)hipGetLastError();
  return from_hip(rfp2::launch_debug_decode_i8(w, N, K, wa_out, wb_out, scales_out, stream));
}

}  // extern "C"
