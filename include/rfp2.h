/*
 * rfp2.h -- C ABI of the ROCmFP2 GEMV / GEMM library for AMD Instinct MI355X
 * (gfx950).
 *
 * The format and the method follow the page "ROCmFP2 codebook research
 * report" (llm.ciru.ai, 2026-07-13):
 *
 *   "01 · Storage": a block stores 32 weights in 10 bytes.  Bytes 0..7 are
 *     code bytes; byte j holds weights 4j..4j+3, weight 4j+i in bits
 *     2i..2i+1.  Byte 8 is the UE4M3 scale of weights 0..15, byte 9 the
 *     scale of weights 16..31.  2.50 bits per weight.
 *   "02 · Quantization": codes 00,01,10,11 mean -4,-1,+1,+4 times the scale
 *     of their half.  A scale byte b (legal 0x00..0x7E) has E = b >> 3,
 *     M = b & 7 and value M * 2^-10 (E == 0) or (8 + M) * 2^(E - 11).
 *     The quantizer starts near max|x|/4, tries legal scales, maps all 16
 *     values of the half to the nearest level (inner when |x/s| <= 2.5) and
 *     keeps the scale with the least squared error.
 *   "03 · Runtime": each code byte becomes four signed int8 lanes, which are
 *     multiplied four at a time with int8 (Q8_1-style) activations and
 *     accumulated in int32 per 16-weight half; the two weight scales and the
 *     activation scale are applied after the integer sum,
 *     d_a * (d_0 * S_0 + d_1 * S_1).  The multi-column kernel expands a
 *     block once and reuses it for every activation column.
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is a DEVICE pointer owned by the caller (the library
 *     allocates nothing, frees nothing and keeps no state between calls
 *     beyond a per-device cache of the GPU's compute-unit count).
 *   - Inputs are never written.  Outputs are overwritten, not accumulated.
 *   - Every call only enqueues work on `stream` (0 = the null stream) and
 *     returns; nothing is synchronised.  Calls are thread-safe.
 *   - Matrices are row-major.  A stored weight matrix of N rows and K columns
 *     is N rows of K/32 blocks, back to back: N * K / 32 * 10 bytes, row n at
 *     byte n * K * 10 / 32.
 *   - Activations are q int8 [M][K] plus d fp32 [M][K/32]: column (token) m
 *     of the product uses q[m][k] * d[m][k/32].
 *   - Argument errors are checked on the host before anything is enqueued;
 *     the call then returns a negative status and launches nothing.
 *   - Data errors are loud on the device: a scale byte outside 0x00..0x7E
 *     makes every output that depends on it NaN.
 */
#ifndef RFP2_H
#define RFP2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rfp2_status {
  RFP2_OK = 0,
  RFP2_E_NULL = -1,   /* a required pointer is null                        */
  RFP2_E_SHAPE = -2,  /* a size is out of range (see each call)            */
  RFP2_E_ALIGN = -3,  /* a pointer is not aligned as the call requires     */
  RFP2_E_LAUNCH = -4  /* the HIP runtime reported an error for the launch  */
} rfp2_status;

#define RFP2_ABI_VERSION 1
#define RFP2_GEMV_MAX_M 8

/* ABI version of the loaded library (RFP2_ABI_VERSION). */
int rfp2_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* rfp2_status_string(int status);

/*
 * rfp2_quantize_acts -- int8 activations, one fp32 scale per 32 values
 * ("03 · Runtime": the int8 activation operand and its scale).
 *   a  [M][K] fp32, 16-byte aligned.   q [M][K] int8, 4-byte aligned.
 *   d  [M][K/32] fp32, 4-byte aligned.
 * Per 32-value block: amax = max|a|, d = amax / 127 (IEEE fp32 division,
 * round to nearest even), q = round(a / d) with halves away from zero,
 * clamped to [-127, 127]; d == 0 gives q = 0.  A block holding a NaN or an
 * infinity gets d = NaN and q = 0.
 * Requires M >= 1, K >= 32, K % 32 == 0.
 */
rfp2_status rfp2_quantize_acts(const float* a, int64_t M, int64_t K,
                               int8_t* q, float* d, hipStream_t stream);

/*
 * rfp2_quantize_weights -- pack fp32 weights into ROCmFP2 blocks
 * ("02 · Quantization": how a block is chosen).
 *   x [N][K] fp32, 4-byte aligned.  w [N * K/32 * 10] bytes, 2-byte aligned.
 * Each 16-weight half gets the legal scale byte with the least squared
 * reconstruction error over all 127 legal bytes (errors summed in fp64 in
 * index order); on an exact tie the byte nearest to the start byte (the one
 * whose scale is nearest max|x|/4, the lower on a tie) wins, the lower one
 * first.  Codes: x < 0 negative, else positive; |x| <= 2.5 * s inner.
 * Non-finite weights give unspecified bytes.
 * Requires N >= 1, K >= 32, K % 32 == 0.
 */
rfp2_status rfp2_quantize_weights(const float* x, int64_t N, int64_t K,
                                  uint8_t* w, hipStream_t stream);

/*
 * rfp2_quantize_weights_imatrix -- rfp2_quantize_weights with the
 * importance-weighted error of "05 · Completed experiment": a candidate
 * scale's error is sum_i imp_i * sqrt(sigma^2 + x_i^2) * (x_i - xhat_i)^2
 * over the half, where imp_i is the importance of the value's input channel
 * and sigma^2 is the mean of x^2 over the half (the page leaves sigma
 * undefined; this is the reading taken).  Weights and errors are fp64, one
 * rounding per step, so the choice is reproducible.  The block layout,
 * codebook and codes are unchanged; only which scale wins can differ.
 *   importance [K] fp32, 4-byte aligned, finite and >= 0 (other values give
 *   unspecified bytes).  x, w and the limits as rfp2_quantize_weights.
 */
rfp2_status rfp2_quantize_weights_imatrix(const float* x, int64_t N, int64_t K,
                                          const float* importance, uint8_t* w,
                                          hipStream_t stream);

/*
 * rfp2_gemv -- y[m][n] = sum_k w[n][k] * q[m][k] * d[m][k/32] for a few
 * activation columns ("03 · Runtime": decode once, reuse for every column).
 *   w [N][K/32][10] bytes, 16-byte aligned.  q [M][K] int8, 16-byte aligned.
 *   d [M][K/32] fp32, 4-byte aligned.         y [M][N] fp32, 4-byte aligned.
 * Requires N >= 1, 1 <= M <= RFP2_GEMV_MAX_M, 256 <= K <= 32768,
 * K % 256 == 0 (a row is then a whole number of 80-byte groups and every row
 * starts 16-byte aligned).
 */
rfp2_status rfp2_gemv(const uint8_t* w, int64_t N, int64_t K,
                      const int8_t* q, const float* d, int64_t M,
                      float* y, hipStream_t stream);

/*
 * rfp2_gemm -- the same product for a batch of M >= 1 activation columns
 * (prompt batches), computed with i8 matrix-core instructions on int32
 * integer sums ("03 · Runtime" applied to a tile of columns).  The UE4M3
 * mantissas of a block's two scales are folded into its int8 weights, so
 * the block is one integer dot product with one power-of-two scale while
 * the two scale exponents differ by at most 2 (as int32 per-half partials
 * otherwise); every such scaled sum is exact and the activation scale is
 * applied to it with one rounding, then added with one more.
 * Layouts and alignment as rfp2_gemv.  Requires N >= 1, M >= 1,
 * 256 <= K <= 2^24, K % 256 == 0.
 */
rfp2_status rfp2_gemm(const uint8_t* w, int64_t N, int64_t K,
                      const int8_t* q, const float* d, int64_t M,
                      float* y, hipStream_t stream);

/*
 * rfp2_gemm_f16 -- the same product as rfp2_gemm, computed on the fp16
 * matrix cores.  Every reconstructed weight (level x UE4M3 scale) and every
 * int8 activation is exactly an fp16 number and every product is exact in
 * fp32, so each 32-weight block's sum s0*S0 + s1*S1 comes out of the matrix
 * core in fp32 (exact while the two scale exponents differ by at most 7;
 * beyond, the core's fp32 accumulation may round, each step within 2^-24 of
 * the running sum) and only the activation scale is applied afterwards: one
 * multiply-add per output and block instead of the int32 path's two.
 * Layouts, alignment and limits as rfp2_gemm.
 */
rfp2_status rfp2_gemm_f16(const uint8_t* w, int64_t N, int64_t K,
                          const int8_t* q, const float* d, int64_t M,
                          float* y, hipStream_t stream);

/*
 * rfp2_moe_gemv -- routed-expert GEMV for one token.
 *   w    E experts back to back, each [N][K/32][10] bytes; 16-byte aligned.
 *   ids  [top_k] int32 on the device: the experts to apply, in output order.
 *   q, d one activation column ([K] int8, [K/32] fp32).
 *   y    [top_k][N] fp32: row j = expert ids[j] applied to the token.
 *   err  nullable device int32: when an id lies outside [0, E) its row of y
 *        is set to NaN and 1 is written to *err (never cleared by the call).
 * Duplicate ids are legal.  Expert offsets are computed in 64 bits.
 * Requires E >= 1, N >= 1, 1 <= top_k <= 65535, 256 <= K <= 32768,
 * K % 256 == 0.
 */
rfp2_status rfp2_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                          const int32_t* ids, int64_t top_k,
                          const int8_t* q, const float* d,
                          float* y, int32_t* err, hipStream_t stream);

/*
 * rfp2_moe_gemv_tokens -- routed-expert GEMV for T tokens at once (e.g. the
 * tokens of a speculative-decoding verification batch).  Slot s = t * top_k
 * + j of token t is routed to expert ids[s]; the slots routed to one expert
 * are computed together, so each expert's rows are expanded once and reused
 * for every token routed to it ("Why AMD-friendly does not mean always
 * faster": expand a block once, reuse it across all activation columns).
 *   w    E experts back to back, each [N][K/32][10] bytes; 16-byte aligned.
 *   ids  [T][top_k] int32 on the device.
 *   q, d [T][K] int8 (16-byte aligned) and [T][K/32] fp32.
 *   y    [T][top_k][N] fp32: row s = expert ids[s] applied to token s / top_k.
 *   err  as rfp2_moe_gemv (an id outside [0, E) gives a NaN row and *err = 1).
 * Duplicate ids are legal.  T = 1 is rfp2_moe_gemv.  Each row of y is within
 * the fp32 bound of the product, but the order of its additions may differ
 * from rfp2_moe_gemv's for the same token.
 * Requires E >= 1, N >= 1, 1 <= T <= RFP2_GEMV_MAX_M, top_k >= 1,
 * T * top_k <= 64, 256 <= K <= 32768, K % 256 == 0.
 */
rfp2_status rfp2_moe_gemv_tokens(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                 const int32_t* ids, int64_t T, int64_t top_k,
                                 const int8_t* q, const float* d, float* y, int32_t* err,
                                 hipStream_t stream);

/*
 * rfp2_moe_sort -- the routed slots grouped by expert, the token order of a
 * prompt batch through the routed experts ("04 · Measured evidence" and
 * "07 · Recipe decision": the method's gain is prefill on large expert
 * tensors; a prefill product takes each expert's tokens together).
 *   ids     [S] int32 on the device: slot s (token s / top_k of a batch) is
 *           routed to expert ids[s].
 *   offsets [E+1] int32 (written): expert e's slots are
 *           order[offsets[e] .. offsets[e+1]); offsets[E] = the routed slots.
 *   order   [S] int32 (written up to offsets[E]): every slot whose id lies in
 *           [0, E), grouped by expert in expert order, increasing slot order
 *           inside an expert (the stable order: deterministic).
 *   err     nullable device int32: set to 1 when an id lies outside [0, E)
 *           (such slots are left out; never cleared by the call).
 * One workgroup; suited to the few thousand slots of a prompt batch.
 * Requires 1 <= S <= 2^24, 1 <= E <= 2048; all pointers 4-byte aligned.
 */
rfp2_status rfp2_moe_sort(const int32_t* ids, int64_t S, int64_t E, int32_t* offsets,
                          int32_t* order, int32_t* err, hipStream_t stream);

/*
 * rfp2_moe_gemm_workspace_bytes -- device bytes rfp2_moe_gemm needs as
 * workspace for E experts and T * top_k slots (0 when the sizes are out of
 * range).
 */
size_t rfp2_moe_gemm_workspace_bytes(int64_t E, int64_t T, int64_t top_k);

/*
 * rfp2_moe_gemm -- routed-expert products for a prompt batch of T tokens on
 * the matrix cores: the slots are sorted by expert (rfp2_moe_sort), then each
 * expert's slots are cut into tiles of 64 tokens and multiplied with that
 * expert's weights as rfp2_gemm_f16 multiplies a dense batch (exact fp16
 * operands, one rescale per output and block).
 *   w    E experts back to back, each [N][K/32][10] bytes; 16-byte aligned.
 *   ids  [T][top_k] int32 on the device; slot s = t * top_k + j.
 *   q, d [T][K] int8 (16-byte aligned) and [T][K/32] fp32.
 *   y    [T][top_k][N] fp32: row s = expert ids[s] applied to token s / top_k
 *        (NaN for an id outside [0, E), and *err = 1 as rfp2_moe_gemv).
 *   workspace  device memory of at least rfp2_moe_gemm_workspace_bytes(E, T,
 *        top_k) bytes, 256-byte aligned, owned by the caller; overwritten.
 *        Calls that share a workspace must not overlap in time.
 * Each output is computed independently of which other slots share its
 * tile, so y does not depend on the routing of the other tokens.
 * Requires 1 <= E <= 2048, N >= 1, T >= 1, top_k >= 1, T * top_k <= 2^24,
 * 256 <= K <= 2^24, K % 256 == 0.
 */
rfp2_status rfp2_moe_gemm(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                          const int32_t* ids, int64_t T, int64_t top_k, const int8_t* q,
                          const float* d, float* y, int32_t* err, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * rfp2_moe_gemm_noalloc -- rfp2_moe_gemm for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same sort and product kernels and the same
 * result, with the sorted slots kept in a device array that the library owns
 * instead of a caller workspace.  The call allocates nothing.
 *   w, ids, q, d, y, err and their layouts, alignment and limits as
 *   rfp2_moe_gemm; in addition rfp2_moe_gemm_workspace_bytes(E, T, top_k)
 *   must not exceed RFP2_MOE_GEMM_NOALLOC_MAX_BYTES (otherwise RFP2_E_SHAPE,
 *   nothing launched).  With 128 experts that allows up to 261,886 routed
 *   slots, e.g. 32,735 tokens at top-8.
 * The array (RFP2_MOE_GEMM_NOALLOC_MAX_BYTES bytes) is held by every GPU the
 * library runs on until the process ends; its device address is looked up on
 * the first call on each device (RFP2_E_LAUNCH if that fails).  All calls on
 * one GPU share it and it keeps the last call's contents: calls that overlap
 * in time on one GPU (several streams, several host threads) race and must be
 * serialised by the caller.
 */
#define RFP2_MOE_GEMM_NOALLOC_MAX_BYTES 1048576
rfp2_status rfp2_moe_gemm_noalloc(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                  const int32_t* ids, int64_t T, int64_t top_k,
                                  const int8_t* q, const float* d, float* y, int32_t* err,
                                  hipStream_t stream);

/*
 * rfp2_quant_gemv -- one token end to end: quantizes the fp32 activations a
 * exactly as rfp2_quantize_acts does, writing q and d, and computes
 * y = W * a as rfp2_gemv does from that q and d ("03 · Runtime": the int8
 * activation operand, its scale, then the product), in a single kernel
 * launch for most K and up to 128 MiB of weights (beyond, the two launches
 * are faster): each wave quantizes the activations it needs while its
 * weights stream in.  q and d are bit-identical to rfp2_quantize_acts.  y is
 * bit-identical to rfp2_gemv with M = 1 on them wherever the single launch
 * splits K as rfp2_gemv does; where rfp2_gemv's split gives a wave more than
 * 4 groups of 256 (K = 6144, 8192, 10240, 12288, 14336, 16384) and the call
 * reads at most 64 MiB, the single launch may split K over more waves or
 * more rows per workgroup, and y then sums in another order (same fp32
 * bound).
 *   w [N][K/32][10] bytes, 16-byte aligned.   a [K] fp32, 16-byte aligned.
 *   q [K] int8, 16-byte aligned (written).     d [K/32] fp32, 4-byte aligned
 *   (written).                                 y [N] fp32, 4-byte aligned.
 * Requires N >= 1, 256 <= K <= 32768, K % 256 == 0.
 */
rfp2_status rfp2_quant_gemv(const uint8_t* w, int64_t N, int64_t K, const float* a,
                            int8_t* q, float* d, float* y, hipStream_t stream);

/*
 * rfp2_quant_moe_gemv -- the routed-expert GEMV of rfp2_moe_gemv for one
 * token given in fp32, with the activation quantization of
 * rfp2_quantize_acts done inside the product launch (as rfp2_quant_gemv).
 * w, ids, y, err and the limits as rfp2_moe_gemv; a, q, d as
 * rfp2_quant_gemv.  q and d are bit-identical to rfp2_quantize_acts, and y
 * to rfp2_moe_gemv on them, with the same exception as rfp2_quant_gemv.
 */
rfp2_status rfp2_quant_moe_gemv(const uint8_t* w, int64_t E, int64_t N, int64_t K,
                                const int32_t* ids, int64_t top_k, const float* a,
                                int8_t* q, float* d, float* y, int32_t* err,
                                hipStream_t stream);

/*
 * rfp2_read_ceiling -- measurement helper, not part of the method: reads
 * `bytes` bytes of buf once with the plainest coalesced 16-byte loads
 * (thread t of the grid reads pieces t, t + T, t + 2T, ... of 16 bytes,
 * T = 256 * min(2048, ceil(bytes / 4096)) threads) and XORs the four words of
 * every piece it reads; a thread whose XOR equals `magic` writes it to
 * out[t], no other thread writes.  Its time is the ceiling for any kernel that
 * must read that many bytes (launch and ramp-up included), the yardstick the
 * products' effective bandwidth is reported against besides the HBM peak.
 *   buf  device bytes, 16-byte aligned.
 *   out  device uint32 [T] (RFP2_READ_CEILING_OUTPUTS at most); only the
 *        entries of threads whose XOR equals magic are written.
 * Requires bytes >= 16, bytes % 16 == 0.
 */
#define RFP2_READ_CEILING_OUTPUTS 524288
rfp2_status rfp2_read_ceiling(const uint8_t* buf, int64_t bytes, uint32_t magic, uint32_t* out,
                              hipStream_t stream);

/*
 * Inspection entry points.  They run the products' own device functions on
 * the register layouts the products use, so what they return is what the
 * products compute internally ("03 · Runtime": SPREAD / PERMUTE expand each
 * code byte into four int8 lanes, DOT4 sums each 16-weight half in int32).
 *
 * rfp2_debug_decode: the GEMV's decode.  The block stream is taken in 80-byte
 * groups of 8 blocks, as a GEMV lane holds them, and each block is decoded as
 * the GEMV decodes block j of its group (the odd blocks start at byte 2 of a
 * dword).  codes_out [N][K] int8: the lane each weight expands to;
 * scales_out [N][K/16] fp32: the scale of each half (NaN for an illegal
 * byte).  Requires N >= 1, K >= 32, K % 32 == 0; w 2-byte aligned, codes_out
 * and scales_out 4-byte aligned.
 *
 * rfp2_debug_half_dots: the GEMV's int32 sum of each 16-weight half against
 * the int8 activations (staged in the GEMV's lane order), sums_out
 * [M][N][K/32][2] int32.  Requires N >= 1, M >= 1, K >= 32, K % 32 == 0,
 * M * N * (K/32) <= 2^40; w 2-byte aligned, q 4-byte aligned.
 *
 * rfp2_debug_half_sums_mf: the same int32 half sums as computed by the
 * GEMV's matrix-core form of two to eight columns (v_mfma_i32_4x4x4_16b_i8
 * over quads of four rows at one 8-block group, one column's activations per
 * lane; "03 · Runtime": the half's int8 products summed in int32 before any
 * scale), sums_out [M][N][K/32][2] int32 as rfp2_debug_half_dots.  Requires
 * N >= 1, M >= 1, K >= 256, K % 256 == 0, M * N * (K/32) <= 2^40; w 2-byte
 * aligned, q 4-byte aligned.
 *
 * rfp2_debug_decode_f16: the fp16 value (level x scale) each weight takes in
 * the fp16 matrix-core products, h_out [N][K] as IEEE half-precision bit
 * patterns in natural order (NaN for both halves of a block with an illegal
 * scale byte).  form 0: the decode of rfp2_gemm_f16 (a thread expands both
 * halves of one block of a 20-byte pair); form 1: the decode of
 * rfp2_moe_gemm (a lane expands one half of a block straight into its
 * matrix-core operand).  Requires N >= 1, K >= 32, K % 32 == 0, form 0 or 1;
 * w and h_out 2-byte aligned.
 */
rfp2_status rfp2_debug_decode(const uint8_t* w, int64_t N, int64_t K,
                              int8_t* codes_out, float* scales_out,
                              hipStream_t stream);
rfp2_status rfp2_debug_half_dots(const uint8_t* w, int64_t N, int64_t K,
                                 const int8_t* q, int64_t M,
                                 int32_t* sums_out, hipStream_t stream);
rfp2_status rfp2_debug_half_sums_mf(const uint8_t* w, int64_t N, int64_t K,
                                    const int8_t* q, int64_t M,
                                    int32_t* sums_out, hipStream_t stream);
rfp2_status rfp2_debug_decode_f16(const uint8_t* w, int64_t N, int64_t K, int form,
                                  uint16_t* h_out, hipStream_t stream);

/*
 * rfp2_debug_decode_i8: the decode of rfp2_gemm (the int8 matrix-core
 * product), as its staging threads run it: blocks taken in dword-aligned
 * 20-byte pairs (the second block of a pair starts at byte 2 of a dword),
 * the scale mantissas folded into the two int8 operands.  Per block, in
 * natural weight order: wa_out [N][K] and wb_out [N][K] int8, the operands
 * whose weight k stands for wa[k] * sA + wb[k] * sB; scales_out
 * [N][K/32][6] fp32 = (s, -1.5*2^23*s, sA, -1.5*2^23*sA, sB,
 * -1.5*2^23*sB), where s = sA = sB when the block is one dot product and
 * s = -sB (negative: the split path) when its halves stay apart; all six
 * are NaN for a block with an illegal scale byte.
 * Requires N >= 1, K >= 32, K % 32 == 0; w 2-byte aligned, the outputs
 * 4-byte aligned.
 */
rfp2_status rfp2_debug_decode_i8(const uint8_t* w, int64_t N, int64_t K, int8_t* wa_out,
                                 int8_t* wb_out, float* scales_out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* RFP2_H */
