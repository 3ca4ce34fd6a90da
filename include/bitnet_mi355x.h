/*
 * bitnet_mi355x.h — C ABI of the H-BitLinear forward library for AMD MI355X (gfx950).
 *
 * The layer (BitNet v2 "H-BitLinear", as restated on the Quillan-Ronin
 * bitnet_v2_engine.py page, class HBitLinear and Eq. 1-7) computes, per token
 * row x of X [M, K]:
 *     x_r  = H_K x                    (orthonormal Walsh-Hadamard, optional)
 *     q, s = per-token quantization   (int8 absmax or int4 absmean*sqrt7)
 *     y    = (q . t^T) * alpha * s / c
 * with t = RoundClip(W / (alpha + eps), -1, 1) the absmean-ternarized weights
 * and alpha = mean|W| (Eq. 1-2). The RMSNorm that precedes the transform in
 * that class is not part of this library: X is taken to be already normalized.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer (HBM of the current HIP device),
 *     row-major, allocated and owned by the caller. The library never
 *     allocates, frees or synchronizes; every call only enqueues kernels on
 *     `stream` (0 = the null stream) and returns.
 *   - Returns BITNET_OK (0) on success. On any error nothing is launched and
 *     bitnet_last_error() returns a message (per calling thread). A failed
 *     kernel launch returns BITNET_ERR_HIP. Device-side faults surface, as for
 *     any HIP work, at the caller's next synchronization.
 *   - Pointers to tensors must be 16-byte aligned; the alpha and scale
 *     pointers 4-byte aligned.
 *   - eps = 1e-7 (BITNET_EPS), the engine page's default for every quantizer.
 *   - Calls that share a workspace must not overlap in time.
 *   - M = 0 or N = 0 is a no-op that returns BITNET_OK.
 *
 * Packed-weight layout ("block-64", 2 bits per weight, 4 weights per byte)
 *   Wpacked is uint8 [N, K/4]. Each ternary weight is stored as the 2-bit
 *   code t + 1 in {0, 1, 2} (3 is never written). K is cut into blocks of 64
 *   consecutive weights; block g of row n occupies bytes 16g .. 16g+15 of that
 *   row, and byte b of the block holds the weights at block offsets
 *   b, 16+b, 32+b, 48+b in its bit pairs 0-1, 2-3, 4-5, 6-7 (LSB first).
 *   Shifting a 32-bit word of the block right by 2j and masking 0x03030303
 *   yields four consecutive weights, which is why this order was chosen.
 *   K must therefore be a multiple of 64.
 */
#ifndef BITNET_MI355X_H
#define BITNET_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNET_ABI_VERSION 4
#define BITNET_EPS 1e-7f
/* Largest K the fused transform + quantizer stages in one CU's LDS (fp32). */
#define BITNET_MAX_K 32768

typedef enum {
  BITNET_OK = 0,
  BITNET_ERR_INVALID_ARG = 1, /* null pointer, negative size, workspace too small */
  BITNET_ERR_NOT_POW2 = 2,    /* hadamard=1 with K not a power of two */
  BITNET_ERR_BAD_BITS = 3,    /* bits not in {4, 8} */
  BITNET_ERR_ALIGN = 4,       /* K not a multiple of 64, or a misaligned pointer */
  BITNET_ERR_UNSUPPORTED = 5, /* K above BITNET_MAX_K, or dtype not supported */
  BITNET_ERR_HIP = 6          /* the HIP runtime rejected a launch */
} bitnet_status;

typedef enum { BITNET_F32 = 0, BITNET_BF16 = 1 } bitnet_dtype;

/* Version of this ABI (BITNET_ABI_VERSION). Makes no HIP call. */
int bitnet_abi_version(void);

/* Message of the last error on the calling thread ("" if none). Makes no HIP call. */
const char* bitnet_last_error(void);

/* ------------------------------------------------------------------------ */
/* Weight preparation                                                        */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace bitnet_ternarize_weights needs for an [N, K] tensor. */
size_t bitnet_ternarize_workspace_bytes(int64_t N, int64_t K);

/* Absmean ternarization and 2-bit packing of fp32 latent weights.
 * Engine page, Eq. 1-2 (quantize_weight_ternary): alpha = mean|W| over the
 * whole tensor, t = RoundClip(W / (alpha + eps), -1, 1) with round-half-even.
 *   W        fp32 [N, K], K contiguous (out_features x in_features).
 *   Wpacked  uint8 [N, K/4], block-64 layout (above). Written.
 *   alpha    one fp32 on the device. Written (stays on the device, so the
 *            forward can consume it without a host round trip).
 *   ws       workspace of at least bitnet_ternarize_workspace_bytes(N, K).
 * The |W| sum is a fixed-order two-stage reduction accumulated in fp64, so
 * results are bitwise reproducible. Requires K % 64 == 0 and N >= 1. */
bitnet_status bitnet_ternarize_weights(const float* W, int64_t N, int64_t K, uint8_t* Wpacked,
                                       float* alpha, void* ws, size_t ws_bytes,
                                       hipStream_t stream);

/* Packs ternary values held one per int8 [N, K] into the block-64 layout:
 * the edge page's I2_S format (bitnet_cpp_edge.py, Table 1: 2 bits per
 * weight, a ternary value per 2-bit field) with the blog page's LUT code
 * w -> w + 1 (youngju.dev BitNet page, LUT simulation). Values are mapped by
 * sign (negative -> -1, zero -> 0, positive -> +1).
 *   T        int8 [N, K], read.   Wpacked  uint8 [N, K/4], written.
 * Requires K % 64 == 0; both pointers 16-byte aligned. N = 0 is a no-op. */
bitnet_status bitnet_pack_2bit(const int8_t* T, int64_t N, int64_t K, uint8_t* Wpacked,
                               hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Forward                                                                   */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace bitnet_hbitlinear_forward needs: the codes, fp32
 * scales and int32 code row sums of the batch (M*K, 4*M and 4*M bytes, each
 * rounded up to 256; with bits = 4, M <= 16 and K % 256 == 0 the codes are
 * held two to a byte and fill half of their part). It is 0
 * when the forward runs as a single fused kernel (M <= 16, M*K <= 16384,
 * K <= 4096, and hadamard = 0 or K <= 256); ws may then be NULL. Returns 0
 * for invalid sizes. */
size_t bitnet_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, int bits, int hadamard);

/* H-BitLinear forward (engine page, HBitLinear.forward after its RMSNorm;
 * Eq. 3-7):
 *   x_r = hadamard ? H_K x : x          fp32, never rounded to a narrower type
 *   bits == 8: s = max|x_r| + eps,  q = RoundClip(127 x_r / s, -128, 127)  (Eq. 5)
 *   bits == 4: s = mean|x_r| + eps, q = RoundClip(sqrt7 x_r / s, -8, 7)    (Eq. 6)
 *   acc = q . t^T                       exact int32
 *   y   = acc * alpha * s / c           fp32, c = 127 or sqrt 7
 *   x        [M, K] in x_dtype (BITNET_F32 or BITNET_BF16).
 *   Wpacked  uint8 [N, K/4], block-64 layout; alpha: one fp32 on the device.
 *   y        fp32 [M, N]. Written.
 *   ws       workspace of at least bitnet_forward_workspace_bytes(...); its
 *            contents on entry do not matter.
 * Requires K % 64 == 0, K <= BITNET_MAX_K, and a power-of-two K when
 * hadamard != 0. */
bitnet_status bitnet_hbitlinear_forward(const void* x, bitnet_dtype x_dtype, int64_t M, int64_t K,
                                        const uint8_t* Wpacked, int64_t N, const float* alpha,
                                        int bits, int hadamard, float* y, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/* The forward, or one of its two stages, on the forward's own kernels and
 * workspace format: stages = BITNET_STAGE_QUANTIZE writes the transform and
 * quantization stage's results (codes, scales, code row sums) into ws;
 * BITNET_STAGE_PRODUCT reads them from ws and writes y; both (3) is exactly
 * bitnet_hbitlinear_forward. Running stage 1 then stage 2 on the same ws
 * gives the forward's y bit for bit. Where the forward runs as one fused
 * kernel (bitnet_forward_workspace_bytes = 0) only stages = 3 is accepted
 * (BITNET_ERR_UNSUPPORTED otherwise). Arguments and errors as for
 * bitnet_hbitlinear_forward; stages outside 1..3 is BITNET_ERR_INVALID_ARG.
 * Used to time each stage's kernel alone. */
#define BITNET_STAGE_QUANTIZE 1
#define BITNET_STAGE_PRODUCT 2
bitnet_status bitnet_hbitlinear_forward_stages(const void* x, bitnet_dtype x_dtype, int64_t M,
                                               int64_t K, const uint8_t* Wpacked, int64_t N,
                                               const float* alpha, int bits, int hadamard,
                                               float* y, void* ws, size_t ws_bytes, int stages,
                                               hipStream_t stream);

/* The two stages of the forward, exposed for inspection and timing. They run
 * the kernels of the forward's two-launch path; where the forward fuses both
 * stages into one kernel (see bitnet_forward_workspace_bytes) that kernel
 * takes the same quantization and product steps in the same precision, and
 * where it passes int4 codes two to a byte (see above) the product's result
 * is the same integer, so the output is the same bit for bit. */

/* Transform + per-token quantization only (Eq. 3-6): writes int8 codes
 * [M, K] and fp32 scales s [M] (s = stat + eps, the value the dequantization
 * multiplies by), and, when rowsum is not NULL, each token's code sum
 * rowsum[m] = sum_k codes[m, k] (int32 [M], exact), which
 * bitnet_ternary_linear_dequant can take instead of summing the codes again.
 * Same requirements as the forward; rowsum 4-byte aligned. */
bitnet_status bitnet_quantize_activations(const void* x, bitnet_dtype x_dtype, int64_t M,
                                          int64_t K, int bits, int hadamard, int8_t* codes,
                                          float* scales, int32_t* rowsum, hipStream_t stream);

/* Exact integer product only: acc[m, n] = sum_k codes[m, k] * t[n, k], int32.
 * This is the engine page's F.linear(x_q, w_q) of HBitLinear.forward before
 * its two scales (the blog page's BitLinear_b158 integer form; the edge
 * page's I2_S multiply-add, Table 1, "lossless"): every sum is exact, since
 * |codes| <= 128 and K <= 32768.
 *   codes    int8 [M, K], values in [-128, 127].
 *   Wpacked  uint8 [N, K/4], block-64 layout.   acc  int32 [M, N], written.
 * Requires K % 64 == 0 and K <= BITNET_MAX_K; codes and Wpacked 16-byte
 * aligned, acc 4-byte aligned. */
bitnet_status bitnet_ternary_gemm_i32(const int8_t* codes, int64_t M, int64_t K,
                                      const uint8_t* Wpacked, int64_t N, int32_t* acc,
                                      hipStream_t stream);

/* Integer product with the fused dequantization epilogue (engine page,
 * HBitLinear.forward's F.linear of the two dequantized operands, rewritten by
 * linearity): y = (codes . t^T) * alpha * scales[m] / c, c = 127 (bits 8) or
 * sqrt 7 (bits 4). rowsum: NULL, or the codes' per-token sums as
 * bitnet_quantize_activations wrote them (int32 [M]); the prefill product
 * then skips summing the codes, which is how the forward runs it. A rowsum
 * that is not the codes' sum gives wrong outputs (it is not checked). */
bitnet_status bitnet_ternary_linear_dequant(const int8_t* codes, const float* scales,
                                            const int32_t* rowsum, int64_t M, int64_t K,
                                            const uint8_t* Wpacked, int64_t N, const float* alpha,
                                            int bits, float* y, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Forward with the layer-input prologue                                     */
/* ------------------------------------------------------------------------ */

/* The whole of the engine page's HBitLinear.forward, with the input
 * prologue the plain forward leaves to the caller:
 *   u   = up ? silu(x) * up : x      BitNetV2FFN.forward: Swish(gate) * up,
 *                                    the input of the H-BitLinear down
 *                                    projection (x is then the gate
 *                                    projection; silu(g) = g / (1 + e^-g))
 *   u   = rmsnorm ? u / sqrt(mean(u^2) + norm_eps) * norm_weight : u
 *                                    HBitLinear.forward step 1, nn.RMSNorm
 *   then exactly the steps of bitnet_hbitlinear_forward on u.
 *   up           NULL, or [M, K] in x_dtype (same layout as x).
 *   rmsnorm      0 or 1.
 *   norm_weight  NULL (all ones, nn.RMSNorm's initial value) or fp32 [K];
 *                read only when rmsnorm = 1.
 *   norm_eps     > 0; the engine page passes the layer's eps (1e-7).
 * The prologue is computed in fp32 as each vector is loaded and is never
 * written to memory; 1/rms enters only the scale and the code multiplier
 * (per-token quantization sees u / stat(u)). Same requirements and errors
 * as bitnet_hbitlinear_forward, except that a workspace of
 * bitnet_forward_prologue_workspace_bytes is always required (the decode
 * shapes the plain forward runs as one kernel run as one kernel here too and
 * leave it untouched); up and norm_weight must be 16-byte aligned;
 * norm_eps <= 0 or rmsnorm not in {0, 1} is BITNET_ERR_INVALID_ARG. */
size_t bitnet_forward_prologue_workspace_bytes(int64_t M, int64_t K, int64_t N, int bits,
                                               int hadamard);
bitnet_status bitnet_hbitlinear_forward_prologue(const void* x, const void* up, bitnet_dtype x_dtype,
                                                 int64_t M, int64_t K, int rmsnorm,
                                                 const float* norm_weight, float norm_eps,
                                                 const uint8_t* Wpacked, int64_t N,
                                                 const float* alpha, int bits, int hadamard,
                                                 float* y, void* ws, size_t ws_bytes,
                                                 hipStream_t stream);

/* Prologue + transform + per-token quantization only; writes the codes and
 * scales bitnet_hbitlinear_forward_prologue multiplies with. */
bitnet_status bitnet_quantize_activations_prologue(const void* x, const void* up,
                                                   bitnet_dtype x_dtype, int64_t M, int64_t K,
                                                   int rmsnorm, const float* norm_weight,
                                                   float norm_eps, int bits, int hadamard,
                                                   int8_t* codes, float* scales,
                                                   hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* TL2 weight code (1.67 bits per weight) for single-token decode            */
/* ------------------------------------------------------------------------ */

/* Edge page (bitnet_cpp_edge.py), module docstring item 2 and class
 * SignedUnsignedWeightPacker: a ternary triplet (w0, w1, w2) is stored as the
 * 4-bit index (0..13) of one of the page's 14 base triplets (all zero, or
 * first non-zero element +1) and a sign bit that negates it, 5 bits per 3
 * weights. Layout per output column: blocks b covering weights 384 b ..
 * 384 b + 383 (triplet j: weights 384 b + 3 j + 0..2; weights past K are
 * zero), each of G groups of 32 triplets: G = 4 for a whole block (80 bytes),
 * and for a partial last block the ceil((K % 384) / 96) groups it reaches,
 * its 20 G bytes rounded up to 16 with zeros. Triplet j = 32 g + 4 i + tt
 * keeps its index in bits 4 (i % 2) .. +3 of byte 16 g + 4 (i / 2) + tt and
 * its sign in bit i of byte 16 G + 4 g + tt. The row of a column is
 * bitnet_tl2_bytes(1, K) bytes (1.67 bits per weight at K = 16384). */

/* Bytes of a TL2 weight buffer for [N, K] (0 for invalid sizes). */
size_t bitnet_tl2_bytes(int64_t N, int64_t K);

/* Re-encode 2-bit packed weights (bitnet_ternarize_weights / bitnet_pack_2bit
 * layout, [N, K/4]) as TL2 ([N, bitnet_tl2_bytes(N, K) / N] bytes, written).
 * Requires K % 64 == 0; both pointers 16-byte aligned. The weights' alpha is
 * unchanged. */
bitnet_status bitnet_pack_tl2(const uint8_t* Wpacked, int64_t N, int64_t K, uint8_t* Wtl2,
                              hipStream_t stream);

/* Single-token decode forward on TL2 weights: the same result as
 * bitnet_hbitlinear_forward with hadamard = 0 and M = 1 (same per-token
 * codes, exact int32 product, y = acc * alpha * s / c), one kernel, no
 * workspace. Requires M <= 1 (BITNET_ERR_UNSUPPORTED otherwise), K % 64 == 0,
 * K <= 4608; x 16-byte aligned, Wtl2 16-byte aligned. */
bitnet_status bitnet_hbitlinear_forward_tl2(const void* x, bitnet_dtype x_dtype, int64_t M,
                                            int64_t K, const uint8_t* Wtl2, int64_t N,
                                            const float* alpha, int bits, float* y,
                                            hipStream_t stream);

/* Batched forward on TL2 weights. Edge page (bitnet_cpp_edge.py), class
 * TL2KernelEdge, method compute_gemv, which takes a batch of tokens x [B, K]:
 * the same result as bitnet_hbitlinear_forward with hadamard = 0 for
 * 1 <= M <= 16 tokens and any K % 64 == 0 up to BITNET_MAX_K (per-token codes,
 * exact int32 product, y = acc * alpha * s / c). One token with
 * K <= 4608 runs the single-token kernel and needs no workspace; otherwise the
 * tokens are quantized into ws (codes in the product's own order, scales and
 * code row sums: bitnet_tl2_forward_workspace_bytes(M, K) bytes, 16-byte
 * aligned, caller-owned, contents undefined afterwards) and the product runs
 * 16 output columns per workgroup. M > 16: BITNET_ERR_UNSUPPORTED. x and Wtl2
 * 16-byte aligned. */
size_t bitnet_tl2_forward_workspace_bytes(int64_t M, int64_t K);
bitnet_status bitnet_hbitlinear_forward_tl2_batched(const void* x, bitnet_dtype x_dtype,
                                                    int64_t M, int64_t K, const uint8_t* Wtl2,
                                                    int64_t N, const float* alpha, int bits,
                                                    float* y, void* ws, size_t ws_bytes,
                                                    hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Low-bit KV cache                                                          */
/* ------------------------------------------------------------------------ */

/* Per-token quantization of post-RoPE keys or values (engine page, module
 * docstring item 5 / Section 3.1, BitNetV2Attention._quantize_kv_head):
 *   kv      [R, D] in x_dtype: the rows of a contiguous [B, H, S, D] tensor,
 *           row r being token r % S of its head (R = B * H * S).
 *   bits    3, 4 or 8 for tokens s >= 1; token 0 (BOS) of every head is
 *           always quantized with the 8-bit absmax rule.
 *             8 (and BOS): s = max|x| + eps,  q = RoundClip(127 x / s, -128, 127)
 *             4:           s = mean|x| + eps, q = RoundClip(sqrt7 x / s, -8, 7)
 *             3:           s = max|x| + eps,  q = RoundClip(3 x / s, -4, 3)
 *   codes   int8 [R, D], written (one code per byte).
 *   scales  fp32 [R], written: s, so that x ~ q * s / c with the token's c.
 * Requires D % 8 == 0, 8 <= D <= 512, S >= 1 and R % S == 0; kv and codes
 * 16-byte aligned. R = 0 is a no-op. bits outside {3, 4, 8} is
 * BITNET_ERR_BAD_BITS. */
bitnet_status bitnet_kv_quantize(const void* kv, bitnet_dtype x_dtype, int64_t R, int64_t D,
                                 int64_t S, int bits, int8_t* codes, float* scales,
                                 hipStream_t stream);

/* The same quantization (same codes and scales) with the 3- or 4-bit codes
 * stored b bits apiece, so that the cache holds b / 8 bytes per element. The
 * page keeps the fake-quantized tensor; this packing is this library's layout:
 *   packed     uint8 [R, D * bits / 8], written: one little-endian bit stream
 *              per token row, code k at stream bits bits*k .. bits*k+bits-1
 *              (stream bit i is bit i % 8 of byte i / 8), two's complement
 *              (at 4 bits: code 2i in the low nibble of byte i, 2i+1 in the
 *              high one). The rows of BOS tokens are zero here.
 *   bos_codes  int8 [R / S, D], written: the BOS token's 8-bit codes of each
 *              head, in head order.
 *   scales     fp32 [R], written, as above (BOS rows included).
 * Requires bits = 3 or 4 (else BITNET_ERR_BAD_BITS), D % 8 == 0 (D % 32 == 0
 * at 3 bits, so that rows are whole 32-bit words; else BITNET_ERR_ALIGN),
 * 8 <= D <= 512, S >= 1, R % S == 0; kv 16-byte, packed 4-byte, bos_codes
 * 8-byte aligned. R = 0 is a no-op. */
bitnet_status bitnet_kv_quantize_packed(const void* kv, bitnet_dtype x_dtype, int64_t R,
                                        int64_t D, int64_t S, int bits, uint8_t* packed,
                                        int8_t* bos_codes, float* scales, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Backward                                                                  */
/* ------------------------------------------------------------------------ */

/* Gradients of the H-BitLinear forward under the engine page's training
 * rules: HadamardTransformFunction's backward applies the transform to the
 * gradient (Eq. 8), and the STE autograd functions of the weight and
 * activation quantizers pass the gradient through unchanged. With the
 * forward's y = F.linear(x_q, w_q), x_q = (scales[m] / c) q, w_q = alpha t:
 *   dx = H (alpha * dy . t)   [M, K] fp32, the gradient with respect to the
 *                             transform's input (H only when hadamard = 1)
 *   dw = dy^T . x_q           [N, K] fp32, the gradient of the latent
 *                             weights
 *   dy       [M, N] in dy_dtype (BITNET_BF16 or BITNET_F32), row-major.
 *   codes    int8 [M, K], scales fp32 [M]: what bitnet_quantize_activations
 *            wrote for the forward's input (read only when dw is set).
 *   Wpacked, alpha: the forward's packed weights [N, K/4] and alpha (read
 *            only when dx is set).
 *   bits     4 or 8 (c = sqrt 7 or 127); hadamard 0 or 1.
 *   dx, dw   outputs, written (not accumulated); either may be NULL to skip
 *            that gradient.
 * Arithmetic: products on bf16 matrix cores with fp32 accumulation; a bf16
 * dy and the ternary weights are exact there; an fp32 dy (for dx) and
 * dy * scales / c (for dw) are split into two bf16 parts (16 significant
 * bits). Workspace: bitnet_backward_workspace_bytes (256-B aligned).
 * Requires K % 64 == 0, N % 64 == 0, M and N below 2^22, and for
 * hadamard = 1 a power-of-two K <= BITNET_MAX_K; dy, codes and ws 16-byte
 * aligned. M = 0 writes dw = 0; N = 0 writes dx = 0. */
size_t bitnet_backward_workspace_bytes(int64_t M, int64_t K, int64_t N, bitnet_dtype dy_dtype,
                                       int want_dx, int want_dw);
bitnet_status bitnet_hbitlinear_backward(const void* dy, bitnet_dtype dy_dtype, int64_t M,
                                         int64_t N, const int8_t* codes, const float* scales,
                                         int64_t K, const uint8_t* Wpacked, const float* alpha,
                                         int bits, int hadamard, float* dx, float* dw, void* ws,
                                         size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Forward for callers that cannot allocate                                  */
/* ------------------------------------------------------------------------ */

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward as bitnet_hbitlinear_forward, with the same kernels, arguments
 * (minus the workspace), results (bit for bit) and errors, whose workspace is
 * a fixed device array inside the library instead of the caller's: the call
 * allocates nothing. Each GPU the library runs on holds its own
 * BITNET_NOALLOC_SCRATCH_BYTES array from the first load of the library's
 * code on it until the process ends; its address on a device is looked up
 * (hipGetSymbolAddress, no allocation) on the first call made with that
 * device current.
 *   Limit: a shape whose bitnet_forward_workspace_bytes exceeds
 *   BITNET_NOALLOC_SCRATCH_BYTES (about M * K > 64 Mi codes) is rejected with
 *   BITNET_ERR_UNSUPPORTED before anything is launched.
 *   Concurrency: every call on one GPU shares that GPU's array, and each
 *   call's quantization stage overwrites all of the workspace it uses before
 *   its product stage reads it (nothing needs clearing). Calls that overlap
 *   in time on one GPU (different streams, or host threads without ordering)
 *   race on the array and give wrong results; calls ordered on one stream do
 *   not. */
#define BITNET_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
bitnet_status bitnet_hbitlinear_forward_noalloc(const void* x, bitnet_dtype x_dtype, int64_t M,
                                                int64_t K, const uint8_t* Wpacked, int64_t N,
                                                const float* alpha, int bits, int hadamard,
                                                float* y, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Measurement and test hooks                                                */
/* ------------------------------------------------------------------------ */

/* Reads `bytes` at p with 16-byte loads and no arithmetic (a plain streaming
 * read, no step of the layer): the bandwidth ceiling the forward's weight
 * stream is measured against, and a way to push a buffer out of the caches.
 * sink (one uint32 on the device) is written only if the XOR of all words
 * read equals a fixed constant. Requires p 16-byte aligned and bytes % 16 == 0;
 * bytes = 0 is a no-op. */
bitnet_status bitnet_stream_read(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream);

/* Test hook: the next entry point on the calling thread that passes its
 * argument checks fails as if its first kernel launch had returned the HIP
 * error code hip_error (BITNET_ERR_HIP, with that code in
 * bitnet_last_error()), and launches nothing; 0 clears a pending error.
 * Makes no HIP call, so error handling can be exercised without a device. */
void bitnet_test_fail_next_launch(int hip_error);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_MI355X_H */
