// Internal launch interface between the C ABI (abi.cpp) and the gfx950 kernels.
// Every launcher enqueues on `stream` and returns the launch status; argument
// validation has already happened in the ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace bitnet {

// Number of fp64 partial sums of |W| the ternarizer's first stage writes.
constexpr int kAbsPartials = 1024;

// Token counts up to this use the weight-streaming (decode) kernels.
constexpr int64_t kDecodeMaxM = 16;

// Largest M*K whose quantization the decode kernel fuses in (the codes of the
// whole batch sit in the workgroup's LDS).
constexpr int64_t kFusedMaxElems = 16384;
// Largest K the fused decode kernel transforms (one wave holds a token row).
constexpr int64_t kFusedHadMaxK = 256;

// Work decomposition of the decode (M <= 16) product. A workgroup owns `ct`
// 16-column tiles and all of K; `sb_waves` waves take interleaved 256-k
// super-blocks (four 64-weight blocks, one per 16-lane group).
struct GemvPlan {
  int ct;          // 16-column tiles per workgroup
  int sb_waves;    // waves that own super-blocks
  int threads;     // workgroup size
  int col_groups;  // workgroups along N
  bool fused;      // x is quantized inside the kernel
};

inline GemvPlan plan_gemv(int64_t M, int64_t K, int64_t N, bool x_given, bool hadamard) {
  GemvPlan p;
  const int64_t nKB = K / 64;
  const int64_t nSB = (nKB + 3) / 4;
  p.sb_waves = (int)(nSB < 16 ? nSB : 16);
  // Fusing keeps every token's codes in LDS and needs one 4-element chunk per
  // thread and row: K <= 4 * 64 * sb_waves, i.e. a single round of waves.
  // With the transform, a whole token row must sit in one wave: K <= 256.
  p.fused = x_given && (!hadamard || K <= kFusedHadMaxK) && M * K <= kFusedMaxElems && nSB <= 16;
  p.ct = 1;
  p.col_groups = (int)((N + 16 * p.ct - 1) / (16 * p.ct));
  int waves = p.sb_waves;
  if (p.fused && waves < 4) waves = 4;
  p.threads = 64 * waves;
  return p;
}

constexpr size_t kWsAlign = 256;
inline size_t ws_round(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Stage 1 of the absmean reduction: partials[i] = sum of |W| over a fixed
// subset of the n elements (n % 4 == 0). Returns the number of partials used.
hipError_t launch_absmean_partial(const float* W, int64_t n, double* partials, int* n_partials,
                                  hipStream_t stream);

// Stage 2 + packing: every workgroup sums the partials in the same order,
// derives alpha and the rounding threshold, and packs its share of W.
hipError_t launch_ternarize_pack(const float* W, int64_t N, int64_t K, const double* partials,
                                 int n_partials, uint8_t* Wpacked, float* alpha,
                                 hipStream_t stream);

hipError_t launch_pack_2bit(const int8_t* T, int64_t N, int64_t K, uint8_t* Wpacked,
                            hipStream_t stream);

// Optional input prologue of the quantizer: the layer input is
// silu(x) * up when `up` is set (x is then the gate projection, `up` has x's
// dtype and shape), followed by RMSNorm when `rms` is set (elementwise weight
// `gamma`, ones when null, and `norm_eps`).
struct Prologue {
  const void* up;
  const float* gamma;
  float norm_eps;
  int rms;
};

#ifdef __HIPCC__
// silu(g) = g / (1 + exp(-g)) on the hardware exponential and reciprocal
// (v_exp_f32 on g * log2(e), v_rcp_f32): about 1e-6 relative error for the
// |g| the layers see, far inside the quantizer's rounding band, at a fifth of
// the operations of the correctly rounded exp and divide. Large |g| saturate
// correctly: exp(-g) -> inf gives 0, exp(-g) -> 0 gives g.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
#endif

// Nibble codes (bits = 4 only, K % 8 == 0): each token row of K codes is
// K / 2 bytes, eight codes to a 32-bit word: byte b of word i holds code
// 8 i + b in its high nibble and code 8 i + 4 + b in its low nibble (two's
// complement). Masking a word with 0xF0F0F0F0 then gives codes 8i .. 8i+3
// times 16 as int8 lanes, and shifting it left by 4 first gives the other
// four: two operations per four codes, half the bytes of int8 codes.
constexpr int kNibbleKMultiple = 256;  // the decode product reads nibble codes when K is a multiple

// FP8 pairs: a code form of the forward's workspace that only the prefill
// product reads. The 4-bit codes of a row are stored one byte each as fp8
// E4M3 (exact for integers up to 16), in the order of the fp4 weight fields
// the product unpacks: byte 32 g + 2 i + h of each 64-weight block holds
// the code of the block's weight 16 g + i + 32 h (g, h < 2, i < 16). The
// transform kernels write them (4-bit codes with the transform), and the
// 128 x 128-tile product reads them, the one that runs when there are fewer
// than 1024 tiles of 256 x 256.
inline bool fp8_pair_gemm_ok(int64_t M, int64_t K, int64_t N, int bits) {
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return bits == 4 && M > kDecodeMaxM && K % 64 == 0 && big_tiles < 1024;
}
inline bool fp8_pair_quant_ok(int bits, int hadamard) { return bits == 4 && hadamard; }

// Fused (optional) prologue + Walsh-Hadamard transform + per-token
// quantization. x_dtype: 0 = fp32, 1 = bf16 bit patterns. pro may be null.
// rowsum, when not null, receives each token's code sum (int32 [M]), which
// the prefill product then needs not compute. nibbles (bits = 4 only):
// write nibble codes instead of int8 codes; fp8_pairs: write fp8 pairs
// (fp8_pair_quant_ok only; K is then a power of two of at least 64).
hipError_t launch_quantize(const void* x, int x_dtype, int64_t M, int K, int bits, int hadamard,
                           int8_t* codes, float* scales, hipStream_t stream,
                           const Prologue* pro = nullptr, int32_t* rowsum = nullptr,
                           bool nibbles = false, bool fp8_pairs = false);

// Low-bit KV cache: rows of D elements, row r being token r % S of its head;
// token 0 int8 absmax, the others bits = 3, 4 or 8. With packed (bits 3 or 4
// only), the non-BOS codes go to packed [R, D * bits / 8] as one bit stream
// per row and codes is the [R / S, D] array of the BOS rows' int8 codes.
hipError_t launch_kv_quantize(const void* kv, int x_dtype, int64_t R, int D, int S, int bits,
                              int8_t* codes, float* scales, hipStream_t stream,
                              uint8_t* packed = nullptr);

// Ternary product from codes. Exactly one of y (dequantized; needs scales,
// alpha, bits) or acc (raw int32) is non-null. rowsum (optional, with y):
// the codes' per-token sums from launch_quantize. nibbles: the codes are
// nibble codes (M <= kDecodeMaxM and K % kNibbleKMultiple == 0 only);
// fp8_pairs: the codes are fp8 pairs (fp8_pair_gemm_ok, with y and rowsum).
hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream,
                                 const int32_t* rowsum = nullptr, bool nibbles = false,
                                 bool fp8_pairs = false);

// The two product shapes behind launch_ternary_matmul.
hipError_t launch_gemv(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream, bool nibbles = false,
                       const int32_t* rowsum = nullptr);
hipError_t launch_gemm(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream, const int32_t* rowsum = nullptr,
                       bool fp8_pairs = false);

// Decode forward with the quantization fused in (plan.fused must hold).
hipError_t launch_fused_decode(const void* x, int x_dtype, int64_t M, int K,
                               const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                               float* y, hipStream_t stream, const Prologue* pro = nullptr,
                               int hadamard = 0);

// ---- Backward -------------------------------------------------------------

// C[R, Cn] = scale * (A + A_lo)[R, Kc] . B[Cn, Kc]^T on bf16 operands
// (uint16 bit patterns, row pitches lda / ldb elements; A_lo may be null),
// fp32 out with pitch ldc; scale = scale_h * *scale_p (scale_p may be null).
// Kc % 64 == 0.
hipError_t launch_bf16_gemm_nt(const uint16_t* A, const uint16_t* A_lo, int64_t lda,
                               const uint16_t* B, int64_t ldb, int64_t R, int64_t Cn, int64_t Kc,
                               float* C, int64_t ldc, const float* scale_p, float scale_h,
                               hipStream_t stream);

// Wt [K, N] bf16 = t^T from the packed weights (N % 64 == 0, K % 64 == 0).
hipError_t launch_expand_transpose(const uint8_t* Wpacked, int64_t N, int64_t K, uint16_t* Wt,
                                   hipStream_t stream);

// fp32 -> hi, lo bf16 (hi + lo equals x to 16 significant bits); n % 8 == 0.
hipError_t launch_split_rows(const float* x, int64_t n, uint16_t* hi, uint16_t* lo,
                             hipStream_t stream);

// phi / plo [N, Mp] = split of dy[m][n] * scales[m] * inv_c, transposed,
// zero for m >= M (Mp % 64 == 0, N % 64 == 0).
hipError_t launch_scale_transpose_split(const void* dy, int dy_dtype, const float* scales,
                                        float inv_c, int64_t M, int64_t N, int64_t Mp,
                                        uint16_t* phi, uint16_t* plo, hipStream_t stream);

// Qt [K, Mp] bf16 = codes^T, zero for m >= M.
hipError_t launch_codes_transpose(const int8_t* codes, int64_t M, int64_t K, int64_t Mp,
                                  uint16_t* Qt, hipStream_t stream);

// Orthonormal Walsh-Hadamard transform of fp32 rows of length K (a power of
// two, 64 .. 32768); out may equal x.
hipError_t launch_fwht_f32(const float* x, int64_t M, int K, float* out, hipStream_t stream);

// TL2 weight code (edge page mirror consolidation, 5 bits per 3 weights):
// blocks of 128 triplets per column (64 index bytes, 16 sign bytes); a
// partial last block holds only its G groups of 32 triplets (96 weights):
// 16 G index bytes, then 4 G sign bytes, rounded up to 16 bytes.
constexpr int kTl2MaxK = 6 * 768;  // single-token TL2 decode: six 768-weight super-blocks
constexpr int kTl2BlockK = 384;     // weights per block
constexpr int kTl2BlockBytes = 80;  // 64 index bytes + 16 sign bytes
__host__ __device__ inline int tl2_last_groups(int64_t K) {  // groups of the last block
  const int r = (int)(K % kTl2BlockK);
  return r ? (r + 95) / 96 : 4;
}
__host__ __device__ inline int64_t tl2_row_bytes(int64_t K) {
  const int g = tl2_last_groups(K);
  return (K / kTl2BlockK) * kTl2BlockBytes + (K % kTl2BlockK ? (20 * g + 15) / 16 * 16 : 0);
}
inline size_t tl2_bytes(int64_t N, int64_t K) { return (size_t)N * (size_t)tl2_row_bytes(K); }
// 2-bit packed weights [N, K/4] -> TL2 [N, tl2_bytes / N].
hipError_t launch_repack_tl2(const uint8_t* Wpacked, int64_t N, int K, uint8_t* Wtl2,
                             hipStream_t stream);
// Per-token quantization (no transform) with the codes in TL2 order: rows of
// tl2_code_row(K) bytes, whole 384-code blocks, the code of weight 3 j + p of
// a block at its byte 128 p + j, the codes past K zero; scales and row sums
// as launch_quantize's.
inline int64_t tl2_code_row(int64_t K) { return (K + kTl2BlockK - 1) / kTl2BlockK * kTl2BlockK; }
hipError_t launch_quantize_tl2_order(const void* x, int x_dtype, int64_t M, int K, int bits,
                                     int8_t* codes, float* scales, int32_t* rowsum,
                                     hipStream_t stream);
// Batched TL2 product (1 <= M <= 16) from TL2-order codes, their scales and
// row sums: y [M, N].
hipError_t launch_tl2_gemv(const int8_t* codes, const float* scales, const int32_t* rowsum,
                           int64_t M, int K, const uint8_t* Wtl2, int64_t N, const float* alpha,
                           int bits, float* y, hipStream_t stream);
// Single-token decode forward (M = 1, no transform, K <= kTl2MaxK) on TL2 weights.
hipError_t launch_tl2_decode(const void* x, int x_dtype, int K, const uint8_t* Wtl2, int64_t N,
                             const float* alpha, int bits, float* y, hipStream_t stream);

// Forward scratch of the entry point that allocates nothing: a fixed device
// array (one per GPU). noalloc_scratch gives its address on the current
// device, looked up once per device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

// Measurement: read `bytes` (a multiple of 16 is read; the tail is ignored)
// with 16-byte loads and no arithmetic; sink receives a word only in the
// (practically never met) case that the data's XOR equals a fixed constant.
hipError_t launch_stream_read(const void* p, size_t bytes, unsigned* sink, hipStream_t stream);

}  // namespace bitnet
