// C ABI of the H-BitLinear library: argument validation, workspace layout and
// dispatch to the gfx950 kernels. No entry point allocates, frees or
// synchronizes; no C++ exception crosses the ABI; nothing is launched when
// validation fails. Loading the library makes no HIP call.
#include "../../include/bitnet_mi355x.h"

#include <climits>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_last_error;
// HIP error the next launch on this thread reports instead of launching (test
// hook; 0 = none).
thread_local int g_injected_error = 0;

bitnet_status fail(bitnet_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bitnet_status ok() {
  g_last_error.clear();
  return BITNET_OK;
}

bitnet_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BITNET_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

// Called by every entry point after its arguments have been validated and
// before its first launch: a pending injected error is reported as that
// launch's failure (BITNET_ERR_HIP) and nothing is launched.
bitnet_status launch_guard(const char* fn) {
  if (g_injected_error == 0) return BITNET_OK;
  const hipError_t e = static_cast<hipError_t>(g_injected_error);
  g_injected_error = 0;
  return hip_status(e, fn);
}

size_t round_up(size_t v) { return bitnet::ws_round(v); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Largest M: the kernels carry token counts, row indices and the prefill
// tile count as 32-bit ints (the tile count (M / 128 + 1) (N / 128 + 1) must
// stay below 2^31 as well; checked with N below).
constexpr int64_t kMaxM = (int64_t)1 << 23;

bitnet_status check_dims(const char* fn, int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0)
    return fail(BITNET_ERR_INVALID_ARG, "%s: negative size (M=%lld K=%lld N=%lld)", fn,
                (long long)M, (long long)K, (long long)N);
  if (K == 0 || K % 64 != 0)
    return fail(BITNET_ERR_ALIGN, "%s: K=%lld must be a positive multiple of 64", fn, (long long)K);
  if (M > kMaxM || N > INT_MAX || (M / 128 + 1) * (N / 128 + 1) >= ((int64_t)1 << 31))
    return fail(BITNET_ERR_UNSUPPORTED, "%s: M=%lld or N=%lld too large", fn, (long long)M,
                (long long)N);
  return BITNET_OK;
}

bitnet_status check_quant_args(const char* fn, int64_t K, int bits, int hadamard, int x_dtype) {
  if (bits != 4 && bits != 8)
    return fail(BITNET_ERR_BAD_BITS, "%s: bits=%d must be 4 or 8", fn, bits);
  if (K > BITNET_MAX_K)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld exceeds BITNET_MAX_K=%d", fn, (long long)K,
                BITNET_MAX_K);
  if (hadamard && !is_pow2(K))
    return fail(BITNET_ERR_NOT_POW2, "%s: K=%lld must be a power of two with hadamard=1", fn,
                (long long)K);
  if (x_dtype != BITNET_F32 && x_dtype != BITNET_BF16)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: unknown x dtype %d", fn, x_dtype);
  return BITNET_OK;
}

// Forward workspace: [codes M*K][scales 4M][code row sums 4M], each part
// 256-B aligned. The fused decode kernel needs none of it. The quantizer
// writes each token's code sum so that the GEMM's epilogue can subtract it
// without summing the codes again.
struct ForwardWorkspace {
  int8_t* codes;
  float* scales;
  int32_t* rowsum;
};

size_t forward_parts_bytes(int64_t M, int64_t K) {
  return round_up((size_t)M * (size_t)K) + 2 * round_up((size_t)M * sizeof(float));
}

// Small batches of int4 codes travel between the quantizer and the
// weight-streaming product as nibble codes: every workgroup of the product
// reads all of the codes, so halving them shortens the product (M = 16,
// K = 16384, N = 4096: 10.0 -> 8.9 us per product launch).
bool use_nibble_codes(int64_t M, int64_t K, int bits) {
  return bits == 4 && M <= bitnet::kDecodeMaxM && K % bitnet::kNibbleKMultiple == 0;
}

// The forward's 4-bit codes go from the transform kernels to the 128 x
// 128-tile product as fp8 pairs when both can take them (one fp8 x fp4 MFMA
// per 64-weight block instead of two int8 ones).
bool use_fp8_pairs(int64_t M, int64_t K, int64_t N, int bits, int hadamard) {
  return bitnet::fp8_pair_quant_ok(bits, hadamard) && bitnet::fp8_pair_gemm_ok(M, K, N, bits);
}

bool forward_is_fused(int64_t M, int64_t K, int64_t N, int hadamard) {
  if (M > bitnet::kDecodeMaxM) return false;
  return bitnet::plan_gemv(M, K, N, true, hadamard != 0).fused;
}

size_t forward_ws_bytes(int64_t M, int64_t K, int64_t N, int hadamard) {
  if (M <= 0 || N <= 0) return 0;
  if (forward_is_fused(M, K, N, hadamard)) return 0;
  return forward_parts_bytes(M, K);
}

ForwardWorkspace carve_forward(void* ws, int64_t M, int64_t K) {
  char* base = static_cast<char*>(ws);
  ForwardWorkspace w;
  w.codes = reinterpret_cast<int8_t*>(base);
  w.scales = reinterpret_cast<float*>(base + round_up((size_t)M * (size_t)K));
  w.rowsum = reinterpret_cast<int32_t*>(base + round_up((size_t)M * (size_t)K) +
                                        round_up((size_t)M * sizeof(float)));
  return w;
}

}  // namespace

extern "C" {

int bitnet_abi_version(void) { return BITNET_ABI_VERSION; }

const char* bitnet_last_error(void) { return g_last_error.c_str(); }

void bitnet_test_fail_next_launch(int hip_error) { g_injected_error = hip_error; }

size_t bitnet_ternarize_workspace_bytes(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return round_up(sizeof(double) * bitnet::kAbsPartials);
}

bitnet_status bitnet_ternarize_weights(const float* W, int64_t N, int64_t K, uint8_t* Wpacked,
                                       float* alpha, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  const char* fn = "bitnet_ternarize_weights";
  if (bitnet_status st = check_dims(fn, 0, K, N)) return st;
  if (N == 0) return fail(BITNET_ERR_INVALID_ARG, "%s: N must be >= 1 (mean of an empty tensor)", fn);
  if (!W || !Wpacked || !alpha || !ws)
    return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (ws_bytes < bitnet_ternarize_workspace_bytes(N, K))
    return fail(BITNET_ERR_INVALID_ARG, "%s: workspace %zu B < required %zu B", fn, ws_bytes,
                bitnet_ternarize_workspace_bytes(N, K));
  if (!aligned(W, 16) || !aligned(Wpacked, 16) || !aligned(ws, 16) || !aligned(alpha, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  double* partials = static_cast<double*>(ws);
  int n_partials = 0;
  hipError_t e = bitnet::launch_absmean_partial(W, N * K, partials, &n_partials, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  e = bitnet::launch_ternarize_pack(W, N, K, partials, n_partials, Wpacked, alpha, stream);
  return hip_status(e, fn);
}

bitnet_status bitnet_pack_2bit(const int8_t* T, int64_t N, int64_t K, uint8_t* Wpacked,
                               hipStream_t stream) {
  const char* fn = "bitnet_pack_2bit";
  if (bitnet_status st = check_dims(fn, 0, K, N)) return st;
  if (N == 0) return ok();
  if (!T || !Wpacked) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(T, 16) || !aligned(Wpacked, 16))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_pack_2bit(T, N, K, Wpacked, stream), fn);
}

size_t bitnet_forward_workspace_bytes(int64_t M, int64_t K, int64_t N, int bits, int hadamard) {
  (void)bits;
  if (M < 0 || K <= 0 || N < 0 || K % 64 != 0) return 0;
  return forward_ws_bytes(M, K, N, hadamard);
}

bitnet_status bitnet_quantize_activations(const void* x, bitnet_dtype x_dtype, int64_t M,
                                          int64_t K, int bits, int hadamard, int8_t* codes,
                                          float* scales, int32_t* rowsum, hipStream_t stream) {
  const char* fn = "bitnet_quantize_activations";
  if (bitnet_status st = check_dims(fn, M, K, 0)) return st;
  if (bitnet_status st = check_quant_args(fn, K, bits, hadamard, x_dtype)) return st;
  if (M == 0) return ok();
  if (!x || !codes || !scales) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(rowsum, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_quantize(x, (int)x_dtype, M, (int)K, bits, hadamard, codes,
                                            scales, stream, nullptr, rowsum),
                    fn);
}

bitnet_status bitnet_ternary_gemm_i32(const int8_t* codes, int64_t M, int64_t K,
                                      const uint8_t* Wpacked, int64_t N, int32_t* acc,
                                      hipStream_t stream) {
  const char* fn = "bitnet_ternary_gemm_i32";
  if (bitnet_status st = check_dims(fn, M, K, N)) return st;
  if (K > BITNET_MAX_K)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld exceeds BITNET_MAX_K=%d", fn, (long long)K,
                BITNET_MAX_K);
  if (M == 0 || N == 0) return ok();
  if (!codes || !Wpacked || !acc) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(codes, 16) || !aligned(Wpacked, 16) || !aligned(acc, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_ternary_matmul(codes, nullptr, M, (int)K, Wpacked, N, nullptr,
                                                  8, nullptr, acc, stream),
                    fn);
}

bitnet_status bitnet_ternary_linear_dequant(const int8_t* codes, const float* scales,
                                            const int32_t* rowsum, int64_t M, int64_t K,
                                            const uint8_t* Wpacked, int64_t N, const float* alpha,
                                            int bits, float* y, hipStream_t stream) {
  const char* fn = "bitnet_ternary_linear_dequant";
  if (bitnet_status st = check_dims(fn, M, K, N)) return st;
  if (bits != 4 && bits != 8) return fail(BITNET_ERR_BAD_BITS, "%s: bits=%d must be 4 or 8", fn, bits);
  if (K > BITNET_MAX_K)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld exceeds BITNET_MAX_K=%d", fn, (long long)K,
                BITNET_MAX_K);
  if (M == 0 || N == 0) return ok();
  if (!codes || !scales || !Wpacked || !alpha || !y)
    return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(codes, 16) || !aligned(Wpacked, 16) || !aligned(y, 4) || !aligned(scales, 4) ||
      !aligned(alpha, 4) || !aligned(rowsum, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_ternary_matmul(codes, scales, M, (int)K, Wpacked, N, alpha,
                                                  bits, y, nullptr, stream, rowsum),
                    fn);
}

}  // extern "C"

namespace {

static_assert(BITNET_NOALLOC_SCRATCH_BYTES == bitnet::kNoAllocScratchBytes,
              "the header's scratch size is the library's");

// The forward, or the stages of it that `stages` selects (both for the
// forward itself). With fixed_scratch the workspace is the library's fixed
// device array instead of the caller's ws (which is then ignored): its size
// is checked with the other arguments, and its address, looked up once per
// device, is taken only after every check has passed.
bitnet_status forward_impl(const char* fn, const void* x, bitnet_dtype x_dtype, int64_t M,
                           int64_t K, const uint8_t* Wpacked, int64_t N, const float* alpha,
                           int bits, int hadamard, float* y, void* ws, size_t ws_bytes, int stages,
                           hipStream_t stream, bool fixed_scratch = false) {
  if (stages < 1 || stages > 3)
    return fail(BITNET_ERR_INVALID_ARG, "%s: stages=%d must be 1, 2 or 3", fn, stages);
  if (bitnet_status st = check_dims(fn, M, K, N)) return st;
  if (bitnet_status st = check_quant_args(fn, K, bits, hadamard, x_dtype)) return st;
  if (M == 0 || N == 0) return ok();
  if (!x || !Wpacked || !alpha || !y)
    return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  const size_t need = forward_ws_bytes(M, K, N, hadamard);
  if (fixed_scratch) {
    if (need > bitnet::kNoAllocScratchBytes)
      return fail(BITNET_ERR_UNSUPPORTED,
                  "%s: M=%lld K=%lld needs %zu B of scratch, above the fixed %zu B", fn,
                  (long long)M, (long long)K, need, bitnet::kNoAllocScratchBytes);
  } else if (need > 0 && (!ws || ws_bytes < need)) {
    return fail(BITNET_ERR_INVALID_ARG, "%s: workspace %zu B < required %zu B", fn,
                ws ? ws_bytes : (size_t)0, need);
  }
  if (!aligned(x, 16) || !aligned(Wpacked, 16) ||
      (need > 0 && !fixed_scratch && !aligned(ws, 16)) || !aligned(y, 4) || !aligned(alpha, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (need == 0 && stages != BITNET_STAGE_QUANTIZE + BITNET_STAGE_PRODUCT)
    return fail(BITNET_ERR_UNSUPPORTED,
                "%s: this shape runs as one fused kernel; its stages cannot run apart", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  if (fixed_scratch && need > 0) {
    if (hipError_t e = bitnet::noalloc_scratch(&ws)) return hip_status(e, fn);
  }
  if (need == 0) {
    return hip_status(bitnet::launch_fused_decode(x, (int)x_dtype, M, (int)K, Wpacked, N, alpha,
                                                  bits, y, stream, nullptr, hadamard),
                      fn);
  }
  const ForwardWorkspace w = carve_forward(ws, M, K);
  const bool nib = use_nibble_codes(M, K, bits);
  const bool f8 = use_fp8_pairs(M, K, N, bits, hadamard);
  hipError_t e = hipSuccess;
  if (stages & BITNET_STAGE_QUANTIZE) {
    e = bitnet::launch_quantize(x, (int)x_dtype, M, (int)K, bits, hadamard, w.codes, w.scales,
                                stream, nullptr, w.rowsum, nib, f8);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  if (stages & BITNET_STAGE_PRODUCT)
    e = bitnet::launch_ternary_matmul(w.codes, w.scales, M, (int)K, Wpacked, N, alpha, bits, y,
                                      nullptr, stream, w.rowsum, nib, f8);
  return hip_status(e, fn);
}

}  // namespace

extern "C" {

bitnet_status bitnet_hbitlinear_forward(const void* x, bitnet_dtype x_dtype, int64_t M, int64_t K,
                                        const uint8_t* Wpacked, int64_t N, const float* alpha,
                                        int bits, int hadamard, float* y, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  return forward_impl("bitnet_hbitlinear_forward", x, x_dtype, M, K, Wpacked, N, alpha, bits,
                      hadamard, y, ws, ws_bytes, BITNET_STAGE_QUANTIZE + BITNET_STAGE_PRODUCT,
                      stream);
}

bitnet_status bitnet_hbitlinear_forward_stages(const void* x, bitnet_dtype x_dtype, int64_t M,
                                               int64_t K, const uint8_t* Wpacked, int64_t N,
                                               const float* alpha, int bits, int hadamard,
                                               float* y, void* ws, size_t ws_bytes, int stages,
                                               hipStream_t stream) {
  return forward_impl("bitnet_hbitlinear_forward_stages", x, x_dtype, M, K, Wpacked, N, alpha,
                      bits, hadamard, y, ws, ws_bytes, stages, stream);
}

bitnet_status bitnet_hbitlinear_forward_noalloc(const void* x, bitnet_dtype x_dtype, int64_t M,
                                                int64_t K, const uint8_t* Wpacked, int64_t N,
                                                const float* alpha, int bits, int hadamard,
                                                float* y, hipStream_t stream) {
  return forward_impl("bitnet_hbitlinear_forward_noalloc", x, x_dtype, M, K, Wpacked, N, alpha,
                      bits, hadamard, y, nullptr, 0, BITNET_STAGE_QUANTIZE + BITNET_STAGE_PRODUCT,
                      stream, /*fixed_scratch=*/true);
}

bitnet_status bitnet_stream_read(const void* p, size_t bytes, uint32_t* sink,
                                 hipStream_t stream) {
  const char* fn = "bitnet_stream_read";
  if (bytes == 0) return ok();
  if (!p || !sink) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(p, 16) || !aligned(sink, 4) || bytes % 16 != 0)
    return fail(BITNET_ERR_ALIGN, "%s: p must be 16-byte aligned and bytes a multiple of 16", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_stream_read(p, bytes, sink, stream), fn);
}

size_t bitnet_forward_prologue_workspace_bytes(int64_t M, int64_t K, int64_t N, int bits,
                                               int hadamard) {
  (void)bits;
  (void)hadamard;
  if (M <= 0 || K <= 0 || N <= 0 || K % 64 != 0) return 0;
  return forward_parts_bytes(M, K);
}

}  // extern "C"

namespace {

// Backward workspace. The dx parts (t^T in bf16; the hi/lo halves of an
// fp32 dy) and the dw parts (hi/lo of dy * s / c transposed; the codes
// transposed) are used one after the other on the stream, so they share the
// same bytes.
constexpr int64_t kMaxGradDim = (int64_t)1 << 22;

struct BackwardWorkspace {
  uint16_t* wt;
  uint16_t* dy_hi;
  uint16_t* dy_lo;
  uint16_t* p_hi;
  uint16_t* p_lo;
  uint16_t* qt;
};

int64_t pad64(int64_t v) { return (v + 63) / 64 * 64; }

size_t backward_dx_bytes(int64_t M, int64_t K, int64_t N, int dy_dtype) {
  size_t b = round_up((size_t)K * N * 2);
  if (dy_dtype == BITNET_F32) b += 2 * round_up((size_t)M * N * 2);
  return b;
}

size_t backward_dw_bytes(int64_t M, int64_t K, int64_t N) {
  const size_t Mp = (size_t)pad64(M);
  return 2 * round_up((size_t)N * Mp * 2) + round_up((size_t)K * Mp * 2);
}

BackwardWorkspace carve_backward(void* ws, int64_t M, int64_t K, int64_t N) {
  BackwardWorkspace w{};
  char* b = static_cast<char*>(ws);
  w.wt = reinterpret_cast<uint16_t*>(b);
  w.dy_hi = reinterpret_cast<uint16_t*>(b + round_up((size_t)K * N * 2));
  w.dy_lo = reinterpret_cast<uint16_t*>(b + round_up((size_t)K * N * 2) + round_up((size_t)M * N * 2));
  const size_t Mp = (size_t)pad64(M);
  w.p_hi = reinterpret_cast<uint16_t*>(b);
  w.p_lo = reinterpret_cast<uint16_t*>(b + round_up((size_t)N * Mp * 2));
  w.qt = reinterpret_cast<uint16_t*>(b + 2 * round_up((size_t)N * Mp * 2));
  return w;
}

}  // namespace

extern "C" {

size_t bitnet_backward_workspace_bytes(int64_t M, int64_t K, int64_t N, bitnet_dtype dy_dtype,
                                       int want_dx, int want_dw) {
  if (M < 0 || K <= 0 || N < 0 || K % 64 != 0 || N % 64 != 0) return 0;
  size_t b = 0;
  if (want_dx) b = backward_dx_bytes(M, K, N, dy_dtype);
  if (want_dw) {
    const size_t d = backward_dw_bytes(M, K, N);
    if (d > b) b = d;
  }
  return b;
}

bitnet_status bitnet_hbitlinear_backward(const void* dy, bitnet_dtype dy_dtype, int64_t M,
                                         int64_t N, const int8_t* codes, const float* scales,
                                         int64_t K, const uint8_t* Wpacked, const float* alpha,
                                         int bits, int hadamard, float* dx, float* dw, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  const char* fn = "bitnet_hbitlinear_backward";
  if (M < 0 || K < 0 || N < 0)
    return fail(BITNET_ERR_INVALID_ARG, "%s: negative size (M=%lld K=%lld N=%lld)", fn,
                (long long)M, (long long)K, (long long)N);
  if (K == 0 || K % 64 != 0 || N % 64 != 0)
    return fail(BITNET_ERR_ALIGN, "%s: K=%lld must be a positive multiple of 64 and N=%lld a "
                "multiple of 64", fn, (long long)K, (long long)N);
  if (M >= kMaxGradDim || N >= kMaxGradDim)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: M=%lld or N=%lld not below 2^22", fn, (long long)M,
                (long long)N);
  if (bits != 4 && bits != 8)
    return fail(BITNET_ERR_BAD_BITS, "%s: bits=%d must be 4 or 8", fn, bits);
  if (hadamard != 0 && hadamard != 1)
    return fail(BITNET_ERR_INVALID_ARG, "%s: hadamard=%d must be 0 or 1", fn, hadamard);
  if (hadamard && (!is_pow2(K) || K > BITNET_MAX_K))
    return fail(BITNET_ERR_NOT_POW2, "%s: K=%lld must be a power of two <= %d with hadamard=1",
                fn, (long long)K, BITNET_MAX_K);
  if (dy_dtype != BITNET_F32 && dy_dtype != BITNET_BF16)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: unknown dy dtype %d", fn, dy_dtype);
  if (!dx && !dw) return ok();
  if (M == 0 && !dw) return ok();  // dx has no elements
  if ((M > 0 && N > 0 && !dy) || (dx && (!Wpacked || !alpha)) || (dw && M > 0 && (!codes || !scales)))
    return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  const size_t need = bitnet_backward_workspace_bytes(M, K, N, dy_dtype, dx != nullptr,
                                                      dw != nullptr);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(BITNET_ERR_INVALID_ARG, "%s: workspace %zu B < required %zu B", fn,
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(dy, 16) || !aligned(codes, 16) || !aligned(Wpacked, 16) || !aligned(ws, 256) ||
      !aligned(dx, 4) || !aligned(dw, 4) || !aligned(scales, 4) || !aligned(alpha, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);

  if (bitnet_status st = launch_guard(fn)) return st;
  const BackwardWorkspace w = carve_backward(ws, M, K, N);
  hipError_t e = hipSuccess;
  if (dx && M > 0) {
    // dx = H (alpha dy . t): t^T expanded to bf16, one product per bf16 part
    // of dy, then the transform of each row.
    e = bitnet::launch_expand_transpose(Wpacked, N, K, w.wt, stream);
    if (e != hipSuccess) return hip_status(e, fn);
    if (dy_dtype == BITNET_BF16) {
      e = bitnet::launch_bf16_gemm_nt(static_cast<const uint16_t*>(dy), nullptr, N, w.wt, N, M, K,
                                      N, dx, K, alpha, 1.0f, stream);
    } else {
      e = bitnet::launch_split_rows(static_cast<const float*>(dy), M * N, w.dy_hi, w.dy_lo, stream);
      if (e == hipSuccess)
        e = bitnet::launch_bf16_gemm_nt(w.dy_hi, w.dy_lo, N, w.wt, N, M, K, N, dx, K, alpha, 1.0f,
                                        stream);
    }
    if (e != hipSuccess) return hip_status(e, fn);
    if (hadamard) {
      e = bitnet::launch_fwht_f32(dx, M, (int)K, dx, stream);
      if (e != hipSuccess) return hip_status(e, fn);
    }
  }
  if (dw) {
    // dw = dy^T x_q = (dy s / c)^T q: both operands transposed so that the
    // tokens are contiguous, dy s / c in two bf16 parts.
    const int64_t Mp = pad64(M);
    const float inv_c = 1.0f / (bits == 8 ? 127.0f : 2.6457513110645906f);
    e = bitnet::launch_scale_transpose_split(dy, (int)dy_dtype, scales, inv_c, M, N, Mp, w.p_hi,
                                             w.p_lo, stream);
    if (e == hipSuccess) e = bitnet::launch_codes_transpose(codes, M, K, Mp, w.qt, stream);
    if (e == hipSuccess)
      e = bitnet::launch_bf16_gemm_nt(w.p_hi, w.p_lo, Mp, w.qt, Mp, N, K, Mp, dw, K, nullptr, 1.0f,
                                      stream);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return ok();
}

}  // extern "C"

namespace {

bitnet_status check_prologue(const char* fn, const void* up, int rmsnorm, const float* norm_weight,
                             float norm_eps) {
  if (rmsnorm != 0 && rmsnorm != 1)
    return fail(BITNET_ERR_INVALID_ARG, "%s: rmsnorm=%d must be 0 or 1", fn, rmsnorm);
  if (rmsnorm && !(norm_eps > 0.0f && norm_eps < 3.0e38f))
    return fail(BITNET_ERR_INVALID_ARG, "%s: norm_eps must be a positive finite value", fn);
  if ((up && !aligned(up, 16)) || (rmsnorm && norm_weight && !aligned(norm_weight, 16)))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned prologue pointer", fn);
  return BITNET_OK;
}

}  // namespace

extern "C" {

bitnet_status bitnet_quantize_activations_prologue(const void* x, const void* up,
                                                   bitnet_dtype x_dtype, int64_t M, int64_t K,
                                                   int rmsnorm, const float* norm_weight,
                                                   float norm_eps, int bits, int hadamard,
                                                   int8_t* codes, float* scales,
                                                   hipStream_t stream) {
  const char* fn = "bitnet_quantize_activations_prologue";
  if (bitnet_status st = check_dims(fn, M, K, 0)) return st;
  if (bitnet_status st = check_quant_args(fn, K, bits, hadamard, x_dtype)) return st;
  if (bitnet_status st = check_prologue(fn, up, rmsnorm, norm_weight, norm_eps)) return st;
  if (M == 0) return ok();
  if (!x || !codes || !scales) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  const bitnet::Prologue pro{up, rmsnorm ? norm_weight : nullptr, norm_eps, rmsnorm};
  return hip_status(bitnet::launch_quantize(x, (int)x_dtype, M, (int)K, bits, hadamard, codes,
                                            scales, stream, &pro),
                    fn);
}

bitnet_status bitnet_hbitlinear_forward_prologue(const void* x, const void* up, bitnet_dtype x_dtype,
                                                 int64_t M, int64_t K, int rmsnorm,
                                                 const float* norm_weight, float norm_eps,
                                                 const uint8_t* Wpacked, int64_t N,
                                                 const float* alpha, int bits, int hadamard,
                                                 float* y, void* ws, size_t ws_bytes,
                                                 hipStream_t stream) {
  const char* fn = "bitnet_hbitlinear_forward_prologue";
  if (bitnet_status st = check_dims(fn, M, K, N)) return st;
  if (bitnet_status st = check_quant_args(fn, K, bits, hadamard, x_dtype)) return st;
  if (bitnet_status st = check_prologue(fn, up, rmsnorm, norm_weight, norm_eps)) return st;
  if (M == 0 || N == 0) return ok();
  if (!x || !Wpacked || !alpha || !y)
    return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  const size_t need = bitnet_forward_prologue_workspace_bytes(M, K, N, bits, hadamard);
  if (!ws || ws_bytes < need)
    return fail(BITNET_ERR_INVALID_ARG, "%s: workspace %zu B < required %zu B", fn,
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(x, 16) || !aligned(Wpacked, 16) || !aligned(ws, 16) || !aligned(y, 4) ||
      !aligned(alpha, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  const bitnet::Prologue pro{up, rmsnorm ? norm_weight : nullptr, norm_eps, rmsnorm};
  if (forward_is_fused(M, K, N, hadamard)) {
    return hip_status(bitnet::launch_fused_decode(x, (int)x_dtype, M, (int)K, Wpacked, N, alpha,
                                                  bits, y, stream, &pro, hadamard),
                      fn);
  }
  const ForwardWorkspace w = carve_forward(ws, M, K);
  const bool nib = use_nibble_codes(M, K, bits);
  const bool f8 = use_fp8_pairs(M, K, N, bits, hadamard);
  hipError_t e = bitnet::launch_quantize(x, (int)x_dtype, M, (int)K, bits, hadamard, w.codes,
                                         w.scales, stream, &pro, w.rowsum, nib, f8);
  if (e != hipSuccess) return hip_status(e, fn);
  e = bitnet::launch_ternary_matmul(w.codes, w.scales, M, (int)K, Wpacked, N, alpha, bits, y,
                                    nullptr, stream, w.rowsum, nib, f8);
  return hip_status(e, fn);
}

namespace {

bitnet_status kv_check(const char* fn, int64_t R, int64_t D, int64_t S, int bits,
                       bitnet_dtype x_dtype, bool packed) {
  if (R < 0 || D < 0 || S < 0)
    return fail(BITNET_ERR_INVALID_ARG, "%s: negative size (R=%lld D=%lld S=%lld)", fn,
                (long long)R, (long long)D, (long long)S);
  if (packed ? (bits != 3 && bits != 4) : (bits != 3 && bits != 4 && bits != 8))
    return fail(BITNET_ERR_BAD_BITS, "%s: bits=%d must be %s", fn, bits, packed ? "3 or 4" : "3, 4 or 8");
  if (D % 8 != 0 || D < 8)
    return fail(BITNET_ERR_ALIGN, "%s: D=%lld must be a positive multiple of 8", fn, (long long)D);
  if (packed && bits == 3 && D % 32 != 0)
    return fail(BITNET_ERR_ALIGN, "%s: D=%lld must be a multiple of 32 for 3-bit packing", fn,
                (long long)D);
  if (D > 512)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: D=%lld exceeds 512", fn, (long long)D);
  if (S < 1 || R % S != 0)
    return fail(BITNET_ERR_INVALID_ARG, "%s: R=%lld must be a multiple of S=%lld >= 1", fn,
                (long long)R, (long long)S);
  if (x_dtype != BITNET_F32 && x_dtype != BITNET_BF16)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, x_dtype);
  if (S > INT_MAX || R > (int64_t)INT_MAX * 64)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: R or S too large", fn);
  return BITNET_OK;
}

}  // namespace

bitnet_status bitnet_kv_quantize(const void* kv, bitnet_dtype x_dtype, int64_t R, int64_t D,
                                 int64_t S, int bits, int8_t* codes, float* scales,
                                 hipStream_t stream) {
  const char* fn = "bitnet_kv_quantize";
  if (bitnet_status st = kv_check(fn, R, D, S, bits, x_dtype, false)) return st;
  if (R == 0) return ok();
  if (!kv || !codes || !scales) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(kv, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_kv_quantize(kv, (int)x_dtype, R, (int)D, (int)S, bits, codes,
                                               scales, stream),
                    fn);
}

bitnet_status bitnet_kv_quantize_packed(const void* kv, bitnet_dtype x_dtype, int64_t R,
                                        int64_t D, int64_t S, int bits, uint8_t* packed,
                                        int8_t* bos_codes, float* scales, hipStream_t stream) {
  const char* fn = "bitnet_kv_quantize_packed";
  if (bitnet_status st = kv_check(fn, R, D, S, bits, x_dtype, true)) return st;
  if (R == 0) return ok();
  if (!kv || !packed || !bos_codes || !scales)
    return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(kv, 16) || !aligned(packed, 4) || !aligned(bos_codes, 8) || !aligned(scales, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_kv_quantize(kv, (int)x_dtype, R, (int)D, (int)S, bits,
                                               bos_codes, scales, stream, packed),
                    fn);
}

size_t bitnet_tl2_bytes(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K % 64 != 0) return 0;
  return bitnet::tl2_bytes(N, K);
}

bitnet_status bitnet_pack_tl2(const uint8_t* Wpacked, int64_t N, int64_t K, uint8_t* Wtl2,
                              hipStream_t stream) {
  const char* fn = "bitnet_pack_tl2";
  if (bitnet_status st = check_dims(fn, 0, K, N)) return st;
  if (N == 0) return ok();
  if (!Wpacked || !Wtl2) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(Wpacked, 16) || !aligned(Wtl2, 16))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_repack_tl2(Wpacked, N, (int)K, Wtl2, stream), fn);
}

bitnet_status bitnet_hbitlinear_forward_tl2(const void* x, bitnet_dtype x_dtype, int64_t M,
                                            int64_t K, const uint8_t* Wtl2, int64_t N,
                                            const float* alpha, int bits, float* y,
                                            hipStream_t stream) {
  const char* fn = "bitnet_hbitlinear_forward_tl2";
  if (bitnet_status st = check_dims(fn, M, K, N)) return st;
  if (bitnet_status st = check_quant_args(fn, K, bits, 0, x_dtype)) return st;
  if (M > 1)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: M=%lld, the TL2 decode takes one token", fn,
                (long long)M);
  if (K > bitnet::kTl2MaxK)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld exceeds %d", fn, (long long)K,
                bitnet::kTl2MaxK);
  if (M == 0 || N == 0) return ok();
  if (!x || !Wtl2 || !alpha || !y) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(x, 16) || !aligned(Wtl2, 16) || !aligned(y, 4) || !aligned(alpha, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  return hip_status(bitnet::launch_tl2_decode(x, (int)x_dtype, (int)K, Wtl2, N, alpha, bits, y,
                                              stream),
                    fn);
}

size_t bitnet_tl2_forward_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 64 != 0 || M > bitnet::kDecodeMaxM) return 0;
  if (M == 1 && K <= bitnet::kTl2MaxK) return 0;  // the single-token kernel
  return round_up((size_t)M * (size_t)bitnet::tl2_code_row(K)) + 2 * round_up((size_t)M * 4);
}

bitnet_status bitnet_hbitlinear_forward_tl2_batched(const void* x, bitnet_dtype x_dtype,
                                                    int64_t M, int64_t K, const uint8_t* Wtl2,
                                                    int64_t N, const float* alpha, int bits,
                                                    float* y, void* ws, size_t ws_bytes,
                                                    hipStream_t stream) {
  const char* fn = "bitnet_hbitlinear_forward_tl2_batched";
  if (bitnet_status st = check_dims(fn, M, K, N)) return st;
  if (bitnet_status st = check_quant_args(fn, K, bits, 0, x_dtype)) return st;
  if (M > bitnet::kDecodeMaxM)
    return fail(BITNET_ERR_UNSUPPORTED, "%s: M=%lld, the TL2 product takes at most %lld tokens",
                fn, (long long)M, (long long)bitnet::kDecodeMaxM);
  if (M == 0 || N == 0) return ok();
  if (!x || !Wtl2 || !alpha || !y) return fail(BITNET_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  const size_t need = bitnet_tl2_forward_workspace_bytes(M, K);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(BITNET_ERR_INVALID_ARG, "%s: workspace %zu B < required %zu B", fn,
                ws ? ws_bytes : (size_t)0, need);
  if (!aligned(x, 16) || !aligned(Wtl2, 16) || (need > 0 && !aligned(ws, 16)) || !aligned(y, 4) ||
      !aligned(alpha, 4))
    return fail(BITNET_ERR_ALIGN, "%s: misaligned pointer", fn);
  if (bitnet_status st = launch_guard(fn)) return st;
  if (need == 0)
    return hip_status(bitnet::launch_tl2_decode(x, (int)x_dtype, (int)K, Wtl2, N, alpha, bits, y,
                                                stream),
                      fn);
  char* base = static_cast<char*>(ws);
  int8_t* codes = reinterpret_cast<int8_t*>(base);
  const size_t cbytes = round_up((size_t)M * (size_t)bitnet::tl2_code_row(K));
  float* scales = reinterpret_cast<float*>(base + cbytes);
  int32_t* rowsum = reinterpret_cast<int32_t*>(base + cbytes + round_up((size_t)M * 4));
  hipError_t e = bitnet::launch_quantize_tl2_order(x, (int)x_dtype, M, (int)K, bits, codes, scales,
                                                   rowsum, stream);
  if (e != hipSuccess) return hip_status(e, fn);
  return hip_status(bitnet::launch_tl2_gemv(codes, scales, rowsum, M, (int)K, Wtl2, N, alpha, bits,
                                            y, stream),
                    fn);
}

}  // extern "C"
