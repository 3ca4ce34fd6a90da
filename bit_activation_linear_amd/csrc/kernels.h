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

// Fused (optional) Walsh-Hadamard transform + per-token quantization.
// x_dtype: 0 = fp32, 1 = bf16 bit patterns.
hipError_t launch_quantize(const void* x, int x_dtype, int64_t M, int K, int bits, int hadamard,
                           int8_t* codes, float* scales, hipStream_t stream);

// Ternary product. Exactly one of y (dequantized, needs scales/alpha/bits) or
// acc (raw int32) is non-null.
hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream);

}  // namespace bitnet
