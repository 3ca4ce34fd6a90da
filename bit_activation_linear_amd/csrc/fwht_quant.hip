// Fused online Walsh-Hadamard transform + per-token activation quantization.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py):
//   - fast_hadamard_transform / Eq. 3-4: the orthonormal Sylvester transform,
//     log2 K stages of (u, v) -> ((u + v)/sqrt2, (u - v)/sqrt2).
//   - quantize_act_int8 / Eq. 5: s = max|x| + eps, q = RoundClip(127 x / s, -128, 127).
//   - quantize_act_int4 / Eq. 6: s = mean|x| + eps, q = RoundClip(sqrt7 x / s, -8, 7).
//
// One workgroup per token row. The row is widened to fp32 and staged in LDS
// (K <= 32768 floats fits the 160 KiB of one CU); it is never rounded to a
// narrower type and never written back to HBM. The transform's stages commute
// (H_K is a Kronecker product of H_2 factors), so they are grouped into passes
// of up to five index bits: each thread pulls a group of 2^nb elements that
// differ only in those bits into registers, runs the nb butterfly stages
// there, and writes them back. The 1/sqrt2 of each stage is folded into one
// multiplier applied with the quantization scale.
//
// LDS layout: element i lives at float index i + i/32 (one pad word per 32),
// which keeps both the unit-stride and the 32-stride passes free of bank
// conflicts.
#include "kernels.h"

#include <cmath>

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr float kEps = 1e-7f;

__device__ __forceinline__ int pad_idx(int i) { return i + (i >> 5); }

template <typename XT>
struct Loader;

template <>
struct Loader<float> {
  // 8 consecutive elements.
  __device__ static void load8(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <>
struct Loader<uint16_t> {
  // 8 consecutive bf16 values: widening is a 16-bit left shift.
  __device__ static void load8(const uint16_t* p, float (&v)[8]) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0];
    const unsigned w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// One pass of NB butterfly stages over index bits [b0, b0 + NB).
template <int NB>
__device__ void fwht_pass(float* lds, int K, int b0) {
  constexpr int R = 1 << NB;
  const int groups = K >> NB;
  const int lo_mask = (1 << b0) - 1;
  for (int g = threadIdx.x; g < groups; g += kThreads) {
    const int base = (g & lo_mask) | ((g >> b0) << (b0 + NB));
    float v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) v[i] = lds[pad_idx(base + (i << b0))];
#pragma unroll
    for (int h = 1; h < R; h <<= 1) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        if ((i & h) == 0) {
          const float a = v[i], b = v[i + h];
          v[i] = a + b;
          v[i + h] = a - b;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i) lds[pad_idx(base + (i << b0))] = v[i];
  }
}

__device__ inline float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename XT, int BITS, bool HAD>
__global__ __launch_bounds__(kThreads) void fwht_quant_kernel(const XT* __restrict__ x, int K,
                                                              int logK, int8_t* __restrict__ codes,
                                                              float* __restrict__ scales) {
  extern __shared__ float lds[];
  __shared__ float red[4];
  const int row = blockIdx.x;
  const XT* xr = x + (size_t)row * (size_t)K;

  // 1. HBM -> fp32 LDS, 16-B (bf16) or 2x16-B (fp32) loads per thread.
  for (int base = threadIdx.x * 8; base < K; base += kThreads * 8) {
    float v[8];
    Loader<XT>::load8(xr + base, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) lds[pad_idx(base + e)] = v[e];
  }
  __syncthreads();

  // 2. Unnormalized butterflies, five index bits per pass.
  float norm = 1.0f;
  if (HAD) {
    for (int b0 = 0; b0 < logK; b0 += 5) {
      const int nb = min(5, logK - b0);
      switch (nb) {
        case 1: fwht_pass<1>(lds, K, b0); break;
        case 2: fwht_pass<2>(lds, K, b0); break;
        case 3: fwht_pass<3>(lds, K, b0); break;
        case 4: fwht_pass<4>(lds, K, b0); break;
        default: fwht_pass<5>(lds, K, b0); break;
      }
      __syncthreads();
    }
    // prod of logK factors 1/sqrt2 = 2^(-logK/2).
    norm = ldexpf(1.0f, -(logK >> 1));
    if (logK & 1) norm *= 0.70710678118654752f;
  }

  // 3. Per-token statistic on the transformed row (fixed-order reduction).
  const int K4 = K >> 2;
  float stat = 0.0f;
  for (int i4 = threadIdx.x; i4 < K4; i4 += kThreads) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = fabsf(lds[pad_idx(4 * i4 + e)]);
      stat = (BITS == 8) ? fmaxf(stat, a) : stat + a;
    }
  }
  stat = (BITS == 8) ? wave_max(stat) : wave_sum(stat);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = stat;
  __syncthreads();
  if (BITS == 8) {
    stat = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  } else {
    stat = ((red[0] + red[1]) + (red[2] + red[3])) / (float)K;
  }
  // s is the scale of the normalized row: stat(H x) = norm * stat(unnormalized).
  const float s = stat * norm + kEps;
  const float c = (BITS == 8) ? 127.0f : 2.6457513110645906f;
  const float mult = (c * norm) / s;
  const float lo = (BITS == 8) ? -128.0f : -8.0f;
  const float hi = (BITS == 8) ? 127.0f : 7.0f;
  if (threadIdx.x == 0) scales[row] = s;

  // 4. Quantize with round-half-even and store four codes per thread.
  int8_t* cr = codes + (size_t)row * (size_t)K;
  for (int i4 = threadIdx.x; i4 < K4; i4 += kThreads) {
    unsigned word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float q = __builtin_rintf(lds[pad_idx(4 * i4 + e)] * mult);
      q = fminf(fmaxf(q, lo), hi);
      word |= ((unsigned)(int)q & 0xFFu) << (8 * e);
    }
    reinterpret_cast<unsigned*>(cr)[i4] = word;
  }
}

template <typename XT, int BITS, bool HAD>
hipError_t launch_one(const void* x, int64_t M, int K, int logK, int8_t* codes, float* scales,
                      hipStream_t stream) {
  const size_t lds_bytes = (size_t)(K + K / 32) * sizeof(float);
  auto kern = fwht_quant_kernel<XT, BITS, HAD>;
  if (lds_bytes > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds_bytes);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)M), dim3(kThreads), lds_bytes, stream>>>(
      reinterpret_cast<const XT*>(x), K, logK, codes, scales);
  return hipGetLastError();
}

template <typename XT>
hipError_t launch_dtype(const void* x, int64_t M, int K, int logK, int bits, int hadamard,
                        int8_t* codes, float* scales, hipStream_t stream) {
  if (bits == 8) {
    return hadamard ? launch_one<XT, 8, true>(x, M, K, logK, codes, scales, stream)
                    : launch_one<XT, 8, false>(x, M, K, logK, codes, scales, stream);
  }
  return hadamard ? launch_one<XT, 4, true>(x, M, K, logK, codes, scales, stream)
                  : launch_one<XT, 4, false>(x, M, K, logK, codes, scales, stream);
}

}  // namespace

hipError_t launch_quantize(const void* x, int x_dtype, int64_t M, int K, int bits, int hadamard,
                           int8_t* codes, float* scales, hipStream_t stream) {
  int logK = 0;
  while ((1 << logK) < K) ++logK;
  if (x_dtype == 1)
    return launch_dtype<uint16_t>(x, M, K, logK, bits, hadamard, codes, scales, stream);
  return launch_dtype<float>(x, M, K, logK, bits, hadamard, codes, scales, stream);
}

}  // namespace bitnet
