// Low-bit KV-cache quantizer.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), module docstring item 5
// (Section 3.1, Tables 2 and 3) and BitNetV2Attention._quantize_kv_head:
// post-RoPE keys and values [B, H, S, D] are quantized per token along the
// head dimension D; token 0 of every head (BOS) keeps the 8-bit absmax
// quantizer (Eq. 5), the others use
//   bits 8: s = max|x| + eps,   q = RoundClip(127 x / s, -128, 127)
//   bits 4: s = mean|x| + eps,  q = RoundClip(sqrt7 x / s, -8, 7)     (Eq. 6)
//   bits 3: s = max|x| + eps,   q = RoundClip(3 x / s, -4, 3)
// and x is recovered as q * s / c.
//
// The pass is bound by HBM (2 or 4 bytes read, 1 byte written per element,
// plus 4 bytes per token). A row of D elements is split over G = D / 8 lanes
// (rounded up to a power of two), each holding one 16-byte (bf16) or two
// 16-byte (fp32) loads, so a wave covers 64 / G tokens and every per-token
// statistic is a butterfly over G lanes of one wave: no LDS, no barrier.
//
// Packed output (PACK, bits 3 and 4): the codes of the non-BOS tokens are
// stored b bits apiece, one little-endian bit stream per token row (code k at
// stream bits b k .. b k + b - 1, two's complement), so the cache holds
// b / 8 bytes per element: a lane's eight codes are one 32-bit word at 4 bits
// and 24 bits at 3 bits, of which four neighbouring lanes make three words.
// BOS rows keep their int8 codes in a separate [R / S, D] array (their slot
// of the packed array is zeroed).
#include "kernels.h"

namespace bitnet {
namespace {

constexpr float kEps = 1e-7f;

__device__ __forceinline__ void load8v(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8v(const uint16_t* p, float* v) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const unsigned w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One token row per group of G lanes; lane j of a group owns elements
// 8j .. 8j+7 (j < D / 8).
template <typename XT, int BITS, int G, bool PACK>
__global__ __launch_bounds__(256) void kv_quant_kernel(const XT* __restrict__ kv, int64_t R, int D,
                                                       int S, int8_t* __restrict__ codes,
                                                       float* __restrict__ scales,
                                                       uint8_t* __restrict__ packed) {
  constexpr int kRowsPerBlock = 256 / G;
  const int t = threadIdx.x;
  const int j = t % G;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + t / G;
  const bool row_ok = row < R;
  const int64_t rc = row_ok ? row : R - 1;
  const bool own = j * 8 < D;
  const int jc = own ? j : 0;
  float v[8];
  load8v(kv + rc * D + 8 * jc, v);

  const bool bos = (rc % S) == 0;
  float st_max = 0.0f, st_sum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    st_max = fmaxf(st_max, fabsf(v[e]));
    st_sum += fabsf(v[e]);
  }
  st_max = group_max<G>(own ? st_max : 0.0f);
  st_sum = group_sum<G>(own ? st_sum : 0.0f);
  // BOS tokens, and every token at 8 bits, use absmax with c = 127.
  float c, lo, hi, st;
  if (bos || BITS == 8) {
    c = 127.0f; lo = -128.0f; hi = 127.0f; st = st_max;
  } else if (BITS == 4) {
    c = 2.6457513110645906f; lo = -8.0f; hi = 7.0f; st = st_sum / (float)D;
  } else {
    c = 3.0f; lo = -4.0f; hi = 3.0f; st = st_max;
  }
  const float s = st + kEps;
  const float mult = c / s;
  int q[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q[e] = (int)fminf(fmaxf(__builtin_rintf(v[e] * mult), lo), hi);
  if (row_ok && j == 0) scales[row] = s;
  unsigned w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e >> 2] |= ((unsigned)q[e] & 0xFFu) << (8 * (e & 3));
  if constexpr (!PACK) {
    if (row_ok && own) *reinterpret_cast<uint2*>(codes + row * D + 8 * j) = make_uint2(w[0], w[1]);
  } else {
    // BOS rows: int8 codes into the BOS array, zeros in the packed slot
    if (row_ok && own && bos)
      *reinterpret_cast<uint2*>(codes + (row / S) * D + 8 * j) = make_uint2(w[0], w[1]);
    unsigned f = 0u;  // the lane's eight b-bit fields, code e at bits b e
#pragma unroll
    for (int e = 0; e < 8; ++e) f |= ((unsigned)q[e] & ((1u << BITS) - 1u)) << (BITS * e);
    if (bos) f = 0u;
    if constexpr (BITS == 4) {
      if (row_ok && own) *reinterpret_cast<unsigned*>(packed + row * (D / 2) + 4 * j) = f;
    } else {
      // lanes 4a .. 4a+3 hold 96 stream bits: lane 4a + b (b < 3) stores
      // word b, the low bits of its own field shifted down and its right
      // neighbour's shifted up
      const unsigned nxt = (unsigned)__shfl_down((int)f, 1, 64);
      const int b = j & 3;
      const unsigned word = (f >> (8 * b)) | (nxt << (24 - 8 * b));
      if (row_ok && own && b < 3)
        *reinterpret_cast<unsigned*>(packed + row * (3 * D / 8) + 12 * (j >> 2) + 4 * b) = word;
    }
  }
}

template <typename XT, int BITS, int G, bool PACK>
hipError_t launch_kv_g(const void* kv, int64_t R, int D, int S, int8_t* codes, float* scales,
                       uint8_t* packed, hipStream_t stream) {
  constexpr int kRowsPerBlock = 256 / G;
  const int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  kv_quant_kernel<XT, BITS, G, PACK><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      reinterpret_cast<const XT*>(kv), R, D, S, codes, scales, packed);
  return hipGetLastError();
}

template <typename XT, int BITS, bool PACK>
hipError_t launch_kv_bits(const void* kv, int64_t R, int D, int S, int8_t* codes, float* scales,
                          uint8_t* packed, hipStream_t stream) {
  const int lanes = D / 8;
  if (lanes <= 1) return launch_kv_g<XT, BITS, 1, PACK>(kv, R, D, S, codes, scales, packed, stream);
  if (lanes <= 2) return launch_kv_g<XT, BITS, 2, PACK>(kv, R, D, S, codes, scales, packed, stream);
  if (lanes <= 4) return launch_kv_g<XT, BITS, 4, PACK>(kv, R, D, S, codes, scales, packed, stream);
  if (lanes <= 8) return launch_kv_g<XT, BITS, 8, PACK>(kv, R, D, S, codes, scales, packed, stream);
  if (lanes <= 16) return launch_kv_g<XT, BITS, 16, PACK>(kv, R, D, S, codes, scales, packed, stream);
  if (lanes <= 32) return launch_kv_g<XT, BITS, 32, PACK>(kv, R, D, S, codes, scales, packed, stream);
  return launch_kv_g<XT, BITS, 64, PACK>(kv, R, D, S, codes, scales, packed, stream);
}

template <typename XT>
hipError_t launch_kv_dtype(const void* kv, int64_t R, int D, int S, int bits, int8_t* codes,
                           float* scales, uint8_t* packed, hipStream_t stream) {
  if (packed) {
    if (bits == 3) return launch_kv_bits<XT, 3, true>(kv, R, D, S, codes, scales, packed, stream);
    if (bits == 4) return launch_kv_bits<XT, 4, true>(kv, R, D, S, codes, scales, packed, stream);
    return hipErrorInvalidValue;
  }
  if (bits == 3) return launch_kv_bits<XT, 3, false>(kv, R, D, S, codes, scales, nullptr, stream);
  if (bits == 4) return launch_kv_bits<XT, 4, false>(kv, R, D, S, codes, scales, nullptr, stream);
  return launch_kv_bits<XT, 8, false>(kv, R, D, S, codes, scales, nullptr, stream);
}

}  // namespace

hipError_t launch_kv_quantize(const void* kv, int x_dtype, int64_t R, int D, int S, int bits,
                              int8_t* codes, float* scales, hipStream_t stream, uint8_t* packed) {
  if (x_dtype == 1) return launch_kv_dtype<uint16_t>(kv, R, D, S, bits, codes, scales, packed, stream);
  return launch_kv_dtype<float>(kv, R, D, S, bits, codes, scales, packed, stream);
}

}  // namespace bitnet
